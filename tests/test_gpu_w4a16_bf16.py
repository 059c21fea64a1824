"""W4A16 with bf16 activations (mq_w4a16_*_bf16) against the CPU oracle on an MI355X.

pymllm Setup and Usage, Overview: BF16 is one of the runtime's schemes beside
W4A16 and W8A8_INT8, so 4-bit layers sit among bf16 activations. The
definition is the fp16 one, y = sum_k x (q - z) s, with x widened exactly from
bf16 (the oracle takes those float32 values) and y rounded to bf16.

1. One-hot activations: every output is one weight rounded once to bf16, in
   every kernel (the GEMM rounds the exact binary32 product (q - z) s to
   bf16 before the MFMA; the GEMVs form it exactly in binary32 and round the
   output), so outputs equal the oracle's exact weights rounded to nearest
   even as bf16, bit for bit.
2. Dense inputs meet the element-wise bound derived from the arithmetic
   (bf16 unit roundoff 2^-8, binary32 2^-24):
     weight-rounding forms (GEMM; 17-64 tokens on the decode layout)
       |y - y64| <= 2^-8 |y64| + (2^-8 + K 2^-24) sum_k |x w| (1 + 2^-7)
     the 128 + q forms (the decode-layout GEMV up to 16 tokens, all
       AWQ-layout GEMVs)
       |y - y64| <= 2^-8 |y64| + 2^-15 * 143 sum_k |x s|
   and, as a statistical check that the bound's slack hides no systematic
   error, relative Frobenius error <= 5e-3 (bf16 rounding of independent
   terms gives about 2e-3).
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits):
    import torch
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _bf16_round(a):
    """float64/float32 values -> float64 of their bf16 rounding (torch CPU: round to nearest even)."""
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


def _values(y):
    import torch
    return y.float().cpu().numpy().astype(np.float64)


def _blocked(x, qweight, scales, qzeros, group):
    return mq.w4a16_gemv_blocked(x, mq.w4a16_block_weights(qweight), scales, qzeros, group)


KERNELS = {"gemm": mq.w4a16_gemm, "gemv": mq.w4a16_gemv, "gemv_blocked": _blocked}


def _run(name, x_bits, d, G, what):
    import torch
    M, K = x_bits.shape
    announce(f"bf16 {name} G={G} {what} M={M} K={K} N={d['scales'].shape[1]}")
    y = KERNELS[name](_bf16_tensor(x_bits), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), G)
    assert y.dtype == torch.bfloat16
    torch.cuda.synchronize()
    return _values(y)


def _rounds_weights(name, M):
    return name == "gemm" or (name == "gemv_blocked" and M > 16)


def _check(name, M, got, x, d, G, what):
    K = x.shape[1]
    ref = oracle.w4a16_ref(x, d["qweight"], d["scales"], d["qzeros"], G)
    w = oracle.dequant_w4(d["qweight"], d["scales"], d["qzeros"], G).astype(np.float64)
    ax = np.abs(x.astype(np.float64))
    if _rounds_weights(name, M):
        slack = (2.0 ** -8 + K * 2.0 ** -24) * (ax @ np.abs(w)) * (1 + 2.0 ** -7)
    else:
        g = np.arange(K) // G
        s_rows = np.abs(d["scales"].astype(np.float64))[g, :]
        slack = 2.0 ** -15 * 143 * (ax @ s_rows)
    bound = 2.0 ** -8 * np.abs(ref) + slack
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = np.max(err / bound)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"bf16 {name} {what}: rel_fro={rel:.3e} max err/bound={worst:.3f}")
    assert worst <= 1.0, f"{what}: element-wise bound exceeded ({worst:.3f}x)"
    assert rel <= 5e-3, f"{what}: rel_fro={rel:.3e}"


@pytest.mark.parametrize("G", [128, 64, 32])
@pytest.mark.parametrize("name,M", [("gemm", 512), ("gemv", 64), ("gemv_blocked", 16), ("gemv_blocked", 64)])
def test_bf16_onehot_weights_rounded_once(name, M, G):
    K, N = 512, 512
    d = synth.w4a16_weights(K, N, G, tag=940 + G, scale_log2=(-16, 8))
    w = oracle.dequant_w4(d["qweight"], d["scales"], d["qzeros"], G)
    want = _bf16_round(w)
    rows = []
    for c in range(K // M):
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), M * c + np.arange(M)] = 1.0
        rows.append(_run(name, synth.bf16_bits(x), d, G, f"one-hot rows {M * c}.."))
    got = np.concatenate(rows, 0)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{name} G={G}: {len(bad)} outputs differ from bf16((q - z) * s), first "
                           f"{[(int(k), int(n), got[k, n], want[k, n]) for k, n in bad[:3]]}")


@pytest.mark.parametrize("name,M,K,N,G", [
    ("gemm", 4, 512, 512, 128), ("gemm", 300, 1024, 1032, 128), ("gemm", 4096, 4096, 4096, 128),
    ("gemm", 2048, 4096, 4096, 128), ("gemm", 577, 1024, 3072, 64), ("gemm", 200, 384, 424, 32),
    ("gemv", 1, 4096, 24576, 128), ("gemv", 4, 4096, 24576, 128), ("gemv", 16, 4096, 24576, 128),
    ("gemv", 40, 4096, 4096, 128), ("gemv", 64, 4096, 6144, 128), ("gemv", 3, 384, 424, 128),
    ("gemv", 17, 384, 424, 64), ("gemv", 5, 2048, 136, 32),
    ("gemv_blocked", 1, 4096, 24576, 128), ("gemv_blocked", 4, 4096, 24576, 128),
    ("gemv_blocked", 16, 4096, 24576, 128), ("gemv_blocked", 8, 12288, 4096, 128),
    ("gemv_blocked", 24, 4096, 6144, 128), ("gemv_blocked", 33, 4096, 4096, 128),
    ("gemv_blocked", 64, 4096, 24576, 128), ("gemv_blocked", 64, 12288, 4096, 128),
    ("gemv_blocked", 1, 1024, 3072, 64), ("gemv_blocked", 48, 1024, 3072, 64), ("gemv_blocked", 16, 1024, 3072, 32)])
def test_bf16_dense(name, M, K, N, G):
    d = synth.w4a16_inputs_bf16(M, K, N, G, outlier_frac=0.005 if M <= 64 else 0.0, tag=950 + M + K + G)
    got = _run(name, d["x_bits"], d, G, "dense")
    _check(name, M, got, d["x"], d, G, f"M={M} K={K} N={N} G={G}")


@pytest.mark.parametrize("name,M", [("gemm", 128), ("gemv", 16), ("gemv_blocked", 16), ("gemv_blocked", 64)])
def test_bf16_scale_range(name, M):
    K, N = 4096, 1024
    d = synth.w4a16_inputs_bf16(M, K, N, 128, tag=960 + M, scale_log2=(-16, -4))
    got = _run(name, d["x_bits"], d, 128, "scales 2^-16..2^-4")
    _check(name, M, got, d["x"], d, 128, f"scale range M={M}")


def test_bf16_linear_and_graph():
    import torch
    d = synth.w4a16_inputs_bf16(8, 4096, 6144, 128, outlier_frac=0.005, tag=970)
    x = _bf16_tensor(d["x_bits"])
    qw, sc, qz = dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"])
    qb = mq.w4a16_block_weights(qw)
    announce("bf16 w4a16_linear decode layout + graph replay")
    y0 = _values(mq.w4a16_linear(x, qw, sc, qz, 128, qweight_blocked=qb))
    _check("gemv_blocked", 8, y0, d["x"], d, 128, "linear")
    out = torch.empty((8, 6144), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(mq.w4a16_gemv_blocked_workspace_bytes(8, 6144, 4096, 128), 16), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.w4a16_gemv_blocked(x, qb, sc, qz, 128, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.w4a16_gemv_blocked(x, qb, sc, qz, 128, out=out, workspace=ws)
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_values(out), y0), f"replay {r} differs from the eager call"
