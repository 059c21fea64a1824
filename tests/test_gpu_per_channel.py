"""W4A16 with per-channel parameters (group -1) against the CPU oracle on an MI355X.

LMDeploy 4-bit deployment guide, section 3.2: a layer's quantization config
gives its bits and group size, -1 meaning no grouping -- one scale and one
zero point per output column over all of K. scales is [1, N] and qzeros
[1, N/8]; y[m,n] = sum_k x[m,k] * (q[k,n] - z[n]) * s[n]. The kernels run
such a layer as groups of 128 rows that all read the one parameter row.

1. Dense layers at decode and prefill shapes (the 8B layers, ragged M and N,
   long K) for the GEMM, both GEMVs and the linear-layer entry, at the
   usual fp16 tolerance (relative Frobenius <= 1e-3, max-abs <= 5e-2 against
   the unrounded float64 oracle) and, with bf16 activations, the element-wise
   bound of the bf16 tests.
2. One-hot rows: every output is one weight; the GEMM and the decode-layout
   GEMV at 17-64 tokens round it once to fp16, the others apply s in
   binary32 and round the output once, so all must equal fp16((q - z) * s)
   of the oracle bit for bit. A kernel that reads the parameters of any row
   other than row 0 would differ (and read past the [1, N] buffers).
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


def _blocked(x, qweight, scales, qzeros, group):
    return mq.w4a16_gemv_blocked(x, mq.w4a16_block_weights(qweight), scales, qzeros, group)


KERNELS = {"gemm": mq.w4a16_gemm, "gemv": mq.w4a16_gemv, "gemv_blocked": _blocked}


def _run(name, d, what):
    announce(f"per-channel {name} {what} M={d['x'].shape[0]} K={d['x'].shape[1]} N={d['scales'].shape[1]}")
    return host(KERNELS[name](dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), -1))


def _ref(d):
    return oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], -1)


@pytest.mark.parametrize("name,M,K,N", [
    ("gemm", 4, 512, 512), ("gemm", 300, 1024, 1032), ("gemm", 2048, 4096, 4096), ("gemm", 577, 1024, 3072),
    ("gemm", 100, 12288, 264),
    ("gemv", 1, 4096, 24576), ("gemv", 4, 4096, 6144), ("gemv", 16, 4096, 4096), ("gemv", 40, 4096, 4096),
    ("gemv", 3, 384, 424), ("gemv", 2, 12288, 4096),
    ("gemv_blocked", 1, 4096, 24576), ("gemv_blocked", 4, 4096, 6144), ("gemv_blocked", 8, 4096, 4096),
    ("gemv_blocked", 16, 4096, 24576), ("gemv_blocked", 48, 4096, 6144), ("gemv_blocked", 64, 12288, 4096),
    ("gemv_blocked", 1, 12288, 4096), ("gemv_blocked", 5, 1024, 3072)])
def test_per_channel_dense(name, M, K, N):
    d = synth.w4a16_inputs(M, K, N, -1, outlier_frac=0.005 if M <= 64 else 0.0, tag=980 + M + N)
    assert d["scales"].shape == (1, N) and d["qzeros"].shape == (1, N // 8)
    assert_fp16_close(_run(name, d, "dense"), _ref(d), f"per-channel {name} M={M} K={K} N={N}")


@pytest.mark.parametrize("name,M", [("gemm", 256), ("gemv", 64), ("gemv", 16), ("gemv_blocked", 16),
                                    ("gemv_blocked", 64)])
def test_per_channel_onehot(name, M):
    K, N = 512, 512
    w = synth.w4a16_weights(K, N, -1, tag=990, scale_log2=(-16, 8))
    want = oracle.dequant_w4(w["qweight"], w["scales"], w["qzeros"], -1).astype(np.float16)
    rows = []
    for c in range(K // M):
        x = np.zeros((M, K), np.float16)
        x[np.arange(M), M * c + np.arange(M)] = 1.0
        rows.append(_run(name, dict(w, x=x), f"one-hot rows {M * c}.."))
    got = np.concatenate(rows, 0)
    bad = np.argwhere(got.astype(np.float64) != want.astype(np.float64))
    assert bad.size == 0, (f"{name}: {len(bad)} weights differ from fp16((q - z) * s), first "
                           f"{[(int(k), int(n), float(got[k, n]), float(want[k, n])) for k, n in bad[:3]]}")


@pytest.mark.parametrize("M", [1, 8, 64, 300])
def test_per_channel_linear(M):
    # the model-facing entry: decode layout up to 64 tokens, GEMM beyond
    K, N = 4096, 6144
    d = synth.w4a16_inputs(M, K, N, -1, outlier_frac=0.005 if M <= 64 else 0.0, tag=995 + M)
    qw = dev(d["qweight"])
    qb = mq.w4a16_block_weights(qw)
    announce(f"per-channel w4a16_linear M={M}")
    y = host(mq.w4a16_linear(dev(d["x"]), qw, dev(d["scales"]), dev(d["qzeros"]), -1, qweight_blocked=qb))
    assert_fp16_close(y, _ref(d), f"per-channel linear M={M}")


@pytest.mark.parametrize("name,M,K,N", [("gemm", 300, 1024, 1032), ("gemv", 16, 4096, 4096),
                                        ("gemv_blocked", 8, 4096, 6144), ("gemv_blocked", 48, 4096, 4096)])
def test_per_channel_bf16(name, M, K, N):
    import torch
    d = synth.w4a16_inputs_bf16(M, K, N, -1, outlier_frac=0.005 if M <= 64 else 0.0, tag=1000 + M)
    x = dev(np.ascontiguousarray(d["x_bits"]).view(np.int16)).view(torch.bfloat16)
    announce(f"per-channel bf16 {name} M={M} K={K} N={N}")
    y = KERNELS[name](x, dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), -1)
    assert y.dtype == torch.bfloat16
    got = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], -1)
    # element-wise bound of the bf16 forms (as in the bf16 W4A16 tests):
    # bf16 output rounding plus the weight rounding (GEMM, decode layout past
    # 32 tokens) or the binary32 accumulation of 128 + q fragments (others)
    w = oracle.dequant_w4(d["qweight"], d["scales"], d["qzeros"], -1).astype(np.float64)
    ax = np.abs(d["x"].astype(np.float64))
    if name == "gemm" or (name == "gemv_blocked" and M > 16):
        slack = (2.0 ** -8 + K * 2.0 ** -24) * (ax @ np.abs(w)) * (1 + 2.0 ** -7)
    else:
        slack = 2.0 ** -15 * 143 * (ax.sum(1, keepdims=True) * np.abs(d["scales"].astype(np.float64)))
    bound = 2.0 ** -8 * np.abs(ref) + slack
    worst = np.max(np.abs(got - ref) / bound)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"per-channel bf16 {name}: rel_fro={rel:.3e} max err/bound={worst:.3f}")
    assert worst <= 1.0 and rel <= 5e-3, (worst, rel)


def test_per_channel_graph_replay():
    import torch
    M, K, N = 4, 4096, 4096
    d = synth.w4a16_inputs(M, K, N, -1, outlier_frac=0.005, tag=1010)
    x, qb = dev(d["x"]), mq.w4a16_block_weights(dev(d["qweight"]))
    sc, qz = dev(d["scales"]), dev(d["qzeros"])
    announce("per-channel decode-layout GEMV graph replay")
    y0 = host(mq.w4a16_gemv_blocked(x, qb, sc, qz, -1))
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = torch.zeros(max(mq.w4a16_gemv_blocked_workspace_bytes(M, N, K, -1), 16), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.w4a16_gemv_blocked(x, qb, sc, qz, -1, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.w4a16_gemv_blocked(x, qb, sc, qz, -1, out=out, workspace=ws)
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), y0), f"replay {r} differs from the eager call"
    assert_fp16_close(y0, _ref(d), "per-channel graph")
