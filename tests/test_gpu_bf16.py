"""bf16 activations on the W8A8_INT8 path (mq_quant_per_token_int8_bf16,
mq_w8a8_scaled_mm_bf16, mq_w8a8_linear_bf16) on an MI355X.

Codes and scales are bit-exact against the oracle's quantizer applied to the
bf16 values (bf16 widens exactly to binary32). The bf16 output is checked
element by element against the unrounded float64 oracle with the bound the
arithmetic gives: three binary32 roundings (under 2^-22 relative together)
and one round-to-nearest-even to bf16 (at most 2^-8 relative), so
|y - y64| <= (2^-8 + 2^-20) |y64|. The fused and two-kernel layers must be
bit-identical to the quantizer followed by the scaled GEMM."""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, host

pytestmark = pytest.mark.gpu

BF16_REL_BOUND = 2.0 ** -8 + 2.0 ** -20


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bf16_host(t):
    import torch
    torch.cuda.synchronize()
    return synth.bf16_values(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check_bf16_output(y, y64, what):
    y64 = np.asarray(y64, dtype=np.float64)
    err = np.abs(y.astype(np.float64) - y64)
    bad = err > BF16_REL_BOUND * np.abs(y64)
    assert not np.any(bad), f"{what}: {int(bad.sum())} outputs beyond 2^-8 relative, first {np.argwhere(bad)[:3]}"
    rel = np.linalg.norm(y.astype(np.float64) - y64) / max(np.linalg.norm(y64), 1e-300)
    print(f"{what}: rel_fro={rel:.2e} max_rel={np.max(err / np.maximum(np.abs(y64), 1e-300)):.2e}")


@pytest.mark.parametrize("MK", [(2048, 4096), (37, 80), (5, 20000), (1, 16)], ids=["c2", "ragged", "stream", "tiny"])
def test_quant_bf16_bitexact(MK):
    M, K = MK
    d = synth.w8a8_inputs_bf16(M, K, 16, outlier_frac=0.01, tag=900 + M)
    announce(f"quant bf16 M={M} K={K}")
    xq, s = mq.quant_per_token_int8(_bf16_dev(d["x_bits"]))
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(d["x"])
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


def test_quant_bf16_edge_rows():
    # exact ties (absmax 127 gives scale 1 exactly; k + 1/2 is exact in bf16),
    # an all-zero row, signed zeros, large and tiny magnitudes
    K = 128
    ties = np.concatenate([[127.0], np.arange(63) + 0.5, -(np.arange(64) + 0.5)]).astype(np.float32)
    rows = [ties, np.zeros(K, np.float32), np.resize(np.array([-0.0, 0.0], np.float32), K),
            np.resize(np.array([3.0e38, -1.0, 2.0 ** -120], np.float32), K),
            np.resize(np.array([2.0 ** -126, -(2.0 ** -125)], np.float32), K)]
    bits = synth.bf16_bits(np.array(rows, np.float32))
    x = synth.bf16_values(bits)
    announce("quant bf16 edge rows")
    xq, s = mq.quant_per_token_int8(_bf16_dev(bits))
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(x)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert host(xq)[0, 1:64].tolist() == [k + (k % 2) for k in range(63)]  # k + 1/2 -> even
    # the one-token fused layer (a layer wide enough for it) quantizes the
    # same rows inside its kernel
    import torch
    rng = np.random.default_rng(3)
    wq = _dev(rng.integers(-127, 128, size=(16384, K)).astype(np.int8))
    s_ch = _dev(rng.uniform(0.001, 0.01, 16384).astype(np.float32))
    xd = _bf16_dev(bits)
    for r in range(len(rows)):
        y1 = mq.w8a8_linear(xd[r:r + 1].contiguous(), wq, s_ch)
        q1, s1 = mq.quant_per_token_int8(xd[r:r + 1].contiguous())
        y2 = mq.w8a8_scaled_mm(q1, s1, wq, s_ch, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"fused layer, edge row {r}"


@pytest.mark.parametrize("MNK", [(8, 4096, 4096), (48, 640, 1024), (300, 640, 1024), (2048, 4096, 4096)],
                         ids=["decode", "gemv64", "tiled", "c2"])
def test_scaled_mm_bf16(MNK):
    M, N, K = MNK
    d = synth.w8a8_inputs_bf16(M, K, N, outlier_frac=0.01, tag=910 + M)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(d["x"])
    announce(f"scaled_mm bf16 M={M} N={N} K={K}")
    import torch
    y = mq.w8a8_scaled_mm(_dev(xq_ref), _dev(s_ref), _dev(wq), _dev(s_ch), out_dtype=torch.bfloat16)
    assert y.dtype == torch.bfloat16
    yh = _bf16_host(y)
    rows = np.arange(M) if M <= 300 else np.random.default_rng(M).choice(M, size=96, replace=False)
    y64 = oracle.w8a8_ref(xq_ref[rows], s_ref[rows], wq, s_ch)
    _check_bf16_output(yh[rows], y64, f"scaled_mm bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 4, 32, 300])
def test_linear_bf16_matches_two_calls_and_oracle(M):
    import torch
    N, K = 1024, 2048
    d = synth.w8a8_inputs_bf16(M, K, N, outlier_frac=0.01, tag=920 + M)
    wq_np, s_ch_np = oracle.quant_per_token_int8_ref(d["wf"])
    x = _bf16_dev(d["x_bits"])
    wq, s_ch = _dev(wq_np), _dev(s_ch_np)
    announce(f"w8a8_linear bf16 M={M}")
    y = mq.w8a8_linear(x, wq, s_ch)
    assert y.dtype == torch.bfloat16
    xq, s = mq.quant_per_token_int8(x)
    y2 = mq.w8a8_scaled_mm(xq, s, wq, s_ch, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "linear differs from quantize + scaled GEMM"
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(d["x"])
    _check_bf16_output(_bf16_host(y), oracle.w8a8_ref(xq_ref, s_ref, wq_np, s_ch_np), f"w8a8_linear bf16 M={M}")


def test_bf16_and_fp16_outputs_share_the_epilogue():
    # the same codes and scales through both output types: each output is the
    # nearest value of its type to one binary32 epilogue result, so the bf16
    # output is within half a bf16 ulp of the fp16 output's value (up to the
    # fp16 rounding)
    import torch
    M, N, K = 64, 2048, 1024
    d = synth.w8a8_inputs_bf16(M, K, N, outlier_frac=0.01, tag=930)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    xq, s = oracle.quant_per_token_int8_ref(d["x"])
    args = (_dev(xq), _dev(s), _dev(wq), _dev(s_ch))
    announce("bf16 vs fp16 epilogue")
    y16 = host(mq.w8a8_scaled_mm(*args)).astype(np.float64)
    yb = _bf16_host(mq.w8a8_scaled_mm(*args, out_dtype=torch.bfloat16)).astype(np.float64)
    assert np.all(np.abs(yb - y16) <= 2.0 ** -8 * np.abs(yb) + 2.0 ** -11 * np.abs(y16) + 2.0 ** -24)
