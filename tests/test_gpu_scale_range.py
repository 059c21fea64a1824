"""W4A16 over the whole fp16 scale range on an MI355X, against the CPU oracle.

LMDeploy toolkit overview, section 2.5 (AWQ group scales) and LMDeploy 4-bit
deployment guide, section 2.2 (the scale is applied inside the matmul
kernel). Real checkpoints hold scales far outside the [0.005, 0.02] of the
benchmark workloads, so the kernels are checked over all of fp16:

1. One-hot activations isolate single weights. With x = I (the GEMM) or rows
   that each select one input channel (the GEMVs), every output is one
   dequantized weight: the GEMM rounds it once, fp16((q - z) * s); the GEMVs
   keep q - z exact and apply s in binary32, then round the output once. Both
   must therefore equal the oracle's exact weight rounded to fp16, bit for bit
   (zeros compared by value). Scales are log-uniform over [2^-24, 2^12] with
   random signs, so products reach fp16 subnormals and 15 * 4096 < 65504.
2. Dense layers with scales log-uniform over [2^-16, 2^-8], and a mixed-range
   case over [2^-20, 2^-4], at the usual tolerance (relative Frobenius error
   <= 1e-3, max-abs error <= 5e-2 against the unrounded float64 oracle).
3. Scales below the fp16 normal range, [2^-24, 2^-14], on the GEMVs, whose
   weights never pass through fp16.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


def _gemv_blocked(x, qweight, scales, qzeros, group):
    return mq.w4a16_gemv_blocked(x, mq.w4a16_block_weights(qweight), scales, qzeros, group)


KERNELS = {"gemm": mq.w4a16_gemm, "gemv": mq.w4a16_gemv, "gemv_blocked": _gemv_blocked}


def _full_range_weights(K, N, G, tag):
    w = synth.w4a16_weights(K, N, G, tag=tag, scale_log2=(-24, 12))
    rng = np.random.default_rng(tag)
    sign = np.where(rng.integers(0, 2, size=w["scales"].shape) == 1, -1, 1).astype(np.float16)
    w["scales"] = (w["scales"] * sign).astype(np.float16)
    return w


def _run(name, x, w, G, what):
    announce(f"{name} G={G} {what} M={x.shape[0]} K={x.shape[1]} N={w['scales'].shape[1]}")
    fn = KERNELS[name]
    return host(fn(dev(x), dev(w["qweight"]), dev(w["scales"]), dev(w["qzeros"]), G))


@pytest.mark.parametrize("G", [128, 64, 32])
@pytest.mark.parametrize("name", ["gemm", "gemv", "gemv_blocked"])
def test_onehot_weights_rounded_once(name, G):
    K, N = 512, 512
    w = _full_range_weights(K, N, G, tag=900 + G)
    want = oracle.dequant_w4(w["qweight"], w["scales"], w["qzeros"], G).astype(np.float16)
    assert np.all(np.isfinite(want.astype(np.float64)))
    if name == "gemm":
        got = _run(name, np.eye(K, dtype=np.float16), w, G, "x = I")
    else:
        # 64 one-hot rows per call (the GEMVs take up to 64 tokens), all K rows covered
        rows = []
        for c in range(K // 64):
            x = np.zeros((64, K), np.float16)
            x[np.arange(64), 64 * c + np.arange(64)] = 1.0
            rows.append(_run(name, x, w, G, f"one-hot rows {64 * c}..{64 * c + 63}"))
        got = np.concatenate(rows, 0)
    assert np.all(np.isfinite(got.astype(np.float64))), f"{name}: non-finite output"
    bad = np.argwhere(got.astype(np.float64) != want.astype(np.float64))
    assert bad.size == 0, (f"{name} G={G}: {len(bad)} weights differ from fp16((q - z) * s), first "
                           f"{[(int(k), int(n), float(got[k, n]), float(want[k, n])) for k, n in bad[:3]]}")


@pytest.mark.parametrize("name,M,K,N", [("gemm", 4, 512, 512), ("gemm", 4096, 4096, 4096), ("gemm", 300, 1024, 1032),
                                        ("gemv", 1, 4096, 4096), ("gemv", 4, 4096, 4096), ("gemv", 16, 4096, 4096),
                                        ("gemv", 64, 4096, 4096), ("gemv", 4, 512, 512), ("gemv", 16, 4096, 24576),
                                        ("gemv_blocked", 1, 4096, 4096), ("gemv_blocked", 4, 4096, 4096),
                                        ("gemv_blocked", 16, 4096, 4096), ("gemv_blocked", 64, 4096, 4096),
                                        ("gemv_blocked", 4, 512, 512), ("gemv_blocked", 16, 4096, 24576)])
def test_small_scales_dense(name, M, K, N):
    d = synth.w4a16_inputs(M, K, N, 128, outlier_frac=0.005, tag=910 + M, scale_log2=(-16, -8))
    got = _run(name, d["x"], d, 128, "scales 2^-16..2^-8")
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], 128)
    assert_fp16_close(got, ref, f"{name} small scales M={M} K={K} N={N}")


@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("name,M", [("gemm", 512), ("gemm", 4), ("gemv", 8), ("gemv_blocked", 8),
                                    ("gemv_blocked", 40)])
def test_mixed_range_scales(name, M, G):
    K, N = 4096, 1024
    d = synth.w4a16_inputs(M, K, N, G, outlier_frac=0.0, tag=920 + M + G, scale_log2=(-20, -4))
    got = _run(name, d["x"], d, G, "scales 2^-20..2^-4")
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], G)
    assert_fp16_close(got, ref, f"{name} mixed scales G={G} M={M}")


@pytest.mark.parametrize("name,M", [("gemv", 1), ("gemv", 16), ("gemv_blocked", 1), ("gemv_blocked", 16)])
def test_subnormal_range_scales_gemv(name, M):
    # weights (q - z) * s below 2^-10: the GEMVs apply s in binary32, so the
    # outputs keep full relative precision; x is scaled up by 2^10 (exact) so
    # that |y| sits in the fp16 normal range, well below 64
    K, N = 4096, 4096
    d = synth.w4a16_inputs(M, K, N, 128, outlier_frac=0.0, tag=930 + M, scale_log2=(-24, -14))
    d["x"] = (d["x"].astype(np.float32) * np.float32(1024.0)).astype(np.float16)
    got = _run(name, d["x"], d, 128, "scales 2^-24..2^-14")
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], 128)
    assert_fp16_close(got, ref, f"{name} subnormal-range scales M={M}")
