"""W4A16 with groups of 32 and 64 rows against the CPU oracle on an MI355X.

LMDeploy's 4-bit deployment guide (section 3.2) quantizes the vision tower's
attention projection with groups of 64 input channels while the language
model keeps 128; the kernels are instantiated for G = 32, 64 and 128. Same
tolerance as every fp16 output: relative Frobenius error <= 1e-3 and max-abs
error <= 5e-2 against the unrounded float64 oracle.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


def _case(M, K, N, G, outliers=0.005, tag=0):
    return synth.w4a16_inputs(M, K, N, group=G, outlier_frac=outliers, tag=tag)


def _run(fn, d, G, what):
    announce(f"{fn.__name__} G={G} {what} M={d['x'].shape[0]} K={d['x'].shape[1]} N={d['scales'].shape[1]}")
    return host(fn(dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), G))


def _ref(d, G):
    return oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], G)


# ViT-L-sized attention projection (hidden 1024, fused qkv N = 3072) at
# decode and prefill token counts, then the language-model shapes.
@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("M,K,N", [(1, 1024, 3072), (4, 1024, 3072), (16, 1024, 3072), (64, 1024, 3072),
                                   (1, 4096, 24576), (16, 4096, 24576), (37, 4096, 6144),
                                   (3, 384, 424), (17, 384, 424), (5, 2048, 136), (13, 1024, 1032),
                                   (2, 12288, 4096), (1, 128, 8)])
def test_gemv_groups(M, K, N, G):
    d = _case(M, K, N, G, tag=M + K + N + G)
    assert_fp16_close(_run(mq.w4a16_gemv, d, G, "gemv"), _ref(d, G), f"gemv G={G} M={M} K={K} N={N}")


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("M,K,N", [(256, 1024, 3072), (577, 1024, 3072), (65, 1024, 1024),
                                   (17, 384, 424), (200, 384, 424), (129, 1024, 1032), (1, 128, 8),
                                   (300, 256, 264)])
def test_gemm_groups(M, K, N, G):
    d = _case(M, K, N, G, outliers=0.0, tag=3 * M + K + N + G)
    assert_fp16_close(_run(mq.w4a16_gemm, d, G, "gemm"), _ref(d, G), f"gemm G={G} M={M} K={K} N={N}")


def test_gemm_group64_prefill_o_proj():
    # the 4096 x 4096 x 4096 prefill shape with groups of 64
    d = _case(4096, 4096, 4096, 64, outliers=0.0, tag=64)
    assert_fp16_close(_run(mq.w4a16_gemm, d, 64, "prefill"), _ref(d, 64), "gemm G=64 4096^3")


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("fn,M,N", [(mq.w4a16_gemv, 2, 264), (mq.w4a16_gemv, 5, 256), (mq.w4a16_gemv, 40, 256),
                                    (mq.w4a16_gemm, 100, 264)],
                         ids=["gemv_regs", "gemv_lds", "gemv_lds_3tiles", "gemm"])
def test_groups_long_k(fn, M, N, G):
    # K = 65536: many groups per split; activations scaled by 1/4 (exact) so
    # |y| stays well below 128, where half an fp16 ulp would exceed 5e-2.
    d = _case(M, 65536, N, G, outliers=0.0, tag=N + M + G)
    d["x"] = (d["x"] * np.float16(0.25)).astype(np.float16)
    assert_fp16_close(_run(fn, d, G, "long K"), _ref(d, G), f"{fn.__name__} G={G} M={M} K=65536 N={N}")


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("fn", [mq.w4a16_gemv, mq.w4a16_gemm], ids=["gemv", "gemm"])
def test_group_boundaries_matter(fn, G):
    # Zero points and scales that change at every group of G rows: one-hot
    # rows of x pick single weights, so a kernel that reads the parameters of
    # the wrong group (e.g. groups of 128) gives a different column.
    M, K, N = 8, 512, 256
    rng = np.random.default_rng(G)
    ks = rng.choice(K, size=M, replace=False)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    d = _case(M, K, N, G, outliers=0.0, tag=G + 5)
    d["x"] = x
    got = _run(fn, d, G, "one-hot rows")
    ref = _ref(d, G)
    assert_fp16_close(got, ref, f"{fn.__name__} G={G} one-hot")
    # each output is one dequantized weight: representable in fp16 and exact
    assert np.array_equal(got.astype(np.float64), ref.astype(np.float16).astype(np.float64))
