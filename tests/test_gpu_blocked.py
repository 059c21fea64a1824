"""Column-blocked W4A16 decode path on an MI355X: the layout conversion is
bit-exact against the oracle's definition of the layout, and the GEMV on
converted weights matches the oracle computed from the original [K, N/8]
weights (relative Frobenius error <= 1e-3, max-abs error <= 5e-2 against the
unrounded float64 result)."""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N", [(4096, 24576), (128, 32), (384, 96), (12288, 4096), (1024, 3072)])
def test_block_weights_bitexact(K, N):
    w = synth.w4a16_weights(K, N, 128, tag=50, seed=K + N)
    announce(f"block_weights K={K} N={N}")
    got = host(mq.w4a16_block_weights(dev(w["qweight"])))
    ref = oracle.block_weights_ref(w["qweight"])
    assert got.shape == ref.shape
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} words differ, first at {bad[:3].tolist()}"


def _run(d, G, what):
    M, K = d["x"].shape
    N = d["scales"].shape[1]
    announce(f"gemv_blocked G={G} {what} M={M} K={K} N={N}")
    qb = mq.w4a16_block_weights(dev(d["qweight"]))
    return host(mq.w4a16_gemv_blocked(dev(d["x"]), qb, dev(d["scales"]), dev(d["qzeros"]), G))


def _ref(d, G):
    return oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], G)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_blocked_decode_gate_up(M):
    d = synth.w4a16_inputs(M, 4096, 24576, group=128, outlier_frac=0.005, tag=1)
    assert_fp16_close(_run(d, 128, "c1"), _ref(d, 128), f"gemv_blocked c1 M={M}")


# layer shapes (one strip per workgroup, or K split for narrow layers), the
# vision tower's qkv, one to four 16-token tiles incl. ragged tails and the
# 32-token passes, the smallest K (one chunk)
@pytest.mark.parametrize("G", [128, 64, 32])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 6144), (8, 4096, 4096), (3, 12288, 4096), (64, 4096, 24576),
                                   (1, 1024, 3072), (16, 1024, 3072), (17, 384, 256), (32, 2048, 1024),
                                   (33, 1024, 3072), (63, 256, 384), (5, 128, 128), (1, 128, 24576),
                                   (2, 640, 640), (7, 384, 32), (40, 640, 96), (1, 4096, 24608),
                                   # workgroups of three (5..16 tokens) or two (17..32) adjacent strips
                                   (12, 640, 96), (9, 4096, 24576), (5, 1024, 3072), (24, 512, 4096),
                                   # 17-64 tokens: six and ten 64-row steps per wavefront (the
                                   # two-step pipeline's tail after two and four steady rounds)
                                   (48, 3072, 4096), (40, 5120, 8192)])
def test_gemv_blocked_shapes(M, K, N, G):
    d = synth.w4a16_inputs(M, K, N, group=G, outlier_frac=0.005, tag=M + K + N + G)
    assert_fp16_close(_run(d, G, "shape"), _ref(d, G), f"gemv_blocked G={G} M={M} K={K} N={N}")


@pytest.mark.parametrize("M", [2, 20])
def test_gemv_blocked_long_k(M):
    # K = 65536: many chunks per wavefront; activations scaled by 1/4 (exact)
    # so |y| stays well below 128
    d = synth.w4a16_inputs(M, 65536, 256, group=128, outlier_frac=0.0, tag=77 + M)
    d["x"] = (d["x"] * np.float16(0.25)).astype(np.float16)
    assert_fp16_close(_run(d, 128, "long K"), _ref(d, 128), f"gemv_blocked M={M} K=65536")


def test_gemv_blocked_one_hot_exact():
    # one-hot token rows pick single dequantized weights: exact in fp16
    M, K, N = 16, 512, 288
    rng = np.random.default_rng(9)
    d = synth.w4a16_inputs(M, K, N, group=64, outlier_frac=0.0, tag=9)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), rng.choice(K, size=M, replace=False)] = 1.0
    d["x"] = x
    got = _run(d, 64, "one-hot")
    ref = _ref(d, 64)
    assert np.array_equal(got.astype(np.float64), ref.astype(np.float16).astype(np.float64))


def test_gemv_blocked_deterministic():
    d = synth.w4a16_inputs(16, 4096, 4096, group=128, outlier_frac=0.005, tag=5)
    qb = mq.w4a16_block_weights(dev(d["qweight"]))
    x, s, z = dev(d["x"]), dev(d["scales"]), dev(d["qzeros"])
    a = host(mq.w4a16_gemv_blocked(x, qb, s, z, 128))
    b = host(mq.w4a16_gemv_blocked(x, qb, s, z, 128))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
