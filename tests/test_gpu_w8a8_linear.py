"""W8A8_INT8 linear layer from fp16 activations (mq_w8a8_linear) on an MI355X.

For one token with K <= 12288, two with K <= 8192 and three or four with
K <= 4096 and N >= 6144 (the token rows held in registers, two, four or
six 16-byte chunks per thread and row) the per-token quantizer runs inside
the decode kernel (a capped grid walks the channel tiles, each workgroup
forming the codes once); the result must equal mq_quant_per_token_int8
followed by mq_w8a8_scaled_mm bit for bit
(same codes, scales and int32 accumulators, same epilogue), and the oracle
within the fp16 tolerance. Otherwise the entry point runs the two kernels
through its workspace.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (1, 4096, 6144), (1, 4096, 24576), (1, 12288, 4096),
                                   (1, 16, 16384), (1, 272, 16392), (1, 1040, 16400), (1, 12288, 16384),
                                   (1, 16, 8), (1, 272, 300), (1, 1040, 37), (1, 81904, 64), (1, 133136, 48),
                                   (4, 4096, 24576), (16, 4096, 4096),
                                   (2, 16, 8), (2, 4096, 24576), (2, 4096, 6144), (2, 12288, 4096),
                                   (2, 40000, 200), (2, 1040, 9000),
                                   (7, 272, 300), (13, 1040, 37), (16, 64, 4112),
                                   (3, 133136, 48),
                                   # fused for 2 tokens up to K = 8192 and 3-4 tokens up to K = 4096
                                   # with N >= 6144 (a fourth row of zeros for 3 tokens); past those,
                                   # two kernels
                                   (3, 1040, 6160), (3, 4096, 4096), (4, 4096, 6144), (4, 4112, 6144),
                                   (2, 8192, 1024), (2, 8208, 64),
                                   # two kernels through the workspace
                                   (17, 512, 264), (64, 4096, 4096), (300, 1024, 640)])
def test_w8a8_linear_matches_two_calls_and_oracle(M, K, N):
    d = synth.w8a8_inputs(M, K, N, outlier_frac=0.01, tag=900 + M + K % 97)
    if K > 100000:
        d["x"] = (d["x"] * np.float16(0.25)).astype(np.float16)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    x, w, s = dev(d["x"]), dev(wq), dev(s_ch)
    announce(f"w8a8_linear M={M} K={K} N={N}")
    y = host(mq.w8a8_linear(x, w, s))
    xq, st = mq.quant_per_token_int8(x)
    y2 = host(mq.w8a8_scaled_mm(xq, st, w, s))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "differs from quant + scaled_mm"
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(d["x"])
    assert_fp16_close(y, oracle.w8a8_ref(xq_ref, s_ref, wq, s_ch), f"w8a8_linear M={M} K={K} N={N}")


@pytest.mark.parametrize("K", [12288, 8208, 8192, 4112, 4096, 12304])
def test_w8a8_linear_fused_long_rows(K):
    # the fused kernel at the row lengths where its register count changes
    # (K = 4096 / 8192 / 12288 the most each form holds; 12304 takes the two
    # kernels), on a wide layer; weights are random codes (not from the
    # quantizer) so the test stays light; bit-identical to the two kernels,
    # the oracle on sampled columns
    N = 16384
    rng = np.random.default_rng(K)
    x = (rng.standard_normal((1, K)) * 0.25).astype(np.float16)
    wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s_ch = rng.uniform(0.001, 0.01, N).astype(np.float32)
    tx, tw, ts = dev(x), dev(wq), dev(s_ch)
    announce(f"w8a8_linear fused long rows K={K}")
    y = host(mq.w8a8_linear(tx, tw, ts))
    xq, st = mq.quant_per_token_int8(tx)
    y2 = host(mq.w8a8_scaled_mm(xq, st, tw, ts))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "fused differs from quant + scaled_mm"
    cols = rng.choice(N, size=64, replace=False)
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(x)
    assert_fp16_close(y[:, cols], oracle.w8a8_ref(xq_ref, s_ref, wq[cols], s_ch[cols]), f"fused K={K}")


def test_w8a8_linear_zero_and_tie_rows():
    # an all-zero token (s = 0, codes 0, output row 0) next to rows of exact
    # ties (x = (j + 0.5) * s for a power-of-two s): the quantizer, separate
    # or fused (one token at a time on a wide layer), must round them half to
    # even like the oracle
    M, K, N = 5, 256, 96
    d = synth.w8a8_inputs(M, K, N, outlier_frac=0.0, tag=31)
    x = d["x"]
    x[1] = 0
    j = np.arange(K) % 127
    x[2] = ((j + 0.5) * 0.25).astype(np.float16)
    x[2, 0] = np.float16(127 * 0.25)  # absmax -> s = 0.25 exactly
    x[3] = -x[2]
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    announce("w8a8_linear zero and tie rows")
    y = host(mq.w8a8_linear(dev(x), dev(wq), dev(s_ch)))
    xq_ref, s_ref = oracle.quant_per_token_int8_ref(x)
    assert s_ref[1] == 0 and s_ref[2] == np.float32(0.25)
    assert np.all(y[1] == 0)
    assert_fp16_close(y, oracle.w8a8_ref(xq_ref, s_ref, wq, s_ch), "w8a8_linear ties")
    # the separate quantizer takes the oracle's codes on these rows (bit-exact
    # elsewhere), and the fused kernel must give the same outputs bit for bit
    xq, st = mq.quant_per_token_int8(dev(x))
    assert np.array_equal(host(xq), xq_ref)
    y2 = host(mq.w8a8_scaled_mm(xq, st, dev(wq), dev(s_ch)))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    rng = np.random.default_rng(31)
    ww = dev(rng.integers(-127, 128, size=(16384, K)).astype(np.int8))
    sw = dev(rng.uniform(0.001, 0.01, 16384).astype(np.float32))
    for r in range(M):
        xr = dev(x[r:r + 1])
        y1 = host(mq.w8a8_linear(xr, ww, sw))
        q1, s1 = mq.quant_per_token_int8(xr)
        assert np.array_equal(y1.view(np.uint16), host(mq.w8a8_scaled_mm(q1, s1, ww, sw)).view(np.uint16)), r
