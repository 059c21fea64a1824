"""Parity on the linear layers of an 8B-shaped GQA decoder layer (hidden 4096,
32 query / 8 KV heads of dim 128): qkv (4096 -> 6144), o_proj (4096 -> 4096),
gate_up (4096 -> 24576) and down (12288 -> 4096), at decode batches 1, 8, 64
and a 2048-token prefill, under W4A16 (group 128) and W8A8_INT8.

W4A16 inputs: decode batches use N(0, 1) activations with 0.5% x20 outlier
channels, the prefill plain N(0, 1); W8A8 uses 1% x20 outlier channels at
every batch. Each case goes through the layer entry point a model would call
(GEMV for M <= 64, GEMM above; quantize + scaled GEMM for W8A8).
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu

LAYERS = list(synth.LAYER_SET.items())
MS = list(synth.LAYER_SET_MS)


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("name,shape", LAYERS, ids=[n for n, _ in LAYERS])
def test_layer_w4a16(name, shape, M):
    K, N = shape["K"], shape["N"]
    d = synth.w4a16_inputs(M, K, N, group=128, outlier_frac=0.0 if M == 2048 else 0.005,
                           tag=100 + K + N, seed=M)
    announce(f"layer w4a16 {name} M={M}")
    y = mq.w4a16_linear(dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), 128)
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], 128)
    assert_fp16_close(host(y), ref, f"w4a16 {name} M={M}")


@pytest.mark.parametrize("M", [m for m in MS if m <= mq.GEMV_MAX_M] + [33, 48])
@pytest.mark.parametrize("name,shape", LAYERS, ids=[n for n, _ in LAYERS])
def test_layer_w4a16_decode_layout(name, shape, M):
    # decode through the layer entry with weights converted once to the
    # decode layout (the path the layer-set timings take)
    K, N = shape["K"], shape["N"]
    d = synth.w4a16_inputs(M, K, N, group=128, outlier_frac=0.005, tag=150 + K + N, seed=M)
    announce(f"layer w4a16 decode layout {name} M={M}")
    qw = dev(d["qweight"])
    y = mq.w4a16_linear(dev(d["x"]), qw, dev(d["scales"]), dev(d["qzeros"]), 128,
                        qweight_blocked=mq.w4a16_block_weights(qw))
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], 128)
    assert_fp16_close(host(y), ref, f"w4a16 decode layout {name} M={M}")


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("name,shape", LAYERS, ids=[n for n, _ in LAYERS])
def test_layer_w8a8(name, shape, M):
    K, N = shape["K"], shape["N"]
    d = synth.w8a8_inputs(M, K, N, outlier_frac=0.01, tag=200 + K + N, seed=M)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    announce(f"layer w8a8 {name} M={M}")
    xq_gpu, s_gpu = mq.quant_per_token_int8(dev(d["x"]))
    y = mq.w8a8_scaled_mm(xq_gpu, s_gpu, dev(wq), dev(s_ch))
    xq, s_tok = oracle.quant_per_token_int8_ref(d["x"])
    assert np.array_equal(host(xq_gpu), xq) and np.array_equal(host(s_gpu), s_tok)
    assert_fp16_close(host(y), oracle.w8a8_ref(xq, s_tok, wq, s_ch), f"w8a8 {name} M={M}")
