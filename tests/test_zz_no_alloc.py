"""The allocation-free W8A8_INT8 layer (mq_w8a8_linear_noalloc) on an MI355X.

Called through the C ABI, it must give the same bits as mq_w8a8_linear with
a caller's workspace (the same kernels; only where the quantizer's codes and
scales live differs), and the oracle's result within the fp16 tolerance
(relative Frobenius error <= 1e-3, max-abs error <= 5e-2), on calls in a row
whose later inputs are smaller (the library's scratch keeps the previous
call's contents), and under HIP graph capture.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host

pytestmark = pytest.mark.gpu


def _case(M, K, N, tag):
    d = synth.w8a8_inputs(M, K, N, outlier_frac=0.01, tag=tag)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    return d["x"], wq, s_ch


def _check(x, wq, s_ch, what):
    M, K = x.shape
    N = wq.shape[0]
    announce(f"w8a8_linear_noalloc {what} M={M} K={K} N={N}")
    tx, twq, ts = dev(x), dev(wq), dev(s_ch)
    y0 = host(mq.w8a8_linear_noalloc(tx, twq, ts))
    y1 = host(mq.w8a8_linear(tx, twq, ts))
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16)), f"{what}: differs from mq_w8a8_linear"
    xq, s_tok = oracle.quant_per_token_int8_ref(x)
    assert_fp16_close(y0, oracle.w8a8_ref(xq, s_tok, wq, s_ch), f"noalloc {what}")


def test_noalloc_calls_in_a_row_shrinking():
    # prefill-sized first, then smaller calls that reuse the scratch: the
    # second reads none of the first call's codes or scales
    for i, (M, K, N) in enumerate([(2048, 4096, 4096), (7, 272, 300), (33, 4096, 1024), (2, 16, 8), (1, 4096, 6144)]):
        _check(*_case(M, K, N, tag=700 + i), what=f"call {i}")


def test_noalloc_largest_scratch():
    # 2048 tokens of the down projection (K = 12288): 24 MiB of codes
    x, wq, s_ch = _case(2048, 12288, 256, tag=710)
    assert mq.w8a8_linear_workspace_bytes(2048, 12288) <= mq.NOALLOC_SCRATCH_BYTES
    _check(x, wq, s_ch, "largest")
    with pytest.raises(mq.MqError) as e:
        mq.w8a8_linear_noalloc(dev(np.zeros((4096, 12288), np.float16)), dev(wq), dev(s_ch))
    assert e.value.status_name == "MQ_ERR_WORKSPACE"


def test_noalloc_graph_capture():
    import torch
    x, wq, s_ch = _case(64, 4096, 4096, tag=720)
    tx, twq, ts = dev(x), dev(wq), dev(s_ch)
    y = torch.empty((64, 4096), dtype=torch.float16, device="cuda")
    ref = host(mq.w8a8_linear(tx, twq, ts))
    announce("w8a8_linear_noalloc graph capture M=64 K=4096 N=4096")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.w8a8_linear_noalloc(tx, twq, ts, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.w8a8_linear_noalloc(tx, twq, ts, out=y)
    other = [tuple(dev(a) for a in _case(5 + r, 272, 40, tag=730 + r)) for r in range(3)]
    for r in range(3):
        y.zero_()
        mq.w8a8_linear_noalloc(*other[r])  # eager work on the same scratch between replays
        torch.cuda.synchronize()
        g.replay()
        got = host(y)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), f"replay {r} differs"
