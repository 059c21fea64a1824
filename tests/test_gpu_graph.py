"""Every entry point captured in a HIP graph and replayed.

The entry points are asynchronous and allocate and clear nothing, so a
caller may capture them (the benchmark does). Here each path is captured
once with static buffers; between replays the test rewrites the inputs with
eager copies and runs the same calls eagerly on other outputs. Every replay
must match the eager result bit for bit (the kernels are deterministic) and
the oracle within the usual tolerance.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_w4a16():
    import torch
    K = 4096
    cases = [("gemv_split", 16, 6144), ("gemv_tiles", 40, 4096), ("gemm", 200, 1024)]
    for name, M, N in cases:
        d = synth.w4a16_inputs(M, K, N, group=128, outlier_frac=0.005, tag=500 + N)
        w = {k: torch.from_numpy(d[k]).cuda() for k in ("qweight", "scales", "qzeros")}
        x = torch.from_numpy(d["x"]).cuda()
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        gemv = M <= mq.GEMV_MAX_M
        ws = torch.empty(max(mq.w4a16_gemv_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")

        def call(out, x=x):
            if gemv:
                mq.w4a16_gemv(x, w["qweight"], w["scales"], w["qzeros"], 128, out=out, workspace=ws)
            else:
                mq.w4a16_gemm(x, w["qweight"], w["scales"], w["qzeros"], 128, out=out)

        announce(f"graph w4a16 {name} M={M} N={N}")
        g = _capture(torch, lambda: call(y))
        rng = np.random.default_rng(7)
        for r in range(REPLAYS):
            xr = rng.standard_normal((M, K)).astype(np.float16)
            x.copy_(torch.from_numpy(xr))
            eager = torch.empty_like(y)
            call(eager)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager), f"{name}: replay {r} differs from the eager call"
            ref = oracle.w4a16_ref(xr, d["qweight"], d["scales"], d["qzeros"], 128)
            assert_fp16_close(y.cpu().numpy(), ref, f"graph {name} replay {r}")


def test_graph_replays_w8a8():
    import torch
    K = 1024
    for name, M, N in (("decode", 8, 4096), ("tiled", 300, 640)):
        d = synth.w8a8_inputs(M, K, N, outlier_frac=0.01, tag=600 + N)
        wq_np, s_ch_np = oracle.quant_per_token_int8_ref(d["wf"])
        wq, s_ch = torch.from_numpy(wq_np).cuda(), torch.from_numpy(s_ch_np).cuda()
        x = torch.from_numpy(d["x"]).cuda()
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        st = torch.empty((M,), dtype=torch.float32, device="cuda")
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda")

        def layer(xq, st, y, acc):
            mq.quant_per_token_int8(x, out=xq, s_out=st)
            mq.w8a8_scaled_mm(xq, st, wq, s_ch, out=y)
            mq.w8a8_mm_i32(xq, wq, out=acc)

        announce(f"graph w8a8 {name} M={M} N={N}")
        g = _capture(torch, lambda: layer(xq, st, y, acc))
        rng = np.random.default_rng(11)
        for r in range(REPLAYS):
            xr = (rng.standard_normal((M, K)) * (1 + r)).astype(np.float16)
            x.copy_(torch.from_numpy(xr))
            e = [torch.empty_like(t) for t in (xq, st, y, acc)]
            layer(*e)
            g.replay()
            torch.cuda.synchronize()
            for got, want, what in zip((xq, st, y, acc), e, ("xq", "s_tok", "y", "acc")):
                assert torch.equal(got, want), f"{name}: replay {r} {what} differs from the eager call"
            xq_ref, s_ref = oracle.quant_per_token_int8_ref(xr)
            assert np.array_equal(xq.cpu().numpy(), xq_ref)
            assert np.array_equal(acc.cpu().numpy().astype(np.int64), oracle.w8a8_acc_ref(xq_ref, wq_np))
            assert_fp16_close(y.cpu().numpy(), oracle.w8a8_ref(xq_ref, s_ref, wq_np, s_ch_np),
                              f"graph w8a8 {name} replay {r}")


def test_graph_replays_blocked():
    # the layout conversion and the blocked GEMV (one launch; K split with a
    # reduce launch; two-tile multi-strip workgroups) in one graph
    import torch
    K = 4096
    for name, M, N, G in (("wide", 1, 24576, 128), ("split", 16, 4096, 128), ("tiles", 24, 3072, 64)):
        d = synth.w4a16_inputs(M, K, N, group=G, outlier_frac=0.005, tag=700 + N)
        qw = torch.from_numpy(d["qweight"]).cuda()
        s = torch.from_numpy(d["scales"]).cuda()
        z = torch.from_numpy(d["qzeros"]).cuda()
        x = torch.from_numpy(d["x"]).cuda()
        qb = torch.empty((K // 64, 8 * N), dtype=torch.int32, device="cuda")
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ws = torch.empty(max(mq.w4a16_gemv_blocked_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8,
                         device="cuda")

        def call(out_qb, out_y, x=x):
            mq.w4a16_block_weights(qw, out=out_qb)
            mq.w4a16_gemv_blocked(x, out_qb, s, z, G, out=out_y, workspace=ws)

        announce(f"graph blocked {name} M={M} N={N} G={G}")
        g = _capture(torch, lambda: call(qb, y))
        rng = np.random.default_rng(13)
        for r in range(REPLAYS):
            xr = rng.standard_normal((M, K)).astype(np.float16)
            x.copy_(torch.from_numpy(xr))
            eb, ey = torch.empty_like(qb), torch.empty_like(y)
            call(eb, ey)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(qb, eb) and torch.equal(y, ey), f"{name}: replay {r} differs from the eager call"
            assert np.array_equal(qb.cpu().numpy(), oracle.block_weights_ref(d["qweight"]))
            ref = oracle.w4a16_ref(xr, d["qweight"], d["scales"], d["qzeros"], G)
            assert_fp16_close(y.cpu().numpy(), ref, f"graph blocked {name} replay {r}")


def test_graph_replays_kv_and_checkpoint():
    # KV-cache quantization (both widths, both row-per-group forms) and the
    # checkpoint-layout conversions in one graph
    import torch
    rng = np.random.default_rng(17)
    xs = [torch.empty((T, 32, 128), dtype=torch.float16, device="cuda") for T in (2100, 7)]
    w_kn = torch.empty((64, 96), dtype=torch.int32, device="cuda")
    w_nk = torch.empty((136, 25), dtype=torch.int32, device="cuda")
    s_nk = torch.empty((70, 130), dtype=torch.float16, device="cuda")
    order = mq.AWQ_FIELD_ORDER

    def outs():
        o = []
        for x in xs:
            for bits in (8, 4):
                o.append(torch.empty(x.shape[:-1] + (128 if bits == 8 else 64,), dtype=torch.uint8, device="cuda"))
                o.append(torch.empty(x.shape[:-1] + (2,), dtype=torch.float32, device="cuda"))
        o.append(torch.empty_like(w_kn))
        o.append(torch.empty((200, 17), dtype=torch.int32, device="cuda"))
        o.append(torch.empty((130, 70), dtype=torch.float16, device="cuda"))
        return o

    def run(o):
        i = 0
        for x in xs:
            for bits in (8, 4):
                mq.kv_quant(x, bits, codes=o[i], params=o[i + 1])
                i += 2
        mq.int4_reorder(w_kn, order, out=o[i])
        mq.int4_transpose(w_nk, order, out=o[i + 1])
        mq.u16_transpose(s_nk, out=o[i + 2])

    announce("graph kv_quant + checkpoint layouts")
    static = outs()
    g = _capture(torch, lambda: run(static))
    for r in range(REPLAYS):
        xr = [(rng.standard_normal(tuple(x.shape)) * (1 + r)).astype(np.float16) for x in xs]
        wk = rng.integers(-2 ** 31, 2 ** 31, size=(64, 96), dtype=np.int64).astype(np.int32)
        wn = rng.integers(-2 ** 31, 2 ** 31, size=(136, 25), dtype=np.int64).astype(np.int32)
        sn = rng.uniform(0.005, 0.02, (70, 130)).astype(np.float16)
        for x, a in zip(xs, xr):
            x.copy_(torch.from_numpy(a))
        w_kn.copy_(torch.from_numpy(wk))
        w_nk.copy_(torch.from_numpy(wn))
        s_nk.copy_(torch.from_numpy(sn))
        eager = outs()
        run(eager)
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(static, eager)):
            assert torch.equal(got, want), f"replay {r}: output {k} differs from the eager call"
        i = 0
        for a in xr:
            for bits in (8, 4):
                rc, rp = oracle.kv_quant_ref(a.reshape(-1, 128), bits)
                assert np.array_equal(static[i].cpu().numpy().reshape(rc.shape), rc)
                assert np.array_equal(static[i + 1].cpu().numpy().reshape(-1, 2).view(np.uint32), rp.view(np.uint32))
                i += 2
        assert np.array_equal(static[i].cpu().numpy(), oracle.reorder_int4_ref(wk, order))
        assert np.array_equal(static[i + 1].cpu().numpy(), oracle.transpose_int4_ref(wn, order))
        assert np.array_equal(static[i + 2].cpu().numpy().view(np.uint16), sn.T.view(np.uint16))


def test_graph_replays_w8a8_bf16():
    # bf16 activations: quantizer, scaled GEMM (decode and tiled kernels) and
    # the one-token fused layer in one graph
    import torch
    K, N = 1024, 640
    rng = np.random.default_rng(19)
    d = synth.w8a8_inputs_bf16(4, K, N, tag=611)
    wq_np, s_ch_np = oracle.quant_per_token_int8_ref(d["wf"])
    wq, s_ch = torch.from_numpy(wq_np).cuda(), torch.from_numpy(s_ch_np).cuda()
    xs = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for M in (8, 300, 1)]
    # the one-token layer on a layer wide enough for the fused kernel
    NW = 16384
    wq_w = torch.from_numpy(rng.integers(-127, 128, size=(NW, K)).astype(np.int8)).cuda()
    s_w = torch.from_numpy(rng.uniform(0.001, 0.01, NW).astype(np.float32)).cuda()

    def outs():
        o = []
        for x in xs[:2]:
            M = x.shape[0]
            o += [torch.empty((M, K), dtype=torch.int8, device="cuda"),
                  torch.empty((M,), dtype=torch.float32, device="cuda"),
                  torch.empty((M, N), dtype=torch.bfloat16, device="cuda")]
        o.append(torch.empty((1, NW), dtype=torch.bfloat16, device="cuda"))
        return o

    def run(o):
        for i, x in enumerate(xs[:2]):
            mq.quant_per_token_int8(x, out=o[3 * i], s_out=o[3 * i + 1])
            mq.w8a8_scaled_mm(o[3 * i], o[3 * i + 1], wq, s_ch, out=o[3 * i + 2])
        mq.w8a8_linear(xs[2], wq_w, s_w, out=o[6])

    announce("graph w8a8 bf16")
    static = outs()
    g = _capture(torch, lambda: run(static))
    for r in range(REPLAYS):
        xr = [synth.bf16_bits((rng.standard_normal(tuple(x.shape)) * (1 + r)).astype(np.float32)) for x in xs]
        for x, b in zip(xs, xr):
            x.copy_(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16))
        eager = outs()
        run(eager)
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(static, eager)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r}: output {k} differs"
        for i in range(2):
            q_ref, s_ref = oracle.quant_per_token_int8_ref(synth.bf16_values(xr[i]))
            assert np.array_equal(static[3 * i].cpu().numpy(), q_ref)
            assert np.array_equal(static[3 * i + 1].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
            y64 = oracle.w8a8_ref(q_ref, s_ref, wq_np, s_ch_np)
            yb = synth.bf16_values(static[3 * i + 2].view(torch.int16).cpu().numpy().view(np.uint16))
            assert np.all(np.abs(yb - y64) <= (2.0 ** -8 + 2.0 ** -20) * np.abs(y64))
