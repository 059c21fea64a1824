"""Parity of the HIP path (through the C ABI) with the CPU oracle on an MI355X.

Bit-exact: int8 codes, fp32 per-token scales, int32 accumulators.
fp16 outputs: relative Frobenius error <= 1e-3 and max-abs error <= 5e-2
against the unrounded float64 oracle.

Inputs come from ``synth`` (seeded) or are built here; no expected value
comes from the HIP path.
"""

import numpy as np
import pytest

import oracle
import synth
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, assert_fp16_close, dev, host
from tests.oracle_pins import loop_pack

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a).view(np.uint32 if np.asarray(a).dtype.itemsize == 4 else np.uint8)


def _quant_check(x, what):
    announce(f"quant {what} M={x.shape[0]} K={x.shape[1]}")
    xq, s = mq.quant_per_token_int8(dev(x))
    xq, s = host(xq), host(s)
    rq, rs = oracle.quant_per_token_int8_ref(x)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), f"{what}: s_tok differs"
    bad = np.argwhere(xq != rq)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:3].tolist()}"


# ---------------------------------------------------------------------------
# per-token int8 quantization: bit-exact
# ---------------------------------------------------------------------------

def test_quant_prefill_c2():
    x = synth.w8a8_inputs(2048, 4096, 8, outlier_frac=0.01, tag=2)["x"]
    _quant_check(x, "c2 prefill")


@pytest.mark.parametrize("M,K", [(1, 16), (37, 272), (5, 512), (3, 4096), (2, 12288),
                                 (3, 16384), (5, 20480), (1, 4096),
                                 # ragged rows at the row-per-workgroup forms' edges
                                 # (256 / 512 / 1024 threads) and past 128 rows
                                 (7, 2064), (9, 4112), (128, 12304), (4, 16368),
                                 (129, 4096)])
def test_quant_shapes(M, K):
    rng = np.random.default_rng(M * 100003 + K)
    x = (rng.standard_normal((M, K)) * rng.uniform(0.01, 30, size=(M, 1))).astype(np.float16)
    _quant_check(x, "shape")


def test_quant_edge_rows():
    rng = np.random.default_rng(17)
    K = 272
    rows = [np.zeros(K),                                     # all zero -> s = 0, q = 0
            np.full(K, -3.0),                                # constant negative
            np.where(np.arange(K) == 5, 65504.0, 0.0),       # single fp16 max
            np.where(np.arange(K) == 7, 6e-8, 0.0),          # single subnormal
            ]
    ties = rng.integers(-127, 128, size=K) * 0.5             # many exact .5 quotients
    ties[3] = 127.0
    rows.append(ties)
    rows.append(rng.integers(-127, 128, size=K) * 2.0 ** -6)
    x = np.stack(rows).astype(np.float16)
    _quant_check(x, "edge rows")


def test_weight_quant_per_channel():
    """Per-output-channel weight quantization is the same quantizer on the rows of W [N, K]."""
    wf = synth.w8a8_inputs(8, 4096, 4096, tag=2)["wf"]
    _quant_check(wf, "weights c2")


# ---------------------------------------------------------------------------
# W8A8 GEMM
# ---------------------------------------------------------------------------

def _w8a8_operands(M, K, N, tag, outliers=0.01):
    d = synth.w8a8_inputs(M, K, N, outlier_frac=outliers, tag=tag)
    xq, s_tok = oracle.quant_per_token_int8_ref(d["x"])
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    return xq, s_tok, wq, s_ch


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 4096), (200, 300, 272), (1, 8, 16), (3, 1, 64),
                                   (129, 257, 4112), (64, 6144, 4096), (300, 1000, 400), (513, 130, 48),
                                   (600, 2050, 96), (1300, 384, 256),
                                   # decode-shaped: one, two and four 16-token tiles, ragged N and K
                                   (1, 6144, 4096), (8, 4096, 12288), (17, 24576, 4096), (33, 1000, 400),
                                   (5, 130, 48), (64, 4096, 16), (16, 17, 4112), (32, 4096, 12288),
                                   (48, 6144, 4096), (20, 6200, 272), (64, 24576, 128),
                                   # up to 16 tokens on 6144+ channels with the codes staged in LDS
                                   (8, 6144, 4096), (5, 24576, 4096), (3, 6160, 12288), (16, 8192, 2048),
                                   (9, 6144, 1024), (16, 6144, 4096), (6, 6144, 12288)])
def test_w8a8_acc_bitexact(M, N, K):
    xq, _, wq, _ = _w8a8_operands(M, K, N, tag=M + N + K)
    announce(f"w8a8 i32 M={M} N={N} K={K}")
    acc = host(mq.w8a8_mm_i32(dev(xq), dev(wq)))
    ref = oracle.w8a8_acc_ref(xq, wq)
    assert acc.dtype == np.int32
    bad = np.argwhere(acc.astype(np.int64) != ref)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 4096), (200, 300, 272), (1, 8, 16), (129, 257, 4112),
                                   (1, 24576, 4096), (8, 6144, 4096), (64, 4096, 12288), (40, 1000, 400),
                                   (64, 8192, 4096), (30, 6176, 4112)])
def test_w8a8_scaled(M, N, K):
    xq, s_tok, wq, s_ch = _w8a8_operands(M, K, N, tag=7 * M + N + K)
    announce(f"w8a8 scaled M={M} N={N} K={K}")
    y = host(mq.w8a8_scaled_mm(dev(xq), dev(s_tok), dev(wq), dev(s_ch)))
    assert_fp16_close(y, oracle.w8a8_ref(xq, s_tok, wq, s_ch), f"w8a8 M={M} N={N} K={K}")


def test_w8a8_extreme_accumulators():
    K = 12288
    xq = np.full((3, K), 127, np.int8)
    xq[1] = -127
    wq = np.full((5, K), 127, np.int8)
    wq[2] = -127
    announce("w8a8 extreme")
    acc = host(mq.w8a8_mm_i32(dev(xq), dev(wq)))
    assert np.array_equal(acc.astype(np.int64), oracle.w8a8_acc_ref(xq, wq))
    assert acc.max() == 16129 * K and acc.min() == -16129 * K


@pytest.mark.parametrize("M", [3, 300], ids=["decode_kernel", "tiled_gemm"])
def test_w8a8_largest_k(M):
    # K = 133136, the largest multiple of 16 whose worst-case accumulator
    # (127 * 127 * K) still fits int32: all +-127 rows hit the bound exactly.
    K, N = 133136, 40
    rng = np.random.default_rng(M)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    xq[0] = 127
    wq[0] = 127
    wq[1] = -127
    announce(f"w8a8 largest K M={M}")
    acc = host(mq.w8a8_mm_i32(dev(xq), dev(wq)))
    ref = oracle.w8a8_acc_ref(xq, wq)
    assert np.array_equal(acc.astype(np.int64), ref)
    assert acc[0, 0] == 16129 * K and acc[0, 1] == -16129 * K


@pytest.mark.parametrize("fn,M,N", [(mq.w4a16_gemv, 2, 264), (mq.w4a16_gemv, 5, 256), (mq.w4a16_gemv, 40, 256),
                                    (mq.w4a16_gemm, 100, 264)],
                         ids=["gemv_regs", "gemv_lds", "gemv_lds_3tiles", "gemm"])
def test_w4a16_long_k(fn, M, N):
    # K = 65536 (512 groups): many splits per strip, long stage loops. The
    # activations are scaled by 1/4 (exact in fp16) and carry no outliers so
    # that |y| stays well below 128: above it half an fp16 ulp (0.0625)
    # alone exceeds the 5e-2 max-abs bound.
    d = _w4(M, 65536, N, outliers=0.0, tag=N + M)
    d["x"] = (d["x"] * np.float16(0.25)).astype(np.float16)
    assert_fp16_close(_run_w4(fn, d, "long K"), _ref_w4(d), f"{fn.__name__} M={M} K=65536 N={N}")


def test_w8a8_linear_end_to_end():
    d = synth.w8a8_inputs(300, 4096, 1024, outlier_frac=0.01, tag=22)
    wq, s_ch = oracle.quant_per_token_int8_ref(d["wf"])
    announce("w8a8 linear")
    y = host(mq.w8a8_linear(dev(d["x"]), dev(wq), dev(s_ch)))
    xq, s_tok = oracle.quant_per_token_int8_ref(d["x"])
    assert_fp16_close(y, oracle.w8a8_ref(xq, s_tok, wq, s_ch), "w8a8 linear")


# ---------------------------------------------------------------------------
# W4A16 GEMV (decode) and GEMM (prefill)
# ---------------------------------------------------------------------------

def _w4(M, K, N, outliers=0.0, tag=0):
    return synth.w4a16_inputs(M, K, N, group=128, outlier_frac=outliers, tag=tag)


def _run_w4(fn, d, what):
    announce(f"{fn.__name__} {what} M={d['x'].shape[0]} K={d['x'].shape[1]} N={d['scales'].shape[1]}")
    y = fn(dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), 128)
    return host(y)


def _ref_w4(d):
    return oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], 128)


@pytest.mark.parametrize("fn", [mq.w4a16_gemv, mq.w4a16_gemm], ids=["gemv", "gemm"])
def test_w4a16_tiny_c0(fn):
    d = _w4(4, 512, 512, tag=0)
    assert_fp16_close(_run_w4(fn, d, "c0"), _ref_w4(d), f"{fn.__name__} c0")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_w4a16_gemv_decode_c1(M):
    d = _w4(M, 4096, 24576, outliers=0.005, tag=1)
    assert_fp16_close(_run_w4(mq.w4a16_gemv, d, "c1"), _ref_w4(d), f"gemv c1 M={M}")


@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (3, 384, 424), (7, 384, 424), (13, 1024, 1032),
                                   (16, 256, 4096), (2, 4096, 6144), (5, 12288, 4096), (16, 128, 24576),
                                   (3, 4096, 128), (5, 2048, 136), (16, 8192, 520),
                                   # two to four 16-token tiles; ragged token tails; N % 32 != 0
                                   # (16-token slices); many and few splits
                                   (17, 384, 424), (32, 4096, 6144), (33, 1024, 1032), (48, 12288, 4096),
                                   (64, 4096, 24576), (64, 4096, 4096), (63, 256, 4096), (40, 2048, 136)])
def test_w4a16_gemv_shapes(M, K, N):
    d = _w4(M, K, N, outliers=0.005, tag=M * 7 + K + N)
    assert_fp16_close(_run_w4(mq.w4a16_gemv, d, "shape"), _ref_w4(d), f"gemv M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (17, 384, 424), (200, 384, 424), (129, 1024, 1032),
                                   (300, 256, 264), (64, 4096, 6144)])
def test_w4a16_gemm_shapes(M, K, N):
    d = _w4(M, K, N, tag=M * 13 + K + N)
    assert_fp16_close(_run_w4(mq.w4a16_gemm, d, "shape"), _ref_w4(d), f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("K", [4096, 12288], ids=["c3a_o_proj", "c3b_down"])
def test_w4a16_gemm_prefill_c3(K):
    d = _w4(4096, K, 4096, tag=3 if K == 4096 else 4)
    assert_fp16_close(_run_w4(mq.w4a16_gemm, d, "c3"), _ref_w4(d), f"gemm c3 K={K}")


@pytest.mark.parametrize("fn", [mq.w4a16_gemv, mq.w4a16_gemm], ids=["gemv", "gemm"])
def test_w4a16_q_equals_z_gives_zero(fn):
    rng = np.random.default_rng(31)
    M, K, N = 5, 384, 264
    z = rng.integers(0, 16, size=(K // 128, N))
    d = {"x": rng.standard_normal((M, K)).astype(np.float16),
         "qweight": loop_pack(np.repeat(z, 128, axis=0)),
         "scales": rng.uniform(0.005, 0.02, size=(K // 128, N)).astype(np.float16),
         "qzeros": loop_pack(z)}
    y = _run_w4(fn, d, "q=z")
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("fn", [mq.w4a16_gemv, mq.w4a16_gemm], ids=["gemv", "gemm"])
def test_w4a16_one_hot_gathers_columns(fn):
    rng = np.random.default_rng(37)
    M, K, N = 3, 512, 136
    perm = rng.integers(0, K, size=N)
    q = np.zeros((K, N), np.int64)
    q[perm, np.arange(N)] = 1
    d = {"x": rng.standard_normal((M, K)).astype(np.float16),
         "qweight": loop_pack(q),
         "scales": np.ones((K // 128, N), np.float16),
         "qzeros": loop_pack(np.zeros((K // 128, N), np.int64))}
    y = _run_w4(fn, d, "one-hot")
    assert np.array_equal(y, d["x"][:, perm])


def test_w4a16_deterministic():
    d = _w4(16, 4096, 6144, outliers=0.005, tag=41)
    a = _run_w4(mq.w4a16_gemv, d, "repeat 1")
    b = _run_w4(mq.w4a16_gemv, d, "repeat 2")
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    a = _run_w4(mq.w4a16_gemm, d, "repeat 1")
    b = _run_w4(mq.w4a16_gemm, d, "repeat 2")
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_linear_dispatch_and_empty():
    import torch
    d = _w4(16, 256, 264, tag=43)
    args = [dev(d[k]) for k in ("qweight", "scales", "qzeros")]
    announce("w4a16_linear dispatch")
    y16 = host(mq.w4a16_linear(dev(d["x"]), *args))
    assert_fp16_close(y16, _ref_w4(d), "linear M=16")
    x17 = np.concatenate([d["x"], d["x"][:1]])
    y17 = host(mq.w4a16_linear(dev(x17), *args))
    assert_fp16_close(y17, oracle.w4a16_ref(x17, d["qweight"], d["scales"], d["qzeros"], 128), "linear M=17")
    x65 = np.concatenate([d["x"]] * 4 + [d["x"][:1]])  # past the GEMV: the GEMM
    y65 = host(mq.w4a16_linear(dev(x65), *args))
    assert_fp16_close(y65, oracle.w4a16_ref(x65, d["qweight"], d["scales"], d["qzeros"], 128), "linear M=65")
    # empty problems: valid, nothing written
    out = torch.full((0, 264), 1.0, dtype=torch.float16, device="cuda")
    x0 = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    assert mq.w4a16_gemm(x0, *args, out=out).shape == (0, 264)
    assert mq.w4a16_gemv(x0, *args, out=out).shape == (0, 264)
    xq0, s0 = mq.quant_per_token_int8(x0)
    assert xq0.shape == (0, 256) and s0.shape == (0,)


def test_gemv_rejects_large_m():
    d = _w4(65, 256, 264, tag=44)
    with pytest.raises(mq.MqError) as e:
        _run_w4(mq.w4a16_gemv, d, "M=65")
    assert e.value.status_name == "MQ_ERR_UNSUPPORTED"


@pytest.mark.parametrize("M,K,N,G", [(2048, 4096, 4096, 128), (577, 1024, 3072, 64), (2048, 12288, 4096, 128),
                                     (100, 4096, 1024, 128), (300, 1024, 1032, 32), (65, 2048, 264, 128)])
def test_w4a16_gemm_split_k(M, K, N, G):
    # small tile grids split K (fp32 partials, then the reduce kernel): the
    # result matches the oracle, and the unsplit call (no workspace) within
    # fp32 summation order
    import torch
    d = synth.w4a16_inputs(M, K, N, group=G, tag=M + K + N)
    splits = mq.w4a16_gemm_workspace_bytes(M, N, K, G) // (4 * M * N)
    announce(f"w4a16_gemm split K={K} M={M} N={N} G={G} splits={splits}")
    args = (dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), dev(d["qzeros"]), G)
    y = host(mq.w4a16_gemm(*args))
    ref = oracle.w4a16_ref(d["x"], d["qweight"], d["scales"], d["qzeros"], G)
    assert_fp16_close(y, ref, f"gemm split M={M} K={K} N={N}")
    y1 = host(mq.w4a16_gemm(*args, workspace=False))
    assert_fp16_close(y1, ref, f"gemm unsplit M={M} K={K} N={N}")
    if M in (2048, 577):
        assert splits >= 2
    y2 = host(mq.w4a16_gemm(*args))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "split GEMM is not deterministic"
