"""Checkpoint-layout adapter (mq_int4_reorder, mq_int4_transpose,
mq_u16_transpose) on an MI355X: bit-exact against the oracle's definitions
at the 8B-shaped layer sizes and at ragged shapes that leave partial tiles,
and a K-packed checkpoint converted and run through the W4A16 GEMM and GEMV
against the oracle on the original values."""

import numpy as np
import pytest

import oracle
import weight_activation_quantized_amd as mq
from tests.gpu_util import MAX_ABS_TOL, REL_FRO_TOL, announce, dev, fp16_errors, host

pytestmark = pytest.mark.gpu

AWQ = mq.AWQ_FIELD_ORDER


def _pack_rows(q, order):
    """Test-side packer: word c of row r holds element 8c + order[j] in field j."""
    q = np.asarray(q, dtype=np.uint64)
    w = np.zeros((q.shape[0], q.shape[1] // 8), dtype=np.uint64)
    for j in range(8):
        w |= q[:, order[j]::8] << np.uint64(4 * j)
    return w.astype(np.uint32).view(np.int32)


def _random_words(rng, shape):
    return rng.integers(-2 ** 31, 2 ** 31, size=shape, dtype=np.int64).astype(np.int32)


@pytest.mark.parametrize("order", [AWQ, tuple(range(8)), (7, 6, 5, 4, 3, 2, 1, 0)], ids=["awq", "plain", "reversed"])
@pytest.mark.parametrize("shape", [(4096, 3072), (128, 768), (7, 3), (1, 1), (5, 9)],
                         ids=["gate_up", "zeros", "ragged21", "one", "ragged45"])
def test_int4_reorder_bitexact(shape, order):
    rng = np.random.default_rng(sum(shape) + order[1])
    w = _random_words(rng, shape)
    announce(f"int4_reorder shape={shape} order={order}")
    got = host(mq.int4_reorder(dev(w), order))
    assert np.array_equal(got, oracle.reorder_int4_ref(w, order))


@pytest.mark.parametrize("order", [AWQ, tuple(range(8))], ids=["awq", "plain"])
@pytest.mark.parametrize("AB", [(6144, 4096), (4096, 1024), (8, 8), (136, 200), (264, 1032), (1024, 8)],
                         ids=["qkv", "vit", "one_word", "ragged", "ragged2", "tall"])
def test_int4_transpose_bitexact(AB, order):
    A, B = AB
    rng = np.random.default_rng(A + B + order[1])
    w = _random_words(rng, (A, B // 8))
    announce(f"int4_transpose A={A} B={B} order={order}")
    got = host(mq.int4_transpose(dev(w), order))
    assert got.shape == (B, A // 8)
    assert np.array_equal(got, oracle.transpose_int4_ref(w, order))


@pytest.mark.parametrize("AB", [(6144, 32), (24576, 32), (70, 130), (1, 1), (64, 64)],
                         ids=["qkv_scales", "gate_up_scales", "ragged", "one", "tile"])
def test_u16_transpose_bitexact(AB):
    rng = np.random.default_rng(sum(AB))
    s = rng.uniform(0.005, 0.02, AB).astype(np.float16)
    s.view(np.uint16)[0, 0] = 0x8000  # a signed zero keeps its bits
    announce(f"u16_transpose shape={AB}")
    got = host(mq.u16_transpose(dev(s)))
    assert np.array_equal(got.view(np.uint16), s.T.view(np.uint16))


@pytest.mark.parametrize("M", [4, 300])
def test_k_packed_checkpoint_through_the_linear_path(M):
    """Weights stored one output channel per row ([N, K/8], AWQ field order),
    scales [N, K/G] and zeros [N/8, K/G] packed along N in the same order:
    converted on the GPU and fed to the W4A16 linear layer, the result
    matches the oracle on the original values."""
    K, N, G = 1024, 768, 128
    rng = np.random.default_rng(M)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(K // G, N))
    s = rng.uniform(0.005, 0.02, (K // G, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w_nk = _pack_rows(q.T, AWQ)                 # [N, K/8] along K
    s_nk = np.ascontiguousarray(s.T)            # [N, K/G]
    z_kn = _pack_rows(z, AWQ)                   # [K/G, N/8] along N
    announce(f"k-packed checkpoint M={M} K={K} N={N}")
    qweight = mq.int4_transpose(dev(w_nk), AWQ)
    scales = mq.u16_transpose(dev(s_nk))
    qzeros = mq.int4_reorder(dev(z_kn), AWQ)
    assert np.array_equal(host(qweight), oracle.pack_int4(q))
    assert np.array_equal(host(qzeros), oracle.pack_int4(z))
    y = host(mq.w4a16_linear(dev(x), qweight, scales, qzeros, G))
    ref = oracle.w4a16_ref(x, oracle.pack_int4(q), s, oracle.pack_int4(z), G)
    rel, mx, _ = fp16_errors(y, ref)
    assert rel <= REL_FRO_TOL and mx <= MAX_ABS_TOL, (rel, mx)
