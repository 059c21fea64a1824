"""Online KV-cache quantization (mq_kv_quant) on an MI355X: codes and
(scale, min) bit-exact against the oracle, INT8 and INT4, at a 4096-token
prefill of a 32-head, 128-dim layer, a decode append, other head sizes and
the edge rows the oracle's pins cover (ties, binary32-sensitive quotients,
constant rows, signed zeros, fp16 extremes)."""

import numpy as np
import pytest

import oracle
import weight_activation_quantized_amd as mq
from tests.gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def _check(x, bits, what):
    announce(f"kv_quant {what} bits={bits} shape={x.shape}")
    codes, params = mq.kv_quant(dev(x), bits)
    codes, params = host(codes), host(params)
    rc, rp = oracle.kv_quant_ref(x.reshape(-1, x.shape[-1]), bits)
    assert np.array_equal(params.reshape(-1, 2).view(np.uint32), rp.view(np.uint32)), f"{what}: params differ"
    bad = np.argwhere(codes.reshape(rc.shape) != rc)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    return codes, params


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("shape", [(4096, 32, 128), (128, 32, 128), (37, 8, 64), (5, 3, 256), (1000, 512),
                                   (7, 8), (3, 16), (9, 32)],
                         ids=["prefill_4k", "decode_128seq", "h64", "h256", "h512", "h8", "h16", "h32"])
def test_kv_quant_bitexact(shape, bits):
    rng = np.random.default_rng(sum(shape) + bits)
    x = (rng.standard_normal(shape) * rng.uniform(0.1, 4, shape[:-1] + (1,))).astype(np.float16)
    _check(x, bits, "random")


@pytest.mark.parametrize("bits", [8, 4])
def test_kv_quant_edge_rows(bits):
    qmax = 2 ** bits - 1
    D = 512
    rows = []
    jj = np.arange(qmax)
    tie = np.concatenate([[0.0, qmax / 8.0], (jj + 0.5) / 8.0])
    rows.append(np.resize(tie, D))                                   # exact ties
    rows.append(np.resize([-1.953125, 3.802734375, 0.9248046875], D))  # binary32-sensitive quotient (8 bits)
    rows.append(np.resize([-3.423828125, 3.794921875, 2.591796875, -2.220703125], D))
    rows.append(np.full(D, 1.5))                                     # constant
    rows.append(np.resize([-0.0, 0.0], D))                           # signed zeros
    rows.append(np.resize([-0.0, 0.0, 1.0, 0.5], D))
    rows.append(np.resize([65504.0, -65504.0, 0.0], D))              # fp16 extremes
    rows.append(np.resize([6e-8, -6e-8, 0.0], D))                    # subnormals
    x = np.array(rows).astype(np.float16)
    codes, params = _check(x, bits, "edge rows")
    assert params[3, 0] == 0 and np.all(codes[3] == 0)
    assert not np.any(np.signbit(params[4]))


@pytest.mark.parametrize("bits", [8, 4])
def test_kv_quant_two_rows_per_group_ragged(bits):
    """Enough rows for two rows per lane group (the large-call form), with a
    ragged last workgroup and the edge rows planted among random ones."""
    qmax = 2 ** bits - 1
    rng = np.random.default_rng(40 + bits)
    x = rng.standard_normal((4099 * 33, 128)).astype(np.float16)
    jj = np.arange(qmax)
    edge = [np.resize(np.concatenate([[0.0, qmax / 8.0], (jj + 0.5) / 8.0]), 128),
            np.full(128, -2.5), np.resize([-0.0, 0.0], 128), np.resize([65504.0, -65504.0, 0.0], 128),
            np.resize([6e-8, -6e-8, 0.0], 128)]
    at = rng.choice(x.shape[0], size=200, replace=False)
    for i, r in enumerate(at):
        x[r] = np.asarray(edge[i % len(edge)], dtype=np.float16)
    x[-1] = np.asarray(edge[0], dtype=np.float16)
    _check(x, bits, "two rows per group, ragged")


def test_kv_quant_dequant_error():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2048, 128)).astype(np.float16)
    for bits in (8, 4):
        codes, params = mq.kv_quant(dev(x), bits)
        xhat = oracle.kv_dequant_ref(host(codes), host(params), bits)
        step = host(params)[:, 0:1].astype(np.float64)
        assert np.all(np.abs(xhat - x.astype(np.float64)) <= 0.5 * step * (1 + 1e-5) + 1e-6)


def _check_bf16(bits16, bits, what):
    import torch
    import synth
    x = torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).cuda().view(torch.bfloat16)
    announce(f"kv_quant bf16 {what} bits={bits} shape={bits16.shape}")
    codes, params = mq.kv_quant(x, bits)
    codes, params = host(codes), host(params)
    xf = synth.bf16_values(bits16).reshape(-1, bits16.shape[-1])
    rc, rp = oracle.kv_quant_ref(xf, bits)
    assert np.array_equal(params.reshape(-1, 2).view(np.uint32), rp.view(np.uint32)), f"{what}: params differ"
    assert np.array_equal(codes.reshape(rc.shape), rc), f"{what}: codes differ"


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("shape", [(4096, 32, 128), (2100, 32, 128), (37, 8, 64), (9, 512)],
                         ids=["prefill_4k", "two_rows_ragged", "h64", "h512"])
def test_kv_quant_bf16_bitexact(shape, bits):
    import synth
    rng = np.random.default_rng(sum(shape) + 100 * bits)
    x = (rng.standard_normal(shape) * rng.uniform(0.1, 4, shape[:-1] + (1,))).astype(np.float32)
    _check_bf16(synth.bf16_bits(x), bits, "random")


@pytest.mark.parametrize("bits", [8, 4])
def test_kv_quant_bf16_edge_rows(bits):
    import synth
    qmax = 2 ** bits - 1
    D = 256
    jj = np.arange(min(qmax, 127))
    rows = [np.resize(np.concatenate([[0.0, qmax / 8.0], (jj + 0.5) / 8.0]), D),   # ties (where bf16 holds them)
            np.full(D, -3.25),                                                     # constant
            np.resize([-0.0, 0.0], D),                                             # signed zeros
            np.resize([0.0, 2.0 ** -130, 2.0 ** -129, 3 * 2.0 ** -131], D),          # subnormal scale
            np.resize([1.0e38, -1.0e38, 0.0], D),                                  # wide but finite span
            np.resize([2.0 ** -126, -(2.0 ** -126), 2.0 ** -127], D)]
    _check_bf16(synth.bf16_bits(np.array(rows, np.float32)), bits, "edge rows")
