"""The CPU oracle against its pins, and the pins against planted mistakes.

The first group runs every pin on the oracle as written. The second plants a
plausible mistake in a copy of one oracle function (on the CPU, never on the
GPU path) and asserts that at least one pin fails, which shows that the pins
can tell a right oracle from a wrong one.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins as P

# ---------------------------------------------------------------------------
# the oracle passes every pin
# ---------------------------------------------------------------------------


def test_nibble_golden():
    P.check_nibble_golden(oracle.unpack_int4)


def test_pack_roundtrip():
    P.check_pack_roundtrip(oracle.unpack_int4)


def test_dequant_exact():
    P.check_dequant_exact(oracle.dequant_w4)


def test_dequant_exact_full_scale_range():
    P.check_dequant_exact_full_range(oracle.dequant_w4)


def test_w4a16_bruteforce():
    P.check_w4a16_bruteforce(oracle.w4a16_ref)


def test_w4a16_special_cases():
    P.check_w4a16_special_cases(oracle.w4a16_ref)


def test_quant_golden():
    P.check_quant_golden(oracle.quant_per_token_int8_ref)


def test_quant_exact_rational():
    P.check_quant_exact_rational(oracle.quant_per_token_int8_ref)


def test_quant_exhaustive():
    P.check_quant_exhaustive(oracle.quant_per_token_int8_ref)


def test_quant_invariants():
    P.check_quant_invariants(oracle.quant_per_token_int8_ref)


def test_acc_bruteforce():
    P.check_acc_bruteforce(oracle.w8a8_acc_ref)


def test_acc_special():
    P.check_acc_special(oracle.w8a8_acc_ref)


def test_w8a8_bruteforce():
    P.check_w8a8_bruteforce(oracle.w8a8_ref)


def test_w8a8_linearity():
    P.check_w8a8_linearity(oracle.w8a8_ref)


def test_block_layout():
    P.check_block_layout(oracle.block_weights_ref)


def test_block_layout_mutants_caught():
    # a transposed index in the layout (h and b swapped, rows reversed in a
    # slot, packed columns rotated, byte index g taken from the wrong lane
    # bits) must fail the pin
    def view6(qw):
        out = oracle.block_weights_ref(qw)
        return out, np.ascontiguousarray(out).view(np.uint8).reshape(out.shape[0], -1, 4, 16, 2, 8)

    def back(v, out):
        return np.ascontiguousarray(v).reshape(-1).view(np.int32).reshape(out.shape)

    def swap_hb(qw):
        out, v = view6(qw)
        return back(v[:, :, [0, 2, 1, 3]], out)

    def reverse_e(qw):
        out, v = view6(qw)
        return back(v[..., ::-1], out)

    def rotate_c(qw):
        out, v = view6(qw)
        j = np.arange(16)
        return back(v[:, :, :, (j // 4) * 4 + (j + 1) % 4], out)

    def swap_g(qw):
        out, v = view6(qw)
        j = np.arange(16)
        return back(v[:, :, :, ((j // 4) ^ 1) * 4 + j % 4], out)

    for mutant in (swap_hb, reverse_e, rotate_c, swap_g):
        with pytest.raises(AssertionError):
            P.check_block_layout(mutant)


def test_kv_quant():
    P.check_kv_quant(oracle.kv_quant_ref)


def test_kv_dequant_inverts_packing():
    rng = np.random.default_rng(5)
    for bits in (8, 4):
        x = rng.standard_normal((6, 64)).astype(np.float16)
        codes, params = oracle.kv_quant_ref(x, bits)
        xhat = oracle.kv_dequant_ref(codes, params, bits)
        assert xhat.shape == x.shape
        assert np.max(np.abs(xhat - x.astype(np.float64))) <= 0.5 * np.max(params[:, 0]) * (1 + 1e-5) + 1e-6


@pytest.mark.parametrize("mode", ["round_half_away", "scale_over_2b", "no_offset", "high_nibble_first",
                                  "float64_divide"])
def test_kv_quant_mutants_caught(mode):
    def mutant(x, bits):
        xf = np.asarray(x).astype(np.float32)
        qmax = np.float32(2 ** bits - (0 if mode == "scale_over_2b" else 1))
        mn, mx = xf.min(1), xf.max(1)
        scale = np.divide(np.subtract(mx, mn, dtype=np.float32), qmax, dtype=np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            sh = xf if mode == "no_offset" else np.subtract(xf, mn[:, None], dtype=np.float32)
            if mode == "float64_divide":
                quo = sh.astype(np.float64) / scale[:, None].astype(np.float64)
            else:
                quo = np.divide(sh, scale[:, None], dtype=np.float32)
            r = np.floor(quo + 0.5) if mode == "round_half_away" else np.rint(quo)
        q = np.where(scale[:, None] > 0, np.clip(np.nan_to_num(r), 0, 2 ** bits - 1), 0).astype(np.int64)
        params = np.stack([scale, mn], 1).astype(np.float32)
        if bits == 8:
            return q.astype(np.uint8), params
        lo, hi = (q[:, 1::2], q[:, 0::2]) if mode == "high_nibble_first" else (q[:, 0::2], q[:, 1::2])
        return (lo | (hi << 4)).astype(np.uint8), params
    with pytest.raises(AssertionError):
        P.check_kv_quant(mutant)


def test_acc_overflow_guard():
    K = (2 ** 31 - 1) // 16129 + 1
    with pytest.raises(OverflowError):
        oracle.w8a8_acc_ref(np.full((1, K), 127, np.int8), np.full((1, K), 127, np.int8))


# ---------------------------------------------------------------------------
# planted mistakes are caught
# ---------------------------------------------------------------------------


def _unpack_reversed(packed):
    words = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    out = np.empty((words.shape[0], words.shape[1] * 8), np.uint8)
    for j in range(8):
        out[:, j::8] = (words >> (4 * (7 - j))) & 0xF
    return out


def _unpack_signed(packed):
    u = oracle.unpack_int4(packed).astype(np.int16)
    return np.where(u >= 8, u - 16, u)


def _unpack_blocked(packed):
    # columns of a word laid out in blocks instead of interleaved
    words = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    R, C = words.shape
    out = np.empty((R, C * 8), np.uint8)
    for j in range(8):
        out[:, j * C:(j + 1) * C] = (words >> (4 * j)) & 0xF
    return out


def _dequant_with(unpack, mode):
    def f(qweight, scales, qzeros, group):
        q = unpack(qweight).astype(np.float32)
        K, N = q.shape
        G = int(group)
        z = unpack(qzeros).astype(np.float32)
        s = np.asarray(scales).astype(np.float32)
        g = np.arange(K) // G
        if mode == "group_mod":
            g = np.arange(K) % (K // G)
        if mode == "no_zero":
            return q * s[g]
        if mode == "plus_zero":
            return (q + z[g]) * s[g]
        if mode == "fp16_product":
            return ((q - z[g]) * s[g]).astype(np.float16).astype(np.float32)
        if mode == "zero_offset":
            return (q - (z[g] + 1)) * s[g]
        return (q - z[g]) * s[g]
    return f


def _w4a16_with(dequant, mode="ok"):
    def f(x, qweight, scales, qzeros, group):
        w = dequant(qweight, scales, qzeros, group)
        if mode == "fp32_acc":
            return (np.asarray(x).astype(np.float32) @ w).astype(np.float64)
        y = np.asarray(x).astype(np.float64) @ w.astype(np.float64)
        if mode == "fp16_out":
            return y.astype(np.float16).astype(np.float64)
        return y
    return f


def _quant_with(mode):
    def f(x):
        xf = np.asarray(x).astype(np.float32)
        a = np.max(np.abs(xf), axis=1)
        s = np.divide(a, np.float32(127.0), dtype=np.float32)
        if mode == "scale_128":
            s = np.divide(a, np.float32(128.0), dtype=np.float32)
        q = np.zeros(xf.shape, np.int8)
        nz = s > 0
        if mode == "mul_recip":
            t = xf[nz] * np.divide(np.float32(127.0), a[nz], dtype=np.float32)[:, None]
        elif mode == "fp64_div":
            t = xf[nz].astype(np.float64) / s[nz, None].astype(np.float64)
        else:
            t = np.divide(xf[nz], s[nz, None], dtype=np.float32)
        if mode == "half_away":
            r = np.sign(t) * np.floor(np.abs(t) + np.float32(0.5))
        elif mode == "trunc":
            r = np.trunc(t)
        else:
            r = np.rint(t)
        q[nz] = np.clip(r, -127, 127).astype(np.int8)
        return q, s
    return f


def _acc_fp32(xq, wq):
    return (np.asarray(xq).astype(np.float32) @ np.asarray(wq).astype(np.float32).T).astype(np.int64)


def _w8a8_with(mode):
    def f(xq, s_tok, wq, s_ch):
        acc = oracle.w8a8_acc_ref(xq, wq).astype(np.float64)
        st = np.asarray(s_tok).astype(np.float64)
        sc = np.asarray(s_ch).astype(np.float64)
        if mode == "swap_scales":
            M, N = acc.shape
            return acc * np.resize(sc, M)[:, None] * np.resize(st, N)[None, :]
        if mode == "fp16_out":
            return (acc * st[:, None] * sc[None, :]).astype(np.float16).astype(np.float64)
        if mode == "tok_only":
            return acc * st[:, None]
        return acc * st[:, None] * sc[None, :]
    return f


def _fails(*checks):
    for check in checks:
        try:
            check()
        except AssertionError:
            return True
    return False


UNPACK_MUTANTS = [_unpack_reversed, _unpack_signed, _unpack_blocked]


@pytest.mark.parametrize("mutant", UNPACK_MUTANTS, ids=lambda f: f.__name__)
def test_unpack_mutants_caught(mutant):
    assert _fails(lambda: P.check_nibble_golden(mutant), lambda: P.check_pack_roundtrip(mutant))


@pytest.mark.parametrize("mode", ["group_mod", "no_zero", "plus_zero", "fp16_product", "zero_offset"])
def test_dequant_mutants_caught(mode):
    d = _dequant_with(oracle.unpack_int4, mode)
    w = _w4a16_with(d)
    assert _fails(lambda: P.check_dequant_exact(d), lambda: P.check_w4a16_bruteforce(w),
                  lambda: P.check_w4a16_special_cases(w))
    assert _fails(lambda: P.check_dequant_exact_full_range(d))


@pytest.mark.parametrize("mode", ["fp32_acc", "fp16_out"])
def test_w4a16_mutants_caught(mode):
    w = _w4a16_with(oracle.dequant_w4, mode)
    assert _fails(lambda: P.check_w4a16_bruteforce(w), lambda: P.check_w4a16_special_cases(w))


def test_w4a16_unpack_mutants_caught_downstream():
    for mutant in UNPACK_MUTANTS:
        w = _w4a16_with(_dequant_with(mutant, "ok"))
        assert _fails(lambda: P.check_w4a16_bruteforce(w), lambda: P.check_w4a16_special_cases(w))


@pytest.mark.parametrize("mode", ["scale_128", "mul_recip", "fp64_div", "half_away", "trunc"])
def test_quant_mutants_caught(mode):
    q = _quant_with(mode)
    assert _fails(lambda: P.check_quant_golden(q), lambda: P.check_quant_invariants(q),
                  lambda: P.check_quant_exact_rational(q), lambda: P.check_quant_exhaustive(q))


def test_quant_correct_copy_passes():
    q = _quant_with("ok")
    P.check_quant_golden(q)
    P.check_quant_exhaustive(q)


def test_acc_mutant_caught():
    assert _fails(lambda: P.check_acc_bruteforce(_acc_fp32), lambda: P.check_acc_special(_acc_fp32))


@pytest.mark.parametrize("mode", ["swap_scales", "fp16_out", "tok_only"])
def test_w8a8_mutants_caught(mode):
    w = _w8a8_with(mode)
    assert _fails(lambda: P.check_w8a8_bruteforce(w), lambda: P.check_w8a8_linearity(w))


def test_int4_checkpoint_layouts():
    P.check_int4_checkpoint(oracle.reorder_int4_ref, oracle.transpose_int4_ref, oracle.pack_int4)


@pytest.mark.parametrize("mode", ["inverse_order", "no_transpose", "order_on_rows", "high_first"])
def test_int4_checkpoint_mutants_caught(mode):
    def fields(words, order):
        f = oracle.unpack_int4(words)
        q = np.empty_like(f)
        inv = [order.index(c) for c in range(8)]
        use = inv if mode == "inverse_order" else list(order)
        for j in range(8):
            q[:, use[j]::8] = f[:, j::8]
        return q

    def pack(q):
        if mode == "high_first":
            q = np.asarray(q)
            q = q.reshape(q.shape[0], -1, 8)[:, :, ::-1].reshape(q.shape[0], -1)
        return oracle.pack_int4(q)

    def reorder(words, order):
        return pack(fields(words, tuple(order)))

    def transpose(words, order):
        order = tuple(order)
        if mode == "order_on_rows":
            q = oracle.unpack_int4(words)
            return pack(np.ascontiguousarray(q.T))
        q = fields(words, order)
        if mode == "no_transpose":
            return pack(q.reshape(q.shape[1], q.shape[0]))
        return pack(np.ascontiguousarray(q.T))

    with pytest.raises(AssertionError):
        P.check_int4_checkpoint(reorder, transpose, pack)


def test_bf16_input_generator():
    # bf16 rounding of the generator: exact values stay, ties go to even,
    # and the values are the upper halves of binary32 words
    x = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 3.0e38, -0.0], np.float32)
    b = synth.bf16_bits(x)
    assert b.tolist() == [0x3F80, 0xC020, 0x3F80, 0x3F82, 0x3F80, 0x7F62, 0x8000]
    v = synth.bf16_values(b)
    assert v[0] == 1.0 and v[1] == -2.5 and v[3] == np.float32(1.0 + 2 ** -6)
    d = synth.w8a8_inputs_bf16(3, 64, 8, tag=9)
    assert np.array_equal(synth.bf16_bits(d["x"]), d["x_bits"])
    x16 = synth.w8a8_inputs(3, 64, 8, tag=9)["x"].astype(np.float32)  # the same draw rounded to fp16
    assert np.all(np.abs(d["x"] - x16) <= 2 ** -7 * np.abs(x16) + 1e-7)
