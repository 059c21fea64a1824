"""Pins for the CPU oracle: checks against values that do not come from it.

Each ``check_*`` takes the oracle function(s) under test as arguments, so the
same check runs on the real oracle (it must pass) and on copies with a
planted mistake (it must fail; see ``test_oracle.py``). Nothing here calls
the oracle's own helpers to produce an expected value: expected values come
from hand-written fixtures under ``tests/golden/``, independent pure-Python
loops, exact rational arithmetic (``fractions.Fraction``), closed forms and
special cases that reduce to a textbook matmul.
"""

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent helpers (pure Python ints / Fractions; no NumPy arithmetic)
# ----------------------------------------------------------------------------

def loop_pack(fields):
    """Pack a [R, 8C] array of 0..15 values into int32 [R, C]; field j of word c = column 8c+j."""
    fields = [[int(v) for v in row] for row in np.asarray(fields)]
    rows = len(fields)
    cols = len(fields[0]) // 8 if rows else 0
    out = np.zeros((rows, cols), dtype=np.int32)
    for r in range(rows):
        for c in range(cols):
            word = 0
            for j in range(8):
                v = fields[r][8 * c + j]
                assert 0 <= v <= 15
                word |= v << (4 * j)
            if word >= 2 ** 31:
                word -= 2 ** 32
            out[r, c] = word
    return out


def loop_field(word, j):
    """Field j of a 32-bit word, computed on a Python int."""
    return (int(word) & 0xFFFFFFFF) >> (4 * j) & 0xF


def round_half_even(fr):
    """Nearest integer to a Fraction, ties to even."""
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_binary32(fr):
    """Correctly rounded IEEE binary32 value (ties to even) of a Fraction in the normal range."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "outside the normal binary32 range"
    ulp = Fraction(2) ** (e - 23)
    m = round_half_even(a / ulp)
    return sign * m * ulp


def exact_quant_row(xs):
    """Per-token quantization of one row, evaluated in exact rational arithmetic.

    s = binary32(absmax / 127); q = clamp(rne(binary32(x / s)), -127, 127).
    """
    fx = [Fraction(float(v)) for v in xs]
    a = max(abs(v) for v in fx)
    if a == 0:
        return [0] * len(fx), Fraction(0)
    s = round_to_binary32(a / 127)
    q = []
    for v in fx:
        t = round_to_binary32(v / s) if v != 0 else Fraction(0)
        q.append(max(-127, min(127, round_half_even(t))))
    return q, s


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _fp16_values_between(lo, hi):
    """Every finite fp16 value v with lo <= v <= hi (lo >= 0)."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    return bits[(bits >= lo) & (bits <= hi)]


# ----------------------------------------------------------------------------
# unpack
# ----------------------------------------------------------------------------

def check_nibble_golden(unpack):
    for line in _read_golden("nibble_layout.txt"):
        word_s, fields_s = line.split(":")
        word = int(word_s.strip(), 16)
        if word >= 2 ** 31:
            word -= 2 ** 32
        expect = [int(v) for v in fields_s.split()]
        got = unpack(np.array([[word]], dtype=np.int32))
        assert got.shape == (1, 8), got.shape
        assert [int(v) for v in got[0]] == expect, (hex(word), got[0], expect)


def check_pack_roundtrip(unpack):
    rng = np.random.default_rng(1234)
    fields = rng.integers(0, 16, size=(7, 48))
    packed = loop_pack(fields)
    got = unpack(packed)
    assert got.shape == fields.shape
    assert np.array_equal(got.astype(np.int64), fields)
    # a single set field at every position of every word
    for j in range(8):
        f = np.zeros((1, 16), dtype=np.int64)
        f[0, j] = 9
        f[0, 8 + j] = 15
        assert np.array_equal(unpack(loop_pack(f)).astype(np.int64), f)
    # all-zero and all-ones words
    assert np.array_equal(unpack(np.zeros((2, 3), np.int32)), np.zeros((2, 24)))
    assert np.array_equal(unpack(np.full((2, 3), -1, np.int32)), np.full((2, 24), 15))


# ----------------------------------------------------------------------------
# dequant and W4A16 matmul
# ----------------------------------------------------------------------------

def check_dequant_exact(dequant):
    """(q - z) * s is exact in float32 for every (q, z) pair and every fp16 scale in [0.005, 0.02]."""
    svals = _fp16_values_between(0.005, 0.02)
    n = (len(svals) + 7) // 8 * 8
    svals = np.concatenate([svals, svals[: n - len(svals)]])
    G = 16
    K = 16 * G  # group g has zero point g; row k has q = k % 16
    q_fields = np.tile((np.arange(K) % 16)[:, None], (1, n))
    z_fields = np.tile(np.arange(16)[:, None], (1, n))
    qweight = loop_pack(q_fields)
    qzeros = loop_pack(z_fields)
    scales = np.tile(svals[None, :], (16, 1)).astype(np.float16)
    w = dequant(qweight, scales, qzeros, G)
    assert w.dtype == np.float32
    diff = (np.arange(K) % 16 - np.arange(K) // G).astype(np.float64)
    expect = diff[:, None] * svals.astype(np.float64)[None, :]
    assert np.array_equal(w.astype(np.float64), expect)


def check_dequant_exact_full_range(dequant):
    """(q - z) * s is exact in float32 for every (q, z) pair and every finite
    fp16 scale of either sign, subnormals included (an 11-bit significand
    times an integer below 16 needs at most 15 bits, and the smallest product,
    2^-24, is a normal binary32)."""
    pos = np.arange(1, 0x7C00, dtype=np.uint16)
    svals = np.concatenate([pos, pos | np.uint16(0x8000)]).view(np.float16)
    n = (len(svals) + 7) // 8 * 8
    svals = np.concatenate([svals, svals[: n - len(svals)]])
    G = 16
    K = 16 * G  # group g has zero point g; row k has q = k % 16
    # every word of a row holds the same eight fields, so pack one word per row and repeat it
    qweight = np.tile(loop_pack(np.tile((np.arange(K) % 16)[:, None], (1, 8))), (1, n // 8))
    qzeros = np.tile(loop_pack(np.tile(np.arange(16)[:, None], (1, 8))), (1, n // 8))
    scales = np.tile(svals[None, :], (16, 1)).astype(np.float16)
    w = dequant(qweight, scales, qzeros, G)
    assert w.dtype == np.float32
    diff = (np.arange(K) % 16 - np.arange(K) // G).astype(np.float64)
    expect = diff[:, None] * svals.astype(np.float64)[None, :]
    assert np.array_equal(w.astype(np.float64), expect)


def _tiny_w4_case(seed, M=3, K=256, N=16, G=128):
    rng = np.random.default_rng(seed)
    rows = 1 if G == -1 else K // G  # G = -1: one scale / zero point per column over all of K
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(rows, N))
    s = rng.uniform(0.005, 0.02, size=(rows, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    return x, q, z, s


def check_w4a16_bruteforce(w4a16):
    for seed, (M, K, N, G) in enumerate([(3, 256, 16, 128), (2, 384, 24, 128), (1, 128, 8, 128),
                                        (2, 64, 16, 32), (2, 256, 16, 64), (2, 256, 16, -1), (1, 384, 8, -1)]):
        x, q, z, s = _tiny_w4_case(seed, M, K, N, G)
        qweight, qzeros = loop_pack(q), loop_pack(z)
        y = w4a16(x, qweight, s, qzeros, G)
        assert y.shape == (M, N) and y.dtype == np.float64
        for m in range(M):
            for n in range(N):
                terms = []
                for k in range(K):
                    g = 0 if G == -1 else k // G  # per-channel: the one parameter row
                    qv = loop_field(qweight[k, n // 8], n % 8)
                    zv = loop_field(qzeros[g, n // 8], n % 8)
                    terms.append(float(x[m, k]) * (qv - zv) * float(s[g, n]))
                ref = math.fsum(terms)
                assert abs(y[m, n] - ref) <= 1e-12 * (1.0 + abs(ref)), (m, n, y[m, n], ref)


def check_w4a16_special_cases(w4a16):
    rng = np.random.default_rng(7)
    M, K, N, G = 4, 256, 32, 128
    x = rng.standard_normal((M, K)).astype(np.float16)
    # q == z everywhere -> y == 0 exactly
    z = rng.integers(0, 16, size=(K // G, N))
    q = np.repeat(z, G, axis=0)
    s = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float16)
    y = w4a16(x, loop_pack(q), s, loop_pack(z), G)
    assert np.array_equal(y, np.zeros((M, N)))
    # z = 0, s = 1, one-hot columns -> y[:, n] = x[:, perm[n]]
    perm = rng.permutation(K)[:N]
    q = np.zeros((K, N), dtype=np.int64)
    q[perm, np.arange(N)] = 1
    ones = np.ones((K // G, N), np.float16)
    zero = np.zeros((K // G, N), np.int64)
    y = w4a16(x, loop_pack(q), ones, loop_pack(zero), G)
    assert np.array_equal(y, x[:, perm].astype(np.float64))
    # x = identity (M = K) -> y = W_deq, built here by loops
    Kc, Nc = 128, 8
    q = rng.integers(0, 16, size=(Kc, Nc))
    z = rng.integers(0, 16, size=(1, Nc))
    s = rng.uniform(0.005, 0.02, size=(1, Nc)).astype(np.float16)
    eye = np.eye(Kc, dtype=np.float16)
    y = w4a16(eye, loop_pack(q), s, loop_pack(z), 128)
    for k in range(Kc):
        for n in range(Nc):
            assert y[k, n] == (int(q[k, n]) - int(z[0, n])) * float(s[0, n])
    # doubling every scale doubles y exactly
    x, q, z, s = _tiny_w4_case(11, 3, 256, 16, 128)
    y1 = w4a16(x, loop_pack(q), s, loop_pack(z), 128)
    y2 = w4a16(x, loop_pack(q), (s.astype(np.float32) * 2).astype(np.float16), loop_pack(z), 128)
    assert np.array_equal(y2, 2.0 * y1)


# ----------------------------------------------------------------------------
# per-token int8 quantization
# ----------------------------------------------------------------------------

def check_quant_golden(quant):
    for line in _read_golden("quant_rows.txt"):
        xs, ss, qs = [p.split() for p in line.split("|")]
        x = np.array([[float(v) for v in xs]], dtype=np.float16)
        assert np.array_equal(x.astype(np.float64)[0], [float(v) for v in xs]), "fixture not exact in fp16"
        q, s = quant(x)
        assert q.dtype == np.int8 and s.dtype == np.float32
        assert s[0] == np.float32(ss[0]), (xs, s[0], ss[0])
        assert [int(v) for v in q[0]] == [int(v) for v in qs], (xs, q[0], qs)


def check_quant_exact_rational(quant):
    """Random rows (with outlier channels) against exact rational arithmetic."""
    rng = np.random.default_rng(99)
    x = rng.standard_normal((6, 96)).astype(np.float32)
    x[:, rng.choice(96, 2, replace=False)] *= 20
    x[3] *= 1e-3
    x[4] *= 300
    x = x.astype(np.float16)
    q, s = quant(x)
    for m in range(x.shape[0]):
        eq, es = exact_quant_row(x[m])
        assert Fraction(float(s[m])) == es, (m, s[m], es)
        assert [int(v) for v in q[m]] == eq, m


def check_quant_exhaustive(quant):
    """One row per absmax a: every fp16 value in [-a, a]; each code against exact arithmetic.

    This covers every element whose binary32 quotient lands on a half-integer
    (decided by round-half-to-even) and every element where dividing by s and
    multiplying by 127/a disagree.
    """
    for a in (1.0, 0.7001953125, 3.0, 57.46875):
        vals = _fp16_values_between(0.0, a)
        row = np.concatenate([vals, -vals[vals > 0]]).astype(np.float16)
        q, s = quant(row[None, :])
        es = round_to_binary32(Fraction(a) / 127)
        assert Fraction(float(s[0])) == es
        sf = float(es)
        for i, v in enumerate(row):
            fv = Fraction(float(v))
            t = round_to_binary32(fv / es) if v != 0 else Fraction(0)
            e = max(-127, min(127, round_half_even(t)))
            if int(q[0, i]) != e:
                raise AssertionError(f"a={a} x={float(v)} q={int(q[0, i])} expected {e} (s={sf})")


def check_quant_invariants(quant):
    rng = np.random.default_rng(5)
    # |x| >= 0.025 so that every power-of-two rescaling below stays exact in fp16
    mag = rng.uniform(0.5, 1.0, size=(8, 200)) * rng.uniform(0.05, 50, size=(8, 1))
    x = (rng.choice([-1.0, 1.0], size=(8, 200)) * mag).astype(np.float16)
    q, s = quant(x)
    # the absmax element maps to +-127
    for m in range(8):
        i = int(np.argmax(np.abs(x[m].astype(np.float32))))
        assert abs(int(q[m, i])) == 127 and np.sign(q[m, i]) == np.sign(x[m, i])
    # odd symmetry
    qn, sn = quant(-x)
    assert np.array_equal(sn, s) and np.array_equal(qn, -q)
    # power-of-two equivariance: quant(2^j x) = (q, 2^j s)
    for j in (-3, -1, 1, 2):
        xj = (x.astype(np.float32) * np.float32(2.0 ** j)).astype(np.float16)
        assert np.array_equal(xj.astype(np.float32), x.astype(np.float32) * np.float32(2.0 ** j))
        qj, sj = quant(xj)
        assert np.array_equal(qj, q) and np.array_equal(sj, s * np.float32(2.0 ** j))
    # rows q0 * 2^-j with |q0| = 127 somewhere round-trip exactly
    for j in range(0, 9):
        q0 = rng.integers(-127, 128, size=(3, 64))
        q0[:, 5] = 127
        q0[1, 5] = -127
        xr = (q0 * 2.0 ** -j).astype(np.float16)
        qr, sr = quant(xr)
        assert np.array_equal(qr.astype(np.int64), q0)
        assert np.all(sr == np.float32(2.0 ** -j))
    # all-zero row
    qz, sz = quant(np.zeros((2, 32), np.float16))
    assert np.all(qz == 0) and np.all(sz == 0)
    # range
    assert q.min() >= -127 and q.max() <= 127


# ----------------------------------------------------------------------------
# int32 accumulator and W8A8 output
# ----------------------------------------------------------------------------

def check_acc_bruteforce(acc_fn):
    rng = np.random.default_rng(3)
    for M, N, K in [(3, 5, 32), (2, 7, 64), (4, 3, 1500)]:
        xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        acc = acc_fn(xq, wq)
        for m in range(M):
            for n in range(N):
                ref = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))
                assert int(acc[m, n]) == ref


def check_acc_special(acc_fn):
    rng = np.random.default_rng(4)
    K = 64
    xq = rng.integers(-127, 128, size=(5, K)).astype(np.int8)
    assert np.array_equal(acc_fn(xq, np.eye(K, dtype=np.int8)), xq.astype(np.int64))
    K = 12288
    plus = np.full((2, K), 127, np.int8)
    minus = np.full((3, K), -127, np.int8)
    assert np.all(acc_fn(plus, minus) == -16129 * K)
    assert np.all(acc_fn(minus, minus) == 16129 * K)
    # the largest K whose worst case still fits int32
    K = (2 ** 31 - 1) // 16129
    assert np.all(acc_fn(np.full((1, K), 127, np.int8), np.full((1, K), 127, np.int8)) == 16129 * K)


def check_w8a8_bruteforce(w8a8):
    rng = np.random.default_rng(8)
    M, N, K = 3, 5, 96
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    st = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sc = rng.uniform(1e-4, 1e-3, size=N).astype(np.float32)
    y = w8a8(xq, st, wq, sc)
    assert y.shape == (M, N) and y.dtype == np.float64
    for m in range(M):
        for n in range(N):
            acc = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))
            exact = Fraction(acc) * Fraction(float(st[m])) * Fraction(float(sc[n]))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def check_w8a8_linearity(w8a8):
    rng = np.random.default_rng(9)
    M, N, K = 4, 6, 128
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    st = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sc = rng.uniform(1e-4, 1e-3, size=N).astype(np.float32)
    y = w8a8(xq, st, wq, sc)
    assert np.array_equal(w8a8(xq, st * np.float32(4), wq, sc), 4 * y)
    assert np.array_equal(w8a8(xq, st, wq, sc * np.float32(0.5)), 0.5 * y)
    # scaling one token's scale scales only that row
    st2 = st.copy()
    st2[1] *= 8
    y2 = w8a8(xq, st2, wq, sc)
    assert np.array_equal(y2[1], 8 * y[1]) and np.array_equal(np.delete(y2, 1, 0), np.delete(y, 1, 0))
    # unit scales give the accumulator itself
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    acc = w8a8(xq, ones_m, wq, ones_n)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))


def check_block_layout(block):
    """The blocked decode layout moves bytes without changing them, puts the
    slots of all strips for one 64-row pair next to each other and gives
    every 16-byte lane slot byte g of eight consecutive rows (twice: two
    32-row blocks) of one packed column, in the order documented in mq.h."""
    for K, N in [(128, 32), (256, 96), (384, 64)]:
        NP = N // 8
        S = N // 32
        kk = np.arange(K)[:, None, None]
        cc = np.arange(NP)[None, :, None]
        gg = np.arange(4)[None, None, :]
        # two encodings of the source position in the byte value itself:
        # (a) the row (K <= 384: row % 256 plus a separate check of row // 256),
        # (b) the packed column and the byte index
        for enc in ("row", "colbyte", "rowhigh"):
            if enc == "row":
                byt = np.broadcast_to(kk % 256, (K, NP, 4))
            elif enc == "colbyte":
                byt = np.broadcast_to(cc * 4 + gg, (K, NP, 4))
            else:
                byt = np.broadcast_to(kk // 256, (K, NP, 4))
            qw = np.ascontiguousarray(byt.astype(np.uint8)).view(np.int32).reshape(K, NP)
            out = block(qw)
            assert out.shape == (K // 64, 8 * N) and out.dtype == np.int32
            ob = np.ascontiguousarray(out).view(np.uint8).reshape(K // 64, S, 4, 16, 2, 8)  # P, s, h, j, b, e
            for s in range(S):
                for P in range(K // 64):
                    for h in range(4):
                        for j in range(16):
                            c, g = 4 * s + j % 4, j // 4
                            for b in range(2):
                                rows = 64 * P + 32 * b + 8 * h + np.arange(8)
                                got = ob[P, s, h, j, b]
                                if enc == "row":
                                    assert np.array_equal(got, rows % 256)
                                elif enc == "colbyte":
                                    assert np.all(got == c * 4 + g)
                                else:
                                    assert np.array_equal(got, rows // 256)
    # bytes are moved, never changed: arbitrary bit patterns survive as a multiset
    rng = np.random.default_rng(3)
    qw = rng.integers(-2 ** 31, 2 ** 31, size=(256, 32), dtype=np.int64).astype(np.int32)
    out = block(qw)
    assert np.array_equal(np.sort(out.view(np.uint8).ravel()), np.sort(qw.view(np.uint8).ravel()))


def _kv_exact(x, bits):
    """kv_quant by exact rational arithmetic with the same IEEE binary32 roundings."""
    from fractions import Fraction
    qmax = 2 ** bits - 1
    codes, params = [], []
    for row in np.asarray(x).astype(np.float32):
        mn, mx = Fraction(float(row.min())), Fraction(float(row.max()))
        span = round_to_binary32(mx - mn) if mx != mn else Fraction(0)
        scale = round_to_binary32(span / qmax) if span != 0 else Fraction(0)
        qs = []
        for v in row:
            if scale == 0:
                qs.append(0)
                continue
            d = Fraction(float(v)) - mn
            d = round_to_binary32(d) if d != 0 else Fraction(0)
            t = round_to_binary32(d / scale) if d != 0 else Fraction(0)
            fl = t.numerator // t.denominator
            frac = t - fl
            r = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            qs.append(min(max(r, 0), qmax))
        codes.append(qs)
        params.append((float(scale), float(mn)))
    return np.array(codes, dtype=np.int64), np.array(params, dtype=np.float64)


def _kv_unpack(codes, bits):
    c = np.asarray(codes).astype(np.int64)
    if bits == 8:
        return c
    q = np.empty((c.shape[0], 2 * c.shape[1]), np.int64)
    q[:, 0::2] = c & 15
    q[:, 1::2] = c >> 4
    return q


def check_kv_quant(kvq):
    rng = np.random.default_rng(11)
    for bits in (8, 4):
        qmax = 2 ** bits - 1
        # exact rational arithmetic on random rows (normal, shifted, wide)
        x = np.concatenate([rng.standard_normal((4, 16)), 3 + 0.01 * rng.standard_normal((2, 16)),
                            rng.uniform(-60, 60, (2, 16))]).astype(np.float16)
        codes, params = kvq(x, bits)
        q = _kv_unpack(codes, bits)
        eq, ep = _kv_exact(x, bits)
        assert np.array_equal(q, eq), bits
        assert np.array_equal(params.astype(np.float64), ep)
        # the row minimum codes to 0 and the maximum to qmax
        for r in range(x.shape[0]):
            assert q[r, np.argmin(x[r].astype(np.float32))] == 0
            assert q[r, np.argmax(x[r].astype(np.float32))] == qmax
        # round trip of values on the code grid: x = mn + j * 2^-e (scale a power of two)
        j = rng.integers(0, qmax + 1, size=(3, 32))
        j[:, 0], j[:, 1] = 0, qmax
        for e, mn in ((3, -1.0), (6, 0.5), (1, -8.0)):
            grid = (mn + j * 2.0 ** -e).astype(np.float16)
            assert np.array_equal(grid.astype(np.float64), mn + j * 2.0 ** -e)  # exact in fp16
            c2, p2 = kvq(grid, bits)
            assert np.all(p2[:, 0] == np.float32(2.0 ** -e * qmax) / np.float32(qmax))
            assert np.array_equal(_kv_unpack(c2, bits), j)
        # exact ties: min 0, max qmax/8 (scale 1/8 exactly), values (j + 1/2)/8:
        # every quotient is j + 1/2, so rounding half to even decides it
        jj = np.arange(qmax)
        tie = np.concatenate([[0.0, qmax / 8.0], (jj + 0.5) / 8.0, [0.0]]).astype(np.float16)[None, :]
        c6, p6 = kvq(tie, bits)
        assert p6[0, 0] == np.float32(0.125) and p6[0, 1] == 0
        want = jj + (jj % 2)  # j + 1/2 -> the even neighbour
        assert np.array_equal(_kv_unpack(c6, bits)[0, 2:2 + qmax], want)
        # every fp16 value in [-1, 1] in one row (min -1, max 1, an inexact
        # scale): against exact rational arithmetic with the same roundings
        if bits == 4:
            h = np.arange(0, 0x3C01, 7, dtype=np.uint16)
        else:
            h = np.arange(0, 0x3C01, 3, dtype=np.uint16)
        vals = np.concatenate([h.view(np.float16), (h | 0x8000).view(np.float16)])
        sweep = np.concatenate([[np.float16(-1), np.float16(1)], vals])
        if sweep.size % 2:
            sweep = np.append(sweep, np.float16(0))
        sweep = sweep[None, :].astype(np.float16)
        c7, p7 = kvq(sweep, bits)
        e7, ep7 = _kv_exact(sweep, bits)
        assert np.array_equal(_kv_unpack(c7, bits), e7) and np.array_equal(p7.astype(np.float64), ep7)
        # rows where the binary32 quotient rounds to a different code than the
        # exact one would (found by searching all fp16 values between a min
        # and a max): the IEEE binary32 division decides
        near = {8: [-1.953125, 3.802734375, 0.9248046875, 0.0],
                4: [-3.423828125, 3.794921875, 2.591796875, -2.220703125]}[bits]
        nr = np.array([near], np.float16)
        c8, p8 = kvq(nr, bits)
        e8, ep8 = _kv_exact(nr, bits)
        assert np.array_equal(_kv_unpack(c8, bits), e8) and np.array_equal(p8.astype(np.float64), ep8)
        # a row whose minimum is -0 stores +0
        z = np.array([[-0.0, 0.0, 1.0, 0.5], [-0.0, 0.0, -0.0, 0.0], [0.0, -0.0, -0.0, -0.0]], np.float16)
        _, pz = kvq(z, bits)
        assert np.all(pz[:, 1] == 0) and not np.any(np.signbit(pz[:, 1]))
        assert np.all(pz[1:, 0] == 0) and not np.any(np.signbit(pz[1:, 0]))
        # constant rows: scale 0, codes 0, offset = the value
        cst = np.full((2, 8), 1.5, np.float16)
        c3, p3 = kvq(cst, bits)
        assert np.all(_kv_unpack(c3, bits) == 0) and np.all(p3[:, 0] == 0) and np.all(p3[:, 1] == 1.5)
        # packing of 4-bit codes: element 2i in the low nibble
        if bits == 4:
            row = np.array([[0, 15, 1, 14, 2, 13, 3, 12]], np.float16)
            c4, _ = kvq(row, 4)
            assert c4.tolist() == [[0xF0, 0xE1, 0xD2, 0xC3]]
        # dequantization error is at most half a step (plus binary32 rounding)
        xs = rng.standard_normal((16, 128)).astype(np.float16)
        c5, p5 = kvq(xs, bits)
        xhat = _kv_unpack(c5, bits) * p5[:, 0:1].astype(np.float64) + p5[:, 1:2].astype(np.float64)
        err = np.abs(xhat - xs.astype(np.float64))
        assert np.all(err <= 0.5 * p5[:, 0:1] * (1 + 1e-5) + 1e-6)


# ----------------------------------------------------------------------------
# checkpoint layouts (field order, packing axis)
# ----------------------------------------------------------------------------

CHECKPOINT_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def _words(vals):
    return np.array([int(v, 16) for v in vals], dtype=np.uint32).view(np.int32)


def _loop_pack_rows(q, order):
    """Explicit loops: word c of row r holds column 8c + order[j] in field j."""
    R, C8 = len(q), len(q[0])
    out = np.zeros((R, C8 // 8), dtype=np.uint32)
    for r in range(R):
        for c in range(C8 // 8):
            w = 0
            for j in range(8):
                w |= int(q[r][8 * c + order[j]]) << (4 * j)
            out[r, c] = w
    return out.view(np.int32)


def _loop_unpack_rows(words):
    """Explicit loops, library order: column 8c + j is field j of word c."""
    u = np.asarray(words).view(np.uint32)
    R, C = u.shape
    return [[(int(u[r, k // 8]) >> (4 * (k % 8))) & 15 for k in range(8 * C)] for r in range(R)]


def check_int4_checkpoint(reorder, transpose, pack):
    for line in _read_golden("checkpoint_words.txt"):
        kind, rest = line.split(None, 1)
        src, dst = [t.split() for t in rest.split("->")]
        if kind == "reorder":
            got = reorder(_words(src).reshape(1, 1), CHECKPOINT_ORDER)
            assert got.view(np.uint32).tolist() == [[int(dst[0], 16)]], line
        else:
            got = transpose(_words(src).reshape(8, 1), tuple(range(8)))
            assert got.view(np.uint32).ravel().tolist() == [int(v, 16) for v in dst], line
    rng = np.random.default_rng(5)
    for order in (CHECKPOINT_ORDER, tuple(range(8)), tuple(rng.permutation(8).tolist())):
        q = rng.integers(0, 16, size=(16, 24))
        src = _loop_pack_rows(q.tolist(), order)
        # reorder keeps the matrix and its shape, in the library's order
        assert _loop_unpack_rows(reorder(src, order)) == q.tolist()
        # transpose gives q^T packed along the new rows
        t = transpose(src, order)
        assert t.shape == (24, 2)
        assert _loop_unpack_rows(t) == q.T.tolist()
    # pack is unpack's inverse (unpack is pinned by nibble_layout.txt)
    q = rng.integers(0, 16, size=(5, 40))
    w = pack(q)
    assert w.dtype == np.int32 and w.shape == (5, 5)
    assert _loop_unpack_rows(w) == q.tolist()
    # the library order is a fixed point; transposing twice is the identity
    w = rng.integers(-2 ** 31, 2 ** 31, size=(16, 4), dtype=np.int64).astype(np.int32)
    assert np.array_equal(reorder(w, tuple(range(8))), w)
    assert np.array_equal(transpose(transpose(w, tuple(range(8))), tuple(range(8))), w)
