"""The W4A16 GEMM's weight-fragment arithmetic, emulated in NumPy float16 (CPU).

LMDeploy 4-bit deployment guide, section 2.2: the group scale is applied
inside the matmul kernel. The GEMM forms each weight operand from its 4-bit
field q, the group's zero point z and the fp16 scale s in three fp16 steps:

1. the field, OR-ed into the bit pattern of a power of two, reads as an
   offset integer: bits 0-3 of a 16-bit half into 1024.0 (0x6400) read
   1024 + q; bits 4-7 into 64.0 (0x5400), whose mantissa step is 1/16, read
   64 + q;
2. the zero point, encoded the same way with the sign set (0xE400 | z or
   0xD400 | z << 4), is added: the sum is q - z exactly;
3. one multiply by s, which rounds once to fp16((q - z) * s).

This test runs those steps for every (q, z) pair and every finite fp16
scale of either sign (subnormals included) and compares each result with
(q - z) * s computed exactly in float64 and rounded once to fp16. A scale
whose product overflows fp16 (|(q - z) * s| >= 65520) is outside the
contract and skipped.

The earlier form read the high field as 1024 + 16q and multiplied by s/16
formed in fp16; for |s| < 2^-10 that quotient is an fp16 subnormal and the
weight was rounded twice. The second test keeps that form as a planted
mistake and shows the comparison catches it.
"""

import numpy as np


def _all_scales():
    pos = np.arange(1, 0x7C00, dtype=np.uint16)
    return np.concatenate([pos, pos | np.uint16(0x8000)]).view(np.float16)


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


def _fragments(q, z, s, odd, legacy=False):
    """The kernel's three fp16 steps, vectorised: q, z int arrays; s fp16."""
    q = q.astype(np.uint16)
    z = z.astype(np.uint16)
    if not odd:
        v = _f16(np.uint16(0x6400) | q)           # 1024 + q
        nz = _f16(np.uint16(0xE400) | z)          # -(1024 + z)
        sc = s
    elif legacy:
        v = _f16(np.uint16(0x6400) | (q << 4))    # 1024 + 16 q
        nz = _f16(np.uint16(0xE400) | (z << 4))   # -(1024 + 16 z)
        sc = (s * np.float16(0.0625)).astype(np.float16)
    else:
        v = _f16(np.uint16(0x5400) | (q << 4))    # 64 + q
        nz = _f16(np.uint16(0xD400) | (z << 4))   # -(64 + z)
        sc = s
    d = (v + nz).astype(np.float16)               # exact
    with np.errstate(over="ignore"):              # out-of-contract products become inf
        return (d * sc).astype(np.float16)        # one rounding (exact product, rounded to fp16)


def _grid():
    s = _all_scales()
    q, z = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    q = q.reshape(-1, 1)
    z = z.reshape(-1, 1)
    exact = (q - z).astype(np.float64) * s.astype(np.float64)[None, :]
    keep = np.abs(exact) < 65520.0
    return q, z, s[None, :], exact, keep


def test_fragment_offsets_exact():
    # step 1 and 2 alone: the offsets read exactly and cancel to q - z
    for q in range(16):
        assert float(_f16(0x6400 | q)) == 1024 + q
        assert float(_f16(0x5400 | (q << 4))) == 64 + q
        for z in range(16):
            assert float(_f16(0x5400 | (q << 4)) + _f16(0xD400 | (z << 4))) == q - z
            assert float(_f16(0x6400 | q) + _f16(0xE400 | z)) == q - z


def test_fragment_rounded_once_every_scale():
    q, z, s, exact, keep = _grid()
    with np.errstate(over="ignore"):
        want = exact.astype(np.float16)
    for odd in (False, True):
        got = _fragments(q, z, s, odd)
        same = (got.view(np.uint16) == want.view(np.uint16)) | (~keep)
        assert same.all(), f"odd={odd}: {int((~same).sum())} weights differ from fp16((q - z) * s)"


def test_legacy_high_field_form_is_caught():
    q, z, s, exact, keep = _grid()
    with np.errstate(over="ignore"):
        want = exact.astype(np.float16)
    got = _fragments(q, z, s, odd=True, legacy=True)
    bad = (got.view(np.uint16) != want.view(np.uint16)) & keep
    assert bad.any()
    # every mismatch has |s| below 2^-10, where s/16 is an fp16 subnormal
    smag = np.abs(np.broadcast_to(s, bad.shape).astype(np.float64))
    assert np.all(smag[bad] < 2.0 ** -10)
