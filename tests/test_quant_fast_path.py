"""The int8 quantizer's fast path, emulated in NumPy (CPU).

pymllm Setup and Usage, section "W8A8 first-run JIT compilation": the per-token
quantizer feeds the int8 scaled matmul; its codes are those of the IEEE
binary32 quotient x / s rounded half to even (the oracle's reading).

The kernel does not divide per element. With r = rcp(s) (the hardware
reciprocal, within one ulp of 1/s) it forms p = fl32(x * r + 128) with one
fused multiply-add and u = rint(p); when |p - u| <= 0.5 - 2^-12 it takes
u - 128 as the code, and only otherwise divides. This test runs that decision
in float32 for each of the three reciprocals one ulp apart around 1/s
(whatever the hardware returns is one of them) and checks every fast-path code
against the oracle's, on the W8A8 activation workload (2048 x 4096 with
outlier channels) and on binary32 values placed next to the rounding
boundaries (the kernel widens fp16 and bf16 exactly, so binary32 inputs cover
both). The second test plants a mistake, no margin at all, and shows that the
near-boundary rows catch it.
"""

import numpy as np

from oracle import quant_per_token_int8_ref
import synth

MARGIN = np.float32(0.5) - np.float32(1.0 / 4096.0)  # 0x3EFFE000, as the kernel folds it


def _fast_codes(x, s, r, margin=MARGIN):
    """(codes, fast mask) of the kernel's fast path for rows x [M, K] float32,
    scales s [M] and reciprocals r [M] (float32)."""
    # fl32(x * r + 128) with one rounding: the float64 product of two binary32
    # values is exact, the sum with 128 is exact in float64, the cast rounds once.
    p = (x.astype(np.float64) * r.astype(np.float64)[:, None] + 128.0).astype(np.float32)
    u = np.rint(p)
    fast = np.abs(p - u) <= margin  # p - u is exact (Sterbenz)
    return (u - np.float32(128)).astype(np.int32), fast


def _reciprocals(s):
    r0 = (np.float32(1.0) / s).astype(np.float32)
    return [np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(np.inf))]


def _near_ties(rng, M=512, K=1024):
    """binary32 rows whose quotients sit within 4e-4 of half-integers."""
    s = rng.uniform(0.005, 0.05, size=M).astype(np.float32)
    k = rng.integers(-127, 127, size=(M, K)).astype(np.float32) + np.float32(0.5)
    eps = (rng.choice([-1, 1], size=(M, K)) * rng.uniform(0, 4e-4, size=(M, K))).astype(np.float32)
    x = ((k + eps) * s[:, None]).astype(np.float32)
    x[:, 0] = np.float32(127) * s  # the row maximum: the oracle's scale is s within an ulp
    return x


def test_fast_path_codes_equal_the_oracle():
    inputs = [synth.w8a8_inputs(2048, 4096, 8, outlier_frac=0.01, tag=2)["x"].astype(np.float32),
              _near_ties(np.random.default_rng(7))]
    for x in inputs:
        q_ref, s = quant_per_token_int8_ref(x)
        assert np.all(s > 0)
        for r in _reciprocals(s):
            codes, fast = _fast_codes(x, s, r)
            assert np.array_equal(codes[fast], q_ref.astype(np.int32)[fast])
            # on the workload the division is the exception (about 1 element
            # in 2000); the near-boundary rows put about 40% of theirs inside it
            assert fast.mean() > 0.999 if x.shape[0] == 2048 else 0.3 < fast.mean() < 0.5


def test_planted_narrow_margin_is_caught():
    # With no margin at all (every element takes u - 128) the near-tie rows
    # disagree with the oracle somewhere for some reciprocal.
    x = _near_ties(np.random.default_rng(11))
    q_ref, s = quant_per_token_int8_ref(x)
    mismatches = 0
    for r in _reciprocals(s):
        codes, fast = _fast_codes(x, s, r, margin=np.float32(0.5))
        mismatches += int(np.sum(codes[fast] != q_ref.astype(np.int32)[fast]))
    assert mismatches > 0
