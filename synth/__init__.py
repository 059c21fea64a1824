"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no packing, unpacking, dequantization, quantization or
matmul). Packed 4-bit tensors are drawn directly as uniformly random 32-bit
words, which is the same as eight independent uniform 4-bit fields per word.

Workload shapes and distributions follow the quantized-linear benchmark
configurations:

* W4A16: activations fp16 ~ N(0, 1), optionally with a fraction of input
  channels (the same channels for every token) multiplied by 20; weights and
  zero points uniform 4-bit; fp16 group scales uniform in [0.005, 0.02]
  (or log-uniform over a stated range of powers of two).
* W8A8: activations fp16 ~ N(0, 1) with 1% outlier channels x20; float
  weights ~ N(0, 0.02) rounded to fp16 (each side quantizes them per output
  channel with its own quantizer). The bf16 form draws the same activations
  and rounds them to bf16 instead.

Every draw comes from ``numpy.random.default_rng`` seeded by a
``SeedSequence`` of integers, with children spawned in a fixed order, so a
(tag, seed) pair always gives the same tensors.
"""

import numpy as np

SCALE_LO = 0.005
SCALE_HI = 0.02
OUTLIER_GAIN = 20.0
WEIGHT_STD = 0.02


def _children(tag, seed, n):
    ss = np.random.SeedSequence([int(tag) & 0xFFFFFFFF, int(seed) & 0xFFFFFFFF])
    return [np.random.default_rng(c) for c in ss.spawn(n)]


def activations(rng_x, rng_idx, M, K, outlier_frac=0.0):
    """fp16 [M, K] ~ N(0, 1); round(outlier_frac*K) channels scaled by 20 in fp32."""
    x = rng_x.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        idx = rng_idx.choice(K, size=n_out, replace=False)
        x[:, idx] *= np.float32(OUTLIER_GAIN)
    return x.astype(np.float16)


def random_words(rng, shape):
    """int32 array whose 4-bit fields are i.i.d. uniform in 0..15."""
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint32).view(np.int32)


def group_scales(rng, shape, scale_log2=None):
    """fp16 group scales: uniform in [0.005, 0.02], or, with
    ``scale_log2 = (lo, hi)``, 2**u with u uniform in [lo, hi] (log-uniform
    magnitudes, as small or large as real checkpoints hold)."""
    if scale_log2 is None:
        return rng.uniform(SCALE_LO, SCALE_HI, size=shape).astype(np.float16)
    lo, hi = scale_log2
    return np.exp2(rng.uniform(lo, hi, size=shape)).astype(np.float16)


def w4a16_inputs(M, K, N, group=128, outlier_frac=0.0, tag=0, seed=0, scale_log2=None):
    """Inputs of one W4A16 layer: dict(x, qweight, scales, qzeros)."""
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    G = K if group == -1 else group
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    r_x, r_idx, r_q, r_s, r_z = _children(tag, seed, 5)
    return {
        "x": activations(r_x, r_idx, M, K, outlier_frac),
        "qweight": random_words(r_q, (K, N // 8)),
        "scales": group_scales(r_s, (K // G, N), scale_log2),
        "qzeros": random_words(r_z, (K // G, N // 8)),
    }


def w4a16_inputs_bf16(M, K, N, group=128, outlier_frac=0.0, tag=0, seed=0, scale_log2=None):
    """As ``w4a16_inputs`` with bf16 activations (the same draws rounded to
    bf16 instead of fp16): dict(x_bits uint16 [M,K], x float32 [M,K] (the
    same values), qweight, scales, qzeros)."""
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    G = K if group == -1 else group
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    r_x, r_idx, r_q, r_s, r_z = _children(tag, seed, 5)
    x = r_x.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        idx = r_idx.choice(K, size=n_out, replace=False)
        x[:, idx] *= np.float32(OUTLIER_GAIN)
    bits = bf16_bits(x)
    return {
        "x_bits": bits, "x": bf16_values(bits),
        "qweight": random_words(r_q, (K, N // 8)),
        "scales": group_scales(r_s, (K // G, N), scale_log2),
        "qzeros": random_words(r_z, (K // G, N // 8)),
    }


def w4a16_weights(K, N, group=128, tag=0, seed=0, scale_log2=None):
    """Weights only (qweight, scales, qzeros), drawn as in ``w4a16_inputs``."""
    G = K if group == -1 else group
    _, _, r_q, r_s, r_z = _children(tag, seed, 5)
    return {
        "qweight": random_words(r_q, (K, N // 8)),
        "scales": group_scales(r_s, (K // G, N), scale_log2),
        "qzeros": random_words(r_z, (K // G, N // 8)),
    }


def w8a8_inputs(M, K, N, outlier_frac=0.01, tag=0, seed=0):
    """Inputs of one W8A8 layer: dict(x fp16 [M,K], wf fp16 [N,K] ~ N(0, 0.02))."""
    r_x, r_idx, r_w = _children(tag, seed, 3)
    wf = r_w.normal(0.0, WEIGHT_STD, size=(N, K)).astype(np.float32)
    return {
        "x": activations(r_x, r_idx, M, K, outlier_frac),
        "wf": wf.astype(np.float16),
    }


def bf16_bits(x32):
    """bfloat16 bit patterns (uint16) of float32 values, rounded to nearest
    even (finite inputs): how a bf16 activation tensor is drawn."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_values(bits):
    """float32 values of bfloat16 bit patterns (exact: the upper half of a binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def w8a8_inputs_bf16(M, K, N, outlier_frac=0.01, tag=0, seed=0):
    """As ``w8a8_inputs`` with bf16 activations: dict(x_bits uint16 [M,K],
    x float32 [M,K] (the same values), wf fp16 [N,K])."""
    r_x, r_idx, r_w = _children(tag, seed, 3)
    x = r_x.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        idx = r_idx.choice(K, size=n_out, replace=False)
        x[:, idx] *= np.float32(OUTLIER_GAIN)
    bits = bf16_bits(x)
    wf = r_w.normal(0.0, WEIGHT_STD, size=(N, K)).astype(np.float32)
    return {"x_bits": bits, "x": bf16_values(bits), "wf": wf.astype(np.float16)}


# Benchmark workloads (name -> shape recipe). Tags keep seeds of different
# workloads apart.
CONFIGS = {
    "c0_w4a16_tiny": dict(kind="w4a16", M=4, K=512, N=512, group=128, outlier_frac=0.0, tag=0),
    "c1_w4a16_gemv": dict(kind="w4a16", Ms=(1, 4, 16), K=4096, N=24576, group=128,
                          outlier_frac=0.005, tag=1),
    "c2_w8a8_prefill": dict(kind="w8a8", M=2048, K=4096, N=4096, outlier_frac=0.01, tag=2),
    "c3a_w4a16_o_proj": dict(kind="w4a16", M=4096, K=4096, N=4096, group=128,
                             outlier_frac=0.0, tag=3),
    "c3b_w4a16_down": dict(kind="w4a16", M=4096, K=12288, N=4096, group=128,
                           outlier_frac=0.0, tag=4),
}

# 8B-shaped GQA decoder layer: hidden 4096, 32 q heads / 8 kv heads, head dim 128.
LAYER_SET = {
    "qkv": dict(K=4096, N=6144),
    "o_proj": dict(K=4096, N=4096),
    "gate_up": dict(K=4096, N=24576),
    "down": dict(K=12288, N=4096),
}
LAYER_SET_MS = (1, 8, 64, 2048)
