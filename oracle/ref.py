"""Plain CPU definitions of the quantized linear layer (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the HIP library never imports it and it imports nothing from the HIP
side.

Sources (pages; each function cites the passage it follows):

* [pymllm-setup]  "pymllm Setup and Usage" -- Overview (BF16, W4A16 and
  W8A8_INT8 schemes; INT8 tensor-core compute), section "W8A8 first-run JIT
  compilation" (per-token int8 activation quantizer; int8 scaled matmul).
* [lmdeploy-ovw]  LMDeploy toolkit overview (devpress) -- section 2.4
  "KV Cache online quantization" (per-head per-token asymmetric INT8/INT4,
  min/max computed online) and section 2.5 "Weight quantization (AWQ)"
  (4-bit weights, group size 128).
* [lmdeploy-hw]   "LMDeploy multimodal LLM 4-bit quantization deployment
  guide" (mlqm) -- section 2.2 (AWQ w4a16; scale and weight consumed in one
  kernel), section 3.2 (per-layer bits / group_size, -1 = no grouping).

Layouts (all row-major, contiguous):
    x        fp16  [M, K]        activations
    qweight  int32 [K, N/8]      uint4 weights, 8 per word along N
    scales   fp16  [K/G, N]      per-group scales
    qzeros   int32 [K/G, N/8]    uint4 zero points, packed like qweight
    xq       int8  [M, K]        quantized activations
    s_tok    fp32  [M]           per-token scales
    wq       int8  [N, K]        int8 weights, one row per output channel
    s_ch     fp32  [N]           per-output-channel scales
"""

import numpy as np

NIBBLES_PER_WORD = 8


def unpack_int4(packed):
    """Split each 32-bit word into its eight 4-bit fields.

    Reading (the pages give no bit layout): field j of word c, counted from
    the least significant bit, is column ``8*c + j``; fields are unsigned
    (0..15). The same layout holds for weights and zero points.

    packed: integer array [R, C] (int32 bit patterns) -> uint8 [R, 8*C].
    """
    packed = np.asarray(packed)
    if packed.ndim != 2:
        raise ValueError("packed must be 2-D")
    words = packed.astype(np.int64) & 0xFFFFFFFF  # reinterpret as unsigned
    rows, cols = words.shape
    out = np.empty((rows, cols * NIBBLES_PER_WORD), dtype=np.uint8)
    for j in range(NIBBLES_PER_WORD):
        out[:, j::NIBBLES_PER_WORD] = (words >> (4 * j)) & 0xF
    return out


def dequant_w4(qweight, scales, qzeros, group):
    """W4A16 group dequantization, w[k, n] = (q[k, n] - z[k // G, n]) * s[k // G, n].

    [lmdeploy-ovw] section 2.5 and [lmdeploy-hw] section 2.2: asymmetric
    4-bit weights with one scale and one zero point per group of G
    consecutive input channels (k) of each output column n. G = 128 on the
    pages; ``group = -1`` ([lmdeploy-hw] section 3.2) means one group
    spanning all of K.

    The product is formed in float32; it is exact there because |q - z| <= 15
    and an fp16 scale has an 11-bit significand (pinned exhaustively in the
    tests). Returns float32 [K, N].
    """
    q = unpack_int4(qweight).astype(np.float32)
    K, N = q.shape
    G = K if group == -1 else int(group)
    if G <= 0 or K % G != 0:
        raise ValueError("K must be a multiple of the group size")
    z = unpack_int4(qzeros).astype(np.float32)
    s = np.asarray(scales).astype(np.float32)
    if z.shape != (K // G, N) or s.shape != (K // G, N):
        raise ValueError("scales / qzeros shape does not match [K/G, N]")
    g = np.arange(K) // G
    return (q - z[g, :]) * s[g, :]


def w4a16_ref(x, qweight, scales, qzeros, group):
    """W4A16 linear layer, y = x @ W_deq, unrounded, in float64.

    [lmdeploy-ovw] section 2.5 (4-bit weights with 16-bit activations) and
    [pymllm-setup] Overview (the W4A16 scheme). Activations are fp16 and are
    widened exactly; the dequantized weights are exact (``dequant_w4``); the
    matmul accumulates in float64. The result is NOT rounded to fp16: a GPU
    output is compared with this value directly.

    x: fp16 [M, K] -> float64 [M, N].
    """
    w = dequant_w4(qweight, scales, qzeros, group).astype(np.float64)
    xf = np.asarray(x).astype(np.float64)
    if xf.ndim != 2 or xf.shape[1] != w.shape[0]:
        raise ValueError("x must be [M, K]")
    return xf @ w


def block_weights_ref(qweight):
    """Column-blocked decode layout of qweight [K, N/8]: its bytes reordered, unchanged.

    [lmdeploy-hw] deployment steps: the AWQ checkpoint is converted once into
    the inference engine's own weight format before serving. The pages do
    not describe that format; the reading here is a byte order in which the
    32 outputs of strip s (packed columns 4s .. 4s+3) over all of K are
    next to each other in memory for every 64 rows. Byte g of word (k, c)
    holds the two 4-bit weights of columns 8c + 2g and 8c + 2g + 1 of row k.
    Rows come in 64-row pairs P; with S = N/32 strips, slot (P, s) holds, for
    lane L = 16h + j (c = j % 4, g = j // 4), 16 bytes, byte 8b + e being
    byte g of word (64P + 32b + 8h + e, 4s + c):

        blocked_bytes[((P * S + s) * 64 + L) * 16 + 8 * b + e]
            = byte g of qweight[64 * P + 32 * b + 8 * h + e, 4 * s + c]

    qweight: int32 [K, N/8] with K % 128 == 0, N % 32 == 0
    -> int32 [K/64, 8 * N] (the same bytes, little-endian words; row P holds
    the 64-row pair P of every strip).
    """
    qw = np.ascontiguousarray(np.asarray(qweight, dtype=np.int32))
    if qw.ndim != 2:
        raise ValueError("qweight must be [K, N/8]")
    K, NP = qw.shape
    if K % 128 or NP % 4:
        raise ValueError("the blocked layout needs K % 128 == 0 and N % 32 == 0")
    S = NP // 4
    by = qw.view(np.uint8).reshape(K, NP, 4)  # little-endian: byte g of word (k, c) = by[k, c, g]
    # index grids over (P, s, h, j, b, e) in the order of the blocked bytes
    P, s, h, j, b, e = np.meshgrid(np.arange(K // 64), np.arange(S), np.arange(4), np.arange(16),
                                   np.arange(2), np.arange(8), indexing="ij")
    rows = 64 * P + 32 * b + 8 * h + e
    cols = 4 * s + j % 4
    g = j // 4
    out = by[rows, cols, g].reshape(K // 64, 64 * S * 16)
    return np.ascontiguousarray(out).view(np.int32)


def pack_int4(q):
    """Pack 4-bit values into words in the library's order: column ``8*c + j``
    of q goes to field j (bits 4j..4j+3) of word c -- the inverse of
    ``unpack_int4``.

    q: integer array [R, 8*C] with values 0..15 -> int32 [R, C].
    """
    q = np.asarray(q).astype(np.int64)
    if q.ndim != 2 or q.shape[1] % NIBBLES_PER_WORD:
        raise ValueError("q must be [R, 8*C]")
    if np.any((q < 0) | (q > 15)):
        raise ValueError("4-bit values must lie in 0..15")
    words = np.zeros((q.shape[0], q.shape[1] // NIBBLES_PER_WORD), dtype=np.int64)
    for j in range(NIBBLES_PER_WORD):
        words |= q[:, j::NIBBLES_PER_WORD] << (4 * j)
    return words.astype(np.uint32).view(np.int32)


def _fields_to_columns(words, field_order):
    """4-bit matrix [R, 8*C] of words whose field j holds column 8*c + field_order[j]."""
    order = [int(v) for v in field_order]
    if sorted(order) != list(range(NIBBLES_PER_WORD)):
        raise ValueError("field_order must be a permutation of 0..7")
    f = unpack_int4(words)  # f[:, 8c + j] = field j of word c
    q = np.empty_like(f)
    for j in range(NIBBLES_PER_WORD):
        q[:, order[j]::NIBBLES_PER_WORD] = f[:, j::NIBBLES_PER_WORD]
    return q


def reorder_int4_ref(words, field_order):
    """Checkpoint words with another field order -> the library's order.

    [lmdeploy-ovw] sections 4.1 and 5.5 load 4-bit checkpoints with
    ``model_format="awq"``, [lmdeploy-hw] converts them with
    ``--model-format awq`` before serving, and [pymllm-setup] loads
    ``compressed-tensors`` checkpoints into its quantized linear path; none
    of the pages gives those formats' bit layouts. Reading: a checkpoint word
    packs 8 consecutive columns of one row in some field order, field j
    holding column ``8*c + field_order[j]``; converting it places each value
    in its column and repacks in the library's order. The values and the
    word shape are unchanged.

    words: int32 [R, C] -> int32 [R, C].
    """
    return pack_int4(_fields_to_columns(words, field_order))


def transpose_int4_ref(words, field_order):
    """A 4-bit matrix packed along its rows' other axis -> transposed, repacked.

    Same passages as ``reorder_int4_ref``. Reading: a checkpoint that stores
    weights one output channel per row, packed along the input dimension
    (words [N, K/8], field j of word c holding k = 8*c + field_order[j]),
    becomes the library's [K, N/8] layout (field j of word c holding
    n = 8*c + j) by transposing the 4-bit matrix.

    words: int32 [A, B/8] -> int32 [B, A/8] (A % 8 == 0).
    """
    q = _fields_to_columns(words, field_order)
    if q.shape[0] % NIBBLES_PER_WORD:
        raise ValueError("the row count must be a multiple of 8")
    return pack_int4(np.ascontiguousarray(q.T))


def quant_per_token_int8_ref(x):
    """Dynamic symmetric per-token int8 quantization.

    [pymllm-setup] Overview (W8A8_INT8 runs activations in int8) and section
    "W8A8 first-run JIT compilation" (the per-token int8 quantizer that feeds
    the int8 scaled matmul). For each row m of x (one token):

        a[m]     = max_k |x[m, k]|                  (exact)
        s[m]     = fl32(a[m] / 127)                 (IEEE binary32 divide)
        q[m, k]  = clamp(rne(fl32(x[m, k] / s[m])), -127, 127)

    Readings (the pages print no formula): divide by the scale rather than
    multiply by 127/a; round half to even; clamp to [-127, 127] (-128 is
    never produced); an all-zero row gets s = 0 and q = 0.

    The same function quantizes int8 weights per output channel when it is
    given the rows of W [N, K].

    x: fp16 (or fp32) [M, K] -> (int8 [M, K], float32 [M]).
    """
    xf = np.asarray(x).astype(np.float32)
    if xf.ndim != 2:
        raise ValueError("x must be 2-D")
    a = np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    s = np.divide(a, np.float32(127.0), dtype=np.float32)
    q = np.zeros(xf.shape, dtype=np.int8)
    nz = s > 0
    if np.any(nz):
        quotient = np.divide(xf[nz], s[nz, None], dtype=np.float32)
        q[nz] = np.clip(np.rint(quotient), -127, 127).astype(np.int8)
    return q, s.astype(np.float32)


def w8a8_acc_ref(xq, wq):
    """Integer accumulator acc[m, n] = sum_k xq[m, k] * wq[n, k].

    [pymllm-setup] Overview (int8 x int8 products on INT8 tensor cores) and
    section "W8A8 first-run JIT compilation" (int8 matmul). Computed as a
    float64 matrix product: every product and every partial sum is an integer
    of magnitude below 2**53, so each float64 operation is exact whatever the
    summation order. The result must fit a signed 32-bit accumulator.

    xq: int8 [M, K], wq: int8 [N, K] -> int64 [M, N].
    """
    a = np.asarray(xq).astype(np.float64)
    b = np.asarray(wq).astype(np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("xq must be [M, K] and wq [N, K]")
    if a.shape[1] * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for exact float64 accumulation")
    acc = (a @ b.T).astype(np.int64)
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    return acc


def w8a8_ref(xq, s_tok, wq, s_ch):
    """W8A8 scaled matmul, y[m, n] = acc[m, n] * s_tok[m] * s_ch[n], unrounded float64.

    [pymllm-setup] section "W8A8 first-run JIT compilation": the int8 GEMM
    with a scale epilogue ("scaled_mm"); per-token activation scales and
    per-output-channel weight scales. Not rounded to fp16.
    """
    acc = w8a8_acc_ref(xq, wq).astype(np.float64)
    st = np.asarray(s_tok).astype(np.float64)
    sc = np.asarray(s_ch).astype(np.float64)
    return acc * st[:, None] * sc[None, :]


def kv_quant_ref(x, bits):
    """Online KV-cache quantization of one head's vector per token.

    [lmdeploy-ovw] section 2.4: the fp16 KV cache is quantized per head and
    per token, asymmetrically, to INT8 or INT4, with min/max scale factors
    computed online (no calibration). Each row of x is one (token, head)
    vector. Readings (the pages give no formula): with b bits and
    qmax = 2**b - 1,

        mn    = min(row), mx = max(row)                      (exact)
        scale = fl32(fl32(mx - mn) / qmax)                   (IEEE binary32)
        q     = clamp(rne(fl32(fl32(x - mn) / scale)), 0, qmax)
        x_hat = q * scale + mn

    a constant row has scale 0 and codes 0 (x_hat = mn exactly); a zero
    minimum or maximum counts as +0 (mn + 0, mx + 0), so a row of signed
    zeros stores (+0, +0). INT4 codes are packed two per byte,
    element 2i in the low nibble.

    x: fp16 [R, D] -> (codes uint8 [R, D] (bits 8) or [R, D/2] (bits 4),
                        params float32 [R, 2] = (scale, mn)).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    xf = np.asarray(x).astype(np.float32)
    if xf.ndim != 2 or (bits == 4 and xf.shape[1] % 2):
        raise ValueError("x must be [R, D] (D even for 4 bits)")
    qmax = np.float32(2 ** bits - 1)
    mn = np.min(xf, axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    mx = np.max(xf, axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    mn = np.add(mn, np.float32(0), dtype=np.float32)  # a zero minimum (maximum) counts as +0
    mx = np.add(mx, np.float32(0), dtype=np.float32)
    span = np.subtract(mx, mn, dtype=np.float32)
    scale = np.divide(span, qmax, dtype=np.float32)
    q = np.zeros(xf.shape, dtype=np.int64)
    nz = scale > 0
    if np.any(nz):
        shifted = np.subtract(xf[nz], mn[nz, None], dtype=np.float32)
        quotient = np.divide(shifted, scale[nz, None], dtype=np.float32)
        q[nz] = np.clip(np.rint(quotient), 0, int(qmax)).astype(np.int64)
    params = np.stack([scale, mn], axis=1).astype(np.float32)
    if bits == 8:
        return q.astype(np.uint8), params
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, params


def kv_dequant_ref(codes, params, bits):
    """x_hat = q * scale + mn in float64 (exact products of the stored values);
    the inverse of kv_quant_ref's packing. Returns float64 [R, D]."""
    c = np.asarray(codes).astype(np.int64)
    if bits == 4:
        q = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.int64)
        q[:, 0::2] = c & 15
        q[:, 1::2] = c >> 4
    else:
        q = c
    p = np.asarray(params).astype(np.float64)
    return q * p[:, 0:1] + p[:, 1:2]
