/*
 * mq.h -- C ABI of the quantized linear layer library (libmq.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * Two paths of the quantized linear layer that LLM inference runtimes use:
 *
 *   W4A16      asymmetric 4-bit weights with per-group fp16 scales and 4-bit
 *              zero points, fp16 activations, fp16 output. A GEMM for
 *              prefill-shaped inputs and a GEMV for decode (M <= 64).
 *              Source: LMDeploy toolkit overview, section 2.5 "Weight
 *              quantization (AWQ)" (4-bit weights, groups of 128); LMDeploy
 *              4-bit deployment guide, section 2.2 (scale and weight are
 *              consumed inside one kernel) and section 3.2 (per-layer group
 *              size, 64 for the vision tower's attention); pymllm Setup and
 *              Usage, Overview (the W4A16 scheme).
 *
 *   W8A8_INT8  dynamic per-token symmetric int8 activation quantization,
 *              then an int8 GEMM with int32 accumulation and a per-token x
 *              per-output-channel scale epilogue to fp16.
 *              Source: pymllm Setup and Usage, Overview (int8 activations
 *              and weights on INT8 matrix units) and section "W8A8 first-run
 *              JIT compilation" (a per-token int8 quantizer feeding an int8
 *              scaled matmul).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - fp16 values are IEEE binary16 passed as uint16_t bit patterns.
 * - Every tensor is row-major and densely packed (no strides).
 * - Every tensor pointer is a DEVICE pointer on the calling thread's current
 *   HIP device, owned by the caller. The library never allocates, frees,
 *   copies to or from the host, or synchronizes. The caller keeps every
 *   buffer alive until the stream has executed the work.
 * - `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream. Work is enqueued asynchronously on it and the call returns.
 *   No memset nodes are issued, so calls may be captured into a HIP graph.
 * - Arguments are validated on the host BEFORE any HIP call. A rejected call
 *   enqueues nothing and leaves every output untouched.
 * - M == 0 (and N == 0 where allowed) is a valid empty problem: MQ_OK,
 *   nothing is enqueued. A pointer may be NULL exactly when its tensor has
 *   no elements (as an empty torch tensor's data pointer is).
 * - Outputs must not overlap any input or each other (MQ_ERR_ALIAS).
 * - Asynchronous device faults are reported by HIP at the caller's next
 *   synchronization, not by these calls.
 * - Thread safety: the library holds no mutable global state besides the
 *   thread-local error message; calls from several threads are safe.
 *   Results are deterministic: the same inputs give the same bits.
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQ_ABI_VERSION 2

typedef enum mq_status {
  MQ_OK = 0,
  MQ_ERR_NULL = 1,        /* a required pointer is NULL */
  MQ_ERR_SHAPE = 2,       /* a size is negative, too large or breaks a divisibility rule */
  MQ_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  MQ_ERR_UNSUPPORTED = 4, /* valid in principle but not provided (e.g. group not in {32, 64, 128, -1}, GEMV M > 64) */
  MQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  MQ_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
  MQ_ERR_HIP = 7          /* the HIP runtime refused the launch (message in mq_last_error) */
} mq_status;

/* MQ_ABI_VERSION of the built library. */
int mq_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* mq_status_string(mq_status s);

/* Detail for the last non-OK call made by this thread ("" if none). The
 * pointer stays valid until this thread's next call into the library. */
const char* mq_last_error(void);

/*
 * Per-token symmetric int8 quantization.
 * Source: pymllm Setup and Usage, section "W8A8 first-run JIT compilation"
 * (the per-token int8 activation quantizer). For each row m:
 *     s_tok[m] = fl32(max_k |x[m,k]| / 127)              (IEEE binary32 divide)
 *     xq[m,k]  = clamp(rne(fl32(x[m,k] / s_tok[m])), -127, 127)
 * with rne = round half to even; an all-zero row gives s_tok = 0, xq = 0.
 * Results are bit-exact to that definition. Inputs must be finite.
 *
 *   x      [M, K] fp16   in
 *   xq     [M, K] int8   out
 *   s_tok  [M]    fp32   out
 * Requires: 0 <= M < 2^31; 16 <= K <= 2^20, K % 16 == 0; x, xq 16-byte
 * aligned; s_tok 4-byte aligned.
 */
mq_status mq_quant_per_token_int8(const uint16_t* x, int8_t* xq, float* s_tok,
                                  int64_t M, int64_t K, void* stream);

/*
 * W8A8 scaled int8 GEMM.
 * Source: pymllm Setup and Usage, section "W8A8 first-run JIT compilation"
 * (int8 GEMM with a scale epilogue). acc[m,n] = sum_k xq[m,k] * wq[n,k] in
 * exact int32, then
 *     y[m,n] = fp16_rne( fl32( fl32(acc[m,n]) * s_tok[m] ) * s_ch[n] )
 *
 *   xq     [M, K] int8   in   (activations, one row per token)
 *   s_tok  [M]    fp32   in   (per-token scales)
 *   wq     [N, K] int8   in   (weights, one row per output channel)
 *   s_ch   [N]    fp32   in   (per-output-channel scales)
 *   y      [M, N] fp16   out
 * Requires: 0 <= M, N < 2^31; 16 <= K <= 133136, K % 16 == 0 (133136 is
 * the largest multiple of 16 with 127*127*K < 2^31); xq, wq, y 16-byte
 * aligned; s_tok, s_ch 4-byte aligned.
 * Codes are expected in [-127, 127], the range the per-token quantizer
 * produces. Any int8 is accepted, but a code of -128 keeps the int32
 * accumulator exact only while 128*128*K < 2^31, i.e. K <= 131056; above
 * that an accumulator fed with -128 codes may wrap.
 * The kernel is chosen by shape (a weight-streaming kernel for up to 32
 * tokens, and for 33-64 tokens while N < 16384; a tiled GEMM otherwise).
 * Both compute the exact accumulator and the same epilogue, so results are
 * identical whichever runs, and deterministic.
 */
mq_status mq_w8a8_scaled_mm(const int8_t* xq, const float* s_tok, const int8_t* wq,
                            const float* s_ch, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Debug entry: the raw int32 accumulator of the W8A8 GEMM,
 *     acc[m,n] = sum_k xq[m,k] * wq[n,k]   (exact)
 * Same operands, layouts and requirements as mq_w8a8_scaled_mm; acc is
 * [M, N] int32, 16-byte aligned.
 */
mq_status mq_w8a8_mm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W8A8_INT8 linear layer from fp16 activations: y = scaled_mm(quant(x)).
 * Source: pymllm Setup and Usage, section "W8A8 first-run JIT compilation"
 * (the per-token quantizer feeding the int8 scaled matmul) and Overview.
 * Same result, bit for bit, as mq_quant_per_token_int8 followed by
 * mq_w8a8_scaled_mm. For one token with K <= 12288, two with K <= 8192,
 * and three or four with K <= 4096 and N >= 6144 it is one kernel: every
 * workgroup forms the tokens' scales itself and quantizes the rows into
 * LDS (IEEE binary32 quotient, round half to even, clamp to [-127, 127]),
 * once for the channel tiles it walks, so xq and s_tok never touch memory
 * and the workspace is not used.
 * Otherwise it runs the two kernels, with xq and s_tok in `workspace`.
 *
 *   x          [M, K] fp16   in,  16-byte aligned
 *   wq, s_ch   as mq_w8a8_scaled_mm
 *   y          [M, N] fp16   out, 16-byte aligned
 *   workspace  >= mq_w8a8_linear_workspace_bytes(M, K) bytes (the size of
 *              the two-kernel path, which does not depend on N; may be NULL
 *              in the one-kernel case), 16-byte aligned, not overlapping any
 *              operand; its contents on entry do not matter.
 * Requires: as mq_w8a8_scaled_mm (K % 16 == 0, K <= 133136).
 */
size_t mq_w8a8_linear_workspace_bytes(int64_t M, int64_t K);
mq_status mq_w8a8_linear(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y,
                         int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bf16 forms of the three entries above, for models whose activations are
 * bf16. Source: pymllm Setup and Usage, Overview (BF16 is one of the
 * runtime's schemes beside W4A16 and W8A8_INT8, so the quantized layers sit
 * among bf16 activations). x is bf16 (raw bits) instead of fp16 and y is
 * bf16 instead of fp16; everything else -- layouts, requirements, errors,
 * workspace sizes and the kernels chosen -- is as in the fp16 entry.
 *   mq_quant_per_token_int8_bf16: bf16 widens exactly to binary32, so the
 *     scales and codes follow the same definition bit for bit.
 *   mq_w8a8_scaled_mm_bf16: y[m,n] = bf16_rne( fl32( fl32(acc) * s_tok[m] ) * s_ch[n] ).
 *   mq_w8a8_linear_bf16: quantizer and scaled GEMM as above, bit-identical to
 *     the two calls in sequence.
 */
mq_status mq_quant_per_token_int8_bf16(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K,
                                       void* stream);
mq_status mq_w8a8_scaled_mm_bf16(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch,
                                 uint16_t* y, int64_t M, int64_t N, int64_t K, void* stream);
mq_status mq_w8a8_linear_bf16(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free form of mq_w8a8_linear (fp16), for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc. Same operands, result (bit for bit),
 * kernels and requirements as mq_w8a8_linear, without the workspace
 * arguments: for more than one token the quantizer's codes and per-token
 * scales go to a scratch array that the library holds on each GPU it runs
 * on, MQ_NOALLOC_SCRATCH_BYTES (32 MiB + 256 KiB) long, from the first call
 * on that device until the process ends. The call allocates nothing and
 * issues no memset (the scratch is fully written before it is read).
 * Requires mq_w8a8_linear_workspace_bytes(M, K) <= MQ_NOALLOC_SCRATCH_BYTES
 * (e.g. 2048 tokens at K = 12288), else MQ_ERR_WORKSPACE before any HIP
 * call. Every call on one GPU shares that GPU's scratch: calls that may
 * overlap in time on one GPU (different streams without ordering, several
 * host threads) race and must be serialized by the caller; calls on one
 * stream are ordered and safe.
 */
#define MQ_NOALLOC_SCRATCH_BYTES 33816576
mq_status mq_w8a8_linear_noalloc(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M,
                                 int64_t N, int64_t K, void* stream);

/*
 * W4A16 GEMM (prefill-shaped M).
 * Source: LMDeploy toolkit overview, section 2.5 (4-bit AWQ weights, group
 * size 128); LMDeploy 4-bit deployment guide, section 2.2 (dequantization
 * fused into the matmul kernel) and section 3.2 (group size per layer: 64
 * for the vision tower's attention projection, 128 for the language model;
 * -1 for no grouping).
 * G = group: the number of consecutive k sharing one scale and zero point;
 * group = -1 means G = K: one scale and zero point per output column
 * (per-channel), scales [1, N] and qzeros [1, N/8]. Every W4A16 entry takes
 * group = -1 and computes it as groups of 128 rows that all read that one
 * row (same arithmetic, same bounds as group 128).
 *     q[k,n]  = field (n % 8) of qweight[k, n/8]     (field j = bits 4j..4j+3)
 *     z[g,n]  = field (n % 8) of qzeros[g, n/8]
 *     w[k,n]  = (q[k,n] - z[k/G,n]) * scales[k/G,n]
 *     y[m,n]  = fp16( sum_k x[m,k] * w[k,n] )   accumulated in fp32
 * The weight is rounded once to fp16, fp16((q - z) * s), before the fp16
 * matrix multiply, for every fp16 scale. Outputs match the exact result
 * within relative Frobenius error 1e-3 and max-abs error 5e-2 at the
 * documented input distributions and for scales down to about 2^-16.
 * Range of the fp16 weight: |(q - z) * s| must stay below 65520 (15 * |s|
 * < 65520 always holds for |s| <= 4096), else that weight becomes +-inf;
 * products below 2^-14 are fp16 subnormals (multiples of 2^-24), so with
 * scales much below 2^-16 the relative error of the weights, and of y,
 * grows. The GEMVs below apply s in fp32 and have neither limit.
 *
 *   x        [M, K]     fp16   in
 *   qweight  [K, N/8]   int32  in   (8 unsigned 4-bit weights per word along N)
 *   scales   [K/G, N]   fp16   in
 *   qzeros   [K/G, N/8] int32  in   (unsigned 4-bit zero points, packed like qweight)
 *   y        [M, N]     fp16   out
 *   workspace  optional (may be NULL). When the 128-token x 512-output
 *              tiles alone leave most CUs idle (fewer than 192 tiles), K is
 *              split across workgroups if a workspace of at least
 *              mq_w4a16_gemm_workspace_bytes(M, N, K, group) bytes is given:
 *              fp32 partial sums go there and a second kernel on the same
 *              stream adds them in split order (deterministic). NULL never
 *              splits. 16-byte aligned, not overlapping any operand; calls
 *              sharing it must be ordered.
 * Requires: group in {32, 64, 128, -1} (anything else ->
 * MQ_ERR_UNSUPPORTED); 0 <= M < 2^31; 8 <= N <= 2^27, N % 8 == 0;
 * 128 <= K <= 2^20, K % 128 == 0 (so K % group == 0); x, scales, y 16-byte
 * aligned; qweight, qzeros 4-byte aligned.
 */
size_t mq_w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);
mq_status mq_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                        const int32_t* qzeros, uint16_t* y,
                        int64_t M, int64_t N, int64_t K, int64_t group,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace size in bytes that mq_w4a16_gemv needs for this problem (0 when
 * it needs none). Returns 0 as well for problems mq_w4a16_gemv rejects.
 * Pure host function.
 */
size_t mq_w4a16_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);

/*
 * W4A16 GEMV for decode (1 <= M <= 64). Same definition, operands and
 * layouts as mq_w4a16_gemm, except that the weights are not rounded to
 * fp16: per group of G rows the kernel forms, in fp32, the sum of
 * x * (q - z) and scales it by s in fp32. (For N % 32 == 0 the sum is
 * taken as sum(x * (1024 + q)) - (1024 + z) * sum(x), with exact fp16
 * products; otherwise (q - z) is formed exactly first.) Outputs meet the
 * same tolerance as mq_w4a16_gemm. K is split across workgroups when N is
 * too narrow to occupy the GPU: each split writes fp32 partial sums to
 * `workspace` and a second kernel on the same stream adds the splits in
 * split order. Results are deterministic. Up to 64 tokens share one pass
 * over the weights (four 16-token MFMA tiles per weight fragment; for
 * N % 32 != 0 the tokens are taken 16 at a time).
 *
 *   workspace        device buffer of at least
 *                    mq_w4a16_gemv_workspace_bytes(M, N, K, group) bytes,
 *                    16-byte aligned; may be NULL when that size is 0.
 *                    Its contents on entry do not matter. It must not
 *                    overlap any operand, and calls sharing a workspace
 *                    must be ordered (same stream or synchronized).
 * Requires: as mq_w4a16_gemm, and M <= 64 (M > 64 -> MQ_ERR_UNSUPPORTED).
 */
mq_status mq_w4a16_gemv(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                        const int32_t* qzeros, uint16_t* y,
                        int64_t M, int64_t N, int64_t K, int64_t group,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Column-blocked weight layout for decode, and the GEMV that reads it.
 * Source: LMDeploy 4-bit deployment guide, deployment steps (the AWQ model
 * is converted once into the inference engine's own weight format before it
 * is served) and section 2.2 (scale and weight consumed in one kernel).
 *
 * mq_w4a16_block_weights reorders the bytes of qweight [K, N/8] (nothing
 * inside a byte changes; byte g of word (k, c) holds the 4-bit weights of
 * columns 8c+2g and 8c+2g+1 of row k) into 1 KB slots, one per 64-row pair
 * P and 32-output strip s (S = N/32 strips), the slots of all strips for one
 * pair next to each other:
 *     blocked_bytes[((P*S + s)*64 + 16h + j)*16 + 8b + e]
 *         = byte (j/4) of qweight[64P + 32b + 8h + e, 4s + j%4]
 * for P < K/64, s < S, h < 4, j < 16, b < 2, e < 8 (little-endian words). Scales and zero points keep their layouts. Run it
 * once when the weights are loaded; the result serves every
 * mq_w4a16_gemv_blocked call on those weights.
 *
 *   qweight          [K, N/8] int32  in,  4-byte aligned
 *   qweight_blocked  K*N/8    int32  out, 16-byte aligned, must not overlap qweight
 * Requires: N % 32 == 0, K % 128 == 0 (-> MQ_ERR_SHAPE otherwise).
 */
mq_status mq_w4a16_block_weights(const int32_t* qweight, int32_t* qweight_blocked, int64_t N, int64_t K,
                                 void* stream);

/* Workspace for mq_w4a16_gemv_blocked (0: none needed, or a rejected problem). */
size_t mq_w4a16_gemv_blocked_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);

/*
 * W4A16 GEMV for decode (1 <= M <= 64) on blocked weights. Same definition,
 * scales, zero points, arithmetic (fp32 group sums of x * (1024 + q), then
 * s * (sum - (1024 + z) * sum(x)) per group) and tolerance as mq_w4a16_gemv;
 * qweight_blocked is the output of mq_w4a16_block_weights for these weights.
 * Each workgroup streams one 32-output strip over its K range as one
 * contiguous run of bytes. When the layer has too few strips for two
 * workgroups per compute unit, up to 8 tokens with K/128 <= 32 take one
 * workgroup of 8 or 16 wavefronts per strip (their sums added in LDS in
 * wavefront order, no workspace); otherwise K is split across workgroups
 * (fp32 partials in `workspace`, added in split order by a second kernel).
 * All M <= 64 tokens share one pass over the weights. For 17-64 tokens the
 * fragments are the weights themselves, rounded once to fp16 as in
 * mq_w4a16_gemm (fp16((q - z) * s), the same range notes apply), accumulated
 * in fp32; up to 16 tokens use the exact (q - z) form with s applied in fp32.
 * Deterministic.
 *
 *   workspace   >= mq_w4a16_gemv_blocked_workspace_bytes(M, N, K, group)
 *               bytes, 16-byte aligned (may be NULL when that is 0); same
 *               rules as mq_w4a16_gemv's workspace.
 * Requires: as mq_w4a16_gemv, and N % 32 == 0 and a scale table
 * (K/group or 1 rows of N fp16) under 2^31 bytes (-> MQ_ERR_SHAPE),
 * qweight_blocked 16-byte aligned.
 */
mq_status mq_w4a16_gemv_blocked(const uint16_t* x, const int32_t* qweight_blocked, const uint16_t* scales,
                                const int32_t* qzeros, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, int64_t group,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * bf16 forms of the three W4A16 entries, for models whose activations are
 * bf16. Source: pymllm Setup and Usage, Overview (BF16 is one of the
 * runtime's schemes beside W4A16 and W8A8_INT8, and the W4A16 layer is
 * chosen from a model's quantization config, so 4-bit layers sit among bf16
 * activations). x and y are bf16 (raw bits); qweight, scales (fp16),
 * qzeros, layouts, workspace sizes, requirements, errors and the kernels
 * chosen are as in the fp16 entry. The definition is the same,
 * y = sum_k x * (q - z) * s with x widened exactly to binary32, y rounded
 * to nearest even as bf16; the arithmetic:
 *   mq_w4a16_gemm_bf16: each weight (q - z) * s is formed exactly in
 *     binary32 and rounded once to bf16 for the bf16 MFMA; fp32 sums.
 *   mq_w4a16_gemv_bf16, mq_w4a16_gemv_blocked_bf16: fragments hold 128 + q
 *     exactly in bf16 and per group the kernel adds, in binary32,
 *     s * (sum(x * (128 + q)) - (128 + z) * sum(x)); on the decode layout
 *     17-64 tokens round each weight once to bf16 as the GEMM does.
 * Error bound, element by element, against the exact sum y64 (derived from
 * that arithmetic: bf16 unit roundoff 2^-8, binary32 2^-24): weight-rounding
 * forms |y - y64| <= 2^-8 |y64| + (2^-8 + K 2^-24) sum_k |x w| (1 + 2^-7);
 * the 128 + q forms |y - y64| <= 2^-8 |y64| + 2^-15 * 143 sum_k |x s|.
 * Scales must keep |(q - z) * s| within the bf16 normal range.
 */
mq_status mq_w4a16_gemm_bf16(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t group,
                             void* workspace, size_t workspace_bytes, void* stream);
mq_status mq_w4a16_gemv_bf16(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t group,
                             void* workspace, size_t workspace_bytes, void* stream);
mq_status mq_w4a16_gemv_blocked_bf16(const uint16_t* x, const int32_t* qweight_blocked, const uint16_t* scales,
                                     const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                     int64_t group, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Online KV-cache quantization, per head and per token.
 * Source: LMDeploy toolkit overview, section 2.4 "KV Cache online
 * quantization" (fp16 KV cache quantized per head per token, asymmetric,
 * to INT8 or INT4, min/max scale factors computed online, no calibration).
 * Each row of x is one (token, head) vector; with b = bits, qmax = 2^b - 1:
 *     mn = min(row) + 0, mx = max(row) + 0          (a zero counts as +0)
 *     scale = fl32(fl32(mx - mn) / qmax)             (IEEE binary32)
 *     q = clamp(rne(fl32(fl32(x - mn) / scale)), 0, qmax); scale 0 -> q = 0
 * and x is recovered as q * scale + mn.
 *
 *   x       [rows, head_dim] fp16  in,  16-byte aligned
 *   codes   bits 8: [rows, head_dim] uint8; bits 4: [rows, head_dim / 2]
 *           uint8, element 2i in the low nibble; out, 8- (bits 8) or
 *           4-byte (bits 4) aligned
 *   params  [rows, 2] fp32 = (scale, mn)  out, 8-byte aligned
 * Requires: bits in {8, 4} (else MQ_ERR_UNSUPPORTED); head_dim a power of
 * two in [8, 512]; 0 <= rows < 2^31 and rows * head_dim < 2^35 (else
 * MQ_ERR_SHAPE). Codes and params are bit-exact.
 */
mq_status mq_kv_quant(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                      int32_t bits, void* stream);

/*
 * bf16 form of mq_kv_quant for a bf16 KV cache: x is bf16 (raw bits), which
 * widens exactly to binary32, so the same definition gives the codes and
 * (scale, min) bit for bit; everything else is as in mq_kv_quant. A row
 * whose scale is subnormal in binary32 is quantized by the IEEE division;
 * rows whose max - min overflows binary32 are outside the contract, as are
 * non-finite inputs.
 */
mq_status mq_kv_quant_bf16(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                           int32_t bits, void* stream);

/*
 * Checkpoint-layout adapter: one-time conversions of 4-bit checkpoint
 * tensors into the layouts above.
 * Source: the LMDeploy overview (sections 4.1 and 5.5) loads 4-bit
 * checkpoints in the AWQ model format and the LMDeploy 4-bit deployment
 * guide converts them before serving; pymllm Setup and Usage loads
 * compressed-tensors checkpoints into its quantized linear path. The pages
 * give none of these formats' bit layouts. Reading: a checkpoint packs 8
 * consecutive 4-bit values of one row into a 32-bit word in some field
 * order -- field j (bits 4j..4j+3) holds element 8c + order[j] of the row --
 * either along the output dimension ([K, N/8], as qweight and qzeros here)
 * or along the input dimension ([N, K/8], one output channel per row).
 * `order` is a HOST pointer to 8 bytes, a permutation of 0..7; NULL means
 * the library's order (order[j] = j). For example AWQ-style words use
 * order = {0, 2, 4, 6, 1, 3, 5, 7}. Results are bit-exact permutations of
 * the input bits; each call is asynchronous on `stream` like the others,
 * and dst must not overlap src (MQ_ERR_ALIAS).
 */

/*
 * src, dst int32 [words], src in `order`, dst in the library's order (same
 * shape). Use on qweight [K, N/8] and qzeros [K/G, N/8] of checkpoints packed
 * along N. 0 <= words < 2^34; src and dst 16-byte aligned; a non-permutation
 * `order` gives MQ_ERR_UNSUPPORTED.
 */
mq_status mq_int4_reorder(const int32_t* src, int32_t* dst, int64_t words, const uint8_t* order, void* stream);

/*
 * src int32 [A, B/8]: a 4-bit matrix [A, B] packed along B in `order`.
 * dst int32 [B, A/8]: its transpose packed along A in the library's order,
 * i.e. field j of dst word (b, c) is element (8c + j, b). Use on weights
 * stored [N, K/8] (A = N, B = K) to get qweight [K, N/8]. A and B
 * non-negative multiples of 8 (else MQ_ERR_SHAPE), A <= 65535 * 128,
 * B < 2^31; src and dst 4-byte aligned.
 */
mq_status mq_int4_transpose(const int32_t* src, int32_t* dst, int64_t A, int64_t B, const uint8_t* order,
                            void* stream);

/*
 * src [A, B] of 16-bit values (fp16 scales as raw bits) -> dst [B, A].
 * Use on scales stored [N, K/G] to get scales [K/G, N]. 0 <= A <= 65535 * 64,
 * 0 <= B <= 2^30; src and dst 2-byte aligned.
 */
mq_status mq_u16_transpose(const uint16_t* src, uint16_t* dst, int64_t A, int64_t B, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
