// Internal launcher declarations shared by the C-ABI layer (mq_api.cpp) and
// the kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mq {

// Per-token int8 quantization of x[M,K] (fp16, or bf16 when bf16) into
// xq[M,K] and s_tok[M].
hipError_t launch_quant_per_token_int8(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K, bool bf16,
                                       hipStream_t stream);

// int8 GEMM acc = xq[M,K] . wq[N,K]^T. Exactly one of y (scaled output,
// fp16 or, when bf16, bf16; needs s_tok and s_ch) and acc (raw int32 output)
// is non-null.
hipError_t launch_w8a8_gemm(const int8_t* xq, const float* s_tok, const int8_t* wq,
                            const float* s_ch, uint16_t* y, int32_t* acc,
                            int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream);

// Decode-shaped form of the same product (M <= kW8A8GemvMaxM), bound by the
// weight stream; launch_w8a8_gemm dispatches to it where w8a8_use_gemv says.
constexpr int64_t kW8A8GemvMaxM = 64;
bool w8a8_use_gemv(int64_t M, int64_t N);
hipError_t launch_w8a8_gemv(const int8_t* xq, const float* s_tok, const int8_t* wq,
                            const float* s_ch, uint16_t* y, int32_t* acc,
                            int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream);

// Quantizer folded into the decode kernel: y = scaled_mm(quant(x), wq, s_ch)
// in one launch, bit-identical to the two separate calls, where
// w8a8_use_fused(M, N, K): one token with K <= 12288, two with K <= 8192,
// three or four with K <= 4096 and N >= 6144 (the token rows held in a
// 256-thread workgroup's registers). Every workgroup forms the tokens'
// scales and codes itself, once for all its tiles, while its first weight
// requests are in flight, which beats the quantizer launch there.
bool w8a8_use_fused(int64_t M, int64_t N, int64_t K);
hipError_t launch_w8a8_gemv_fused(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y,
                                  int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream);

// Device address of the library-owned scratch array on the current device
// (looked up once per device), kNoallocScratchBytes long, 256-byte aligned.
constexpr size_t kNoallocScratchBytes = 33816576;  // MQ_NOALLOC_SCRATCH_BYTES
hipError_t noalloc_scratch(void** ptr);

// Online KV-cache quantization of rows x [rows, head_dim] fp16 to codes
// (uint8 [rows, head_dim] for 8 bits, packed [rows, head_dim/2] for 4) and
// params fp32 [rows, 2] = (scale, min); head_dim a power of two in [8, 512];
// x is fp16, or bf16 when bf16.
hipError_t launch_kv_quant(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                           int bits, bool bf16, hipStream_t stream);

// Checkpoint-layout adapter (one-time conversions, exact bit permutations).
// order[j] = the element (0..7 within the word's span) that field j of a
// source word holds; the result is in the library's order (field j = element j).
hipError_t launch_int4_reorder(const int32_t* src, int32_t* dst, int64_t words, const uint8_t (&order)[8],
                               hipStream_t stream);
// src [A, B/8] packed along B in `order` -> dst [B, A/8] packed along A.
hipError_t launch_int4_transpose(const int32_t* src, int32_t* dst, int64_t A, int64_t B, const uint8_t (&order)[8],
                                 hipStream_t stream);
constexpr int64_t kInt4TransposeMaxA = int64_t{65535} * 128;
// src [A, B] 16-bit -> dst [B, A].
hipError_t launch_u16_transpose(const uint16_t* src, uint16_t* dst, int64_t A, int64_t B, hipStream_t stream);
constexpr int64_t kU16TransposeMaxA = int64_t{65535} * 64;
constexpr int64_t kU16TransposeMaxB = int64_t{1} << 30;

// W4A16 GEMM y[M,N] = x[M,K] . dequant(qweight, scales, qzeros), groups of
// `group` rows (32, 64 or 128; K % 128 == 0). With a workspace of
// w4a16_gemm_workspace(M, N, K) bytes, K is split w4a16_gemm_splits ways
// when the tiles alone leave most CUs idle (fp32 partials, then a reduce
// kernel); a NULL workspace never splits.
int w4a16_gemm_splits(int64_t M, int64_t N, int64_t K);
size_t w4a16_gemm_workspace(int64_t M, int64_t N, int64_t K);
// bf16: x and y are bf16 (the weight is rounded once to bf16 instead of fp16).
// per_channel: scales / qzeros hold one row used for every group (the
// kernel runs with `group` rows per group, 128 for per-channel layers).
hipError_t launch_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, int64_t group, bool per_channel, void* workspace,
                             bool bf16, hipStream_t stream);

// Largest token count the W4A16 GEMV takes (four 16-token MFMA tiles).
constexpr int64_t kGemvMaxM = 64;

// W4A16 GEMV launch plan: K is cut into `splits` slices across workgroups,
// each workgroup has `waves` wavefronts that share its K slice.
struct GemvPlan {
  int splits;
  int waves;  // wavefronts per workgroup (register-staged kernel)
  size_t workspace_bytes;
  bool lds;   // LDS-staged kernel (N % 32 == 0)
  int group;  // rows per group: 32, 64 or 128
  int strips_per_unit = 1;  // blocked GEMV: adjacent 32-output strips per workgroup
  bool per_channel = false; // one scale / zero-point row for all of K (group runs as 128)
};
GemvPlan plan_w4a16_gemv(int64_t M, int64_t N, int64_t K, int64_t group);

// Column-blocked weight layout for the decode GEMV (N % 128 == 0,
// K % 128 == 0): conversion from [K, N/8], plan and launch.
hipError_t launch_w4a16_block_weights(const int32_t* qweight, int32_t* blocked, int64_t N, int64_t K,
                                      hipStream_t stream);
GemvPlan plan_w4a16_gemv_blocked(int64_t M, int64_t N, int64_t K, int64_t group);
size_t w4a16_gemv_blocked_workspace(int64_t M, int64_t N, int64_t K, int64_t group);
hipError_t launch_w4a16_gemv_blocked(const uint16_t* x, const int32_t* blocked, const uint16_t* scales,
                                     const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                     const GemvPlan& plan, void* workspace, bool bf16, hipStream_t stream);

hipError_t launch_w4a16_gemv(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, const GemvPlan& plan,
                             void* workspace, bool bf16, hipStream_t stream);

}  // namespace mq
