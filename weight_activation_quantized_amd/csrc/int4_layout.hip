// Checkpoint-layout adapter for 4-bit weights on gfx950.
//
// Source: the LMDeploy overview (sections 4.1 and 5.5) loads 4-bit
// checkpoints in the AWQ model format, the LMDeploy 4-bit deployment guide
// converts them (--model-format awq) before serving, and pymllm loads
// compressed-tensors checkpoints into its quantized linear path. None of the
// pages gives those formats' bit layouts; the reading here is that a
// checkpoint packs 8 consecutive 4-bit values of one row into a 32-bit word
// in some field order (field j holding element 8c + order[j]), along the
// output dimension ([K, N/8], like the library) or along the input
// dimension ([N, K/8], one output channel per row). Three one-time
// conversions bring such tensors into the library's layout:
//   * int4_reorder:   words in another field order -> library order (same shape),
//   * int4_transpose: a 4-bit matrix [A, B] packed along B -> [B, A] packed
//                     along A, library order,
//   * u16_transpose:  fp16 scales [N, K/G] -> [K/G, N].
// All three are exact permutations of bits, bound by HBM.
#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

// Field j of w moved to field dst_field[j]; dst_field[j] = 4 * order[j] is
// passed as 8 nibbles of `order` and expanded once per lane.
__device__ __forceinline__ uint32_t move_fields(uint32_t w, const uint32_t (&sh)[8]) {
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) out |= ((w >> (4 * j)) & 15u) << sh[j];
  return out;
}

__device__ __forceinline__ void field_shifts(uint32_t order, uint32_t (&sh)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) sh[j] = 4u * ((order >> (4 * j)) & 15u);
}

// One lane per 16 bytes (4 words); the last lane of a ragged count takes the
// remaining 1-3 words one at a time.
__global__ __launch_bounds__(256) void int4_reorder_kernel(const uint32_t* __restrict__ src,
                                                           uint32_t* __restrict__ dst, int64_t words,
                                                           uint32_t order) {
  uint32_t sh[8];
  field_shifts(order, sh);
  const int64_t i = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (i + 4 <= words) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = move_fields(v[e], sh);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + i));
  } else {
    for (int64_t k = i; k < words; ++k) dst[k] = move_fields(src[k], sh);
  }
}

// Tile of 128 source rows (a) by 128 columns (b, 16 words per row). The
// source words are staged in LDS as they are (row stride padded to 17
// words); destination word (b, aw) gathers element b of rows 8aw .. 8aw+7,
// i.e. field inv[b % 8] of word b / 8 of those rows, where inv is the
// inverse of the source field order (passed as 8 nibbles of `inv`).
constexpr int kTA = 128, kTB = 128, kTW = kTB / 8, kLdsStride = kTW + 1;

__global__ __launch_bounds__(256) void int4_transpose_kernel(const uint32_t* __restrict__ src,
                                                             uint32_t* __restrict__ dst, int64_t A, int64_t B,
                                                             uint32_t inv) {
  __shared__ uint32_t tile[kTA * kLdsStride];
  const int64_t a0 = static_cast<int64_t>(blockIdx.y) * kTA;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kTB;
  const int64_t src_words = B / 8, dst_words = A / 8;
  const int t = threadIdx.x;
  // 128 rows x 16 words: lane t loads word t % 16 of rows t / 16 + 16 k
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = t / kTW + 16 * k, w = t % kTW;
    const int64_t a = a0 + r, cw = b0 / 8 + w;
    uint32_t v = 0;
    if (a < A && cw < src_words) v = src[a * src_words + cw];
    tile[r * kLdsStride + w] = v;
  }
  __syncthreads();
  // 128 rows (b) x 16 words (a / 8): lane t writes word t % 16 of rows t / 16 + 16 k
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int bl = t / kTW + 16 * k, aw = t % kTW;
    const int64_t b = b0 + bl, dw = a0 / 8 + aw;
    const uint32_t shift = 4u * ((inv >> (4 * (bl % 8))) & 15u);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) out |= ((tile[(8 * aw + i) * kLdsStride + bl / 8] >> shift) & 15u) << (4 * i);
    if (b < B && dw < dst_words) dst[b * dst_words + dw] = out;
  }
}

// 64 x 64 tile of 16-bit values through LDS (row stride 65), 256 lanes,
// 16 values each.
__global__ __launch_bounds__(256) void u16_transpose_kernel(const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ dst, int64_t A, int64_t B) {
  __shared__ uint16_t tile[64 * 65];
  const int64_t a0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = t / 64 + 4 * k, c = t % 64;
    const int64_t a = a0 + r, b = b0 + c;
    tile[r * 65 + c] = (a < A && b < B) ? src[a * B + b] : uint16_t{0};
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = t / 64 + 4 * k, c = t % 64;  // r: b within the tile, c: a within the tile
    const int64_t b = b0 + r, a = a0 + c;
    if (a < A && b < B) dst[b * A + a] = tile[c * 65 + r];
  }
}

uint32_t pack_nibbles(const uint8_t (&v)[8]) {
  uint32_t p = 0;
  for (int j = 0; j < 8; ++j) p |= static_cast<uint32_t>(v[j] & 15u) << (4 * j);
  return p;
}

}  // namespace

hipError_t launch_int4_reorder(const int32_t* src, int32_t* dst, int64_t words, const uint8_t (&order)[8],
                               hipStream_t stream) {
  const int64_t lanes = (words + 3) / 4;
  const int64_t blocks = (lanes + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  return launch_kernel(int4_reorder_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), words,
                       pack_nibbles(order));
}

hipError_t launch_int4_transpose(const int32_t* src, int32_t* dst, int64_t A, int64_t B, const uint8_t (&order)[8],
                                 hipStream_t stream) {
  uint8_t inv[8];
  for (int j = 0; j < 8; ++j) inv[order[j] & 7] = static_cast<uint8_t>(j);
  const int64_t gx = (B + kTB - 1) / kTB, gy = (A + kTA - 1) / kTA;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  return launch_kernel(int4_transpose_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy)), dim3(256),
                       0, stream, reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), A, B,
                       pack_nibbles(inv));
}

hipError_t launch_u16_transpose(const uint16_t* src, uint16_t* dst, int64_t A, int64_t B, hipStream_t stream) {
  const int64_t gx = (B + 63) / 64, gy = (A + 63) / 64;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  return launch_kernel(u16_transpose_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy)), dim3(256),
                       0, stream, src, dst, A, B);
}

}  // namespace mq
