// Per-token symmetric int8 quantization for gfx950.
//
// Source: pymllm Setup and Usage, section "W8A8 first-run JIT compilation"
// (per-token int8 activation quantizer in front of the int8 scaled matmul).
// For every row m: s[m] = fl32(absmax(x[m,:]) / 127) and
// q[m,k] = clamp(rne(fl32(x[m,k] / s[m])), -127, 127); all-zero rows give
// s = 0, q = 0. The codes are those of the IEEE binary32 quotient rounded
// half to even, bit for bit: a reciprocal product decides every element that
// is not close to a half-integer, the IEEE division the rest.
//
// x is fp16 or bf16 (both widen exactly to binary32, so the same codes and
// scales follow from the same arithmetic).
// Up to 128 rows: one workgroup per row (quant_row_wg). Otherwise one
// wavefront per row, four rows per workgroup. Each lane holds its share
// of the row in registers (16-byte chunks of 8 values), so x is read from HBM
// exactly once: absmax by a wavefront butterfly, then quantize from registers
// and store 8 codes per 8-byte store. Rows longer than 64*8*32 elements take
// a two-pass variant that re-reads x.
#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

constexpr int kRowsPerBlock = 4;

template <bool kBf16>
__device__ __forceinline__ float chunk_absmax(u32x4 v, float m) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float lo, hi;
    word_to_floats<kBf16>(v[w], lo, hi);
    m = fmaxf(m, fabsf(lo));
    m = fmaxf(m, fabsf(hi));
  }
  return m;
}

// Distance from a half-integer below which an element takes the IEEE
// division (see quant_chunk).
constexpr float kTieMargin = 1.0f / 4096.0f;

// The reciprocal quant_chunk multiplies by: rcp(s) for a normal s; infinity
// for a binary32-subnormal s (then every product is non-finite and each
// element takes the division).
__device__ __forceinline__ float code_rcp(float s) {
  return s < 1.17549435e-38f ? __builtin_inff() : __builtin_amdgcn_rcpf(s);
}

// Codes of one 16-byte chunk (8 values) as 8 bytes: rne(fl32(v / s)) for
// s > 0, clamped to [-127, 127]; 0 for s = 0. Each element forms
// u = rint(v * r + 128) with one fused multiply-add (r = rcp(s), within 1 ulp
// of 1/s). The product differs from the exact quotient v / s by at most 2^-22
// relative (< 3.1e-5 for quotients up to 127.5), the rounded sum adds at most
// 2^-17, and the correctly rounded quotient is within half an ulp (< 3.9e-6)
// of the exact one. So when v * r + 128 is more than kTieMargin away from
// every half-integer, the rounded quotient lies on the same side of the
// nearest half-integer and u - 128 is its code; the rest (about 1 element in
// 2000, and every non-finite product) take the IEEE division, whose correctly
// rounded result decides ties. Codes in [-127, 127] are u in [1, 255]; one
// unsigned 8-bit conversion per element packs u, and flipping bit 7 of each
// byte gives the two's-complement code u - 128.
template <bool kBf16>
__device__ __forceinline__ u32x2 quant_chunk(u32x4 v, float s, float r) {
  if (!(s > 0.f)) return u32x2{0u, 0u};
  float f[8], u[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) word_to_floats<kBf16>(v[w], f[2 * w], f[2 * w + 1]);
  bool slow = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = fmaf(f[e], r, 128.f);
    u[e] = rintf(p);
    slow |= !(fabsf(p - u[e]) <= 0.5f - kTieMargin);
  }
  if (slow) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fmaf(f[e], r, 128.f);
      if (!(fabsf(p - u[e]) <= 0.5f - kTieMargin)) u[e] = rintf(f[e] / s) + 128.f;
    }
  }
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    w[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(u[e], 1.f, 255.f), e & 3, w[e >> 2]);
  return u32x2{w[0] ^ 0x80808080u, w[1] ^ 0x80808080u};
}

// CPL = 16-byte chunks per lane kept in registers (row length <= 512*CPL).
template <int CPL, bool kBf16>
__global__ __launch_bounds__(256) void quant_rows_regs(const uint16_t* __restrict__ x,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ s_tok, int M, int K) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nchunk = K >> 3;
  const uint16_t* xr = x + static_cast<size_t>(row) * K;
  int8_t* qr = xq + static_cast<size_t>(row) * K;

  u32x4 v[CPL];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    if (c < nchunk) {
      v[i] = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    } else {
      v[i] = u32x4{0u, 0u, 0u, 0u};
    }
    amax = chunk_absmax<kBf16>(v[i], amax);
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  const float r = code_rcp(s);
  if (lane == 0) s_tok[row] = s;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    if (c < nchunk) *reinterpret_cast<u32x2*>(qr + 8 * c) = quant_chunk<kBf16>(v[i], s, r);
  }
}

// Any row length: absmax pass, then a second pass that re-reads x.
template <bool kBf16>
__global__ __launch_bounds__(256) void quant_rows_stream(const uint16_t* __restrict__ x,
                                                         int8_t* __restrict__ xq,
                                                         float* __restrict__ s_tok, int M, int K) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nchunk = K >> 3;
  const uint16_t* xr = x + static_cast<size_t>(row) * K;
  int8_t* qr = xq + static_cast<size_t>(row) * K;
  float amax = 0.f;
  for (int c = lane; c < nchunk; c += kWave)
    amax = chunk_absmax<kBf16>(*reinterpret_cast<const u32x4*>(xr + 8 * c), amax);
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  const float r = code_rcp(s);
  if (lane == 0) s_tok[row] = s;
  for (int c = lane; c < nchunk; c += kWave)
    *reinterpret_cast<u32x2*>(qr + 8 * c) = quant_chunk<kBf16>(*reinterpret_cast<const u32x4*>(xr + 8 * c), s, r);
}

// Few rows (decode batches): one workgroup of kTh / 64 wavefronts per row
// (four; eight or sixteen for longer rows), CPT 16-byte chunks per thread in
// registers, so a row's loads and codes are spread over 256-1024 lanes
// instead of 64 and the call's latency shrinks; the absmax is a wavefront
// butterfly and then a maximum over the wavefronts through LDS (max is exact
// and order-free, so s is the same).
template <int CPT, bool kBf16, int kTh = 256>
__global__ __launch_bounds__(kTh) void quant_row_wg(const uint16_t* __restrict__ x, int8_t* __restrict__ xq,
                                                    float* __restrict__ s_tok, int M, int K) {
  __shared__ float wmax[kTh / 64];
  const int row = static_cast<int>(blockIdx.x);
  const int nchunk = K >> 3;
  const uint16_t* xr = x + static_cast<size_t>(row) * K;
  int8_t* qr = xq + static_cast<size_t>(row) * K;
  u32x4 v[CPT];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = static_cast<int>(threadIdx.x) + kTh * i;
    v[i] = c < nchunk ? *reinterpret_cast<const u32x4*>(xr + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    amax = chunk_absmax<kBf16>(v[i], amax);
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kTh / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float s = amax / 127.0f;
  const float r = code_rcp(s);
  if (threadIdx.x == 0) s_tok[row] = s;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = static_cast<int>(threadIdx.x) + kTh * i;
    if (c < nchunk) *reinterpret_cast<u32x2*>(qr + 8 * c) = quant_chunk<kBf16>(v[i], s, r);
  }
  (void)M;
}

// Rows at or below which each row gets a workgroup of its own (fewer rows
// than CUs leave most of the GPU idle with one wavefront per row).
constexpr int64_t kRowWgMaxM = 128;

template <bool kBf16>
hipError_t launch_quant(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K, hipStream_t stream) {
  const int m = static_cast<int>(M), k = static_cast<int>(K);
  const int per_thread = ((k >> 3) + 255) / 256;
  // Rows of 4097-16384 values take 1024 threads (one or two 16-byte loads
  // each; 8 tokens at K = 12288: 4.2 -> 3.35 us); up to 2048 values keep 256.
  if (M <= kRowWgMaxM && per_thread > 2 && per_thread <= 8) {
    const dim3 grid(static_cast<uint32_t>(m)), block(1024);
    return launch_kernel(quant_row_wg<2, kBf16, 1024>, grid, block, 0, stream, x, xq, s_tok, m, k);
  }
  // Rows of 2049-4096 values: 512 threads, one load each (16 / 128 tokens at
  // K = 4096: 0.1-0.2 us faster than 256 threads with two).
  if (M <= kRowWgMaxM && per_thread == 2) {
    const dim3 grid(static_cast<uint32_t>(m)), block(512);
    return launch_kernel(quant_row_wg<1, kBf16, 512>, grid, block, 0, stream, x, xq, s_tok, m, k);
  }
  if (M <= kRowWgMaxM && per_thread <= 8) {
    const dim3 grid(static_cast<uint32_t>(m)), block(256);
    switch (per_thread) {
      case 1:
        return launch_kernel(quant_row_wg<1, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
      case 2:
        return launch_kernel(quant_row_wg<2, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
      case 3:
      case 4:
        return launch_kernel(quant_row_wg<4, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
      default:
        return launch_kernel(quant_row_wg<8, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
    }
  }
  const dim3 grid((m + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
  const int per_lane = ((k >> 3) + kWave - 1) / kWave;
  if (per_lane <= 1) {
    return launch_kernel(quant_rows_regs<1, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else if (per_lane <= 2) {
    return launch_kernel(quant_rows_regs<2, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else if (per_lane <= 4) {
    return launch_kernel(quant_rows_regs<4, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else if (per_lane <= 8) {
    return launch_kernel(quant_rows_regs<8, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else if (per_lane <= 16) {
    return launch_kernel(quant_rows_regs<16, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else if (per_lane <= 32) {
    return launch_kernel(quant_rows_regs<32, kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  } else {
    return launch_kernel(quant_rows_stream<kBf16>, grid, block, 0, stream, x, xq, s_tok, m, k);
  }
}

}  // namespace

hipError_t launch_quant_per_token_int8(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K, bool bf16,
                                       hipStream_t stream) {
  return bf16 ? launch_quant<true>(x, xq, s_tok, M, K, stream) : launch_quant<false>(x, xq, s_tok, M, K, stream);
}

}  // namespace mq
