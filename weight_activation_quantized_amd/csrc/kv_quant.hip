// Online KV-cache quantization for gfx950.
//
// Source: LMDeploy toolkit overview, section 2.4 "KV Cache online
// quantization": the fp16 KV cache is quantized per head and per token,
// asymmetrically, to INT8 or INT4, with min/max scale factors computed on
// the fly. One row = one (token, head) vector of D values. With b bits and
// qmax = 2^b - 1 (the pages give no formula; this is the plain reading):
//   scale = fl32(fl32(max - min) / qmax),
//   q     = clamp(rne(fl32(fl32(x - min) / scale)), 0, qmax)   (IEEE binary32),
// a constant row giving scale 0 and q = 0; (scale, min) are stored per row
// in fp32 (a zero minimum or maximum counting as +0) and INT4 codes two per
// byte, element 2i in the low nibble.
//
// The kernel is a single pass bound by HBM: a group of D/8 lanes holds one
// row (one 16-byte load of 8 values per lane, up to two rows in flight per
// group), min and max come from a butterfly within the group, and each lane
// writes its 8 codes (8 bytes, or 4 packed bytes for INT4). The codes come
// from a reciprocal product, with the IEEE division only near half-integers
// (one branch per lane's 8 values); min and max within 16-lane rows by DPP.
// x is fp16 or bf16 (both widen exactly to binary32). x is read once;
// nothing else is.
#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

// Minimum / maximum over a group of kL consecutive lanes (every lane of the
// group gets it): DPP steps within 16-lane rows (quad permutes, half-row and
// row mirrors) for up to 16 lanes, then shuffles across rows. Exact and
// order-free.
template <int kL, bool kMax>
__device__ __forceinline__ float group_reduce(float v) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : fminf(a, b); };
  if constexpr (kL >= 2) v = op(v, dpp_f32<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  if constexpr (kL >= 4) v = op(v, dpp_f32<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  if constexpr (kL >= 8) v = op(v, dpp_f32<0x141>(v));  // row_half_mirror
  if constexpr (kL >= 16) v = op(v, dpp_f32<0x140>(v));  // row_mirror
#pragma unroll
  for (int off = 16; off < kL; off <<= 1) v = op(v, __shfl_xor(v, off, kWave));
  return v;
}

// Distance from a half-integer below which a code takes the IEEE division.
// With r = rcp(scale) (within 1 ulp), p = d * r is within 2^-22 relative of
// the exact quotient d / scale, i.e. under 6.1e-5 for quotients up to 255.5,
// and the correctly rounded quotient is within half an ulp (under 1.6e-5) of
// the exact one; so when p is more than this margin away from every
// half-integer, rint(p) is the code of the IEEE quotient. Only codes inside
// the margin (ties among them) take the division.
constexpr float kKvTieMargin = 1.0f / 4096.0f;

// Codes of the 8 values d[] = x - min of a lane, clamped to [0, kQmax]: the
// reciprocal product everywhere, then, in one branch per 8 values, the IEEE
// division for those within the margin (written so that a non-finite p also
// divides: a binary32-subnormal scale, possible for bf16 rows, gets an
// infinite reciprocal from kv_rcp).
template <int kBits>
__device__ __forceinline__ void kv_codes(const float (&d)[8], float scale, float r, float (&q)[8]) {
  constexpr float kQmax = static_cast<float>((1 << kBits) - 1);
  bool slow = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = d[e] * r;
    q[e] = rintf(p);
    slow |= !(fabsf(p - q[e]) <= 0.5f - kKvTieMargin);
  }
  if (slow) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = d[e] * r;
      if (!(fabsf(p - q[e]) <= 0.5f - kKvTieMargin)) q[e] = rintf(d[e] / scale);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(q[e], 0.f, kQmax);
}

__device__ __forceinline__ float kv_rcp(float scale) {
  return scale < 1.17549435e-38f ? __builtin_inff() : __builtin_amdgcn_rcpf(scale);
}

// kL lanes per row (head_dim = 8 kL), kBits = 8 or 4, kR rows per lane group.
// 256 threads: kR * 256 / kL rows per workgroup; the kR loads of a lane are
// issued before any is used, and for each r the workgroup's 256 lanes read
// one contiguous 4 KB span.
template <int kL, int kBits, int kR, bool kBf16>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                       float* __restrict__ params, int64_t rows) {
  constexpr int kD = 8 * kL;
  constexpr int kRowsPerPass = 256 / kL;
  constexpr float kQmax = static_cast<float>((1 << kBits) - 1);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (kR * kRowsPerPass) + threadIdx.x / kL;
  const int lig = threadIdx.x % kL;  // lane within the row's group
  u32x4 v[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t row = row0 + r * kRowsPerPass;
    v[r] = u32x4{0u, 0u, 0u, 0u};
    if (row < rows) v[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + row * kD + 8 * lig));
  }
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t row = row0 + r * kRowsPerPass;
    float f[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) word_to_floats<kBf16>(v[r][w], f[2 * w], f[2 * w + 1]);
    float mn = f[0], mx = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      mn = fminf(mn, f[e]);
      mx = fmaxf(mx, f[e]);
    }
    // every lane of a group takes part; a zero minimum or maximum becomes +0
    mn = group_reduce<kL, false>(mn) + 0.0f;
    mx = group_reduce<kL, true>(mx) + 0.0f;
    if (row >= rows) continue;
    const float scale = (mx - mn) / kQmax;  // IEEE binary32 subtraction and division
    float q[8];
    if (scale > 0.f) {
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = f[e] - mn;
      kv_codes<kBits>(d, scale, kv_rcp(scale), q);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = 0.f;
    }
    if constexpr (kBits == 8) {
      // codes in [0, 255]: one unsigned 8-bit conversion per code packs them
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(q[e], e & 3, w[e >> 2]);
      __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(codes + row * kD + 8 * lig));
    } else {
      uint32_t out = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) out |= static_cast<uint32_t>(q[e]) << (4 * e);
      __builtin_nontemporal_store(out, reinterpret_cast<uint32_t*>(codes + row * (kD / 2) + 4 * lig));
    }
    if (lig == 0) {
      float2 p;
      p.x = scale;
      p.y = mn;
      *reinterpret_cast<float2*>(params + 2 * row) = p;
    }
  }
}

template <int kBits, int kR, bool kBf16>
hipError_t launch_rows(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                       hipStream_t stream) {
  const int64_t lanes = head_dim / 8;
  const int64_t rows_per_block = kR * (256 / lanes);
  const dim3 grid(static_cast<uint32_t>((rows + rows_per_block - 1) / rows_per_block)), block(256);
  switch (lanes) {
    case 1: return launch_kernel(kv_quant_kernel<1, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 2: return launch_kernel(kv_quant_kernel<2, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 4: return launch_kernel(kv_quant_kernel<4, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 8: return launch_kernel(kv_quant_kernel<8, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 16: return launch_kernel(kv_quant_kernel<16, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 32: return launch_kernel(kv_quant_kernel<32, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    case 64: return launch_kernel(kv_quant_kernel<64, kBits, kR, kBf16>, grid, block, 0, stream, x, codes, params, rows);
    default: return hipErrorInvalidValue;
  }
}

// Two rows per lane group once that still gives at least 2048 workgroups
// (eight per CU); smaller calls keep one row per group so every CU has work.
// Measured at 131072 rows of 128 (INT8 / INT4): one row 12.7 / 12.1 us, two
// 12.0 / 11.9, four 12.8 / 14.1, eight 15.2 / 15.3.
template <int kBits, bool kBf16>
hipError_t launch_bits(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                       hipStream_t stream) {
  const int64_t rows_per_pass = 256 / (head_dim / 8);
  if (rows >= 2048 * 2 * rows_per_pass)
    return launch_rows<kBits, 2, kBf16>(x, codes, params, rows, head_dim, stream);
  return launch_rows<kBits, 1, kBf16>(x, codes, params, rows, head_dim, stream);
}

}  // namespace

hipError_t launch_kv_quant(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                           int bits, bool bf16, hipStream_t stream) {
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  if (bits == 8)
    return bf16 ? launch_bits<8, true>(x, codes, params, rows, head_dim, stream)
                : launch_bits<8, false>(x, codes, params, rows, head_dim, stream);
  if (bits == 4)
    return bf16 ? launch_bits<4, true>(x, codes, params, rows, head_dim, stream)
                : launch_bits<4, false>(x, codes, params, rows, head_dim, stream);
  return hipErrorInvalidValue;
}

}  // namespace mq
