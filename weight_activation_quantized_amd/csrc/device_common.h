// Device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// LDS (address space 3) views for the direct global -> LDS loads.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;

// A float from another lane of the same 16-lane row, by DPP control kCtrl
// (every lane's source is valid for the controls used here).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  const int b = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, kCtrl, 0xF, 0xF, false));
}

// Maximum over the wavefront, the same value in every lane: DPP steps within
// each row of 16 lanes (quad permutes, then the half-row and row mirrors),
// then the four rows' maxima read from lanes 15, 31, 47 and 63. No LDS round
// trips; max is exact and order-free.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror: every lane holds its row's maximum
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// A binary32 rounded to nearest even as fp16 or bf16, returned as raw bits.
template <bool kBf16>
__device__ __forceinline__ uint16_t half_bits(float v) {
  if constexpr (kBf16) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<f16>(v));
  }
}

// Two binary32 values rounded to nearest even as a bf16 pair (lo in bits
// 0-15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 16-bit MFMAs on operands carried as f16x8 bit patterns: fp16, or bf16
// when kBf16 (the same bits reinterpreted).
template <bool kBf16>
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  if constexpr (kBf16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
}
template <bool kBf16>
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  if constexpr (kBf16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
}

// The two 16-bit values of a word (fp16, or bf16 = the upper half of a
// binary32) as floats; both widen exactly.
template <bool kBf16>
__device__ __forceinline__ void word_to_floats(uint32_t w, float& lo, float& hi) {
  if constexpr (kBf16) {
    lo = __builtin_bit_cast(float, w << 16);
    hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    lo = static_cast<float>(h[0]);
    hi = static_cast<float>(h[1]);
  }
}

// Byte permute of two dwords: output byte i = byte sel[i] of the 8-byte value
// {hi:lo} (selectors 0-3 pick bytes of lo, 4-7 bytes of hi).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two packed fp16 values built from two 4-bit fields sitting in bits 0-3 (or
// 4-7) of each 16-bit half: OR-ing them into the mantissa of 1024.0 (0x6400)
// gives exactly 1024 + q (or 1024 + 16*q).
__device__ __forceinline__ uint32_t nib_lo_to_f16x2(uint32_t v) {
  return (v & 0x000F000Fu) | 0x64006400u;
}
__device__ __forceinline__ uint32_t nib_hi_to_f16x2(uint32_t v) {
  return (v & 0x00F000F0u) | 0x64006400u;
}

// s_waitcnt with vmcnt <= VM and lgkmcnt <= LGKM (gfx9 encoding), bracketed
// by compiler memory barriers so no memory access moves across it.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (whose
// release would wait for every LDS DMA in flight). Callers first wait for
// the counters they need with wait_counts.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mq

#include <tuple>
#include <utility>

namespace mq {

// Launch `kernel` and return the launch status directly (no reliance on the
// thread's sticky last-error state). Arguments are converted to the kernel's
// parameter types first.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  std::tuple<KArgs...> values(static_cast<KArgs>(std::forward<Args>(args))...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, values);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
}

}  // namespace mq
