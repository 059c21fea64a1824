// Split-K plumbing shared by the W4A16 decode kernels: the workgroup ->
// (strip, split) map and the kernel that adds the splits' fp32 partial sums.
// K is split across workgroups when a problem has too few column strips to
// occupy the GPU; each split writes fp32 partial sums [split, M, N] and the
// reduction adds them in split order, so results are deterministic.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

constexpr int kXcds = 8;  // workgroups are dispatched round-robin over 8 XCDs

// Work item -> (strip, split). XCD x owns a contiguous block of strips with
// all their splits, so the reduce kernel finds a strip's partial sums in
// that XCD's L2; within an XCD, consecutive workgroups take neighbouring
// strips of one split, so concurrently running workgroups read adjacent
// row segments.
struct XcdMap {
  int strips_per_xcd;
};

__device__ __forceinline__ bool decode_work(int block, int strips_per_xcd, int strips, int splits, int& strip,
                                            int& split) {
  const int xcd = block % kXcds;
  const int slot = block / kXcds;
  const int local = slot % strips_per_xcd;
  split = slot / strips_per_xcd;
  strip = xcd * strips_per_xcd + local;
  return strip < strips && split < splits;
}

// ---------------------------------------------------------------------------
// Split reduction: y = fp16(sum over splits of partial[split]) in split
// order. Thread t of the block sums 4 consecutive outputs of one token row
// of one strip; blocks are mapped to the XCD that wrote that strip.
// ---------------------------------------------------------------------------
template <int S, bool kBF>
__global__ __launch_bounds__(256) void w4a16_gemv_reduce(const float* __restrict__ partial,
                                                         uint16_t* __restrict__ y, int M, int N,
                                                         int strip_cols, int strips_per_xcd,
                                                         int blocks_per_xcd, int splits) {
  const int xcd = blockIdx.x % kXcds;
  const int local = (blockIdx.x / kXcds) * 256 + threadIdx.x;  // 4-output unit within the XCD
  const int units_per_row = strips_per_xcd * strip_cols / 4;    // per token row
  const int m = local / units_per_row;
  const int u = local % units_per_row;
  if (m >= M) return;
  const int n = xcd * strips_per_xcd * strip_cols + u * 4;  // first output column
  if (n >= N) return;
  (void)blocks_per_xcd;
  const size_t stride = static_cast<size_t>(M) * N;
  const float* src = partial + static_cast<size_t>(m) * N + n;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  if constexpr (S > 0) {
    f32x4 v[S > 1 ? S - 1 : 1];
#pragma unroll
    for (int s = 1; s < S; ++s) v[s - 1] = *reinterpret_cast<const f32x4*>(src + s * stride);
#pragma unroll
    for (int s = 1; s < S; ++s) acc += v[s - 1];
  } else {
    for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const f32x4*>(src + s * stride);
  }
  const uint32_t lo = half_bits<kBF>(acc[0]) | (static_cast<uint32_t>(half_bits<kBF>(acc[1])) << 16);
  const uint32_t hi = half_bits<kBF>(acc[2]) | (static_cast<uint32_t>(half_bits<kBF>(acc[3])) << 16);
  *reinterpret_cast<u32x2*>(y + static_cast<size_t>(m) * N + n) = u32x2{lo, hi};
}

template <bool kBF>
hipError_t launch_gemv_reduce_t(const float* part, uint16_t* y, int m, int n, int cols8, int sps, int bpx,
                                int splits, dim3 rgrid, hipStream_t stream) {
  switch (splits) {
    case 2:
      return launch_kernel(w4a16_gemv_reduce<2, kBF>, rgrid, dim3(256), 0, stream, part, y, m, n, cols8, sps, bpx,
                           splits);
    case 4:
      return launch_kernel(w4a16_gemv_reduce<4, kBF>, rgrid, dim3(256), 0, stream, part, y, m, n, cols8, sps, bpx,
                           splits);
    case 8:
      return launch_kernel(w4a16_gemv_reduce<8, kBF>, rgrid, dim3(256), 0, stream, part, y, m, n, cols8, sps, bpx,
                           splits);
    case 16:
      return launch_kernel(w4a16_gemv_reduce<16, kBF>, rgrid, dim3(256), 0, stream, part, y, m, n, cols8, sps, bpx,
                           splits);
    default:
      return launch_kernel(w4a16_gemv_reduce<0, kBF>, rgrid, dim3(256), 0, stream, part, y, m, n, cols8, sps, bpx,
                           splits);
  }
}

// The reduction for `splits` partial sums, output fp16 or (bf16) bf16.
inline hipError_t launch_gemv_reduce(const float* part, uint16_t* y, int m, int n, int cols8, int sps, int bpx,
                                     int splits, bool bf16, dim3 rgrid, hipStream_t stream) {
  return bf16 ? launch_gemv_reduce_t<true>(part, y, m, n, cols8, sps, bpx, splits, rgrid, stream)
              : launch_gemv_reduce_t<false>(part, y, m, n, cols8, sps, bpx, splits, rgrid, stream);
}

}  // namespace
}  // namespace mq
