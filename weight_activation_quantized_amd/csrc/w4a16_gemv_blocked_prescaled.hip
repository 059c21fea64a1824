// W4A16 decode GEMV on the column-blocked layout, 33-64 tokens (three or four
// 16-token tiles, weights pre-scaled in the fragments). Kept in its own
// translation unit: its MFMA results stay in the accumulation registers
// (the VGPR form of the other tiles measured slower here).
#include "w4a16_gemv_blocked.h"

namespace mq {
namespace {

template <int kT, int kGS, bool kBF>
hipError_t launch_blocked_scaled(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                                 uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                                 XcdMap map, dim3 grid, hipStream_t stream) {
  // two LDS slots of 16 kT token rows x 256 bytes per wavefront (the x DMA)
  const size_t lds = static_cast<size_t>(plan.waves) * 2 * kT * 4096;
  if constexpr (kGS >= 64) {
    if (plan.strips_per_unit == 3)
      return launch_blocked_xl<kT, kGS, 3, false, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, lds,
                                                  stream);
    if (plan.strips_per_unit == 2)
      return launch_blocked_xl<kT, kGS, 2, false, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, lds,
                                                  stream);
  }
  return launch_blocked_xl<kT, kGS, 1, false, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, lds,
                                              stream);
}

template <int kGS, bool kBF>
hipError_t launch_scaled_group(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                               uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                               XcdMap map, dim3 grid, hipStream_t stream) {
  if (m > 48) return launch_blocked_scaled<4, kGS, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
  return launch_blocked_scaled<3, kGS, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
}

}  // namespace

hipError_t launch_w4a16_gemv_blocked_prescaled(const uint16_t* x, const u32x4* qb, const uint16_t* scales,
                                               const uint32_t* qz, uint16_t* y, float* part, int m, int n, int k,
                                               const GemvPlan& plan, int units, int strips_per_xcd, dim3 grid,
                                               bool bf16, hipStream_t stream) {
  if (m <= 32 || m > kGemvMaxM) return hipErrorInvalidValue;
  XcdMap map;
  map.strips_per_xcd = strips_per_xcd;
  switch (plan.group * 2 + (bf16 ? 1 : 0)) {
    case 64:
      return launch_scaled_group<32, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 65:
      return launch_scaled_group<32, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 128:
      return launch_scaled_group<64, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 129:
      return launch_scaled_group<64, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 256:
      return launch_scaled_group<128, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 257:
      return launch_scaled_group<128, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mq
