// W4A16 decode GEMV on the column-blocked layout: layout conversion, launch
// plan and the forms with one or two 16-token tiles (up to 32 tokens). The
// layout, the kernel and its arithmetic are described in w4a16_gemv_blocked.h.
#include "w4a16_gemv_blocked.h"

namespace mq {
namespace {

// ---------------------------------------------------------------------------
// Layout conversion: one thread per 16-byte lane slot of the blocked layout.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4a16_block_weights_kernel(const uint32_t* __restrict__ qw,
                                                                  u32x4* __restrict__ qb, int K, int NP,
                                                                  int64_t slots) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= slots) return;
  const int L = static_cast<int>(t & 63);
  const int64_t ps = t >> 6;  // P * S + s
  const int S = NP / kBStrip;
  const int64_t P = ps / S;
  const int64_t s = ps % S;
  const int j = L & 15, h = L >> 4;
  const int c = j & 3, g = j >> 2;
  const uint32_t* col = qw + s * kBStrip + c;
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // word w: block b = w / 2, rows e = 4 (w % 2) .. +3
    const int64_t k0 = 64 * P + 32 * (w >> 1) + 8 * h + 4 * (w & 1);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= ((col[(k0 + e) * NP] >> (8 * g)) & 0xFFu) << (8 * e);
    v[w] = word;
  }
  qb[t] = v;
}

// Bytes of LDS a one-tile call stages (0: x, scales and zero points are
// loaded per chunk): the token rows of x over the split's K range, then the
// unit's scales and zero-point words, if all of it fits beside the static
// reduction buffer in a workgroup's 160 KB.
int64_t blocked_x_lds_bytes(int64_t M, int64_t K, int64_t group, int splits, int waves, int strips_per_unit) {
  const int64_t kr = K / splits;
  const int64_t xb = std::min<int64_t>(M, 16) * (2 * kr + kXLdsPad);
  // the tables take whole 16-group loads
  const int64_t szb = ((kr / group + 15) / 16 * 16) * strips_per_unit * (64 + 16);
  // x staged up front only where a unit has a single strip (several strips
  // share the per-chunk DMA slots instead), and in whole 1 KB loads per row
  if (strips_per_unit > 1 || kr % 512) return 0;
  const int64_t red = int64_t{waves} * 16 * strips_per_unit * kBOut * 4;
  // the one-workgroup-per-strip form (8 or 16 wavefronts) stages up to 8
  // tokens: it has no stream to hold back before the copy
  const int64_t max_tokens = waves >= 8 ? kWideMaxTokens : kXLdsMaxTokens;
  if (M > max_tokens || xb + szb + red > kLdsPerWorkgroup) return 0;
  return xb + szb;
}

template <int kT, int kGS, int kSP, bool kBF>
hipError_t launch_blocked_main(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                               uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                               XcdMap map, dim3 grid, hipStream_t stream) {
  if constexpr (kT == 1 && kSP == 1) {  // x staged up front: one-strip units only
    const int64_t lds = blocked_x_lds_bytes(m, k, kGS, plan.splits, plan.waves, kSP);
    if (lds > 0)
      return launch_blocked_xl<kT, kGS, kSP, true, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid,
                                                   static_cast<size_t>(lds), stream);
  }
  // two LDS slots of 16 kT token rows x 256 bytes per wavefront (the x DMA);
  // with up to 4 / 8 tokens one / two loads per chunk fill the rows in use,
  // and a single token also skips the per-group update of unused rows
  const size_t lds = static_cast<size_t>(plan.waves) * 2 * kT * 4096;
  if constexpr (kT == 1) {
    if (m == 1)
      return launch_blocked_xl<kT, kGS, kSP, false, kBF, 0>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid,
                                                        lds, stream);
    if (m <= 4)
      return launch_blocked_xl<kT, kGS, kSP, false, kBF, 1>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid,
                                                        lds, stream);
    if (m <= 8)
      return launch_blocked_xl<kT, kGS, kSP, false, kBF, 2>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid,
                                                        lds, stream);
  }
  return launch_blocked_xl<kT, kGS, kSP, false, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, lds,
                                                stream);
}

template <int kGS, bool kBF>
hipError_t launch_blocked_group(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                                uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                                XcdMap map, dim3 grid, hipStream_t stream) {
  if (m > 16) return hipErrorInvalidValue;  // 17-64 tokens: the pre-scaled kernel
  if constexpr (kGS == 32) {
    // groups of 32: one strip per workgroup (the multi-strip forms do not
    // fit the register file with four groups per chunk)
    return launch_blocked_main<1, kGS, 1, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
  } else {
    switch (plan.strips_per_unit) {
      case 3:
        return launch_blocked_main<1, kGS, 3, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
      case 2:
        return launch_blocked_main<1, kGS, 2, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
      default:
        return launch_blocked_main<1, kGS, 1, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    }
  }
}

}  // namespace

constexpr int64_t kBlockedMinWgs = 512;  // two workgroups per CU before K is split
constexpr int kCUs = 256;

GemvPlan plan_w4a16_gemv_blocked(int64_t M, int64_t N, int64_t K, int64_t group) {
  GemvPlan plan{1, 1, 0, false, static_cast<int>(group)};
  const int64_t strips = N / kBOut;
  const int64_t chunks = K / kBChunkRows;
  const int64_t mt = std::min(M, kGemvMaxM);
  // Narrow layers with up to 8 tokens (fewer strips than CUs) and short K:
  // one workgroup of 16 (else 8) wavefronts per strip takes all of K, each
  // wavefront one or two chunks, with x staged in LDS, and their sums meet
  // in LDS. One launch with every chunk in flight at once, instead of K
  // split across workgroups with fp32 partial sums and a second kernel to
  // add them (8B qkv at one token 7.6 -> 6.3 us, o_proj 6.5 -> 5.8 us).
  // With six chunks per wavefront (K = 12288) it measured slower than the
  // split.
  if (mt <= kWideMaxTokens && strips < kCUs) {
    for (int w : {16, 8}) {
      if (chunks % w || chunks / w > 2 || blocked_x_lds_bytes(M, K, group, 1, w, 1) == 0) continue;
      plan.waves = w;
      return plan;  // splits = 1, no workspace
    }
  }
  // Every workgroup loads all of x for its K range, so a workgroup takes
  // several adjacent strips that share those loads through its LDS slots
  // (three for one 16-token tile, where that divides the strips; at
  // N = 24576: 4 tokens 12.8 -> 11.5 us, one token 11.9 -> 11.3 us with
  // three strips against one strip with x staged up front).
  // With two to four tiles (17-64 tokens, the pre-scaled kernel) a
  // workgroup takes most of a CU, and the x fragments, read once per strip
  // group, cost more than the weights: the unit takes the most strips (3,
  // then 2) for which splitting K still reaches one workgroup per CU with
  // at least two chunks per split (measured at 64 tokens, 8B layers: qkv
  // 22.7 -> 18.3, o_proj 15.1 -> 13.5, down 30.7 -> 23.7 us against one
  // strip per unit).
  int sp = 1;
  if (mt > 16) {
    for (int cand = (group >= 64 ? 3 : 1); cand > 1; --cand) {
      if (strips % cand) continue;
      bool fits = false;
      for (int64_t s = 1; s <= chunks / 2 && !fits; ++s) fits = chunks % s == 0 && (strips / cand) * s >= kCUs;
      if (fits || strips / cand >= kCUs) {
        sp = cand;
        break;
      }
    }
  } else if (group >= 64) {
    if (strips % 3 == 0) {
      sp = 3;
    } else if (mt > kXLdsMaxTokens && strips % 2 == 0) {
      sp = 2;
    }
  }
  plan.strips_per_unit = sp;
  const int64_t units = strips / sp;
  // Split K only when there are too few units for two single-strip
  // workgroups (one multi-strip or many-token workgroup) per CU: the
  // smallest divisor of the chunk count that gets there (else the largest);
  // four wavefronts per workgroup when the split's chunks allow.
  const int64_t min_wgs = sp == 1 && mt <= 32 ? kBlockedMinWgs : kBlockedMinWgs / 2;
  for (int64_t s = 1; s <= chunks; ++s) {
    if (chunks % s) continue;
    plan.splits = static_cast<int>(s);
    if (units * s >= min_wgs) break;
  }
  const int64_t cps = chunks / plan.splits;
  plan.waves = cps % 4 == 0 ? 4 : (cps % 2 == 0 ? 2 : 1);
  // 17-64 tokens: eight wavefronts (two per SIMD) where the split's chunks
  // allow
  if (mt > 16 && cps % 8 == 0) plan.waves = 8;
  plan.workspace_bytes = plan.splits > 1 ? static_cast<size_t>(plan.splits) * mt * N * sizeof(float) : 0;
  return plan;
}

size_t w4a16_gemv_blocked_workspace(int64_t M, int64_t N, int64_t K, int64_t group) {
  return plan_w4a16_gemv_blocked(M, N, K, group).workspace_bytes;
}

hipError_t launch_w4a16_block_weights(const int32_t* qweight, int32_t* blocked, int64_t N, int64_t K,
                                      hipStream_t stream) {
  if (N % kBOut || K % kBChunkRows) return hipErrorInvalidValue;
  const int64_t slots = (N / 8) * K / 4;  // 16-byte slots
  const int64_t blocks = (slots + 255) / 256;
  return launch_kernel(w4a16_block_weights_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<u32x4*>(blocked),
                       static_cast<int>(K), static_cast<int>(N / 8), slots);
}

hipError_t launch_w4a16_gemv_blocked(const uint16_t* x, const int32_t* blocked, const uint16_t* scales,
                                     const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                     const GemvPlan& plan, void* workspace, bool bf16, hipStream_t stream) {
  if (N % kBOut || K % kBChunkRows || M < 1 || M > kGemvMaxM || plan.waves < 1) return hipErrorInvalidValue;
  if (plan.group != 32 && plan.group != 64 && plan.group != 128) return hipErrorInvalidValue;
  if ((K / kBChunkRows) % (static_cast<int64_t>(plan.splits) * plan.waves)) return hipErrorInvalidValue;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const int units = static_cast<int>(N / kBOut / plan.strips_per_unit);
  XcdMap map;
  map.strips_per_xcd = (units + kXcds - 1) / kXcds;
  const dim3 grid(static_cast<uint32_t>(kXcds * map.strips_per_xcd * plan.splits));
  const u32x4* qb = reinterpret_cast<const u32x4*>(blocked);
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  float* part = static_cast<float*>(workspace);
  hipError_t err;
  if (m > 16) {  // two to four token tiles
    err = launch_w4a16_gemv_blocked_prescaled(x, qb, scales, qz, y, part, m, n, k, plan, units, map.strips_per_xcd,
                                              grid, bf16, stream);
  } else {
    switch (plan.group * 2 + (bf16 ? 1 : 0)) {
      case 64:
        err = launch_blocked_group<32, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
      case 65:
        err = launch_blocked_group<32, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
      case 128:
        err = launch_blocked_group<64, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
      case 129:
        err = launch_blocked_group<64, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
      case 257:
        err = launch_blocked_group<128, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
      default:
        err = launch_blocked_group<128, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
        break;
    }
  }
  if (err != hipSuccess || plan.splits == 1) return err;
  const int cols8 = kBOut * plan.strips_per_unit;
  const int64_t units_per_xcd = static_cast<int64_t>(map.strips_per_xcd) * cols8 / 4 * M;
  const int blocks_per_xcd = static_cast<int>((units_per_xcd + 255) / 256);
  const dim3 rgrid(static_cast<uint32_t>(kXcds * blocks_per_xcd));
  const int sps = map.strips_per_xcd;
  return launch_gemv_reduce(part, y, m, n, cols8, sps, blocks_per_xcd, plan.splits, bf16, rgrid, stream);
}

}  // namespace mq
