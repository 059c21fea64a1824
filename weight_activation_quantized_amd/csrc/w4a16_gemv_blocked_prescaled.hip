// W4A16 decode GEMV on the column-blocked layout, 17-64 tokens (two to four
// 16-token tiles). Same operation and layout as w4a16_gemv_blocked.h (LMDeploy
// 4-bit deployment guide, section 2.2: scale and weight consumed in one
// kernel): y[m,n] = sum_k x[m,k] * fp16((q - z) * s) over groups of G rows.
//
// The one-tile kernel's per-group partial sums and sums of x do not fit the
// register file with several tiles and strips, so this kernel forms the
// weight fragments themselves, fp16((q - z) * s) rounded once (the GEMM's
// arithmetic, with the 64 + q high field), and accumulates the MFMAs straight
// into the running sums: one pass over the weights for all tokens, several
// strips per workgroup sharing every x fragment a wavefront reads.
//
// Eight wavefronts per workgroup, two per SIMD, so one's unpack (VALU)
// runs under the other's MFMAs and memory waits: each wavefront walks a
// contiguous eighth of the workgroup's K range in 64-row steps (one pair of
// the layout), two steps in flight: per step its 16-byte slot of each strip
// in registers, the step's x rows (all token tiles x 64 values) and group
// parameters in one of its two LDS slots by DMA.
//
// Kept in its own translation unit: built without the VGPR form of MFMA
// results that the one-tile kernel uses (with eight wavefronts the compiler
// keeps these accumulators in VGPRs anyway).
#include "w4a16_gemv_blocked.h"

namespace mq {
namespace {

constexpr int kStepRows = 64;  // rows per step: one pair of the blocked layout
constexpr int kRing = 2;       // steps in flight per wavefront

// Pre-scaled B fragments of one 32-row block: each fragment element is the
// weight itself, fp16((q - z) * s), rounded once: field 2g reads 1024 + q
// (pattern of 1024.0), field 2g+1 reads 64 + q (pattern of 64.0, no factor
// 16); adding -(1024 + z) / -(64 + z) leaves q - z exactly, and one multiply
// by s rounds. nz[f] / s2[f]: the encoded negated zero point and the scale of
// field f, both replicated in the two fp16 halves.
// kBF: nz[f] / s2[f] hold binary32 bits of -(offset + z) * s and of s; one
// fused multiply-add per weight gives (q - z) * s exactly in binary32 and
// the pair conversion rounds it once to bf16.
template <bool kBF>
__device__ __forceinline__ void unpack_block_scaled(uint32_t w0, uint32_t w1, const NibConst& c,
                                                    const uint32_t (&nz)[2], const uint32_t (&s2)[2],
                                                    f16x8 (&bf)[2]) {
  const uint32_t ws[2] = {w0, w1};
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t v = byte_perm(ws[q], ws[q], t ? 0x0C030C02u : 0x0C010C00u);
      f16x2 lo, hi;
      if constexpr (kBF) {
        const f16x2 ol = as_f16x2((v & c.lo) | c.magic), oh = as_f16x2((v & c.hi) | c.magic64);
        const float sl = __builtin_bit_cast(float, s2[0]), cl = __builtin_bit_cast(float, nz[0]);
        const float sh = __builtin_bit_cast(float, s2[1]), ch = __builtin_bit_cast(float, nz[1]);
        lo = as_f16x2(bf16x2_bits(fmaf(static_cast<float>(ol[0]), sl, cl), fmaf(static_cast<float>(ol[1]), sl, cl)));
        hi = as_f16x2(bf16x2_bits(fmaf(static_cast<float>(oh[0]), sh, ch), fmaf(static_cast<float>(oh[1]), sh, ch)));
      } else {
        lo = (as_f16x2((v & c.lo) | c.magic) + as_f16x2(nz[0])) * as_f16x2(s2[0]);
        hi = (as_f16x2((v & c.hi) | c.magic64) + as_f16x2(nz[1])) * as_f16x2(s2[1]);
      }
      bf[0][4 * q + 2 * t] = lo[0];
      bf[0][4 * q + 2 * t + 1] = lo[1];
      bf[1][4 * q + 2 * t] = hi[0];
      bf[1][4 * q + 2 * t + 1] = hi[1];
    }
}

// The encoded parameters of one group for unpack_block_scaled: sv holds the
// scales of fields 2g and 2g+1, byte g_lane of zw their zero points.
template <bool kBF>
__device__ __forceinline__ void scaled_params(uint32_t sv_bits, uint32_t zw, int g_lane, uint32_t (&nz)[2],
                                              uint32_t (&s2)[2]) {
  const f16x2 sv = as_f16x2(sv_bits);
  const uint32_t zb = (zw >> (8 * g_lane)) & 0xFFu;
  if constexpr (kBF) {
    const float sl = static_cast<float>(sv[0]), sh = static_cast<float>(sv[1]);
    nz[0] = __builtin_bit_cast(uint32_t, -(1024.0f + static_cast<float>(zb & 15u)) * sl);
    nz[1] = __builtin_bit_cast(uint32_t, -(64.0f + static_cast<float>(zb >> 4)) * sh);
    s2[0] = __builtin_bit_cast(uint32_t, sl);
    s2[1] = __builtin_bit_cast(uint32_t, sh);
  } else {
    f16x2 s_lo, s_hi;
    s_lo[0] = s_lo[1] = sv[0];
    s_hi[0] = s_hi[1] = sv[1];
    const uint32_t e_lo = (zb & 0x0Fu) | 0xE400u, e_hi = (zb & 0xF0u) | 0xD400u;
    nz[0] = e_lo | (e_lo << 16);
    nz[1] = e_hi | (e_hi << 16);
    s2[0] = as_u32(s_lo);
    s2[1] = as_u32(s_hi);
  }
}

// One step's register operands of a lane: its 16-byte slot of the pair for
// each strip (words 2b, 2b+1 hold block b). The group parameters go to LDS
// with the x rows: scale pairs and zero-point words loaded into registers
// were copied between registers by the compiler across the loop, which
// waits for the loads in flight.
template <int kSP>
struct PStep {
  u32x4 w[kSP];
};

struct PLane {
  const u32x4* qb;           // the lane's slot of the unit's first strip in pair 0
  size_t pair_stride;        // slots from one pair to the next (S * 64)
  __amdgpu_buffer_rsrc_t xr;  // x, M rows (rows past M read as zero)
  uint32_t xdma[2];          // load q's byte offset at step 0: xdma[q % 2] + (q / 2) * xtile
  uint32_t xtile;            // 16 token rows of x in bytes
  __amdgpu_buffer_rsrc_t sr;  // scales
  __amdgpu_buffer_rsrc_t zr;  // qzeros
  uint32_t s_off, z_off;     // the lane's scale pair / zero-point word in group row 0, bytes
  uint32_t s_row, z_row;     // bytes between group rows (0: per-channel)
};

// Slot of a step (per wavefront): x, then the group parameters. x: tile t
// at 2048 t, token row r of the tile at 128 r, its 16-byte chunk c (8
// values) at 16 (c ^ ((r >> 1) & 7)), so the 16 rows a fragment read touches
// fall on 16 different bank groups; load q (tile q / 2, rows 8 (q % 2) .. +7)
// writes 1 KB: lane l the physical chunk l % 8 of row 8 (q % 2) + l / 8.
// Parameters at kT * 2048: for group gi of the step and strip sp, 256 bytes
// of scale pairs then 256 bytes of zero-point words, one word per lane.
template <int kT, int kGS, int kSP>
constexpr int slot_bytes() {
  return kT * 2048 + kSP * (kGS >= kStepRows ? 1 : kStepRows / kGS) * 512;
}

// with_params: also the step's group parameters (groups of 128 rows span
// two steps: only the even step loads them).
template <int kT, int kGS, int kSP>
__device__ __forceinline__ void load_step(PStep<kSP>& st, const PLane& L, int pair, lds_u8* slot, bool with_params) {
  constexpr int kGPS = kGS >= kStepRows ? 1 : kStepRows / kGS;
  const u32x4* wp = L.qb + static_cast<size_t>(pair) * L.pair_stride;
  // The weights are read once per call: non-temporal loads.
#pragma unroll
  for (int sp = 0; sp < kSP; ++sp) st.w[sp] = __builtin_nontemporal_load(wp + 64 * sp);
  // The slot's previous contents were read by the compute before this call;
  // lgkmcnt(0) makes sure those reads have returned.
  wait_counts<63, 0>();
#pragma unroll
  for (int q = 0; q < 2 * kT; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.xr, (lds_void*)(slot + 1024 * q), 16,
                                             L.xdma[q % 2] + (q / 2) * L.xtile + 2u * kStepRows * pair, 0, 0, 0);
  if (!with_params) return;
#pragma unroll
  for (int gi = 0; gi < kGPS; ++gi) {
    const uint32_t grp = static_cast<uint32_t>(pair) * kStepRows / kGS + gi;
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp) {
      lds_u8* const ps = slot + kT * 2048 + (gi * kSP + sp) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(L.sr, (lds_void*)(ps), 4, L.s_off + grp * L.s_row + 2u * kBOut * sp,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(L.zr, (lds_void*)(ps + 256), 4,
                                               L.z_off + grp * L.z_row + 4u * kBStrip * sp, 0, 0, 0);
    }
  }
}

// One step: two 32-row blocks; each block's x fragments are read once and
// shared by the strips. nz / s2 carry the encoded group parameters from step
// to step: encode = false (the odd step of a 128-row group) reuses them.
template <int kT, int kGS, int kSP, bool kBF>
__device__ __forceinline__ void compute_step(const PStep<kSP>& st, const NibConst& nc, int lane,
                                             f32x4 (&tot)[kT][kSP][2], const lds_u8* slot, const int (&xo)[2],
                                             uint32_t (&nz)[kSP][2], uint32_t (&s2)[kSP][2], bool encode) {
  constexpr int kGPS = kGS >= kStepRows ? 1 : kStepRows / kGS;
  const int g_lane = (lane & 15) >> 2;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if ((b == 0 && encode) || kGPS == 2) {
      const int gi = b & (kGPS - 1);
#pragma unroll
      for (int sp = 0; sp < kSP; ++sp) {
        const lds_u8* const ps = slot + kT * 2048 + (gi * kSP + sp) * 512 + 4 * lane;
        scaled_params<kBF>(*(const lds_u32*)(ps), *(const lds_u32*)(ps + 256), g_lane, nz[sp], s2[sp]);
      }
    }
    f16x8 xa[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) xa[t] = *(const lds_f16x8*)(slot + 2048 * t + xo[b]);
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp) {
      f16x8 bf[2];
      unpack_block_scaled<kBF>(st.w[sp][2 * b], st.w[sp][2 * b + 1], nc, nz[sp], s2[sp], bf);
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int f = 0; f < 2; ++f) tot[t][sp][f] = mfma_16x16x32<kBF>(xa[t], bf[f], tot[t][sp][f]);
    }
  }
}

// Bytes of a wavefront's sums (kT x kSP x 2 vectors of 16 bytes per lane).
template <int kT, int kSP>
constexpr int sums_bytes() {
  return kT * kSP * 2 * 64 * 16;
}

// LDS of a workgroup: its wavefronts' slots, or, if more, the regions the
// end of the call adds the sums in (max(kW / 2, 1) of them).
template <int kT, int kGS, int kSP>
constexpr size_t prescaled_lds_bytes(int waves) {
  const size_t slots = static_cast<size_t>(waves) * kRing * slot_bytes<kT, kGS, kSP>();
  const size_t sums = static_cast<size_t>(waves >= 2 ? waves / 2 : 1) * sums_bytes<kT, kSP>();
  return slots > sums ? slots : sums;
}

// kT 16-token tiles (3 or 4), groups of kGS rows, kW wavefronts per
// workgroup (each a contiguous part of the workgroup's K range; eight run two
// per SIMD), kSP adjacent strips per workgroup. `units` counts kSP-strip units.
template <int kT, int kGS, int kW, int kSP, bool kBF>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(kW >= 8 ? 2 : 1))) void w4a16_gemv_prescaled_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ qb, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ partial, int M, int N, int K,
    int units, int splits, XcdMap map, int gstep) {
  constexpr int kGPS = kGS >= kStepRows ? 1 : kStepRows / kGS;  // groups per step
  constexpr bool kHalf = kGS == 2 * kStepRows;                   // a group spans two steps
  // vector-memory loads of a step with / without group parameters; the
  // steps alternate from an even one (each wavefront starts on a 128-row
  // boundary), and the waits count the loads of the next three steps
  constexpr int kLp = kSP + 2 * kT + 2 * kSP * kGPS;
  constexpr int kLn = kHalf ? kSP + 2 * kT : kLp;
  constexpr int kWaitEven = kLn;  // before an even step: the next (odd) step's loads
  constexpr int kWaitOdd = kLp;   // before an odd step
  static_assert(kT >= 2 && kT <= 4 && kSP >= 1 && kSP <= 4, "17-64 tokens, at most four strips");
  static_assert(kRing == 2 && kLp + kLn <= 63, "loads in flight within the vmcnt range");
  constexpr int kSlot = slot_bytes<kT, kGS, kSP>();  // bytes per step and wavefront
  extern __shared__ __attribute__((aligned(16))) uint8_t x_dyn[];  // kW * kRing slots

  int unit, split;
  if (!decode_work(blockIdx.x, map.strips_per_xcd, units, splits, unit, split)) return;
  const int strip = unit * kSP;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, h = lane >> 4;
  const int c = j & 3, g = j >> 2;
  const int NP = N >> 3;
  const int cps = (K / kBChunkRows) / splits;  // 128-row chunks per split (plan: divides)
  const int cpw = cps / kW;                    // chunks per wavefront (plan: divides, >= 1)
  const int n = 2 * cpw;                       // steps of this wavefront (even)
  const int p0 = 2 * (split * cps + wave * cpw);  // its first pair
  const int col = strip * kBStrip + c;

  PLane L;
  L.qb = qb + static_cast<size_t>(strip) * 64 + lane;
  L.pair_stride = static_cast<size_t>(NP / kBStrip) * 64;
  {
    const int grows = gstep ? K / kGS : 1;  // parameter rows
    L.sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, grows * N * 2, 0x00020000);
    L.zr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qz), 0, grows * NP * 4, 0x00020000);
    L.s_off = static_cast<uint32_t>(col * 8 + 2 * g) * 2u;
    L.z_off = static_cast<uint32_t>(col) * 4u;
    L.s_row = static_cast<uint32_t>(gstep * N) * 2u;
    L.z_row = static_cast<uint32_t>(gstep * NP) * 4u;
  }
  L.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, M * K * 2, 0x00020000);
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int r = 8 * hq + lane / 8;  // token row within the tile
    L.xdma[hq] = static_cast<uint32_t>(r * K + 8 * ((lane % 8) ^ ((r >> 1) & 7))) * 2u;
  }
  L.xtile = static_cast<uint32_t>(16 * K) * 2u;
  lds_u8* slot[kRing];
#pragma unroll
  for (int q = 0; q < kRing; ++q) slot[q] = (lds_u8*)(x_dyn) + (wave * kRing + q) * kSlot;
  // the lane's 16 bytes of block b in a tile: token row j, chunk 4b + h
  int xo[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) xo[b] = 128 * j + 16 * ((4 * b + h) ^ ((j >> 1) & 7));

  const NibConst nc = nib_const();
  f32x4 tot[kT][kSP][2];
#pragma unroll
  for (int t = 0; t < kT; ++t)
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp)
#pragma unroll
      for (int f = 0; f < 2; ++f) tot[t][sp][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    PStep<kSP> st[kRing];
    uint32_t nz[kSP][2], s2[kSP][2];  // encoded group parameters, carried
    // Prologue: steps 0 and 1 (a wavefront has an even number of steps).
#pragma unroll
    for (int q = 0; q < kRing; ++q) {
      load_step<kT, kGS, kSP>(st[q], L, p0 + min(q, n - 1), slot[q], !kHalf || q % 2 == 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Loads complete in issue order. Before step s is computed, the loads
    // of step s+1 were issued after its own: where it exists, waiting down
    // to its count leaves only those in flight; otherwise (the last step)
    // wait for all. Step s uses buffer and slot s % 2, and its parity is
    // that of s - i (i is even).
    auto run = [&](int u, int s, bool steady, bool refill) {
      const int q = u % kRing;
      const bool even = u % 2 == 0;
      if (steady || s + kRing - 1 < n) {
        if (even) {
          wait_counts<kWaitEven, 15>();
        } else {
          wait_counts<kWaitOdd, 15>();
        }
      } else {
        wait_counts<0, 15>();
      }
      compute_step<kT, kGS, kSP, kBF>(st[q], nc, lane, tot, slot[q], xo, nz, s2, !kHalf || even);
      __builtin_amdgcn_sched_barrier(0);
      if (refill) load_step<kT, kGS, kSP>(st[q], L, p0 + s + kRing, slot[q], !kHalf || even);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Steady loop: every refill is in range, so the requests are
    // unconditional (a conditional one inside the loop makes the compiler
    // copy the buffer at the back edge, which waits for every load).
    int i = 0;
    for (; i + 2 * kRing <= n; i += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) run(u, i + u, true, true);
    }
    // The last two steps (n is even); both are in flight.
#pragma unroll
    for (int u = 0; u < 2 * kRing - 2; ++u)
      if (i + u < n) run(u, i + u, false, i + u + kRing < n);
  }

  // Every load has landed (the last step waited for all); lgkmcnt(0) and a
  // barrier make sure no wavefront still reads its slots. With two or more
  // wavefronts, those in the upper half first add their sums into the lower
  // half's (wavefront w + kW/2 into w, through LDS regions of sums_bytes), then
  // the lower half's sums are added in wavefront order and stored.
  wait_counts<63, 0>();
  __syncthreads();
  lds_u8* const base = (lds_u8*)(x_dyn);
  constexpr int kSums = sums_bytes<kT, kSP>();
  constexpr int kR = kW >= 2 ? kW / 2 : 1;
  if constexpr (kW >= 2) {
    if (wave >= kR) {
      lds_u8* const red = base + (wave - kR) * kSums;
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int sp = 0; sp < kSP; ++sp)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            *(lds_f32x4*)(red + (((t * kSP + sp) * 2 + f) * 64 + lane) * 16) = tot[t][sp][f];
    }
    __syncthreads();
    if (wave < kR) {
      const lds_u8* const red = base + wave * kSums;
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int sp = 0; sp < kSP; ++sp)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            tot[t][sp][f] += *(const lds_f32x4*)(red + (((t * kSP + sp) * 2 + f) * 64 + lane) * 16);
    }
    // each lower wavefront rewrites only the region it has just read
  }
  store_unit_sums<kT, kSP, kW, kBF, kR>(tot, base, kSums, wave, lane, M, N, strip, split, splits, y, partial);
}

template <int kT, int kGS, int kSP, bool kBF>
hipError_t launch_ps_waves(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz, uint16_t* y,
                           float* part, int m, int n, int k, const GemvPlan& plan, int units, XcdMap map, dim3 grid,
                           hipStream_t stream) {
  const size_t lds = prescaled_lds_bytes<kT, kGS, kSP>(plan.waves);
  const int gstep = plan.per_channel ? 0 : 1;
  switch (plan.waves) {
    case 1:
      return launch_kernel(w4a16_gemv_prescaled_kernel<kT, kGS, 1, kSP, kBF>, grid, dim3(64), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, gstep);
    case 2:
      return launch_kernel(w4a16_gemv_prescaled_kernel<kT, kGS, 2, kSP, kBF>, grid, dim3(128), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, gstep);
    case 4:
      return launch_kernel(w4a16_gemv_prescaled_kernel<kT, kGS, 4, kSP, kBF>, grid, dim3(256), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, gstep);
    case 8:
      return launch_kernel(w4a16_gemv_prescaled_kernel<kT, kGS, 8, kSP, kBF>, grid, dim3(512), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, gstep);
    default:
      return hipErrorInvalidValue;
  }
}

template <int kT, int kGS, bool kBF>
hipError_t launch_ps_strips(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                            uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                            XcdMap map, dim3 grid, hipStream_t stream) {
  if constexpr (kGS >= 64) {
    if (plan.strips_per_unit == 3)
      return launch_ps_waves<kT, kGS, 3, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    if (plan.strips_per_unit == 2)
      return launch_ps_waves<kT, kGS, 2, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
  }
  if (plan.strips_per_unit != 1) return hipErrorInvalidValue;
  return launch_ps_waves<kT, kGS, 1, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
}

template <int kGS, bool kBF>
hipError_t launch_ps_group(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                           uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units, XcdMap map,
                           dim3 grid, hipStream_t stream) {
  if (m > 48) return launch_ps_strips<4, kGS, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
  if (m > 32) return launch_ps_strips<3, kGS, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
  return launch_ps_strips<2, kGS, kBF>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
}

}  // namespace

hipError_t launch_w4a16_gemv_blocked_prescaled(const uint16_t* x, const u32x4* qb, const uint16_t* scales,
                                               const uint32_t* qz, uint16_t* y, float* part, int m, int n, int k,
                                               const GemvPlan& plan, int units, int strips_per_xcd, dim3 grid,
                                               bool bf16, hipStream_t stream) {
  if (m <= 16 || m > kGemvMaxM) return hipErrorInvalidValue;
  XcdMap map;
  map.strips_per_xcd = strips_per_xcd;
  switch (plan.group * 2 + (bf16 ? 1 : 0)) {
    case 64:
      return launch_ps_group<32, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 65:
      return launch_ps_group<32, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 128:
      return launch_ps_group<64, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 129:
      return launch_ps_group<64, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 256:
      return launch_ps_group<128, false>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    case 257:
      return launch_ps_group<128, true>(x, qb, scales, qz, y, part, m, n, k, plan, units, map, grid, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mq
