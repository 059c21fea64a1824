// W4A16 GEMV for decode (M <= 64) on gfx950.
//
// Source: LMDeploy toolkit overview, section 2.5 (AWQ 4-bit weights, group
// size 128, 4-bit inference speedup from the smaller weight stream) and
// LMDeploy 4-bit deployment guide, section 2.2 (scale and weight consumed in
// one kernel) and section 3.2 (per-layer group size: 64 for the vision
// tower's attention, 128 for the language model).
// y[m,n] = sum_k x[m,k] * (q[k,n] - z[k/G,n]) * s[k/G,n], G in {32, 64, 128};
// every kernel is instantiated per group size.
//
// Decode reads every weight once and does little arithmetic per weight, so
// the kernel is bound by the HBM weight stream. Common to both kernels:
//  * the M <= 16 tokens ride on the 16-row side of v_mfma_f32_16x16x32_f16,
//    so a weight costs only its unpack on the vector ALU, not M
//    multiply-adds (token rows >= M read a valid row and are never stored;
//    an MFMA output row depends on its own A row only);
//  * a wavefront owns 16 packed columns (128 outputs): lane (j = lane%16,
//    h = lane/16) needs word j of rows 8h..8h+7 of each 32-row step and
//    turns them into B fragments in registers;
//  * each group's sum over its 128 rows is formed in fp32 by the MFMA and
//    scaled in fp32 once per group;
//  * HBM streams well only when a workgroup reads >= 256 contiguous bytes
//    of each row it touches, so workgroups cover wide column strips and K
//    is split across workgroups to occupy every compute unit. Each split
//    writes fp32 partial sums to the workspace and a small second kernel
//    adds the splits in split order (the kernel boundary publishes them; a
//    device-scope fence inside the kernel would write back and invalidate
//    the whole L2 per workgroup). Results are deterministic.
//
// Main kernel (N % 32 == 0): the weight stream goes global -> LDS with
// global_load_lds (no registers held while loads are in flight) through a
// ring of stages, 64 packed columns (256 B) x 32 rows per stage, so several
// stages per workgroup are in flight. The zero point is folded into a
// per-group correction: fragments hold 1024 + q (the fp16 bit trick without
// a subtraction), one extra MFMA against a fragment of ones gives the
// group's per-token sum X of x, and the group adds s * (acc - (1024+z) * X).
//
// General kernel (any N % 8 == 0): the same math with (q - z) formed exactly
// in the fragments and a register-staged double buffer per wavefront.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"
#include "w4a16_split.h"

namespace mq {
namespace {

constexpr int kWaveCols = 16;        // packed columns per wavefront (128 outputs)

template <bool kBF>
__device__ __forceinline__ void store_f16x8(uint16_t* dst, const float (&v)[8]) {
  u32x4 out;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    out[t] = half_bits<kBF>(v[2 * t]) | (static_cast<uint32_t>(half_bits<kBF>(v[2 * t + 1])) << 16);
  *reinterpret_cast<u32x4*>(dst) = out;
}

// Lane (j, h) holds tokens m0+4h..m0+4h+3 of packed column c in tot[p][q]
// (field p, token m0 + 4h + q): write them as fp16 to y, or as fp32 to the
// split's partial-sum slice.
template <bool kBF>
__device__ __forceinline__ void write_out(const f32x4 (&tot)[8], uint16_t* __restrict__ y,
                                          float* __restrict__ partial, int M, int N, int c, int h, int split,
                                          int splits, int m0 = 0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = m0 + 4 * h + q;
    if (m >= M) continue;
    if (splits == 1) {
      float v[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) v[p] = tot[p][q];
      store_f16x8<kBF>(y + static_cast<size_t>(m) * N + 8 * c, v);
    } else {
      float* dst = partial + (static_cast<size_t>(split) * M + m) * N + 8 * c;
      *reinterpret_cast<f32x4*>(dst) = f32x4{tot[0][q], tot[1][q], tot[2][q], tot[3][q]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{tot[4][q], tot[5][q], tot[6][q], tot[7][q]};
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel: LDS-staged, N % 32 == 0.
//
// LDS layouts (chunks are 16 bytes):
//  * weights, per stage: 32 rows x 16 chunks; chunk c of row r is stored at
//    position r*16 + (c ^ (((r >> 3) & 3) << 2)), so the 64 lanes of a
//    fragment read (word j of rows 8h+e, h = 0..3) hit 64 distinct banks;
//  * x, per stage: 16 tokens x 4 chunks (32 fp16); chunk c of token i at
//    i*4 + (c ^ ((i >> 2) & 3)) so a 16-lane fragment read is conflict-free;
//  * scales and zero points of all groups of the split, loaded up front.
// ---------------------------------------------------------------------------

constexpr int kLStrip = 64;                     // packed columns per workgroup
constexpr int kLRows = 32;                      // rows per stage (one MFMA k-step)
constexpr int kLStageWords = kLRows * kLStrip;  // 2048 words = 8 KB
constexpr int kLXWords = 16 * kLRows / 2;       // 256 words = 1 KB
constexpr int kLMaxRows = 1024;                 // rows per split (their scales and zero points sit in LDS)
constexpr int kLStages = 3;  // ring depth (4, 6 and 8 stages measured slower)
// Per lane and stage: 2 x 16 B of weights + 4 B of x per 16-token tile.
template <int T>
constexpr int lds_loads_per_stage() { return 2 + T; }

// B fragments of 1024 + q (even p) or 1024 + 16 q (odd p) for one 32-row
// step: w[e] is the lane's word of row 8h + e. The masks and the 1024.0
// pattern come in registers (NibConst), so the compiler forms each
// (v & mask) | magic as one v_and_or_b32 of its own; the fragments feed MFMA
// operands, and only for its own instructions does the compiler insert the
// wait states a VALU write needs before an MFMA reads the register.
// kBF: bf16 fragments of 128 + q for every field (the high fields shifted
// down first; see NibConst).
template <bool kBF>
__device__ __forceinline__ void unpack_step_biased(const uint32_t (&w)[8], const NibConst& c, f16x8 (&b)[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = byte_perm(w[2 * t + 1], w[2 * t], 0x05040100u);  // bytes 0,1 of both rows
    const uint32_t hi = byte_perm(w[2 * t + 1], w[2 * t], 0x07060302u);  // bytes 2,3 of both rows
    const uint32_t lo8 = lo >> 8, hi8 = hi >> 8;
    uint32_t v[8];
    if constexpr (kBF) {
      const uint32_t m = c.bmagic;
      v[0] = (lo & c.lo) | m;
      v[1] = ((lo >> 4) & c.lo) | m;
      v[2] = (lo8 & c.lo) | m;
      v[3] = ((lo >> 12) & c.lo) | m;
      v[4] = (hi & c.lo) | m;
      v[5] = ((hi >> 4) & c.lo) | m;
      v[6] = (hi8 & c.lo) | m;
      v[7] = ((hi >> 12) & c.lo) | m;
    } else {
      v[0] = (lo & c.lo) | c.magic;
      v[1] = (lo & c.hi) | c.magic;
      v[2] = (lo8 & c.lo) | c.magic;
      v[3] = (lo8 & c.hi) | c.magic;
      v[4] = (hi & c.lo) | c.magic;
      v[5] = (hi & c.hi) | c.magic;
      v[6] = (hi8 & c.lo) | c.magic;
      v[7] = (hi8 & c.hi) | c.magic;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 d = as_f16x2(v[p]);
      b[p][2 * t] = d[0];
      b[p][2 * t + 1] = d[1];
    }
  }
}

// Byte offset of the 16-byte chunk lane `lane` of wavefront `wave` loads
// for DMA instruction l of a stage: LDS position p = l*256 + wave*64 + lane
// holds chunk (p & 15) ^ swizzle(row) of row p >> 4.
__device__ __forceinline__ uint32_t lds_weight_offset(int l, int wave, int lane, int valid_chunks, int chunk0,
                                                      int NP) {
  const int p = l * 256 + wave * 64 + lane;
  const int row = p >> 4;
  const int logical = (p & 15) ^ (((row >> 3) & 3) << 2);
  const int cl = min(logical, valid_chunks - 1);
  return static_cast<uint32_t>(row) * static_cast<uint32_t>(NP) * 4u + static_cast<uint32_t>(chunk0 + cl) * 16u;
}

// Start the DMA of stage st (32 rows of the strip + the matching x slice of
// each 16-token tile) into its ring slot: 2 x 16 B of weights and 4 B of x
// per tile and lane. row_begin is the split's first row.
template <int T>
__device__ __forceinline__ void lds_issue_stage(int st, int row_begin, int NP, int wave, const char* qwb,
                                                const char* xb, uint32_t woff0, uint32_t woff1,
                                                const uint32_t (&xoff)[T], lds_u32* s_w, lds_u32* s_x) {
  const int slot = st % kLStages;
  const int k0 = row_begin + st * kLRows;
  const char* wbase = qwb + static_cast<size_t>(k0) * NP * 4;
  lds_u32* wdst = s_w + slot * kLStageWords + wave * 256;
  __builtin_amdgcn_global_load_lds(wbase + woff0, wdst, 16, 0, 0);
  __builtin_amdgcn_global_load_lds(wbase + woff1, wdst + 1024, 16, 0, 0);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    lds_u32* xdst = s_x + (slot * T + t) * kLXWords + wave * 64;
    __builtin_amdgcn_global_load_lds(xb + static_cast<size_t>(k0) * 2 + xoff[t], xdst, 4, 0, 0);
  }
}

// kT = number of 16-token tiles (M <= 16 kT); every weight fragment, once
// unpacked, feeds the MFMAs of all kT tiles. kGS = group size (a multiple
// of the 32-row step).
template <int kT, int kGS, bool kBF>
__global__ __launch_bounds__(256) void w4a16_gemv_lds_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz,
    uint16_t* __restrict__ y, float* __restrict__ partial, int M, int N, int K, int strips, int splits,
    XcdMap map, int gstep) {
  constexpr int kLLoadsPerStage = lds_loads_per_stage<kT>();
  constexpr int kSPG = kGS / kLRows;             // 32-row steps per group
  constexpr int kMaxGroups = kLMaxRows / kGS;    // groups per split held in LDS
  static_assert(kGS % kLRows == 0 && kLMaxRows % kGS == 0, "group size");
  __shared__ __attribute__((aligned(16))) uint32_t s_w[kLStages * kLStageWords];
  __shared__ __attribute__((aligned(16))) uint32_t s_x[kLStages * kT * kLXWords];
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[kMaxGroups * 256];
  __shared__ __attribute__((aligned(16))) uint32_t s_z[kMaxGroups * 64];

  int strip, split;
  if (!decode_work(blockIdx.x, map.strips_per_xcd, strips, splits, strip, split)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int j = lane & 15;
  const int h = lane >> 4;
  const int NP = N >> 3;
  const int NC = NP >> 2;  // 16-byte chunks per row
  const int G = K / kGS;
  const int g_begin = static_cast<int>(static_cast<int64_t>(split) * G / splits);
  const int g_end = static_cast<int>(static_cast<int64_t>(split + 1) * G / splits);
  const int Gs = g_end - g_begin;  // <= kMaxGroups (plan)
  const int T = Gs * kSPG;
  const int row_begin = g_begin * kGS;
  const int chunk0 = strip * (kLStrip / 4);
  const int valid_chunks = min(kLStrip / 4, NC - chunk0);  // >= 1
  const int valid_cols = valid_chunks * 4;

  const char* qwb = reinterpret_cast<const char*>(qw);
  const char* xb = reinterpret_cast<const char*>(x);

  // Per-lane global byte offsets, constant over stages. Columns past N
  // re-read the strip's last valid chunk (never stored).
  const uint32_t woff0 = lds_weight_offset(0, wave, lane, valid_chunks, chunk0, NP);
  const uint32_t woff1 = lds_weight_offset(1, wave, lane, valid_chunks, chunk0, NP);
  uint32_t xoff[kT];
  {
    const int q = wave * 64 + lane;
    const int i = q >> 4;
    const int c = ((q >> 2) & 3) ^ ((i >> 2) & 3);
#pragma unroll
    for (int t = 0; t < kT; ++t)
      xoff[t] = static_cast<uint32_t>((min(16 * t + i, M - 1) * K + c * 8 + (q & 3) * 2) * 2);
  }
  lds_u32* const s_w_lds = (lds_u32*)(s_w);
  lds_u32* const s_x_lds = (lds_u32*)(s_x);

  // Prologue: scales (512 fp16 = 64 chunks) and zero points (64 words) of
  // every group of the split; wavefront w loads groups w, w+4, ...
  {
    const int pc = min(lane, valid_cols - 1);
    for (int gi = wave; gi < Gs; gi += 4) {
      const size_t g = static_cast<size_t>(gstep) * static_cast<size_t>(g_begin + gi);  // gstep 0: per-channel
      const char* sp = reinterpret_cast<const char*>(scales) + (g * N + static_cast<size_t>(strip) * 512) * 2;
      __builtin_amdgcn_global_load_lds(sp + pc * 16, (lds_u32*)(s_sc) + gi * 256, 16, 0, 0);
      const char* zp = reinterpret_cast<const char*>(qz) + (g * NP + static_cast<size_t>(strip) * kLStrip) * 4;
      __builtin_amdgcn_global_load_lds(zp + pc * 4, (lds_u32*)(s_z) + gi * 64, 4, 0, 0);
    }
  }
  const int pre = min(kLStages - 1, T);
  for (int st = 0; st < pre; ++st)
    lds_issue_stage(st, row_begin, NP, wave, qwb, xb, woff0, woff1, xoff, s_w_lds, s_x_lds);

  // Fragment read offsets (words within a stage).
  const int wchunk = (4 * wave + (j >> 2)) ^ (h << 2);
  const int wread = (8 * h) * 64 + wchunk * 4 + (j & 3);
  const int xread = j * 16 + ((h ^ ((j >> 2) & 3)) * 4);
  const int col = 16 * wave + j;  // packed column within the strip
  const NibConst nc = nib_const();
  const f16x8 ones = ones_fragment<kBF>();

  f32x4 tot[kT][8];
#pragma unroll
  for (int t = 0; t < kT; ++t)
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[t][p][q] = 0.f;

  for (int gi = 0; gi < Gs; ++gi) {
    f32x4 acc[kT][8];
    f32x4 accx[kT];  // per-token sum of x over the group's rows
#pragma unroll
    for (int ks = 0; ks < kSPG; ++ks) {
      const int it = gi * kSPG + ks;
      if (it + kLStages - 2 < T) {
        wait_counts<(kLStages - 2) * kLLoadsPerStage, 0>();
      } else {
        wait_counts<0, 0>();
      }
      bare_barrier();
      if (it + kLStages - 1 < T)
        lds_issue_stage(it + kLStages - 1, row_begin, NP, wave, qwb, xb, woff0, woff1, xoff, s_w_lds, s_x_lds);
      const int slot = it % kLStages;
      const uint32_t* wst = s_w + slot * kLStageWords + wread;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = wst[e * 64];
      f16x8 a[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t) a[t] = *reinterpret_cast<const f16x8*>(&s_x[(slot * kT + t) * kLXWords + xread]);
      f16x8 b[8];
      unpack_step_biased<kBF>(w, nc, b);
      const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        accx[t] = mfma_16x16x32<kBF>(a[t], ones, ks == 0 ? zero4 : accx[t]);
#pragma unroll
        for (int p = 0; p < 8; ++p) acc[t][p] = mfma_16x16x32<kBF>(a[t], b[p], ks == 0 ? zero4 : acc[t][p]);
      }
    }
    // tot += s * (acc - (1024 + z) * X); odd fields carry 16 (q - z), so
    // their scale is s / 16 (exact). bf16: tot += s * (acc - (128 + z) * X).
    const uint32_t zw = s_z[gi * 64 + col];
    const u32x4 sv = *reinterpret_cast<const u32x4*>(&s_sc[gi * 256 + col * 4]);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 s2 = as_f16x2(sv[p >> 1]);
      const float zf = static_cast<float>((zw >> (4 * p)) & 15u);
      const float sc = static_cast<float>(s2[p & 1]) * ((p & 1) && !kBF ? 0.0625f : 1.0f);
      const float bias = kBF ? 128.0f + zf : ((p & 1) ? 1024.0f + 16.0f * zf : 1024.0f + zf);
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[t][p][q] = fmaf(sc, fmaf(-bias, accx[t][q], acc[t][p][q]), tot[t][p][q]);
    }
  }

  const int c = strip * kLStrip + col;
  if (c < NP) {
#pragma unroll
    for (int t = 0; t < kT; ++t) write_out<kBF>(tot[t], y, partial, M, N, c, h, split, splits, 16 * t);
  }
}

// ---------------------------------------------------------------------------
// General kernel: register-staged, any N % 8 == 0.
// ---------------------------------------------------------------------------

// One group's operands for one lane: S steps (S = G / 32) x 8 rows of its
// packed column, the S matching activation fragments, the zero-point word
// and 8 scales.
template <int S>
struct GroupRegs {
  uint32_t w[S][8];
  f16x8 a[S];
  uint32_t zw;
  u32x4 sv;
};

// Pointers are kept as wavefront-uniform bases plus 32-bit per-lane offsets,
// so every load is a scalar-base global load with no per-load address math.
struct GemvLane {
  const char* qw;     // qweight (uniform)
  const char* x;      // x (uniform)
  const char* qz;     // qzeros (uniform)
  const char* sc;     // scales (uniform)
  uint32_t w_off;     // byte offset of word (row 8h, column) in a group
  uint32_t x_off;     // byte offset of (token, 8h) in x
  uint32_t z_off;     // byte offset of the lane's word in a qzeros row
  uint32_t s_off;     // byte offset of the lane's 8 scales in a scales row
  size_t row_bytes;   // NP * 4
  size_t zrow_bytes;  // NP * 4, or 0 for per-channel zero points
  size_t srow_bytes;  // N * 2, or 0 for per-channel scales
};

template <typename T>
__device__ __forceinline__ T load_at(const char* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

template <int S>
__device__ __forceinline__ void load_group(GroupRegs<S>& r, const GemvLane L, int g) {
  const char* wg = L.qw + static_cast<size_t>(g) * (32 * S) * L.row_bytes;
#pragma unroll
  for (int ks = 0; ks < S; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) r.w[ks][e] = load_at<uint32_t>(wg + (ks * 32 + e) * L.row_bytes, L.w_off);
  const char* xg = L.x + static_cast<size_t>(g) * (32 * S) * 2;
#pragma unroll
  for (int ks = 0; ks < S; ++ks) r.a[ks] = load_at<f16x8>(xg + ks * 64, L.x_off);
  r.zw = load_at<uint32_t>(L.qz + static_cast<size_t>(g) * L.zrow_bytes, L.z_off);
  r.sv = load_at<u32x4>(L.sc + static_cast<size_t>(g) * L.srow_bytes, L.s_off);
}

// bf16 (kBF): bf16 has no packed subtraction to form q - z exactly, so the
// fragments hold 128 + q and the group adds s * (acc - (128 + z) * X), with X
// the per-token sum of x from one more MFMA against ones (as the LDS kernel).
template <int S, bool kBF>
__device__ __forceinline__ void compute_group(const GroupRegs<S>& r, f32x4 (&tot)[8]) {
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc[8];
  if constexpr (kBF) {
    const NibConst nc = nib_const();
    const f16x8 ones = ones_fragment<true>();
    f32x4 accx;
#pragma unroll
    for (int ks = 0; ks < S; ++ks) {
      f16x8 b[8];
      unpack_step_biased<true>(r.w[ks], nc, b);
      accx = mfma_16x16x32<true>(r.a[ks], ones, ks == 0 ? zero4 : accx);
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[p] = mfma_16x16x32<true>(r.a[ks], b[p], ks == 0 ? zero4 : acc[p]);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 s2 = as_f16x2(r.sv[p >> 1]);
      const float sc = static_cast<float>(s2[p & 1]);
      const float bias = 128.0f + static_cast<float>((r.zw >> (4 * p)) & 15u);
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[p][q] = fmaf(sc, fmaf(-bias, accx[q], acc[p][q]), tot[p][q]);
    }
  } else {
    uint32_t negz[8];
    zero_bias(r.zw, negz);
#pragma unroll
    for (int ks = 0; ks < S; ++ks) {
      f16x8 b[8];
      unpack_step(r.w[ks], negz, b);
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[p] = mfma_16x16x32<false>(r.a[ks], b[p], ks == 0 ? zero4 : acc[p]);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 s2 = as_f16x2(r.sv[p >> 1]);
      const float sc = static_cast<float>(s2[p & 1]) * ((p & 1) ? 0.0625f : 1.0f);
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[p][q] = fmaf(acc[p][q], sc, tot[p][q]);
    }
  }
}

// The wavefronts of a workgroup sit side by side in N (NWC x 64 contiguous
// bytes per row) and walk the split's groups (of kGS rows) together.
template <int NWC, int kGS, bool kBF>
__global__ __launch_bounds__(NWC * 64) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz,
    uint16_t* __restrict__ y, float* __restrict__ partial, int M, int N, int K, int strips, int splits,
    XcdMap map, int gstep) {
  int strip, split;
  if (!decode_work(blockIdx.x, map.strips_per_xcd, strips, splits, strip, split)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int j = lane & 15;
  const int h = lane >> 4;
  const int NP = N >> 3;
  const int c = (strip * NWC + wave) * kWaveCols + j;
  const bool cvalid = c < NP;
  const int cc = cvalid ? c : NP - 1;
  constexpr int kSPG = kGS / 32;  // 32-row MFMA steps per group
  const int G = K / kGS;
  const int g_begin = static_cast<int>(static_cast<int64_t>(split) * G / splits);
  const int g_end = static_cast<int>(static_cast<int64_t>(split + 1) * G / splits);

  GemvLane L;
  L.qw = reinterpret_cast<const char*>(qw);
  L.x = reinterpret_cast<const char*>(x);
  L.qz = reinterpret_cast<const char*>(qz);
  L.sc = reinterpret_cast<const char*>(scales);
  L.w_off = static_cast<uint32_t>(8 * h * NP + cc) * 4u;
  L.x_off = static_cast<uint32_t>((j < M ? j : M - 1) * K + 8 * h) * 2u;
  L.z_off = static_cast<uint32_t>(cc) * 4u;
  L.s_off = static_cast<uint32_t>(cc) * 16u;
  L.row_bytes = static_cast<size_t>(NP) * 4;
  L.zrow_bytes = static_cast<size_t>(gstep) * NP * 4;
  L.srow_bytes = static_cast<size_t>(gstep) * N * 2;

  f32x4 tot[8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[p][q] = 0.f;

  // The groups of this split, in order. Two register buffers: group i+1 is
  // loaded while group i is computed; inside the loop every prefetch is
  // unconditional, and sched_barrier keeps the compiler from sinking it
  // below the math it is meant to overlap.
  const int n = g_end - g_begin;
  {
    GroupRegs<kSPG> ra, rb;
    load_group(ra, L, g_begin);
    int i = 0;
    for (; i + 2 < n; i += 2) {
      load_group(rb, L, g_begin + i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute_group<kSPG, kBF>(ra, tot);
      load_group(ra, L, g_begin + i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute_group<kSPG, kBF>(rb, tot);
    }
    if (i + 1 < n) {
      load_group(rb, L, g_begin + i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute_group<kSPG, kBF>(ra, tot);
      compute_group<kSPG, kBF>(rb, tot);
    } else {
      compute_group<kSPG, kBF>(ra, tot);
    }
  }
  if (cvalid) write_out<kBF>(tot, y, partial, M, N, c, h, split, splits);
}

}  // namespace

constexpr int kGemvWaves = 4;         // register-staged kernel: wavefronts per workgroup
constexpr int64_t kTargetWgs = 384;   // 1.5 workgroups per CU (192: slower; 768: no faster)

GemvPlan plan_w4a16_gemv(int64_t M, int64_t N, int64_t K, int64_t group) {
  GemvPlan plan{1, kGemvWaves, 0, false, static_cast<int>(group)};
  plan.lds = (N / 8) % 4 == 0;
  const int64_t strip_cols = plan.lds ? int64_t{kLStrip} : int64_t{kWaveCols} * plan.waves;
  const int64_t strips = (N / 8 + strip_cols - 1) / strip_cols;
  const int64_t G = K / group;
  const int64_t max_groups = kLMaxRows / group;  // per split, LDS kernel
  // Split K only as far as needed to reach the target workgroup count: the
  // smallest divisor of the group count that gets there (and, for the LDS
  // kernel, that leaves at most kLMaxRows rows per split).
  int64_t splits = 1;
  while (strips * splits < kTargetWgs && splits < G) {
    ++splits;
    while (G % splits) ++splits;
  }
  if (plan.lds) {
    while (G / splits > max_groups) {
      ++splits;
      while (G % splits) ++splits;
    }
    if (M > 16) {
      // More tokens: each split's fp32 partial sums (M x N, written and read
      // once) grow with M while the weight stream does not, and the MFMA work
      // per workgroup grows too. Pick the split count (a divisor of the group
      // count, at most kLMaxRows rows per split) with the smallest modelled
      // time: max(HBM bytes / 5 TB/s, MFMA work / (busy CUs x 2.25 TFLOP/s))
      // plus about 2 us for the reduce kernel. Both rates are the ones this
      // kernel pair reaches on the MI355X (stream and 16x16x32 fp16 MFMA with
      // the unpack).
      const double mpad = static_cast<double>((M + 15) / 16 * 16);
      double best = 1e30;
      int64_t best_s = splits;
      for (int64_t s = splits; s <= G; ++s) {
        if (G % s) continue;
        const double bytes = static_cast<double>(K) * N / 2 + (s > 1 ? 2.0 * s * M * N * 4 : 0.0);
        const double wgs = static_cast<double>(strips * s < 256 ? strips * s : 256);
        const double t = std::max(bytes / 5e12, 2.0 * mpad * N * K / (wgs * 2.25e12)) + (s > 1 ? 2e-6 : 0.0);
        if (t < best) {
          best = t;
          best_s = s;
        }
      }
      splits = best_s;
    }
  }
  plan.splits = static_cast<int>(splits);
  plan.workspace_bytes = splits > 1 ? static_cast<size_t>(splits) * M * N * sizeof(float) : 0;
  return plan;
}

namespace {

template <int kGS, bool kBF>
hipError_t launch_gemv_main(const uint16_t* x, const uint32_t* qw, const uint16_t* scales, const uint32_t* qz,
                            uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int strips,
                            XcdMap map, dim3 grid, hipStream_t stream) {
  if (plan.lds) {
    switch ((m + 15) / 16) {
      case 1:
        return launch_kernel(w4a16_gemv_lds_kernel<1, kGS, kBF>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part,
                             m, n, k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
      case 2:
        return launch_kernel(w4a16_gemv_lds_kernel<2, kGS, kBF>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part,
                             m, n, k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
      case 3:
        return launch_kernel(w4a16_gemv_lds_kernel<3, kGS, kBF>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part,
                             m, n, k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
      default:
        return launch_kernel(w4a16_gemv_lds_kernel<4, kGS, kBF>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part,
                             m, n, k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
    }
  }
  switch (plan.waves) {
    case 2:
      return launch_kernel(w4a16_gemv_kernel<2, kGS, kBF>, grid, dim3(128), 0, stream, x, qw, scales, qz, y, part, m, n,
                           k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
    case 8:
      return launch_kernel(w4a16_gemv_kernel<8, kGS, kBF>, grid, dim3(512), 0, stream, x, qw, scales, qz, y, part, m, n,
                           k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
    default:
      return launch_kernel(w4a16_gemv_kernel<4, kGS, kBF>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part, m, n,
                           k, strips, plan.splits, map, plan.per_channel ? 0 : 1);
  }
}

}  // namespace

hipError_t launch_w4a16_gemv(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, const GemvPlan& plan,
                             void* workspace, bool bf16, hipStream_t stream) {
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const int64_t strip_cols = plan.lds ? int64_t{kLStrip} : int64_t{kWaveCols} * plan.waves;
  const int strips = static_cast<int>((N / 8 + strip_cols - 1) / strip_cols);
  XcdMap map;
  map.strips_per_xcd = (strips + kXcds - 1) / kXcds;
  const dim3 grid(static_cast<uint32_t>(kXcds * map.strips_per_xcd * plan.splits));
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  float* part = static_cast<float*>(workspace);
  if (plan.group != 32 && plan.group != 64 && plan.group != 128) return hipErrorInvalidValue;
  if (K % plan.group || M < 1 || M > kGemvMaxM) return hipErrorInvalidValue;
  if (plan.lds && (K / plan.group / plan.splits > kLMaxRows / plan.group || (N / 8) % 4 != 0))
    return hipErrorInvalidValue;
  if (!plan.lds && M > 16) {
    // The register-staged kernel takes 16 tokens at a time: run it on
    // consecutive 16-token slices (same stream, so they share the workspace).
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
      const int64_t ms = M - m0 < 16 ? M - m0 : 16;
      GemvPlan sub = plan_w4a16_gemv(ms, N, K, plan.group);
      sub.per_channel = plan.per_channel;
      const hipError_t e = launch_w4a16_gemv(x + m0 * K, qweight, scales, qzeros, y + m0 * N, ms, N, K, sub,
                                             workspace, bf16, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  hipError_t err;
  switch (plan.group * 2 + (bf16 ? 1 : 0)) {
    case 64:
      err = launch_gemv_main<32, false>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
    case 65:
      err = launch_gemv_main<32, true>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
    case 128:
      err = launch_gemv_main<64, false>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
    case 129:
      err = launch_gemv_main<64, true>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
    case 257:
      err = launch_gemv_main<128, true>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
    default:
      err = launch_gemv_main<128, false>(x, qw, scales, qz, y, part, m, n, k, plan, strips, map, grid, stream);
      break;
  }
  if (err != hipSuccess || plan.splits == 1) return err;
  // 4-output units per XCD: its strips' columns for every token row.
  const int cols8 = static_cast<int>(strip_cols) * 8;  // output columns per strip
  const int64_t units_per_xcd = static_cast<int64_t>(map.strips_per_xcd) * cols8 / 4 * M;
  const int blocks_per_xcd = static_cast<int>((units_per_xcd + 255) / 256);
  const dim3 rgrid(static_cast<uint32_t>(kXcds * blocks_per_xcd));
  const int sps = map.strips_per_xcd;
  return launch_gemv_reduce(part, y, m, n, cols8, sps, blocks_per_xcd, plan.splits, bf16, rgrid, stream);
}

}  // namespace mq
