// W4A16 decode GEMV on a column-blocked weight layout (gfx950).
//
// Source: LMDeploy 4-bit deployment guide, deployment steps (the AWQ model is
// converted once into the inference engine's own format before serving) and
// section 2.2 (scale and weight consumed in one kernel); LMDeploy toolkit
// overview, section 2.5 (4-bit weights in groups; the weight stream is what
// decode pays for). Same result as the GEMV on the [K, N/8] layout:
// y[m,n] = sum_k x[m,k] * (q[k,n] - z[k/G,n]) * s[k/G,n], G in {32, 64, 128}.
//
// Why a second layout: in [K, N/8] a column strip is a few hundred bytes of
// every 4*N/8-byte row, so reading it at full HBM speed needs wide strips,
// and wide strips leave too few workgroups for the GPU unless K is split
// across workgroups (fp32 partial sums and a second kernel). In the blocked
// layout a wavefront's share of the weights is one contiguous run of bytes,
// so a workgroup can own a narrow strip over all of K and no split is needed
// for wide layers.
//
// Blocked layout (the bytes of qweight reordered, nothing inside a byte
// changes; byte g of word (k, c) holds the weights of columns 8c+2g (low
// nibble) and 8c+2g+1 (high nibble) of row k):
//   strip s = packed columns 4s .. 4s+3 (32 outputs), S = N/32 strips; the
//   rows come in 64-row pairs P; for lane L = 16h + j (h = 0..3, j = 0..15,
//   c = j % 4, g = j / 4) the slot (P, s) holds 16 bytes, byte 8b + e
//   (b = 0, 1, e = 0..7) being byte g of qweight[64P + 32b + 8h + e, 4s + c]:
//     blocked_bytes[((P * S + s) * 64 + L) * 16 + 8b + e]
//   A wavefront's 1 KB of a pair is contiguous, and the slots of all strips
//   for one pair are adjacent, so workgroups working on the same rows read
//   neighbouring memory (as a sweep over the rows of [K, N/8] does).
//
// Kernel: a workgroup owns one strip (and, for narrow layers, one of
// `splits` K ranges); its wavefronts take that range's 128-row chunks in
// turn (wavefront w: chunks w, w + W, ...), each chunk a contiguous run of
// bytes streamed into registers (two chunks in flight per wavefront). Lane
// (j, h) of an MFMA B fragment (v_mfma_f32_16x16x32_f16, column j,
// k = 8h..8h+7 of a 32-row block) gets from its 8 bytes of the
// block both field 2g (tile 0) and field 2g+1 (tile 1) of packed column c:
// one byte permute per row pair spreads two bytes into the two fp16 halves,
// and one v_and_or_b32 per field makes 1024 + q (low nibble) or 1024 + 16 q
// (high nibble). Tokens ride on the 16-row side (rows >= M are zero and
// never stored). Per group the kernel adds s * (acc - (1024+z) * X) with X
// the per-token sum of x over the group (one more MFMA against a fragment of
// ones per block). The wavefronts' sums are added in LDS in wavefront
// order, so results are deterministic. 32-output strips give 768
// workgroups for a 24576-wide layer: every CU streams the same share.
// With 17-64 tokens (two to four tiles) a second kernel
// (w4a16_gemv_blocked_prescaled.hip) forms the weights themselves,
// fp16((q - z) * s) rounded once, and accumulates the MFMAs straight into
// the running sums: one pass over the weights for all tokens, with several
// strips per workgroup sharing the x fragments.
//
// This header holds the one-tile kernel and what the two translation units
// share: w4a16_gemv_blocked.hip (layout conversion, plan, up to 16 tokens)
// and w4a16_gemv_blocked_prescaled.hip (17-64 tokens), built with different
// register forms for the MFMA results.
#pragma once

#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"
#include "w4a16_split.h"

namespace mq {
namespace {


constexpr int kBStrip = 4;         // packed columns per strip (32 outputs)
constexpr int kBOut = kBStrip * 8;  // outputs per strip
constexpr int kBChunkRows = 128;    // rows per chunk (two 64-row pairs, four 32-row blocks)

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// x staged in LDS up front (one-tile, one-strip forms): the workgroup's
// token rows over its K range, row pitch = 2 * range + 16 bytes (the 16
// spreads the rows over the banks), plus its strips' scales and zero
// points. Used for one token where a unit has a single strip (groups of 32,
// or strip counts 3 does not divide): there the per-chunk x DMA was slower
// (12.5 against 11.4 us at N = 24576), while with 2-4 tokens it was faster
// (12.5 against 12.8 us). The one-workgroup-per-strip form of narrow layers
// stages up to 8 tokens this way.
constexpr int kXLdsPad = 16;
constexpr int64_t kXLdsMaxTokens = 1;
constexpr int64_t kWideMaxTokens = 8;  // one-workgroup-per-strip form (see the plan)
constexpr int64_t kLdsPerWorkgroup = 160 * 1024;

// One chunk (128 rows) of a lane's operands for kSP adjacent strips: 32
// weight bytes per strip (two 16-byte pair slots) and per strip the two
// scales and the zero-point byte of each group (x comes from LDS).
template <int kT, int kGPC, int kSP>
struct BChunk {
  u32x4 w[kSP][2];
  uint32_t sv[kSP][kGPC];  // fp16 pair: s of field 2g, s of field 2g+1
  uint32_t zw[kSP][kGPC];  // zero-point word of the packed column (byte g used)
};

struct BLane {
  const u32x4* qb;        // the lane's 16-byte slot of the strip's first pair
  size_t pair_stride;     // slots from one 64-row pair to the next (S * 64)
  // Without kXL, x moves into the wavefront's LDS slot by DMA. xr covers
  // the M token rows (rows past M read as zero); load q of a chunk fills
  // slot rows 4q .. 4q+3 and reads from byte xdma[q % 4] + (q / 4) * xtile
  // + 256 * chunk.
  __amdgpu_buffer_rsrc_t xr;
  uint32_t xdma[4];
  uint32_t xtile;         // 16 token rows of x in bytes
  const uint16_t* sc;     // scales + 8 * packed column + 2g
  const uint32_t* qz;     // qzeros + packed column
  int N, NP;  // row strides of scales and qzeros between groups (0: per-channel)
};

// Part kPart of a chunk's loads. Part 0: without kXL, the chunk's x rows by
// DMA; part 1: pair 0 of every strip's slot; part 2: pair 1 and the group
// parameters. The steady loop issues part 0 of the next chunk in a buffer
// once the compute has read its x fragments, part 1 once it has used pair 0
// and part 2 when it is done, so fewer requests wait behind the math. (The
// parameters go last: copying them out of the registers the next chunk's
// loads write would make the loop wait for those loads.)
template <int kPart, int kT, int kGS, int kSP, bool kXL, int kXQ>
__device__ __forceinline__ void load_part(BChunk<kT, kBChunkRows / kGS, kSP>& ch, const BLane& L, int chunk,
                                          lds_u8* xslot) {
  constexpr int kGPC = kBChunkRows / kGS;
  // The weights are read once per call: non-temporal loads (about 1% faster
  // than ordinary ones, measured) keep them from displacing cached data.
  // The unit's strips are adjacent in a pair, so each pair's slots go out as
  // one contiguous run of requests.
  if constexpr (kPart > 0) {
    const u32x4* wp = L.qb + static_cast<size_t>(2 * chunk + kPart - 1) * L.pair_stride;
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp) ch.w[sp][kPart - 1] = __builtin_nontemporal_load(wp + 64 * sp);
  }
  // With x staged up front (kXL) the fragments are read at use from there;
  // otherwise the chunk's 16 token rows per tile x 128 values move into the
  // wavefront's slot by DMA, 1 KB per load (full cache lines, where register
  // loads of the fragments would each take 16 half lines): the slot's
  // previous contents were read by the compute before this call, and
  // lgkmcnt(0) makes sure those reads have returned. The last tile takes
  // only its first kXQ loads (tokens 0 .. 4 kXQ - 1 of it; kXQ = 0: one
  // load for a single token); the kernel zeroes the slot rows past them
  // once at its start.
  if constexpr (kPart == 0 && !kXL) {
    wait_counts<63, 0>();
#pragma unroll
    for (int q = 0; q < 4 * (kT - 1) + (kXQ == 0 ? 1 : kXQ); ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(L.xr, (lds_void*)(xslot + 1024 * q), 16,
                                               L.xdma[q % 4] + (q / 4) * L.xtile + 256u * chunk, 0, 0, 0);
  }
  if constexpr (kPart == 2 && !kXL) {  // with kXL the scales and zero points are staged in LDS too
#pragma unroll
    for (int g = 0; g < kGPC; ++g) {
      const size_t grp = static_cast<size_t>(chunk) * kGPC + g;
#pragma unroll
      for (int sp = 0; sp < kSP; ++sp) {
        ch.sv[sp][g] = *reinterpret_cast<const uint32_t*>(L.sc + grp * L.N + kBOut * sp);
        ch.zw[sp][g] = L.qz[grp * L.NP + kBStrip * sp];
      }
    }
  }
}

template <int kT, int kGS, int kSP, bool kXL, int kXQ>
__device__ __forceinline__ void load_chunk(BChunk<kT, kBChunkRows / kGS, kSP>& ch, const BLane& L, int chunk,
                                           lds_u8* xslot = nullptr) {
  load_part<1, kT, kGS, kSP, kXL, kXQ>(ch, L, chunk, xslot);
  load_part<0, kT, kGS, kSP, kXL, kXQ>(ch, L, chunk, xslot);
  load_part<2, kT, kGS, kSP, kXL, kXQ>(ch, L, chunk, xslot);
}

// B fragments of one 32-row block from the lane's two words of it (rows
// 8h+0..3 and 8h+4..7, byte g of each): tile 0 gets 1024 + q of field 2g,
// tile 1 gets 1024 + 16 q of field 2g+1. The masks and the 1024.0 pattern
// come in registers (NibConst), so the compiler forms each (v & mask) |
// magic as one v_and_or_b32 itself. It must be the compiler's instruction,
// not inline asm: the fragments feed MFMA operands directly, and only for
// its own instructions does the compiler insert the wait states a VALU
// write needs before an MFMA reads the register (with an asm v_and_or_b32
// the MFMA was measured to read the register's old value).
// kBF: bf16 fragments of 128 + q for both fields (the high nibble shifted
// down first).
template <bool kBF>
__device__ __forceinline__ void unpack_block(uint32_t w0, uint32_t w1, const NibConst& c, f16x8 (&bf)[2]) {
  const uint32_t ws[2] = {w0, w1};
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // bytes 2t, 2t+1 (rows 4q+2t, 4q+2t+1) into bits 0-7 and 16-23
      const uint32_t v = byte_perm(ws[q], ws[q], t ? 0x0C030C02u : 0x0C010C00u);
      const f16x2 lo = as_f16x2((v & c.lo) | (kBF ? c.bmagic : c.magic));
      const f16x2 hi = as_f16x2(kBF ? ((v >> 4) & c.lo) | c.bmagic : (v & c.hi) | c.magic);
      bf[0][4 * q + 2 * t] = lo[0];
      bf[0][4 * q + 2 * t + 1] = lo[1];
      bf[1][4 * q + 2 * t] = hi[0];
      bf[1][4 * q + 2 * t + 1] = hi[1];
    }
}

// The x fragments of a chunk (all four 32-row blocks): from the staged x
// (kXL; xl is the lane's 16 bytes of block 0, its token row, rows 8h..8h+7,
// or nullptr for lanes past the last token) or from the chunk's slot (token
// row 16t + j, rows 8h.. of block b at xs + xo[b]).
template <int kT, bool kXL>
__device__ __forceinline__ void read_x(f16x8 (&xa)[kT][4], const lds_u8* xl, const lds_u8* xs, const int (&xo)[4]) {
#pragma unroll
  for (int t = 0; t < kT; ++t)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if constexpr (kXL) {
        xa[t][b] = xl ? *reinterpret_cast<const lds_f16x8*>(xl + 64 * b) : f16x8{};
      } else {
        xa[t][b] = *(const lds_f16x8*)(xs + 4096 * t + xo[b]);
      }
    }
}

// Blocks kB0 .. kB1 - 1 of a chunk: MFMAs into the group's sums acc (and
// accx, the sums of x against ones), and at each group's last block
// tot += s * (acc - (1024 + z) * X). acc and accx are carried between the
// two halves of a chunk when a group spans both (groups of 128).
// kLaneRows: tokens 4h .. 4h + kLaneRows - 1 of a lane's four are in use
// (1 for a single token: the per-group update of the other three is
// skipped). scl / zl (kXL): the lane's scale pair and zero-point word of the
// chunk's first group for strip 0 in the staged tables (groups kSP * 64 /
// kSP * 16 bytes apart, strips 64 / 16 bytes apart).
template <int kB0, int kB1, int kT, int kGS, int kSP, bool kXL, bool kBF, int kLaneRows>
__device__ __forceinline__ void compute_blocks(const BChunk<kT, kBChunkRows / kGS, kSP>& ch, const NibConst& nc,
                                               const f16x8 ones, int g_lane, f32x4 (&tot)[kT][kSP][2],
                                               f32x4 (&acc)[kT][kSP][2], f32x4 (&accx)[kT],
                                               const f16x8 (&xa)[kT][4], const lds_u8* scl, const lds_u8* zl) {
  constexpr int kBPG = kGS / 32;  // 32-row blocks per group
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = kB0; b < kB1; ++b) {  // block within the chunk: pair b / 2, half b % 2
    const int g = b / kBPG, bb = b % kBPG;
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp) {
      f16x8 bf[2];
      unpack_block<kBF>(ch.w[sp][b >> 1][2 * (b & 1)], ch.w[sp][b >> 1][2 * (b & 1) + 1], nc, bf);
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[t][sp][f] = mfma_16x16x32<kBF>(xa[t][b], bf[f], bb == 0 ? zero4 : acc[t][sp][f]);
    }
#pragma unroll
    for (int t = 0; t < kT; ++t) accx[t] = mfma_16x16x32<kBF>(xa[t][b], ones, bb == 0 ? zero4 : accx[t]);
    if (bb != kBPG - 1) continue;
    // tot += s * (acc - (1024 + z) * X); field 2g+1 carries 16 (q - z), so
    // its scale is s / 16 (exact). bf16: both fields carry 128 + q.
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp) {
      uint32_t sv, zw;
      if constexpr (kXL) {
        sv = *(const lds_u32*)(scl + (g * kSP + sp) * 64);
        zw = *(const lds_u32*)(zl + (g * kSP + sp) * 16);
      } else {
        sv = ch.sv[sp][g];
        zw = ch.zw[sp][g];
      }
      const f16x2 s2 = as_f16x2(sv);
      const uint32_t zb = (zw >> (8 * g_lane)) & 0xFFu;
      const float sc[2] = {static_cast<float>(s2[0]), static_cast<float>(s2[1]) * (kBF ? 1.0f : 0.0625f)};
      const float bias[2] = {(kBF ? 128.0f : 1024.0f) + static_cast<float>(zb & 15u),
                             kBF ? 128.0f + static_cast<float>(zb >> 4) : 1024.0f + static_cast<float>(zb & 0xF0u)};
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int i = 0; i < kLaneRows; ++i)
            tot[t][sp][f][i] = fmaf(sc[f], fmaf(-bias[f], accx[t][i], acc[t][sp][f][i]), tot[t][sp][f][i]);
    }
  }
}

// The end of a call: add the sums of wavefronts 0 .. kR-1 of a unit in
// wavefront order and store them (kW wavefronts in the workgroup take part;
// kR = kW unless the caller has folded the others in first). Lane (j, h)
// holds token 16t + 4h + i of output 32sp + 8c + 2g + f of the unit in
// tot[t][sp][f][i]. Each of those wavefronts stores its sums as one 16-byte
// vector (tokens 4h..4h+3) per lane and (t, sp, f) into its own region
// (region_bytes apart from base, at least kT * kSP * 2 KB), consecutive
// lanes at consecutive addresses (no bank conflicts), all at once; after one
// barrier a thread adds the kR vectors of one (t, sp, lane) for both f and
// writes its four tokens' two adjacent outputs as pairs (fp16 / bf16 pairs,
// or fp32 partial sums of split `split` when K is split). The caller makes
// sure the regions are free.
template <int kT, int kSP, int kW, bool kBF, int kR = kW>
__device__ __forceinline__ void store_unit_sums(const f32x4 (&tot)[kT][kSP][2], lds_u8* base, int region_bytes,
                                                int wave, int lane, int M, int N, int strip, int split, int splits,
                                                uint16_t* __restrict__ y, float* __restrict__ partial) {
  if (wave < kR) {
    lds_u8* const red = base + wave * region_bytes;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int sp = 0; sp < kSP; ++sp)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          *(lds_f32x4*)(red + (((t * kSP + sp) * 2 + f) * 64 + lane) * 16) = tot[t][sp][f];
  }
  __syncthreads();
  const int rows = min(M, 16 * kT);
  for (int e = threadIdx.x; e < kT * kSP * 64; e += kW * 64) {
    const int ln = e & 63, tsp = e >> 6;  // tsp = t * kSP + sp
    const int m0 = 16 * (tsp / kSP) + 4 * (ln >> 4);
    if (m0 >= rows) continue;
    f32x4 v[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int off = ((tsp * 2 + f) * 64 + ln) * 16;
      v[f] = *(const lds_f32x4*)(base + off);
#pragma unroll
      for (int w = 1; w < kR; ++w) v[f] += *(const lds_f32x4*)(base + w * region_bytes + off);
    }
    const int jj = ln & 15;
    const size_t o = static_cast<size_t>(strip) * kBOut + kBOut * (tsp % kSP) + 8 * (jj & 3) + 2 * (jj >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + i;
      if (m >= rows) break;
      if (splits == 1) {
        *reinterpret_cast<uint32_t*>(y + static_cast<size_t>(m) * N + o) =
            half_bits<kBF>(v[0][i]) | (static_cast<uint32_t>(half_bits<kBF>(v[1][i])) << 16);
      } else {
        *reinterpret_cast<f32x2*>(partial + (static_cast<size_t>(split) * M + m) * N + o) = f32x2{v[0][i], v[1][i]};
      }
    }
  }
}

// kT 16-token tiles, groups of kGS rows, kW wavefronts per workgroup, kSP
// adjacent strips per workgroup (they share every x fragment a wavefront
// loads). `units` counts kSP-strip units.
// Three wavefronts per SIMD for the one-strip, one-tile forms with groups of
// 64 or 128: a 24576-wide layer has three such workgroups per CU, and all of
// them must be resident at once for every CU to stream an equal share.
// kXL (one-tile, one-strip forms): right behind its first weight requests
// the workgroup moves its token rows of x over its K range (rows of
// 2 * range + 16 bytes), then its strip's scales and zero-point words, into
// LDS (dynamic shared memory) by DMA, and reads the MFMA A
// fragments and the group parameters from there, so the weight stream has
// the vector-memory queue to itself (per-chunk x loads cost about 2 us and
// the scale and zero-point loads about 0.7 us of a 13 us call at N = 24576).
// Two to four tiles (17-64 tokens) take the pre-scaled kernel of
// w4a16_gemv_blocked_prescaled.hip instead.
template <int kT, int kGS, int kW, int kSP, bool kXL, bool kBF, int kXQ>
__global__ __launch_bounds__(kW * 64)
__attribute__((amdgpu_waves_per_eu(kW >= 8 ? kW / 4 : (kT == 1 && kSP == 1 && kGS >= 64 ? 3 : 1)))) void w4a16_gemv_blocked_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ qb, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ partial, int M, int N, int K,
    int units, int splits, XcdMap map, int gstep) {
  constexpr int kGPC = kBChunkRows / kGS;
  constexpr int kUOut = kSP * kBOut;  // outputs per unit
  static_assert(kT == 1, "two to four tiles take the pre-scaled kernel");
  // kXL: the wavefronts' sums meet here (the other forms reuse their x slots)
  __shared__ float s_red[kXL ? kW * 16 * kT * kUOut : 1];
  static_assert(kXL || kSP <= 4, "a wavefront's sums must fit its two x slots");
  extern __shared__ __attribute__((aligned(16))) uint8_t x_dyn[];  // kXL: M rows of staged x

  int unit, split;
  if (!decode_work(blockIdx.x, map.strips_per_xcd, units, splits, unit, split)) return;
  const int strip = unit * kSP;  // first strip of the unit
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int c = j & 3, g = j >> 2;
  const int NP = N >> 3;
  const int chunks = K / kBChunkRows;
  const int cps = chunks / splits;  // chunks per split (plan: divides)
  const int cpw = cps / kW;         // chunks per wavefront (plan: divides, >= 1)
  // Wavefront w takes chunks w, w + kW, w + 2 kW, ... of the split, so the
  // workgroup's requests in flight fall on neighbouring rows of the weights
  // (one narrow band of memory for all workgroups) rather than on kW bands a
  // quarter of the range apart: 1 / 4 / 16 tokens at N = 24576 went from
  // 11.06 / 11.42 / 12.12 to 10.61 / 10.96 / 11.83 us.
  const int c0 = split * cps + wave;
  auto chunk_of = [&](int i) { return c0 + i * kW; };
  const int col = strip * kBStrip + c;  // packed column of the lane

  BLane L;
  L.qb = qb + static_cast<size_t>(strip) * 64 + lane;
  L.pair_stride = static_cast<size_t>(NP / kBStrip) * 64;
  L.sc = scales + static_cast<size_t>(col) * 8 + 2 * g;
  L.qz = qz + col;
  // Without kXL each wavefront has two LDS slots (one per chunk buffer)
  // of 16 kT rows x 256 bytes. Load q fills rows 4q .. 4q+3: lane l writes
  // physical 16-byte chunk l % 16 of row 4q + l / 16 and fetches the logical
  // chunk (l % 16) ^ (row % 16) there, so the fragment reads (16 rows of one
  // logical chunk per 16 lanes) fall on 16 different bank groups.
  lds_u8* xslot[2] = {nullptr, nullptr};
  const lds_u8* xs[2] = {nullptr, nullptr};
  int xo[4] = {0, 0, 0, 0};
  if constexpr (!kXL) {
    L.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, M * K * 2, 0x00020000);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 4 * qq + lane / 16;  // row within a 16-row tile (= row mod 16)
      L.xdma[qq] = static_cast<uint32_t>(r * K + 8 * ((lane % 16) ^ r)) * 2u;
    }
    L.xtile = static_cast<uint32_t>(16 * K) * 2u;
    lds_u8* const base = (lds_u8*)(x_dyn) + wave * 2 * (kT * 4096);
    xslot[0] = base;
    xslot[1] = base + kT * 4096;
    xs[0] = xslot[0] + 256 * j;
    xs[1] = xslot[1] + 256 * j;
    if constexpr (kXQ < 4) {
      // token rows 4 max(kXQ, 1) .. 15 of the last tile are never loaded:
      // zero them in both slots (they only feed output rows not stored)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int r = 4 * (kXQ == 0 ? 1 : kXQ); r < 16; r += 4)
          *(lds_u32x4*)(xslot[sl] + 4096 * (kT - 1) + 256 * (r + lane / 16) + 16 * (lane % 16)) = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) xo[b] = 16 * ((4 * b + h) ^ j);
  }
  // gstep = 1: group g's scales and zero points are row g; gstep = 0
  // (per-channel parameters): every group reads the one row.
  L.N = gstep * N;
  L.NP = gstep * NP;
  const int sN = L.N, sNP = L.NP;

  const NibConst nc = nib_const();
  const f16x8 ones = ones_fragment<kBF>();

  f32x4 tot[kT][kSP][2];
#pragma unroll
  for (int t = 0; t < kT; ++t)
#pragma unroll
    for (int sp = 0; sp < kSP; ++sp)
#pragma unroll
      for (int f = 0; f < 2; ++f) tot[t][sp][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two chunks in flight per wavefront: a buffer's next chunk is requested
  // part by part as the buffer is consumed (x once its fragments are in
  // registers, pair 0 once blocks 0-1 are done, the rest at the end: 1 / 8
  // / 16 tokens at N = 24576 10.64 / 11.12 / 11.69 -> 10.51 / 10.85 / 11.42
  // us against the whole chunk after the compute); sched_barrier keeps each
  // request ahead of the math it is meant to overlap. The steady loop only
  // runs while both of its requests are in range, so they are
  // unconditional (a conditional request inside the loop makes the compiler
  // copy the buffer at the back edge, which waits for every load in
  // flight); the last two or three chunks are finished after the loop with
  // at most one more request. No chunk is requested twice (except when a
  // wavefront has a single chunk). More bytes in flight per wavefront
  // (a third buffer, or eight wavefronts per workgroup) measured slower.
  {
    BChunk<kT, kGPC, kSP> ca, cb;
    load_chunk<kT, kGS, kSP, kXL, kXQ>(ca, L, chunk_of(0), xslot[0]);
    __builtin_amdgcn_sched_barrier(0);
    load_chunk<kT, kGS, kSP, kXL, kXQ>(cb, L, chunk_of(min(1, cpw - 1)), xslot[1]);
    __builtin_amdgcn_sched_barrier(0);
    // Staged x: the lane's row (token j, rows 8h.. of each block) at the
    // split's first chunk; lanes past the last token read nothing.
    const lds_u8* xrow = nullptr;
    const lds_u8* sc_lane = nullptr;
    const lds_u8* z_lane = nullptr;
    const int kbase = split * cps;  // first chunk of the split
    if constexpr (kXL) {
      // The token rows of x (1 KB per load: row m, bytes 1024 v ..), the
      // unit's scale pairs ([group][32] fp16, 16 groups per load) and
      // zero-point words ([group][4], 16 groups per load) over the K range
      // move into LDS by DMA right behind the first weight requests. Nothing
      // waits for them before the compute, which needs those weights anyway
      // (register loads of the same values made the copy wait for the
      // weights first and then start its own requests).
      static_assert(!kXL || kSP == 1, "x is staged up front only for one-strip units");
      lds_u8* const xs = (lds_u8*)(x_dyn);
      const int kr = cps * kBChunkRows;  // K range of the split (host: a multiple of 512)
      const int pitch = 2 * kr + kXLdsPad;
      const int mt = min(M, 16);
      const int ngr = kr / kGS;
      const int ngr16 = (ngr + 15) / 16 * 16;  // the tables are allocated in steps of 16 groups
      lds_u8* const sct = xs + mt * pitch;
      lds_u8* const zt = sct + ngr16 * 64;
      const int grp0 = kbase * kGPC;
      const int grows = gstep ? K / kGS : 1;
      const __amdgpu_buffer_rsrc_t rsx =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, M * K * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t rss =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, grows * N * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t rsz =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qz), 0, grows * NP * 4, 0x00020000);
      const int xper = kr / 512;  // 1 KB loads per row
      const int nx = mt * xper, ns = ngr16 / 16;
      for (int q = wave; q < nx + 2 * ns; q += kW) {
        if (q < nx) {
          const int m = q / xper, v = q % xper;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsx, (lds_void*)(xs + m * pitch + 1024 * v), 16,
              static_cast<uint32_t>(m * K + kbase * kBChunkRows + 512 * v + 8 * lane) * 2u, 0, 0, 0);
        } else if (q < nx + ns) {
          // groups past the range (padding, never read) may wrap to any
          // offset: the descriptor's size turns reads past the table into 0
          const int gl = 16 * (q - nx) + lane / 4;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rss, (lds_void*)(sct + 1024 * (q - nx)), 16,
              (static_cast<uint32_t>(grp0 + gl) * static_cast<uint32_t>(sN) + strip * kBOut + 8 * (lane % 4)) * 2u,
              0, 0, 0);
        } else {
          const int gl = 16 * (q - nx - ns) + lane / 4;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsz, (lds_void*)(zt + 256 * (q - nx - ns)), 4,
              (static_cast<uint32_t>(grp0 + gl) * static_cast<uint32_t>(sNP) + strip * kBStrip + lane % 4) * 4u,
              0, 0, 0);
        }
      }
      wait_counts<0, 15>();
      __syncthreads();
      if (j < M) xrow = xs + j * pitch + 16 * h;
      sc_lane = sct + 16 * c + 4 * g;
      z_lane = zt + 4 * c;
    }
    auto xl = [&](int chunk) -> const lds_u8* {
      return (kXL && xrow) ? xrow + (chunk - kbase) * (2 * kBChunkRows) : nullptr;
    };
    auto sl = [&](int chunk) -> const lds_u8* { return sc_lane + (chunk - kbase) * kGPC * kSP * 64; };
    auto zl = [&](int chunk) -> const lds_u8* { return z_lane + (chunk - kbase) * kGPC * kSP * 16; };
    // Without kXL, before a buffer's compute its DMA must have landed.
    // Loads complete in issue order, and every load of the other buffer's
    // next chunk was issued after this one's (sched_barrier between the
    // requests): waiting down to that chunk's count (kChunkLoads) leaves
    // only those in flight; where no later chunk was requested, wait for all.
    constexpr int kChunkLoads = 2 * kSP + 4 * (kT - 1) + (kXQ == 0 ? 1 : kXQ) + 2 * kSP * kGPC;
    static_assert(kXL || kChunkLoads < 64, "vmcnt range");
    constexpr int kLR = kXQ == 0 ? 1 : 4;
    // a whole chunk (the last two or three of a wavefront)
    auto compute = [&](const BChunk<kT, kGPC, kSP>& ch, int chunk, int buf) {
      f32x4 acc[kT][kSP][2], accx[kT];
      f16x8 xa[kT][4];
      read_x<kT, kXL>(xa, xl(chunk), xs[buf], xo);
      compute_blocks<0, 4, kT, kGS, kSP, kXL, kBF, kLR>(ch, nc, ones, g, tot, acc, accx, xa, sl(chunk), zl(chunk));
    };
    // a chunk of the steady loop: the buffer's next chunk is requested in
    // three parts, x once this chunk's x fragments are in registers, pair 0
    // once the compute has used pair 0, pair 1 and the parameters when it is
    // done
    auto compute_refill = [&](BChunk<kT, kGPC, kSP>& ch, int chunk, int buf, int next) {
      f32x4 acc[kT][kSP][2], accx[kT];
      f16x8 xa[kT][4];
      read_x<kT, kXL>(xa, xl(chunk), xs[buf], xo);
      __builtin_amdgcn_sched_barrier(0);
      load_part<0, kT, kGS, kSP, kXL, kXQ>(ch, L, next, xslot[buf]);
      __builtin_amdgcn_sched_barrier(0);
      compute_blocks<0, 2, kT, kGS, kSP, kXL, kBF, kLR>(ch, nc, ones, g, tot, acc, accx, xa, sl(chunk), zl(chunk));
      __builtin_amdgcn_sched_barrier(0);
      load_part<1, kT, kGS, kSP, kXL, kXQ>(ch, L, next, xslot[buf]);
      __builtin_amdgcn_sched_barrier(0);
      compute_blocks<2, 4, kT, kGS, kSP, kXL, kBF, kLR>(ch, nc, ones, g, tot, acc, accx, xa, sl(chunk), zl(chunk));
      __builtin_amdgcn_sched_barrier(0);
      load_part<2, kT, kGS, kSP, kXL, kXQ>(ch, L, next, xslot[buf]);
      __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + 3 < cpw; i += 2) {
      if constexpr (!kXL) wait_counts<kChunkLoads, 15>();
      compute_refill(ca, chunk_of(i), 0, chunk_of(i + 2));
      if constexpr (!kXL) wait_counts<kChunkLoads, 15>();
      compute_refill(cb, chunk_of(i + 1), 1, chunk_of(i + 3));
    }
    // chunks i and (if in range) i + 1 are in flight; at most i + 2 is left
    if constexpr (!kXL) wait_counts<kChunkLoads, 15>();
    compute(ca, chunk_of(i), 0);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < cpw) load_chunk<kT, kGS, kSP, kXL, kXQ>(ca, L, chunk_of(i + 2), xslot[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!kXL) wait_counts<0, 15>();
    if (i + 1 < cpw) compute(cb, chunk_of(i + 1), 1);
    if (i + 2 < cpw) compute(ca, chunk_of(i + 2), 0);
  }

  // Add the wavefronts' sums and store (see store_unit_sums). Forms
  // without x staged up front store into the wavefront's own x slots: every
  // DMA into them has landed (the last computes waited for all vector-memory
  // loads) and lgkmcnt(0) makes sure the slots' last reads have returned.
  if constexpr (kXL) {
    store_unit_sums<kT, kSP, kW, kBF>(tot, (lds_u8*)(s_red), 16 * kT * kUOut * 4, wave, lane, M, N, strip, split,
                                      splits, y, partial);
  } else {
    wait_counts<63, 0>();
    store_unit_sums<kT, kSP, kW, kBF>(tot, (lds_u8*)(x_dyn), 2 * (kT * 4096), wave, lane, M, N, strip, split, splits,
                                      y, partial);
  }
}

template <int kT, int kGS, int kSP, bool kXL, bool kBF, int kXQ = 4>
hipError_t launch_blocked_xl(const uint16_t* x, const u32x4* qb, const uint16_t* scales, const uint32_t* qz,
                             uint16_t* y, float* part, int m, int n, int k, const GemvPlan& plan, int units,
                             XcdMap map, dim3 grid, size_t lds, hipStream_t stream) {
  switch (plan.waves) {
    case 1:
      return launch_kernel(w4a16_gemv_blocked_kernel<kT, kGS, 1, kSP, kXL, kBF, 4>, grid, dim3(64), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, plan.per_channel ? 0 : 1);
    case 2:
      return launch_kernel(w4a16_gemv_blocked_kernel<kT, kGS, 2, kSP, kXL, kBF, 4>, grid, dim3(128), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, plan.per_channel ? 0 : 1);
    case 8:
    case 16:
      // only the one-strip forms with x staged in LDS (up to 4 tokens,
      // narrow layers) are built for 8 and 16 wavefronts
      if constexpr (kT == 1 && kSP == 1 && kXL) {
        if (plan.waves == 8)
          return launch_kernel(w4a16_gemv_blocked_kernel<kT, kGS, 8, kSP, kXL, kBF, 4>, grid, dim3(512), lds, stream, x,
                               qb, scales, qz, y, part, m, n, k, units, plan.splits, map, plan.per_channel ? 0 : 1);
        return launch_kernel(w4a16_gemv_blocked_kernel<kT, kGS, 16, kSP, kXL, kBF, 4>, grid, dim3(1024), lds, stream, x,
                             qb, scales, qz, y, part, m, n, k, units, plan.splits, map, plan.per_channel ? 0 : 1);
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return launch_kernel(w4a16_gemv_blocked_kernel<kT, kGS, 4, kSP, kXL, kBF, kXQ>, grid, dim3(256), lds, stream, x, qb,
                           scales, qz, y, part, m, n, k, units, plan.splits, map, plan.per_channel ? 0 : 1);
  }
}

}  // namespace

// The forms with two to four token tiles (17-64 tokens), defined in
// w4a16_gemv_blocked_prescaled.hip.
hipError_t launch_w4a16_gemv_blocked_prescaled(const uint16_t* x, const u32x4* qb, const uint16_t* scales,
                                               const uint32_t* qz, uint16_t* y, float* part, int m, int n, int k,
                                               const GemvPlan& plan, int units, int strips_per_xcd, dim3 grid,
                                               bool bf16, hipStream_t stream);

}  // namespace mq
