// W4A16 GEMM for prefill-shaped M on gfx950.
//
// Source: LMDeploy toolkit overview, section 2.5 (AWQ 4-bit weights, group
// size 128) and LMDeploy 4-bit deployment guide, sections 2.2-2.3 (scales
// and weights consumed inside the matmul kernel; a real low-bit kernel rather
// than fake quantization) and section 3.2 (group size 64 for the vision
// tower's attention). y[m,n] = sum_k x[m,k] * fp16((q - z) * s) with one
// (s, z) per group of G = 32, 64 or 128 consecutive k; the kernel is
// instantiated per group size.
//
// Design:
// - v_mfma_f32_32x32x16_f16 (on gfx950 about 1.5x the rate of the 16x16x32
//   form). A workgroup computes 128 tokens x 512 outputs with eight
//   wavefronts side by side in N, two per SIMD; a wavefront owns 128 x 64
//   (four 32-token A fragments x two B tiles, 128 fp32 accumulators per
//   lane), so every weight is dequantized exactly once per workgroup and
//   each dequantized fragment feeds four MFMAs. The unpack arithmetic is
//   what bounds this kernel (the MFMAs of a k-step take 8 x 32 cycles per
//   wavefront, its unpack about 4 vector operations per MFMA), and with two
//   wavefronts per SIMD one's unpack runs under the other's MFMAs.
// - B tiles: lane (j = lane%32, h = lane/32) of tile t takes packed column
//   j%8 of the wavefront's 8 and field f = 2(j/8) + t, rows 8h..8h+7 of a
//   16-row k-step: the two tiles hold the two nibbles of byte j/8 of the
//   lane's words. For each row pair one byte permute moves that byte of the
//   two rows into the two fp16 halves, and it serves both tiles. A field in
//   bits 0-3 of a half, OR-ed into the pattern of 1024.0, reads as
//   1024 + q; a field in bits 4-7, OR-ed into the pattern of 64.0, reads as
//   64 + q (the mantissa step at 64 is 1/16). Subtracting 1024 + z (64 + z)
//   leaves q - z exactly, and the one multiply by s rounds each weight once,
//   to fp16((q - z) * s), for every fp16 scale (subnormal products
//   included).
// - Everything moves HBM -> LDS with buffer_load ... lds through a ring of
//   kStages 32-row stages: the x rows (shared by all wavefronts) and, per
//   32-column area, its raw packed words, scales and zero points. The first
//   four wavefronts issue all the fills (32 x rows and half an area's weight
//   rows each); the other four only compute. Loads past a buffer
//   descriptor's size return zero (ragged M); columns past N read valid
//   memory and are never stored.
// - x rows are 64 bytes per stage with the 16-byte chunk index XOR-swizzled
//   by the row (conflict-free fragment reads). Raw weight rows are 128
//   bytes; k-row r is stored at LDS row r with bits 0 and 3 swapped, so the
//   two lane halves (rows 8h + e) read opposite halves of the banks.
// - The output tile is staged in LDS as fp16 and written as whole rows.
// - Workgroups are dispatched round-robin over the 8 XCDs; tiles are
//   remapped so an XCD runs consecutive token tiles of one weight tile.
#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"

namespace mq {
namespace {

constexpr int kBM = 128;        // tokens per workgroup tile
constexpr int kAreas = 2;       // DMA areas of 32 packed columns (128-byte weight rows)
constexpr int kAreaCols = 32;   // packed columns per area
constexpr int kTileCols = kAreas * kAreaCols;  // 64 packed columns (512 outputs)
constexpr int kWaves = 8;       // four per area (8 packed columns each), two per SIMD
constexpr int kWaveCols = 8;    // packed columns per wavefront
constexpr int kFillers = 4;     // wavefronts that issue the fills
constexpr int kGroupM = 8;      // token tiles per group in the tile order
constexpr int kAFrags = kBM / 32;  // 32-token A fragments per wavefront
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32;       // K rows per stage (two 16-row MFMA k-steps)
constexpr int kStages = 8;      // LDS ring depth (stages)
constexpr int kABytes = kBM * kRows * 2;         // x rows: 128 x 64 B
constexpr int kBBytes = kRows * kAreaCols * 4;   // an area's raw words: 32 x 128 B
constexpr int kSBytes = 1024;                    // an area's scales (512 B used)
constexpr int kZBytes = 256;                     // an area's zero points (128 B used)
constexpr int kAreaBytes = kBBytes + kSBytes + kZBytes;
constexpr int kSlotBytes = kABytes + kAreas * kAreaBytes;
constexpr int kLoadsW = 4;  // per filling wavefront and stage: 2 x, 2 weights
                            // (+ 1 scales or zero-point load at a group's first stage)
constexpr int kOutPitch = kTileCols * 8 * 2 + 16;  // bytes per staged output row
static_assert(kStages >= 2 && (kStages - 1) * (kLoadsW + 1) < 64, "ring depth / vmcnt range");
static_assert(kStages * kSlotBytes <= 160 * 1024, "LDS capacity");
static_assert(kBM * kOutPitch <= kStages * kSlotBytes, "output staging fits the ring");
static_assert(kFillers * 2 * 16 == kBM && kFillers == 2 * kAreas, "fill split: 32 x rows, half an area each");

constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3 (raw 32-bit data)

typedef __attribute__((address_space(3))) int8_t lds_i8;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) uint32_t lds_word;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// XOR applied to the 16-byte chunk index of x row r (64-byte rows): any 8 or
// 16 consecutive rows of a fragment read land on distinct bank groups.
__device__ __forceinline__ int chunk_swizzle(int r) { return ((r >> 2) & 3) ^ (r & 2); }

// LDS row of k-row r within a stage (an involution: bits 0 and 3 swapped).
__device__ __forceinline__ int raw_row(int r) { return (r & ~9) | ((r & 1) << 3) | ((r >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n), kBufferFlags);
}

// What a lane needs to unpack its fields: fields 2g and 2g + 1 (tiles 0
// and 1) of its packed column are the low and high nibble of byte g of a
// word. sel is the byte-permute selector that moves byte g of rows e and
// e + 1 into bytes 0 and 2; mask[t] keeps tile t's nibble in each half and
// magic[t] is the pattern of 1024.0 (low nibble) or 64.0 (high nibble).
struct LaneFields {
  uint32_t sel;
  uint32_t mask[2], magic[2];
  int g;
};

__device__ __forceinline__ LaneFields lane_fields(int g) {
  LaneFields lf;
  lf.g = g;
  const uint32_t b = static_cast<uint32_t>(g);
  lf.sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);  // 0x0C selects a zero byte
  // In registers: gfx9 VOP3 takes no literal, so each nibble-to-fp16 step
  // stays one v_and_or_b32.
  asm("v_mov_b32 %0, 0x000f000f" : "=v"(lf.mask[0]));
  asm("v_mov_b32 %0, 0x00f000f0" : "=v"(lf.mask[1]));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(lf.magic[0]));  // 1024.0: a field in bits 0-3 reads 1024 + q
  asm("v_mov_b32 %0, 0x54005400" : "=v"(lf.magic[1]));  // 64.0: a field in bits 4-7 reads 64 + q
  return lf;
}

// Per group and tile t: negz[t] = -(1024 + z) (t = 0) or -(64 + z) (t = 1)
// in both fp16 halves, and sc2[t] = s in both halves.
// bf16 activations (kBF): the weight is formed in binary32 and rounded once
// to bf16 instead; negz[t] then holds the binary32 bits of -(1024 + z) * s
// (or -(64 + z) * s) and sc2[t] those of s, both exact (an 11-bit integer
// times an 11-bit significand).
struct GroupParams {
  uint32_t negz[2];
  uint32_t sc2[2];
};

// Zero point z of field 2g + t sits in nibble t of byte g of zw: masked in
// place and OR-ed into the sign and exponent of -1024.0 (0xE400) or -64.0
// (0xD400) it reads as -(1024 + z) or -(64 + z), the same encodings as the
// weight fields. sd holds the scales of fields 2g and 2g + 1 in its halves.
template <bool kBF>
__device__ __forceinline__ void make_group_params(uint32_t zw, uint32_t sd, const LaneFields& lf, GroupParams& gp) {
  const uint32_t zb = (zw >> (8 * lf.g)) & 0xFFu;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t sh = (sd >> (16 * t)) & 0xFFFFu;  // the field's fp16 scale
    if constexpr (kBF) {
      const float sf = static_cast<float>(__builtin_bit_cast(f16, static_cast<uint16_t>(sh)));
      const uint32_t zf = (zb >> (4 * t)) & 15u;
      const float off = t ? 64.0f : 1024.0f;
      gp.negz[t] = __builtin_bit_cast(uint32_t, -(off + static_cast<float>(zf)) * sf);
      gp.sc2[t] = __builtin_bit_cast(uint32_t, sf);
    } else {
      const uint32_t e = (zb & (t ? 0xF0u : 0x0Fu)) | (t ? 0xD400u : 0xE400u);
      gp.negz[t] = e | (e << 16);
      gp.sc2[t] = sh | (sh << 16);
    }
  }
}

// Fragments fp16((q - z) * s) of the lane's two fields for one 16-row
// k-step: w[e] is the lane's word of row 8h + e. For each row pair one byte
// permute gathers byte g of both rows; per tile one v_and_or_b32 keeps the
// tile's nibble under its magic pattern, and a packed add and multiply
// subtract the zero point and apply the scale.
// kBF: the offset integer (an exact fp16) times s plus -(offset + z) * s in
// one binary32 fused multiply-add (v_fma_mix_f32 reads the fp16 half
// directly) is exactly (q - z) * s, rounded once to bf16 by the pair
// conversion.
template <bool kBF>
__device__ __forceinline__ void unpack_fields(const uint32_t (&w)[8], const GroupParams& gp, const LaneFields& lf,
                                              f16x8 (&b)[2]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t r = byte_perm(w[2 * p + 1], w[2 * p], lf.sel);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t v = (r & lf.mask[t]) | lf.magic[t];
      f16x2 d;
      if constexpr (kBF) {
        const f16x2 o = as_f16x2(v);
        const float sf = __builtin_bit_cast(float, gp.sc2[t]);
        const float cf = __builtin_bit_cast(float, gp.negz[t]);
        d = as_f16x2(bf16x2_bits(fmaf(static_cast<float>(o[0]), sf, cf), fmaf(static_cast<float>(o[1]), sf, cf)));
      } else {
        d = (as_f16x2(v) + as_f16x2(gp.negz[t])) * as_f16x2(gp.sc2[t]);
      }
      b[t][2 * p] = d[0];
      b[t][2 * p + 1] = d[1];
    }
  }
}

// kSPG = 32-row stages per group (group size 32 kSPG).
// With splits > 1 the workgroup takes K range `split` of `splits` equal
// ranges and writes fp32 partial sums to partial[split, M, N] (a second
// kernel adds them in split order); with splits == 1 it writes y.
template <int kSPG, bool kBF>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qz,
                                                         uint16_t* __restrict__ y, float* __restrict__ partial,
                                                         int M, int N, int K, int tiles_m, int tiles_n,
                                                         int per_xcd, int splits, int gstep) {
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kSlotBytes];
  lds_i8* const sm = (lds_i8*)(smem);

  // Tile of this workgroup: each XCD takes a contiguous run of tile ids,
  // and ids run over groups of kGroupM token tiles, token tiles fastest
  // within a group. An XCD's 32 concurrent workgroups then cover a block of
  // about 8 token tiles x 4 weight tiles, so its L2 fetches each x row block
  // and each weight tile once for several workgroups (with whole columns of
  // token tiles per XCD every XCD would stream all of x).
  const int w_id = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  const int tiles = tiles_m * tiles_n;
  if (w_id >= tiles * splits) return;
  const int split = w_id / tiles;
  const int t_id = w_id % tiles;
  const int group_tiles = kGroupM * tiles_n;
  const int tgroup = t_id / group_tiles;
  const int first_m = tgroup * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int in_group = t_id - tgroup * group_tiles;
  const int m0 = (first_m + in_group % gm) * kBM;
  const int c0 = (in_group / gm) * kTileCols;  // first packed column
  const int k_len = K / splits;                 // multiple of 128 (host plan)
  const int k_base = split * k_len;
  constexpr int kGS = kSPG * kRows;  // rows per group
  static_assert(4 % kSPG == 0, "a group is 1, 2 or 4 stages");
  const int NP = N >> 3;
  // gstep = 1: group g's scales and zero points are row g; gstep = 0
  // (per-channel parameters): every group reads the one row.
  const int G = gstep ? K / kGS : 1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // x: one descriptor for the tile's rows (rows past M read as zero). The
  // weight, scale and zero-point descriptors are re-based at each stage's
  // first row (group), so every offset stays far below 2^31 for any legal
  // shape; columns past N read valid memory of the next row (never stored)
  // or, past the last row, zero.
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + static_cast<size_t>(m0) * K, static_cast<int64_t>(min(kBM, M - m0)) * K * 2);

  // DMA: wavefront f < kFillers fills x rows 32f .. 32f+31 and weight rows
  // 16(f%2) .. 16(f%2)+15 of area f/2 of every stage, and at a group's first
  // stage that area's scales (f even) or zero points (f odd); the other four
  // only compute.
  const bool filler = wave < kFillers;
  const int ff = filler ? wave : 0;
  const int fa = ff >> 1;  // area
  //  x: load u fills rows 32f + 16u .. +15; lane L -> row 32f + 16u + L/4,
  //     physical chunk L%4, which holds logical chunk (L%4) ^ swizzle(row).
  uint32_t xa_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 32 * ff + 16 * u + lane / 4;
    xa_off[u] = static_cast<uint32_t>(row * K + 8 * ((lane % 4) ^ chunk_swizzle(row))) * 2u;
  }
  //  weights: load u fills LDS rows 8v .. 8v+7 of the area (v = 2(f%2) + u);
  //     lane L -> LDS row 8v + L/8 = k-row raw_row(.), 16-byte chunk L%8
  //     (words 4(L%8)..).
  uint32_t wr_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = 2 * (ff & 1) + u;
    wr_off[u] = static_cast<uint32_t>(raw_row(8 * v + lane / 8) * NP + kAreaCols * fa + 4 * (lane % 8)) * 4u;
  }
  //  scales: lane L -> the 8 scales of packed column (L % 32) of the area;
  //  zero points: lane L -> word (L % 32).
  const bool fills_scales = (ff & 1) == 0;
  const uint32_t s_off = static_cast<uint32_t>(8 * (kAreaCols * fa + lane % 32)) * 2u;
  const uint32_t z_off = static_cast<uint32_t>(kAreaCols * fa + lane % 32) * 4u;
  lds_i8* const fill_area = sm + kABytes + fa * kAreaBytes;  // + slot offset

#define MQ_ISSUE(ST, SZ)                                                                             \
  do {                                                                                               \
    const int k0_ = k_base + (ST) * kRows;                                                           \
    const int g_ = gstep * (k0_ / kGS);                                                              \
    const int so_ = ((ST) % kStages) * kSlotBytes;                                                   \
    const __amdgpu_buffer_rsrc_t rw_ =                                                               \
        rsrc(qw + static_cast<size_t>(k0_) * NP + c0, (static_cast<int64_t>(K - k0_) * NP - c0) * 4); \
    _Pragma("unroll") for (int u = 0; u < 2; ++u)                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sm + so_ + (2 * ff + u) * 1024), 16, \
                                                 xa_off[u] + k0_ * 2, 0, 0, 0);                      \
    _Pragma("unroll") for (int u = 0; u < 2; ++u)                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                    \
            rw_, (lds_void*)(fill_area + so_ + (2 * (ff & 1) + u) * 1024), 16, wr_off[u], 0, 0, 0);  \
    if (SZ) {                                                                                        \
      if (fills_scales) {                                                                            \
        const __amdgpu_buffer_rsrc_t rs_ = rsrc(scales + static_cast<size_t>(g_) * N + c0 * 8,       \
                                                (static_cast<int64_t>(G - g_) * N - c0 * 8) * 2);     \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (lds_void*)(fill_area + so_ + kBBytes), 16,    \
                                                 s_off, 0, 0, 0);                                    \
      } else {                                                                                       \
        const __amdgpu_buffer_rsrc_t rz_ = rsrc(qz + static_cast<size_t>(g_) * NP + c0,              \
                                                (static_cast<int64_t>(G - g_) * NP - c0) * 4);       \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rz_, (lds_void*)(fill_area + so_ + kBBytes + kSBytes), \
                                                 4, z_off, 0, 0, 0);                                 \
      }                                                                                              \
    }                                                                                                \
  } while (0)

  // Compute: wavefront w takes packed columns 8w .. 8w+7 of the tile
  // (columns 8(w % 4) .. of area w / 4). Lane (j = lane%32, h = lane/32) of
  // B tile t takes packed column 8w + j%8 and field 2(j/8) + t, so the two
  // tiles cover the eight fields of the wavefront's 8 columns.
  const int fi = lane & 31, fh = lane >> 5;
  const int col_in_area = kWaveCols * (wave & 3) + (fi & 7);
  const LaneFields lf = lane_fields(fi >> 3);
  // x fragments: row fi (+32a) of the tile, k-step t -> logical chunk 2t + fh.
  int xoff[kAFrags][2];
#pragma unroll
  for (int a = 0; a < kAFrags; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 32 * a + fi;
      xoff[a][t] = row * 64 + 16 * ((2 * t + fh) ^ chunk_swizzle(row));
    }
  // raw words: k-row 16t + 8fh + e of the lane's packed column.
  const int area = kABytes + (wave >> 2) * kAreaBytes;
  const int wbase = area + 4 * col_in_area;
  // the lane's scale word (fields 2g and 2g + 1 of its column)
  const int sbase = area + kBBytes + 16 * col_in_area + 4 * lf.g;

  f32x16 acc[kAFrags][2];
#pragma unroll
  for (int a = 0; a < kAFrags; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[a][t] = f32x16{};

  const int nst = k_len / kRows;

  // Operands of one 16-row k-step: the four x fragments and the two
  // dequantized weight fragments.
#define MQ_READ_A(S, T, AF)                                                                      \
  do {                                                                                           \
    const lds_i8* const sl_ = sm + ((S) % kStages) * kSlotBytes;                                 \
    _Pragma("unroll") for (int a = 0; a < kAFrags; ++a) AF[a] = *(const lds_f16x8*)(sl_ + xoff[a][T]); \
  } while (0)
#define MQ_READ_W(S, T, W)                                                                       \
  do {                                                                                           \
    const lds_i8* const sl_ = sm + ((S) % kStages) * kSlotBytes;                                 \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                \
        W[e] = *(const lds_word*)(sl_ + wbase + raw_row(16 * (T) + 8 * fh + e) * 128);            \
  } while (0)
#define MQ_READ_GP(S, GP)                                                                        \
  do {                                                                                           \
    const lds_i8* const sl_ = sm + ((S) % kStages) * kSlotBytes;                                 \
    const uint32_t sd_ = *(const lds_word*)(sl_ + sbase);                                      \
    const uint32_t zw_ = *(const lds_word*)(sl_ + area + kBBytes + kSBytes + 4 * col_in_area);   \
    make_group_params<kBF>(zw_, sd_, lf, GP);                                                    \
  } while (0)
#define MQ_MFMAS(AF, B)                                                                          \
  do {                                                                                           \
    _Pragma("unroll") for (int a = 0; a < kAFrags; ++a) _Pragma("unroll") for (int t = 0; t < 2; ++t) \
        acc[a][t] = mfma_32x32x16<kBF>(AF[a], B[t], acc[a][t]);                                  \
  } while (0)
// Keeps the unpacked fragments in the block that computes them (otherwise
// they are sunk next to their use, out of reach of the MFMAs they are meant
// to overlap).
#define MQ_PIN(B) _Pragma("unroll") for (int t_ = 0; t_ < 2; ++t_) asm volatile("" : "+v"(B[t_]))
// Schedule of a block: each of its 8 MFMAs followed by a share of the LDS
// reads (consumed only in the next block) and of the unpack arithmetic.
// Spreading the reads measured 3-5% faster than issuing them all first.
#define MQ_INTERLEAVE(NDS, NVALU)                                                                \
  do {                                                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, (NDS + 7) / 8, 0);                             \
      __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);                                     \
    }                                                                                            \
  } while (0)

  // Software pipeline, per stage s (two 16-row k-steps):
  //   barrier: stage s + 1 has landed (every filler's share) and every wave
  //            is done with stage s - 1, whose slot takes stage s + 7;
  //   block A: read the x fragments of (s, k1) and the raw words of
  //            (s + 1, k0); unpack the raw words of (s, k1), read one block
  //            earlier; MFMAs of (s, k0);
  //   block B: read the x fragments of (s + 1, k0) and the raw words of
  //            (s + 1, k1); unpack the raw words of (s + 1, k0); MFMAs of
  //            (s, k1).
  // Every LDS read lands a full block before its use, so neither the unpack
  // nor the MFMAs of a block wait on LDS, and the two wavefronts of a SIMD
  // overlap one's unpack with the other's MFMAs. A group is kSPG stages:
  // its scales and zero points are loaded with its first stage only, read
  // from LDS in the block before their first use and turned into the lanes'
  // factors once per group. The stage loop runs four stages per iteration,
  // unrolled, so which stages start a group is known at compile time
  // (K % 128 == 0). After the last stage the blocks read a slot they do not
  // use.
  // Wait counts: a stage carries kLoadsW loads, plus 1 when it starts a
  // group. Before block A of stage s, stages s+2 .. s+6 may stay in flight
  // (stages 2 .. 7 after the prologue). Any run of n consecutive stages
  // holds at least n / kSPG group starts, so waiting down to that many
  // loads never leaves a load of stage s + 1 outstanding (at most one load
  // of stage s + 2 is waited for too early).
  constexpr int kStartsIn2to7 = (kStages - 1) / kSPG - (1 / kSPG);  // exact: stages kSPG, 2 kSPG, .. in 2..7
  constexpr int kWaitPrologue = (kStages - 2) * kLoadsW + kStartsIn2to7;
  constexpr int kWaitLoop = (kStages - 3) * kLoadsW + (kStages - 3) / kSPG;
  static_assert(kWaitPrologue < 64 && kWaitLoop < 64, "vmcnt range");
  if (filler) {
#pragma unroll
    for (int st = 0; st < kStages; ++st)
      if (st < nst) MQ_ISSUE(st, st % kSPG == 0);
  }
  if (nst >= kStages) {
    wait_counts<kWaitPrologue, 0>();
  } else {
    wait_counts<0, 0>();
  }
  bare_barrier();

  GroupParams gp;
  f16x8 a0[kAFrags], b0[2];
  uint32_t wk1[8];  // raw words of (s, k1), unpacked in block A of stage s
  {
    uint32_t w[8];
    MQ_READ_GP(0, gp);
    MQ_READ_A(0, 0, a0);
    MQ_READ_W(0, 0, w);
    MQ_READ_W(0, 1, wk1);
    unpack_fields<kBF>(w, gp, lf, b0);
  }
  for (int s0 = 0; s0 < nst; s0 += 4) {
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const int s = s0 + ss;
      if (s > 0) {
        if (s + kStages - 2 < nst) {
          wait_counts<kWaitLoop, 0>();
        } else {
          wait_counts<0, 0>();
        }
        bare_barrier();
        if (filler && s + kStages - 1 < nst) MQ_ISSUE(s + kStages - 1, (ss + kStages - 1) % kSPG == 0);
      }
      const bool new_group = ss % kSPG == kSPG - 1;  // stage s + 1 starts a group (folded when unrolled)
      // block A
      f16x8 a1[kAFrags], b1[2];
      uint32_t wk0[8];  // raw words of (s + 1, k0)
      uint32_t sd_next, zw_next;
      {
        __builtin_amdgcn_sched_barrier(0);
        MQ_READ_A(s, 1, a1);
        MQ_READ_W(s + 1, 0, wk0);
        if (new_group) {
          const lds_i8* const sl_ = sm + ((s + 1) % kStages) * kSlotBytes;
          sd_next = *(const lds_word*)(sl_ + sbase);
          zw_next = *(const lds_word*)(sl_ + area + kBBytes + kSBytes + 4 * col_in_area);
        }
        unpack_fields<kBF>(wk1, gp, lf, b1);
        MQ_MFMAS(a0, b0);
        MQ_PIN(b1);
        if (new_group) {
          MQ_INTERLEAVE(14, kBF ? 5 : 4);
        } else {
          MQ_INTERLEAVE(12, kBF ? 5 : 4);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // block B
      {
        __builtin_amdgcn_sched_barrier(0);
        MQ_READ_A(s + 1, 0, a0);
        MQ_READ_W(s + 1, 1, wk1);
        if (new_group) make_group_params<kBF>(zw_next, sd_next, lf, gp);
        unpack_fields<kBF>(wk0, gp, lf, b0);
        MQ_MFMAS(a1, b1);
        MQ_PIN(b0);
        if (new_group) {
          MQ_INTERLEAVE(12, kBF ? 6 : 5);
        } else {
          MQ_INTERLEAVE(12, kBF ? 5 : 4);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#undef MQ_READ_A
#undef MQ_READ_W
#undef MQ_READ_GP
#undef MQ_MFMAS
#undef MQ_INTERLEAVE
#undef MQ_PIN
#undef MQ_ISSUE

  // Epilogue. D[m][j] of a 32x32 tile: lane (jj, hh) register r holds token
  // 8 (r / 4) + 4 hh + r % 4 of B column jj, i.e. output 8 (8 w + jj % 8)
  // + 2 (jj / 8) + t of the tile. The tile is staged in LDS as fp16 and
  // written out as whole rows with 16-byte stores (fp32 partial sums: 32
  // rows at a time, staged and written the same way); the fp16 rows go out
  // as non-temporal stores (about 1% faster at 4096^3, same-box A/B).
  wait_counts<0, 0>();
  bare_barrier();  // every wave is done reading the ring
  const int jj = lane & 31, hh = lane >> 5;
  const int ncol = 8 * (kWaveCols * wave + (jj & 7)) + 2 * (jj >> 3);
  if (splits > 1) {
    constexpr int kPitch32 = kTileCols * 8 * 4 + 16;  // bytes per staged fp32 row
    static_assert(32 * kPitch32 <= kStages * kSlotBytes, "fp32 32-row block fits the ring");
#pragma unroll
    for (int a = 0; a < kAFrags; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = 8 * (r / 4) + 4 * hh + (r % 4);
        lds_i8* const row = sm + lr * kPitch32;
#pragma unroll
        for (int t = 0; t < 2; ++t) *(__attribute__((address_space(3))) float*)(row + 4 * (ncol + t)) = acc[a][t][r];
      }
      wait_counts<0, 0>();
      bare_barrier();
      constexpr int kPieces32 = kTileCols * 2;  // 16-byte pieces (4 outputs) per row
      for (int i = threadIdx.x; i < 32 * kPieces32; i += kThreads) {
        const int lr = i / kPieces32, pc = i % kPieces32;
        const int m = m0 + 32 * a + lr, c = c0 + pc / 2;
        if (m >= M || c >= NP) continue;
        *reinterpret_cast<u32x4*>(partial + (static_cast<size_t>(split) * M + m) * N + 8 * c0 + 4 * pc) =
            *(const lds_u32x4*)(sm + lr * kPitch32 + 16 * pc);
      }
      wait_counts<0, 0>();
      bare_barrier();  // the next block reuses the staging rows
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < kAFrags; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mt = 32 * a + 8 * (r / 4) + 4 * hh + (r % 4);
      lds_i8* const row = sm + mt * kOutPitch;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *(__attribute__((address_space(3))) uint16_t*)(row + 2 * (ncol + t)) = half_bits<kBF>(acc[a][t][r]);
    }
  wait_counts<0, 0>();
  bare_barrier();
  constexpr int kPieces = kTileCols;  // 16-byte pieces (8 outputs) per row
  for (int i = threadIdx.x; i < kBM * kPieces; i += kThreads) {
    const int mt = i / kPieces, pc = i % kPieces;
    const int m = m0 + mt, c = c0 + pc;
    if (m >= M || c >= NP) continue;
    const u32x4 v_ = *(const lds_u32x4*)(sm + mt * kOutPitch + 16 * pc);
    __builtin_nontemporal_store(v_, reinterpret_cast<u32x4*>(y + static_cast<size_t>(m) * N + 8 * c));
  }
}


// Adds the splits' fp32 partial sums in split order and rounds to fp16 (or
// bf16); one thread per 4 outputs.
template <bool kBF>
__global__ __launch_bounds__(256) void w4a16_gemm_reduce(const float* __restrict__ partial,
                                                         uint16_t* __restrict__ y, int64_t mn4, int splits) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= mn4) return;
  const size_t stride = static_cast<size_t>(mn4) * 4;
  const float* src = partial + static_cast<size_t>(t) * 4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int sp = 1; sp < splits; ++sp) acc += *reinterpret_cast<const f32x4*>(src + sp * stride);
  const uint32_t lo = half_bits<kBF>(acc[0]) | (static_cast<uint32_t>(half_bits<kBF>(acc[1])) << 16);
  const uint32_t hi = half_bits<kBF>(acc[2]) | (static_cast<uint32_t>(half_bits<kBF>(acc[3])) << 16);
  *reinterpret_cast<u32x2*>(y + static_cast<size_t>(t) * 4) = u32x2{lo, hi};
}

}  // namespace

int w4a16_gemm_splits(int64_t M, int64_t N, int64_t K) {
  // Split K only when the tiles leave most CUs idle: the smallest divisor of
  // K/128 that gives >= 256 workgroups, keeping >= 512 rows (16 stages) per
  // split and at most 8 splits.
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N / 8 + kTileCols - 1) / kTileCols);
  if (tiles >= 192) return 1;
  const int64_t chunks = K / 128;
  int best = 1;
  for (int64_t s = 2; s <= 8 && K / s >= 512; ++s) {
    if (chunks % s) continue;
    best = static_cast<int>(s);
    if (tiles * s >= 256) break;
  }
  return best;
}

size_t w4a16_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  const int s = w4a16_gemm_splits(M, N, K);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

template <bool kBF>
hipError_t launch_w4a16_gemm_t(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                               const int32_t* qzeros, uint16_t* y,
                               int64_t M, int64_t N, int64_t K, int64_t group, bool per_channel, void* workspace,
                               hipStream_t stream) {
  const int gstep = per_channel ? 0 : 1;
  if (K % 128 || (group != 32 && group != 64 && group != 128)) return hipErrorInvalidValue;
  const int splits = workspace ? w4a16_gemm_splits(M, N, K) : 1;
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N / 8 + kTileCols - 1) / kTileCols);
  const int64_t work = static_cast<int64_t>(tiles_m) * tiles_n * splits;
  const int per_xcd = static_cast<int>((work + 7) / 8);
  const dim3 grid(static_cast<uint32_t>(8 * per_xcd));
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  float* part = static_cast<float*>(workspace);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  hipError_t err;
  switch (group) {
    case 32:
      err = launch_kernel(w4a16_gemm_kernel<1, kBF>, grid, dim3(kThreads), 0, stream, x, qw, scales, qz, y, part, m, n, k,
                          tiles_m, tiles_n, per_xcd, splits, gstep);
      break;
    case 64:
      err = launch_kernel(w4a16_gemm_kernel<2, kBF>, grid, dim3(kThreads), 0, stream, x, qw, scales, qz, y, part, m, n, k,
                          tiles_m, tiles_n, per_xcd, splits, gstep);
      break;
    default:
      err = launch_kernel(w4a16_gemm_kernel<4, kBF>, grid, dim3(kThreads), 0, stream, x, qw, scales, qz, y, part, m, n, k,
                          tiles_m, tiles_n, per_xcd, splits, gstep);
      break;
  }
  if (err != hipSuccess || splits == 1) return err;
  const int64_t mn4 = M * N / 4;
  return launch_kernel(w4a16_gemm_reduce<kBF>, dim3(static_cast<uint32_t>((mn4 + 255) / 256)), dim3(256), 0, stream,
                       part, y, mn4, splits);
}

hipError_t launch_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t group,
                             bool per_channel, void* workspace, bool bf16, hipStream_t stream) {
  return bf16 ? launch_w4a16_gemm_t<true>(x, qweight, scales, qzeros, y, M, N, K, group, per_channel, workspace, stream)
              : launch_w4a16_gemm_t<false>(x, qweight, scales, qzeros, y, M, N, K, group, per_channel, workspace,
                                           stream);
}

}  // namespace mq
