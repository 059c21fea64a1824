// W4A16 GEMM for prefill-shaped M on gfx950.
//
// Source: LMDeploy toolkit overview, section 2.5 (AWQ 4-bit weights, group
// size 128) and LMDeploy 4-bit deployment guide, sections 2.2-2.3 (scales
// and weights consumed inside the matmul kernel; a real low-bit kernel rather
// than fake quantization). y[m,n] = sum_k x[m,k] * fp16((q - z) * s).
//
// Design:
// - v_mfma_f32_32x32x16_f16 (on gfx950 about 1.5x the rate of the 16x16x32
//   form). A workgroup computes 64 tokens x 1024 outputs with four
//   wavefronts side by side in N; a wavefront owns 64 x 256 (two 32-token
//   A fragments x eight field tiles, 256 fp32 accumulators per lane), so
//   every weight is dequantized exactly once per workgroup.
// - Field tiles: lane (j = lane%32, h = lane/32) of the B operand takes word
//   j (packed column j of the wavefront) of rows 8h..8h+7 of a 16-row k-step
//   and unpacks it into eight fp16 fragments, one per 4-bit field p; tile p
//   then covers outputs 8c + p of the 32 packed columns c. The unpack is
//   exact and each weight is rounded once, to fp16((q - z) * s).
// - Everything moves HBM -> LDS with buffer_load ... lds through a ring of
//   kStages 32-row stages: the x rows (shared by the four wavefronts), each
//   wavefront's raw packed words, scales and zero points. Loads past a
//   buffer descriptor's size return zero (ragged M); columns past N read
//   valid memory and are never stored.
// - x rows are 64 bytes per stage with the 16-byte chunk index XOR-swizzled
//   by the row (conflict-free fragment reads). Raw weight rows are 128
//   bytes; k-row r is stored at LDS row r with bits 0 and 3 swapped, so the
//   two lane halves (rows 8h + e) read opposite halves of the banks.
// - Workgroups are dispatched round-robin over the 8 XCDs; tiles are
//   remapped so an XCD runs consecutive token tiles of one weight tile.
#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"

namespace mq {
namespace {

constexpr int kBM = 64;                    // tokens per workgroup tile
constexpr int kWaves = 4;                  // side by side in N
constexpr int kWaveCols = 32;              // packed columns per wavefront (256 outputs)
constexpr int kTileCols = kWaves * kWaveCols;  // 128 packed columns (1024 outputs)
constexpr int kRows = 32;                  // K rows per stage (two 16-row MFMA k-steps)
#ifndef MQ_W4_STAGES
#define MQ_W4_STAGES 6
#endif
constexpr int kStages = MQ_W4_STAGES;
constexpr int kABytes = kBM * kRows * 2;       // x rows: 64 x 64 B
constexpr int kBBytes = kRows * kWaveCols * 4;  // a wavefront's raw words: 32 x 128 B
constexpr int kSBytes = 1024;                   // a wavefront's scales (512 B used)
constexpr int kZBytes = 256;                    // a wavefront's zero points (128 B used)
constexpr int kWaveBytes = kBBytes + kSBytes + kZBytes;
constexpr int kSlotBytes = kABytes + kWaves * kWaveBytes;
constexpr int kLoads = 7;  // per wavefront per stage: 1 x, 4 weights, 1 scales, 1 zero points
static_assert(kStages >= 2 && (kStages - 2) * kLoads < 64, "ring depth / vmcnt range");
static_assert(kStages * kSlotBytes <= 160 * 1024, "LDS capacity");

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

struct GroupParams {
  uint32_t negz[8];  // -(1024 + z) (even p) or -(1024 + 16 z) (odd p), both halves
  uint32_t sc2[8];   // s (even p) or s / 16 (odd p), both halves
};

__device__ __forceinline__ void make_group_params(uint32_t zw, u32x4 sv, GroupParams& gp) {
  zero_bias(zw, gp.negz);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const f16x2 s2 = as_f16x2(sv[p >> 1]);
    f16 s = s2[p & 1];
    if (p & 1) s = s * static_cast<f16>(0.0625f);  // exact: power-of-two rescale of a normal fp16
    f16x2 rep;
    rep[0] = s;
    rep[1] = s;
    gp.sc2[p] = as_u32(rep);
  }
}

__global__ __launch_bounds__(256) void w4a16_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qz,
                                                         uint16_t* __restrict__ y, int M, int N, int K,
                                                         int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kSlotBytes];
  lds_i8* const sm = (lds_i8*)(smem);

  // Tile of this workgroup: each XCD takes a contiguous run of tiles, token
  // tiles fastest, so its workgroups share weight tiles.
  const int t_id = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (t_id >= tiles_m * tiles_n) return;
  const int m0 = (t_id % tiles_m) * kBM;
  const int c0 = (t_id / tiles_m) * kTileCols;  // first packed column
  const int NP = N >> 3;
  const int G = K / kGroup;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // x: one descriptor for the tile's rows (rows past M read as zero). The
  // weight, scale and zero-point descriptors are re-based at each stage's
  // first row (group), so every offset stays far below 2^31 for any legal
  // shape; columns past N read valid memory of the next row (never stored)
  // or, past the last row, zero.
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + static_cast<size_t>(m0) * K, static_cast<int64_t>(min(kBM, M - m0)) * K * 2);

  // Per-lane parts of the DMA source offsets.
  //  x: wave w fills rows 16w .. 16w+15; lane L -> row 16w + L/4, physical
  //     chunk L%4, which holds logical chunk (L%4) ^ swizzle(row).
  const int xa_row = 16 * wave + lane / 4;
  const uint32_t xa_off = static_cast<uint32_t>(xa_row * K + 8 * ((lane % 4) ^ chunk_swizzle(xa_row))) * 2u;
  //  weights: load u fills LDS rows 8u .. 8u+7 of the wave's area; lane L ->
  //     LDS row 8u + L/8 = k-row raw_row(.), 16-byte chunk L%8 (words 4(L%8)..).
  uint32_t wr_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    wr_off[u] = static_cast<uint32_t>(raw_row(8 * u + lane / 8) * NP + kWaveCols * wave + 4 * (lane % 8)) * 4u;
  //  scales: lane L -> the 8 scales of packed column (L % 32) of the wave;
  //  zero points: lane L -> word (L % 32).
  const uint32_t s_off = static_cast<uint32_t>(8 * (kWaveCols * wave + lane % 32)) * 2u;
  const uint32_t z_off = static_cast<uint32_t>(kWaveCols * wave + lane % 32) * 4u;

  lds_i8* const wave_area = sm + kABytes + wave * kWaveBytes;  // + slot offset

#define MQ_ISSUE(ST)                                                                                 \
  do {                                                                                               \
    const int k0_ = (ST) * kRows;                                                                    \
    const int g_ = k0_ / kGroup;                                                                     \
    const int so_ = ((ST) % kStages) * kSlotBytes;                                                   \
    const __amdgpu_buffer_rsrc_t rw_ =                                                               \
        rsrc(qw + static_cast<size_t>(k0_) * NP + c0, (static_cast<int64_t>(K - k0_) * NP - c0) * 4); \
    const __amdgpu_buffer_rsrc_t rs_ = rsrc(scales + static_cast<size_t>(g_) * N + c0 * 8,           \
                                            (static_cast<int64_t>(G - g_) * N - c0 * 8) * 2);         \
    const __amdgpu_buffer_rsrc_t rz_ =                                                               \
        rsrc(qz + static_cast<size_t>(g_) * NP + c0, (static_cast<int64_t>(G - g_) * NP - c0) * 4);  \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sm + so_ + wave * 1024), 16,            \
                                             xa_off + k0_ * 2, 0, 0, 0);                             \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw_, (lds_void*)(wave_area + so_ + u * 1024), 16,   \
                                                 wr_off[u], 0, 0, 0);                                \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, (lds_void*)(wave_area + so_ + kBBytes), 16, s_off, \
                                             0, 0, 0);                                               \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rz_, (lds_void*)(wave_area + so_ + kBBytes + kSBytes), 4, \
                                             z_off, 0, 0, 0);                                        \
  } while (0)

  // Fragment read offsets within a slot.
  const int fi = lane & 31, fh = lane >> 5;
  // x fragments: row fi (+32) of the tile, k-step t -> logical chunk 2t + fh.
  int xoff[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 32 * a + fi;
      xoff[a][t] = row * 64 + 16 * ((2 * t + fh) ^ chunk_swizzle(row));
    }
  // raw words: k-row 16t + 8fh + e of packed column fi.
  const int wbase = kABytes + wave * kWaveBytes + 4 * fi;

  f32x16 acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int p = 0; p < 8; ++p) acc[a][p] = f32x16{};

  const int nst = K / kRows;

  // Operands of one 16-row k-step: the two x fragments and the eight
  // dequantized weight fragments.
#define MQ_READ_A(S, T, AF)                                                                      \
  do {                                                                                           \
    const lds_i8* const sl_ = sm + ((S) % kStages) * kSlotBytes;                                 \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) AF[a] = *(const lds_f16x8*)(sl_ + xoff[a][T]);  \
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
    const u32x4 sv_ = *(const lds_u32x4*)(sl_ + wbase - 4 * fi + kBBytes + 16 * fi);             \
    const uint32_t zw_ = *(const lds_word*)(sl_ + wbase + kBBytes + kSBytes);                    \
    make_group_params(zw_, sv_, GP);                                                             \
  } while (0)
#define MQ_MFMAS(AF, B)                                                                          \
  do {                                                                                           \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) _Pragma("unroll") for (int p = 0; p < 8; ++p)  \
        acc[a][p] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AF[a], B[p], acc[a][p], 0, 0, 0);     \
  } while (0)
// Keeps the unpacked fragments in the block that computes them (otherwise
// they are sunk next to their use, out of reach of the MFMAs they are meant
// to overlap).
#define MQ_PIN(B) _Pragma("unroll") for (int p_ = 0; p_ < 8; ++p_) asm volatile("" : "+v"(B[p_]))
// Schedule of a block: its LDS reads first, then the 16 MFMAs each followed
// by a share of the unpack arithmetic.
#define MQ_INTERLEAVE(NDS, NVALU)                                                                \
  do {                                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < 16; ++i_) {                                          \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);                                     \
    }                                                                                            \
  } while (0)

  // Software pipeline: the weights of the next k-step are unpacked while the
  // current k-step's MFMAs run, in the same basic block, so the VALU and the
  // matrix unit overlap within the single wavefront per SIMD. Stage s + 1 is
  // waited for (and the slot of stage s refilled) in the middle of stage s.
  // The prologue fills every slot.
#pragma unroll
  for (int st = 0; st < kStages; ++st)
    if (st < nst) MQ_ISSUE(st);
  if (nst >= kStages) {
    wait_counts<(kStages - 1) * kLoads, 0>();
  } else {
    wait_counts<0, 0>();
  }
  bare_barrier();

  GroupParams gp;
  f16x8 a0[2], b0[8];
  {
    uint32_t w[8];
    MQ_READ_GP(0, gp);
    MQ_READ_A(0, 0, a0);
    MQ_READ_W(0, 0, w);
    unpack_step_scaled(w, gp.negz, gp.sc2, b0);
  }
  for (int s = 0; s < nst; ++s) {
    // k-step 1 of stage s: unpack while k-step 0's MFMAs run.
    f16x8 a1[2], b1[8];
    {
      __builtin_amdgcn_sched_barrier(0);
      uint32_t w[8];
      MQ_READ_A(s, 1, a1);
      MQ_READ_W(s, 1, w);
      unpack_step_scaled(w, gp.negz, gp.sc2, b1);
      MQ_MFMAS(a0, b0);
      MQ_PIN(b1);
      MQ_INTERLEAVE(10, 7);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Stage s + 1 must have landed (every wave's share), and every wave is
    // done reading stage s, whose slot takes stage s + kStages. (After the
    // last stage this reads a slot it does not use.)
    if (s + kStages - 1 < nst) {
      wait_counts<(kStages - 2) * kLoads, 0>();
    } else {
      wait_counts<0, 0>();
    }
    bare_barrier();
    if (s + kStages < nst) MQ_ISSUE(s + kStages);
    // k-step 0 of stage s + 1: unpack while k-step 1's MFMAs run.
    {
      __builtin_amdgcn_sched_barrier(0);
      uint32_t w[8];
      MQ_READ_GP(s + 1, gp);
      MQ_READ_A(s + 1, 0, a0);
      MQ_READ_W(s + 1, 0, w);
      unpack_step_scaled(w, gp.negz, gp.sc2, b0);
      MQ_MFMAS(a1, b1);
      MQ_PIN(b0);
      MQ_INTERLEAVE(12, 10);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef MQ_READ_A
#undef MQ_READ_W
#undef MQ_READ_GP
#undef MQ_MFMAS
#undef MQ_INTERLEAVE
#undef MQ_PIN
#undef MQ_ISSUE

  // D[m][c] of a 32x32 tile: lane (jj, hh) register r holds token
  // 8 (r / 4) + 4 hh + r % 4 of packed column jj; the eight field tiles give
  // the column's 8 consecutive outputs.
  const int jj = lane & 31, hh = lane >> 5;
  const int c = c0 + kWaveCols * wave + jj;
  if (c >= NP) return;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * a + 8 * (r / 4) + 4 * hh + (r % 4);
      if (m >= M) continue;
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x2 pr;
        pr[0] = static_cast<f16>(acc[a][2 * q][r]);
        pr[1] = static_cast<f16>(acc[a][2 * q + 1][r]);
        out[q] = as_u32(pr);
      }
      *reinterpret_cast<u32x4*>(y + static_cast<size_t>(m) * N + 8 * c) = out;
    }
}

}  // namespace

hipError_t launch_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N / 8 + kTileCols - 1) / kTileCols);
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int per_xcd = static_cast<int>((tiles + 7) / 8);
  return launch_kernel(w4a16_gemm_kernel, dim3(static_cast<uint32_t>(8 * per_xcd)), dim3(256), 0, stream, x,
                       reinterpret_cast<const uint32_t*>(qweight), scales,
                       reinterpret_cast<const uint32_t*>(qzeros), y, static_cast<int>(M),
                       static_cast<int>(N), static_cast<int>(K), tiles_m, tiles_n, per_xcd);
}

}  // namespace mq
