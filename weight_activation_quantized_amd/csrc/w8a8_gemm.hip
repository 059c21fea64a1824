// W8A8 int8 GEMM with int32 accumulation and a per-token x per-channel
// scale epilogue, for gfx950.
//
// Source: pymllm Setup and Usage, Overview (int8 activations and weights on
// INT8 matrix units) and section "W8A8 first-run JIT compilation" (int8
// scaled matmul). acc[m,n] = sum_k xq[m,k] * wq[n,k] (exact int32);
// y[m,n] = fp16(fl32(fl32(acc) * s_tok[m]) * s_ch[n]).
//
// Design:
// - v_mfma_i32_32x32x32_i8. On gfx950 it sustains about twice the int8 rate
//   of the 16x16x64 form. Both operands are K-contiguous ([M,K] and [N,K])
//   and lane (i = lane%32, h = lane/32) of either operand supplies 16
//   consecutive k of row i, so a fragment is one 16-byte LDS read per lane.
// - The weight rows are the MFMA's A operand and the token rows its B
//   operand, so the 32x32 result tile is D[n][m]: a lane holds four
//   consecutive output channels of one token.
// - A workgroup computes 256 tokens x 128 channels with eight wavefronts in
//   two groups of four. Within a group the wavefronts split the tile 2 x 2
//   (128 x 64 each, 128 int32 accumulators per lane); group g takes the k
//   half g of every stage. Each SIMD runs one wavefront of each group, so
//   while one waits on LDS or a barrier the other keeps the matrix unit
//   busy. The groups' partial sums are added (exact int32) through LDS at
//   the end.
// - Tiles move HBM -> LDS with buffer_load ... lds (no register staging)
//   into a ring of three 128-byte-deep stages (48 KB each): each load
//   instruction fills 8 rows x 128 bytes. On the MI355X a compute unit
//   streams such tiles from L2 at about 94 GB/s, against about 57 GB/s for
//   16 rows x 64 bytes, and the fill rate bounds this kernel. Two stages are
//   in flight while one is computed. Buffer loads past the descriptor's size
//   return zero, so ragged M, N and K edges arrive as zero rows and columns
//   with no per-lane predication.
// - LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled by the
//   row so that the 32 rows of a fragment read fall on distinct banks.
// - The epilogue stages the workgroup's output tile in LDS and writes whole
//   rows with 16-byte stores.
// - Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a
//   contiguous run of output tiles, ordered in groups of kGroupM token
//   tiles, so the operands a run shares stay in that XCD's L2.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

constexpr int kBM = 256;        // tokens per workgroup tile
constexpr int kBN = 128;        // output channels per workgroup tile
constexpr int kGroupWaves = 4;  // wavefronts per group (2 x 2 of 128 tokens x 64 channels)
constexpr int kWaves = 2 * kGroupWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kGroupM = 4;   // token tiles per group in the tile order
constexpr int kBK = 128;     // K bytes per stage (128-byte row segments)
constexpr int kSlots = 3;    // LDS ring depth (stages)
constexpr int kChunks = kBK / 16;                      // 16-byte chunks per tile row
constexpr int kRowsPerLoad = 1024 / kBK;               // rows one 64 x 16 B load fills
// Group 0 issues every fill (group 1 never waits on the texture unit, so
// its MFMAs keep running while group 0 stalls on a full fill queue).
constexpr int kLoadsX = kBM / kRowsPerLoad / kGroupWaves;  // per filling wave per stage
constexpr int kLoadsW = kBN / kRowsPerLoad / kGroupWaves;
constexpr int kLoads = kLoadsX + kLoadsW;
constexpr int kStageBytes = (kBM + kBN) * kBK;
constexpr int kSubPerGroup = kBK / 2 / 32;  // MFMA k-steps per group and stage
static_assert(kLoads < 32 && kLoads % 2 == 0, "vmcnt range / two bursts per round");
static_assert(kSlots * kStageBytes <= 160 * 1024, "LDS capacity");
static_assert(kSubPerGroup == 2, "a round below is written for two k-steps per group");

constexpr uint32_t kOob = 0x80000000u;    // a buffer offset past every tile: the load returns 0
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3 (raw 32-bit data)

typedef __attribute__((address_space(3))) int8_t lds_i8;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// XOR applied to the 16-byte chunk index of tile row r (128-byte rows).
// A fragment read takes one chunk of 32 consecutive rows; rows 2 apart share
// banks, and (r / 2) mod 8 spreads any 16 consecutive rows over the 16
// distinct 16-byte bank groups of a 256-byte window. Depends on r mod 16.
__device__ __forceinline__ int chunk_swizzle(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const int8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), 0, bytes, kBufferFlags);
}

template <bool kScaled, bool kBf16>
__global__ __launch_bounds__(kThreads) void w8a8_gemm_kernel(const int8_t* __restrict__ xq,
                                                             const float* __restrict__ s_tok,
                                                             const int8_t* __restrict__ wq,
                                                             const float* __restrict__ s_ch,
                                                             uint16_t* __restrict__ y,
                                                             int32_t* __restrict__ acc_out,
                                                             int M, int N, int K,
                                                             int tiles_m, int tiles_n, int per_xcd) {
  // After the main loop the same LDS holds group 1's partial sums (int32)
  // and then the output tile.
  typedef typename std::conditional<kScaled, uint16_t, int32_t>::type OutT;
  constexpr int kPartPitch = kBN * 4 + 16;  // padding staggers the rows over the banks
  constexpr int kRowBytes = kBN * static_cast<int>(sizeof(OutT));
  constexpr int kPitch = kRowBytes + 16;
  static_assert(kBM * kPartPitch <= kSlots * kStageBytes, "partial sums fit the ring");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kSlots * kStageBytes];
  lds_i8* const sm = (lds_i8*)(smem);

  // Output tile of this workgroup (XCD-contiguous, grouped by token tiles).
  const int t_id = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (t_id >= tiles_m * tiles_n) return;
  const int group_tiles = kGroupM * tiles_n;
  const int tgroup = t_id / group_tiles;
  const int first_m = tgroup * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int in_group = t_id - tgroup * group_tiles;
  const int m0 = (first_m + in_group % gm) * kBM;
  const int n0 = (in_group / gm) * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int g = wave / kGroupWaves;  // 0: even stages, 1: odd stages
  const int r = wave % kGroupWaves;  // position in the group; SIMD r hosts waves r and r + 4
  const int wm = r >> 1, wn = r & 1;

  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xq + static_cast<size_t>(m0) * K, min(kBM, M - m0) * K);
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wq + static_cast<size_t>(n0) * K, min(kBN, N - n0) * K);

  // Fill l of group 0's wave r (l < kLoadsX: token rows, else channel rows)
  // covers tile rows (r + 4u) * kRowsPerLoad .. with u = l or l - kLoadsX;
  // lane L writes physical chunk L % kChunks of row L / kChunks, so it
  // fetches the logical chunk that the swizzle places there.
  uint32_t loff[kLoads];
  int lk[kLoads];
#pragma unroll
  for (int l = 0; l < kLoads; ++l) {
    const int u = l < kLoadsX ? l : l - kLoadsX;
    const int row = (r + kGroupWaves * u) * kRowsPerLoad + lane / kChunks;
    lk[l] = 16 * ((lane % kChunks) ^ chunk_swizzle(row));
    loff[l] = static_cast<uint32_t>(row * K + lk[l]);
  }

  // Fragment reads: group g takes chunks 4g .. 4g + 3 of each stage; for its
  // k-step t lane (fi, fh) reads chunk 4g + 2t + fh of row fi (+32 b).
  const int fi = lane & 31, fh = lane >> 5;
  int coff[kSubPerGroup];
#pragma unroll
  for (int t = 0; t < kSubPerGroup; ++t) coff[t] = 16 * ((4 * g + 2 * t + fh) ^ chunk_swizzle(fi));
  const int xrow0 = (wm * 128 + fi) * kBK;
  const int wrow0 = kBM * kBK + (wn * 64 + fi) * kBK;

  i32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = i32x16{};

  const int nst = (K + kBK - 1) / kBK;

  // Fills [L0, L1) of stage S (issued by group 0's waves).
#define MQ_ISSUE(S, L0, L1)                                                                      \
  do {                                                                                           \
    const int k0_ = (S) * kBK;                                                                   \
    const int krem_ = K - k0_;                                                                   \
    lds_i8* const dst_ = sm + ((S) % kSlots) * kStageBytes;                                      \
    _Pragma("unroll") for (int l = (L0); l < (L1); ++l) {                                        \
      const uint32_t off_ = lk[l] < krem_ ? loff[l] + k0_ : kOob;                                \
      if (l < kLoadsX) {                                                                         \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
            rx, (lds_void*)(dst_ + (r + kGroupWaves * l) * 1024), 16, off_, 0, 0, 0);            \
      } else {                                                                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
            rw, (lds_void*)(dst_ + kBM * kBK + (r + kGroupWaves * (l - kLoadsX)) * 1024), 16,    \
            off_, 0, 0, 0);                                                                      \
      }                                                                                          \
    }                                                                                            \
  } while (0)

#define MQ_READ_FRAGS(S, T, FX, FW)                                                     \
  do {                                                                                  \
    const lds_i8* const src_ = sm + ((S) % kSlots) * kStageBytes + coff[T];             \
    _Pragma("unroll") for (int b = 0; b < 4; ++b) FX[b] =                               \
        *(const lds_i32x4*)(src_ + xrow0 + b * 32 * kBK);                               \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) FW[a] =                               \
        *(const lds_i32x4*)(src_ + wrow0 + a * 32 * kBK);                               \
  } while (0)

#define MQ_MFMAS(FX, FW)                                                                          \
  do {                                                                                            \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) _Pragma("unroll") for (int b = 0; b < 4; ++b)   \
        acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(FW[a], FX[b], acc[a][b], 0, 0, 0);      \
  } while (0)

#define MQ_MFMAS_HALF(FX, FW, A)                                                                  \
  do {                                                                                            \
    _Pragma("unroll") for (int b = 0; b < 4; ++b)                                                 \
        acc[A][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(FW[A], FX[b], acc[A][b], 0, 0, 0);      \
  } while (0)

  // Stage s sits in slot s % 3. Both groups compute every stage, group g on
  // its k half. Round s: group 0's waves issue the fills of stage s + 2 into
  // the slot of stage s - 1 (which every wave finished reading before the
  // barrier that ended round s - 1); every wave computes its half of stage
  // s; group 0's waves wait for their own loads of stage s + 1 (loads
  // complete in issue order, so only stage s + 2 stays in flight; group 1
  // has none to wait for) and all meet the barrier, after which stage s + 1
  // is complete and readable.
  if (g == 0) {
    MQ_ISSUE(0, 0, kLoads);
    if (1 < nst) MQ_ISSUE(1, 0, kLoads);
  }
  if (1 < nst) {
    wait_counts<kLoads, 0>();
  } else {
    wait_counts<0, 0>();
  }
  bare_barrier();

  i32x4 fx0[4], fw0[2], fx1[4], fw1[2];
  MQ_READ_FRAGS(0, 0, fx0, fw0);

  // Steady rounds (stages s + 1 and s + 2 exist): no branches, so the
  // compiler waits for exactly the LDS reads each MFMA needs. Half of the
  // second k-step's MFMAs are issued before the barrier and half after it,
  // under the reads of stage s + 1's first fragments.
  int s = 0;
  // One steady round; FILL: this wave issues fills (group 0). Half of the
  // fills of stage s + 2 go out at the start of each k-step: one burst of
  // all of them stalls the wave on the texture unit's full command queue
  // for longer, and single fills between MFMAs stall it more often.
#define MQ_STEADY(FILL) \
  for (; s + 2 < nst; ++s) { \
    __builtin_amdgcn_sched_barrier(0); \
    if (FILL) MQ_ISSUE(s + 2, 0, kLoads / 2); \
    __builtin_amdgcn_sched_barrier(0); \
    MQ_READ_FRAGS(s, 1, fx1, fw1); \
    MQ_MFMAS(fx0, fw0); \
    _Pragma("unroll") for (int i_ = 0; i_ < 3; ++i_) { \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); \
    } \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); \
    __builtin_amdgcn_sched_barrier(0); \
    if (FILL) MQ_ISSUE(s + 2, kLoads / 2, kLoads); \
    __builtin_amdgcn_sched_barrier(0); \
    MQ_MFMAS_HALF(fx1, fw1, 0); \
    __builtin_amdgcn_sched_barrier(0); \
    wait_counts<kLoads, 0>(); \
    bare_barrier(); \
    MQ_READ_FRAGS(s + 1, 0, fx0, fw0); \
    MQ_MFMAS_HALF(fx1, fw1, 1); \
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0); \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); \
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0); \
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0); \
    __builtin_amdgcn_sched_barrier(0); \
  }
  if (g == 0) {
    MQ_STEADY(true)
  } else {
    MQ_STEADY(false)
  }
#undef MQ_STEADY
  // Last two stages (or fewer): nothing left to fill.
  for (; s < nst; ++s) {
    MQ_READ_FRAGS(s, 1, fx1, fw1);
    MQ_MFMAS(fx0, fw0);
    if (s + 1 < nst) {
      wait_counts<0, 0>();
      bare_barrier();
      MQ_READ_FRAGS(s + 1, 0, fx0, fw0);
    }
    MQ_MFMAS(fx1, fw1);
  }
#undef MQ_ISSUE
#undef MQ_READ_FRAGS
#undef MQ_MFMAS
#undef MQ_MFMAS_HALF

  // Epilogue. D[n][m] of a 32x32 tile: lane (j, h) register r holds channel
  // 8 (r / 4) + 4 h + r % 4 of token j, so the lane's tokens are
  // wm*128 + 32 b + j and its channels wn*64 + 32 a + 8 q + 4 h + i.
  const int j = lane & 31, h = lane >> 5;
  // Each group finishes two of the four 32-token blocks b of its wave's
  // 128 x 64 block: group 0 blocks 0 and 1, group 1 blocks 2 and 3. It
  // hands its partial sums of the other two blocks to the other group
  // through LDS (exact int32 adds), then scales and stages its own two.
  float sc[2][4][4], st[4];
  if (kScaled) {
    // Every scale is loaded up front (indices clamped into range; results
    // out of range are not stored) and consumed after the partial-sum
    // exchange, so the loads overlap it.
    const int nb = n0 + wn * 64 + 4 * h, mb = m0 + wm * 128 + j;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[a][q][i] = s_ch[min(nb + 32 * a + 8 * q + i, N - 1)];
#pragma unroll
    for (int b = 0; b < 4; ++b) st[b] = s_tok[min(mb + 32 * b, M - 1)];
  }

  // The waits below are for LDS traffic only (vmcnt 63: the scale loads
  // stay in flight).
#define MQ_PART_WRITE(B)                                                                             \
  _Pragma("unroll") for (int a = 0; a < 2; ++a) _Pragma("unroll") for (int q = 0; q < 4; ++q) {      \
    const int row = wm * 128 + 32 * (B) + j, col = wn * 64 + 32 * a + 8 * q + 4 * h;                \
    *(lds_i32x4*)(sm + row * kPartPitch + col * 4) =                                                \
        i32x4{acc[a][B][4 * q], acc[a][B][4 * q + 1], acc[a][B][4 * q + 2], acc[a][B][4 * q + 3]};   \
  }
#define MQ_PART_ADD(B)                                                                               \
  _Pragma("unroll") for (int a = 0; a < 2; ++a) _Pragma("unroll") for (int q = 0; q < 4; ++q) {      \
    const int row = wm * 128 + 32 * (B) + j, col = wn * 64 + 32 * a + 8 * q + 4 * h;                \
    const i32x4 v = *(const lds_i32x4*)(sm + row * kPartPitch + col * 4);                           \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[a][B][4 * q + i] += v[i];                      \
  }
#define MQ_STAGE(B)                                                                                  \
  _Pragma("unroll") for (int a = 0; a < 2; ++a) _Pragma("unroll") for (int q = 0; q < 4; ++q) {      \
    const int row = wm * 128 + 32 * (B) + j, col = wn * 64 + 32 * a + 8 * q + 4 * h;                \
    lds_i8* const dst = sm + row * kPitch + col * static_cast<int>(sizeof(OutT));                   \
    if constexpr (kScaled) {                                                                         \
      uint32_t hv[4];                                                                                \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                \
        const float v = (static_cast<float>(acc[a][B][4 * q + i]) * st[B]) * sc[a][q][i];            \
        hv[i] = half_bits<kBf16>(v);                                                                 \
      }                                                                                              \
      *(lds_u32x2*)(dst) = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};                      \
    } else {                                                                                         \
      *(lds_i32x4*)(dst) =                                                                           \
          i32x4{acc[a][B][4 * q], acc[a][B][4 * q + 1], acc[a][B][4 * q + 2], acc[a][B][4 * q + 3]}; \
    }                                                                                                \
  }

  wait_counts<63, 0>();  // every wave is done reading the ring
  bare_barrier();
  if (g == 0) {
    MQ_PART_WRITE(2)
    MQ_PART_WRITE(3)
  } else {
    MQ_PART_WRITE(0)
    MQ_PART_WRITE(1)
  }
  wait_counts<63, 0>();
  bare_barrier();
  if (g == 0) {
    MQ_PART_ADD(0)
    MQ_PART_ADD(1)
  } else {
    MQ_PART_ADD(2)
    MQ_PART_ADD(3)
  }
  wait_counts<63, 0>();  // the partial sums are consumed before the area is reused
  bare_barrier();
  if constexpr (kScaled) {
    // Settle the scale loads here (vmcnt also counts stores, so a wait
    // among the stores below would drain them as well).
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(sc[a][q][i]));
#pragma unroll
    for (int b = 0; b < 4; ++b) asm volatile("" : "+v"(st[b]));
  }
  if (g == 0) {
    MQ_STAGE(0)
    MQ_STAGE(1)
  } else {
    MQ_STAGE(2)
    MQ_STAGE(3)
  }
#undef MQ_PART_WRITE
#undef MQ_PART_ADD
#undef MQ_STAGE
  wait_counts<0, 0>();
  bare_barrier();

  // All eight waves write the tile out as whole rows, 16 bytes per lane;
  // non-temporal stores (the output is not read back by this kernel), 1-4%
  // faster than ordinary ones across the prefill shapes (same-box A/B).
  constexpr int kPerChunk = 16 / static_cast<int>(sizeof(OutT));  // outputs per 16-byte piece
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  OutT* const out = kScaled ? reinterpret_cast<OutT*>(y) : reinterpret_cast<OutT*>(acc_out);
  const int c = threadIdx.x % kChunksPerRow;
  const int n = n0 + c * kPerChunk;
  const bool whole = (N % kPerChunk) == 0;  // rows start 16-byte aligned; a piece is all in or all out
#pragma unroll 4
  for (int rr = threadIdx.x / kChunksPerRow; rr < kBM; rr += kRowsPerPass) {
    const int m = m0 + rr;
    if (m >= M || n >= N) continue;
    const u32x4 v = *(const lds_u32x4*)(sm + rr * kPitch + c * 16);
    OutT* const o = out + static_cast<size_t>(m) * N + n;
    if (whole) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(o));
    } else {
#pragma unroll
      for (int i = 0; i < kPerChunk; ++i) {
        if (n + i >= N) break;
        if constexpr (kScaled) {
          o[i] = static_cast<OutT>(v[i / 2] >> (16 * (i % 2)));
        } else {
          o[i] = static_cast<OutT>(v[i]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_w8a8_gemm(const int8_t* xq, const float* s_tok, const int8_t* wq,
                            const float* s_ch, uint16_t* y, int32_t* acc,
                            int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream) {
  if (w8a8_use_gemv(M, N)) return launch_w8a8_gemv(xq, s_tok, wq, s_ch, y, acc, M, N, K, bf16, stream);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int per_xcd = static_cast<int>((tiles + 7) / 8);
  const dim3 grid(static_cast<uint32_t>(8 * per_xcd)), block(kThreads);
  if (y != nullptr && bf16)
    return launch_kernel(w8a8_gemm_kernel<true, true>, grid, block, 0, stream, xq, s_tok, wq, s_ch, y,
                         static_cast<int32_t*>(nullptr), m, n, k, tiles_m, tiles_n, per_xcd);
  if (y != nullptr)
    return launch_kernel(w8a8_gemm_kernel<true, false>, grid, block, 0, stream, xq, s_tok, wq, s_ch, y,
                         static_cast<int32_t*>(nullptr), m, n, k, tiles_m, tiles_n, per_xcd);
  return launch_kernel(w8a8_gemm_kernel<false, false>, grid, block, 0, stream, xq, s_tok, wq, s_ch,
                       static_cast<uint16_t*>(nullptr), acc, m, n, k, tiles_m, tiles_n, per_xcd);
}

}  // namespace mq
