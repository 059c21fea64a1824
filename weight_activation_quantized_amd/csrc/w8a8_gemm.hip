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
// - A workgroup of four wavefronts computes 256 tokens x 128 channels; each
//   wavefront owns 128 x 64 (2 x 4 MFMA tiles, 128 int32 accumulators per
//   lane). That is 85 int8 ops per LDS byte read.
// - Tiles move HBM -> LDS with buffer_load ... lds (no register staging)
//   into a ring of kStages stages of kBK bytes of K. Buffer loads past the
//   descriptor's size return zero, so ragged M, N and K edges arrive as
//   zero rows and columns with no per-lane predication.
// - One wavefront per SIMD: the fills of a stage are spread over the MFMA
//   k-steps of the stage computed two iterations earlier, so the wave never
//   stalls on a long run of load issues while the matrix unit idles.
// - The epilogue stages the workgroup's output tile in LDS and writes whole
//   rows with 16-byte stores.
// - LDS rows are kBK bytes; the 16-byte chunk index is XOR-swizzled by the
//   row so that the 32 rows of a fragment read fall on distinct banks.
// - Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a
//   contiguous run of output tiles, ordered in groups of kGroupM token
//   tiles, so the operands a run shares stay in that XCD's L2.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

#ifndef MQ_W8A8_BK
#define MQ_W8A8_BK 128
#endif
#ifndef MQ_W8A8_STAGES
#define MQ_W8A8_STAGES 3
#endif

constexpr int kBM = 256;    // tokens per workgroup tile
constexpr int kBN = 128;    // output channels per workgroup tile
constexpr int kWaves = 4;   // 2 x 2 wavefronts of 128 tokens x 64 channels
constexpr int kGroupM = 4;  // token tiles per group in the tile order
constexpr int kBK = MQ_W8A8_BK;          // K bytes per pipeline stage
constexpr int kStages = MQ_W8A8_STAGES;  // LDS ring depth
constexpr int kChunks = kBK / 16;                     // 16-byte chunks per tile row
constexpr int kRowsPerLoad = 1024 / kBK;              // rows one 64 x 16 B load fills
constexpr int kLoadsX = kBM / kRowsPerLoad / kWaves;  // loads per wave per stage
constexpr int kLoadsW = kBN / kRowsPerLoad / kWaves;
constexpr int kLoads = kLoadsX + kLoadsW;
constexpr int kStageBytes = (kBM + kBN) * kBK;
constexpr int kSub = kBK / 32;  // MFMA k-steps per stage
static_assert(kBK == 64 || kBK == 128, "stage depth");
static_assert(kStages >= 3 && kStages * kStageBytes <= 160 * 1024, "ring depth / LDS capacity");
static_assert(kLoads % kSub == 0 && (kStages - 2) * kLoads < 64, "load split / vmcnt range");
constexpr int kLoadsPerSub = kLoads / kSub;  // fills issued per MFMA k-step

constexpr uint32_t kOob = 0x80000000u;    // a buffer offset past every tile: the load returns 0
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3 (raw 32-bit data)

typedef __attribute__((address_space(3))) int8_t lds_i8;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// XOR applied to the 16-byte chunk index of tile row r. For the fragment
// reads (32 rows, one chunk each) it makes any 8 and any 16 consecutive rows
// land on distinct 16-byte bank groups of a 128- or 256-byte LDS window.
__device__ __forceinline__ int chunk_swizzle(int r) {
  if constexpr (kBK == 64) {
    return ((r >> 2) & 3) ^ (r & 2);
  } else {
    return (r & 7) ^ ((r >> 3) & 1);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const int8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), 0, bytes, kBufferFlags);
}

template <bool kScaled>
__global__ __launch_bounds__(256) void w8a8_gemm_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ s_tok,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ s_ch,
                                                        uint16_t* __restrict__ y,
                                                        int32_t* __restrict__ acc_out,
                                                        int M, int N, int K,
                                                        int tiles_m, int tiles_n, int per_xcd) {
  // The output tile is staged in the same LDS after the main loop.
  typedef typename std::conditional<kScaled, uint16_t, int32_t>::type OutT;
  constexpr int kRowBytes = kBN * static_cast<int>(sizeof(OutT));
  constexpr int kPitch = kRowBytes + 16;  // padding staggers the rows over the banks
  constexpr int kSmemBytes = kStages * kStageBytes > kBM * kPitch ? kStages * kStageBytes : kBM * kPitch;
  static_assert(kSmemBytes <= 160 * 1024, "LDS capacity");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kSmemBytes];
  lds_i8* const sm = (lds_i8*)(smem);

  // Output tile of this workgroup (XCD-contiguous, grouped by token tiles).
  const int t_id = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (t_id >= tiles_m * tiles_n) return;
  const int group_tiles = kGroupM * tiles_n;
  const int group = t_id / group_tiles;
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int in_group = t_id - group * group_tiles;
  const int m0 = (first_m + in_group % gm) * kBM;
  const int n0 = (in_group / gm) * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xq + static_cast<size_t>(m0) * K, min(kBM, M - m0) * K);
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wq + static_cast<size_t>(n0) * K, min(kBN, N - n0) * K);

  // Fill l of this wave (l < kLoadsX: token rows, else channel rows) covers
  // tile rows (wave + 4u) * kRowsPerLoad .. with u = l or l - kLoadsX; lane
  // L writes physical chunk L % kChunks of row L / kChunks, so it fetches
  // the logical chunk that the swizzle places there.
  uint32_t loff[kLoads];
  int lk[kLoads];
#pragma unroll
  for (int l = 0; l < kLoads; ++l) {
    const int u = l < kLoadsX ? l : l - kLoadsX;
    const int row = (wave + kWaves * u) * kRowsPerLoad + lane / kChunks;
    lk[l] = 16 * ((lane % kChunks) ^ chunk_swizzle(row));
    loff[l] = static_cast<uint32_t>(row * K + lk[l]);
  }

  // Fragment reads: lane (fi, fh) reads chunk 2t + fh of row fi (+32 b).
  const int fi = lane & 31, fh = lane >> 5;
  int coff[kSub];
#pragma unroll
  for (int t = 0; t < kSub; ++t) coff[t] = 16 * ((2 * t + fh) ^ chunk_swizzle(fi));
  const int xrow0 = (wm * 128 + fi) * kBK;
  const int wrow0 = kBM * kBK + (wn * 64 + fi) * kBK;

  i32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = i32x16{};

  const int nst = (K + kBK - 1) / kBK;

  // Fills [L0, L1) of stage S.
#define MQ_ISSUE(S, L0, L1)                                                                       \
  do {                                                                                            \
    const int k0_ = (S) * kBK;                                                                    \
    const int krem_ = K - k0_;                                                                    \
    lds_i8* const dst_ = sm + ((S) % kStages) * kStageBytes;                                      \
    _Pragma("unroll") for (int l = (L0); l < (L1); ++l) {                                         \
      const uint32_t off_ = lk[l] < krem_ ? loff[l] + k0_ : kOob;                                 \
      if (l < kLoadsX) {                                                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(dst_ + (wave + kWaves * l) * 1024), \
                                                 16, off_, 0, 0, 0);                              \
      } else {                                                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                 \
            rw, (lds_void*)(dst_ + kBM * kBK + (wave + kWaves * (l - kLoadsX)) * 1024), 16, off_,  \
            0, 0, 0);                                                                             \
      }                                                                                           \
    }                                                                                             \
  } while (0)

#define MQ_READ_FRAGS(SLOT, T, FX, FW)                                                  \
  do {                                                                                  \
    const lds_i8* const src_ = sm + (SLOT) * kStageBytes + coff[T];                     \
    _Pragma("unroll") for (int b = 0; b < 4; ++b) FX[b] =                               \
        *(const lds_i32x4*)(src_ + xrow0 + b * 32 * kBK);                               \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) FW[a] =                               \
        *(const lds_i32x4*)(src_ + wrow0 + a * 32 * kBK);                               \
  } while (0)

  // Prologue: stages 0 .. kStages - 2. Iteration s then fills stage
  // s + kStages - 1 into the slot of stage s - 1 (free since the barrier that
  // ended iteration s - 1), kLoadsPerSub fills per k-step so they interleave
  // with the MFMAs. Loads complete in issue order.
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nst) MQ_ISSUE(st, 0, kLoads);
  if (nst >= kStages - 1) {
    wait_counts<(kStages - 2) * kLoads, 0>();
  } else {
    wait_counts<0, 0>();
  }
  bare_barrier();

  i32x4 fx0[4], fw0[2], fx1[4], fw1[2];
  MQ_READ_FRAGS(0, 0, fx0, fw0);

  for (int s = 0; s < nst; ++s) {
    const int slot = s % kStages;
    const int fill = s + kStages - 1;
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
      if (fill < nst) MQ_ISSUE(fill, t * kLoadsPerSub, (t + 1) * kLoadsPerSub);
      // Prefetch the next k-step's fragments into the other register set.
      if (t + 1 < kSub) {
        if (t & 1) {
          MQ_READ_FRAGS(slot, t + 1, fx0, fw0);
        } else {
          MQ_READ_FRAGS(slot, t + 1, fx1, fw1);
        }
      } else if (s + 1 < nst) {
        // Stage s + 1 must have landed (every wave's share) and every wave
        // must be done reading stage s before the next iteration refills it.
        if (fill < nst) {
          wait_counts<(kStages - 2) * kLoads, 0>();
        } else {
          wait_counts<0, 0>();
        }
        bare_barrier();
        const int nslot = (s + 1) % kStages;
        if (t & 1) {
          MQ_READ_FRAGS(nslot, 0, fx0, fw0);
        } else {
          MQ_READ_FRAGS(nslot, 0, fx1, fw1);
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (t & 1) {
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw1[a], fx1[b], acc[a][b], 0, 0, 0);
          } else {
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw0[a], fx0[b], acc[a][b], 0, 0, 0);
          }
        }
    }
  }
#undef MQ_ISSUE
#undef MQ_READ_FRAGS

  // Epilogue. D[n][m] of a 32x32 tile: lane (j, h) register r holds channel
  // 8 (r / 4) + 4 h + r % 4 of token j, so the lane's tokens are
  // wm*128 + 32 b + j and its channels wn*64 + 32 a + 8 q + 4 h + i. The
  // results (fp16 after scaling, or int32) are staged in LDS as the
  // workgroup's 256 x 128 output tile, then written out as whole rows in
  // 16-byte pieces.
  const int j = lane & 31, h = lane >> 5;
  float sc[2][4][4], st[4];
  if constexpr (kScaled) {
    // Every scale is loaded up front (indices clamped into range; results
    // out of range are not stored), then consumed by empty asm statements so
    // the loads settle before any store (vmcnt also counts stores).
    const int nb = n0 + wn * 64 + 4 * h, mb = m0 + wm * 128 + j;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[a][q][i] = s_ch[min(nb + 32 * a + 8 * q + i, N - 1)];
#pragma unroll
    for (int b = 0; b < 4; ++b) st[b] = s_tok[min(mb + 32 * b, M - 1)];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(sc[a][q][i]));
#pragma unroll
    for (int b = 0; b < 4; ++b) asm volatile("" : "+v"(st[b]));
  }
  wait_counts<0, 0>();  // every wave is done reading the ring
  bare_barrier();
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int row = wm * 128 + 32 * b + j;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * 64 + 32 * a + 8 * q + 4 * h;
        lds_i8* const dst = sm + row * kPitch + col * static_cast<int>(sizeof(OutT));
        if constexpr (kScaled) {
          uint32_t hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = (static_cast<float>(acc[a][b][4 * q + i]) * st[b]) * sc[a][q][i];
            hv[i] = __builtin_bit_cast(uint16_t, static_cast<f16>(v));
          }
          *(lds_u32x2*)(dst) = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
        } else {
          *(lds_i32x4*)(dst) = i32x4{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                                     acc[a][b][4 * q + 3]};
        }
      }
  }
  wait_counts<0, 0>();
  bare_barrier();

  constexpr int kPerChunk = 16 / static_cast<int>(sizeof(OutT));  // outputs per 16-byte piece
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kRowsPerPass = 256 / kChunksPerRow;
  OutT* const out = kScaled ? reinterpret_cast<OutT*>(y) : reinterpret_cast<OutT*>(acc_out);
  const int c = threadIdx.x % kChunksPerRow;
  const int n = n0 + c * kPerChunk;
  const bool whole = (N % kPerChunk) == 0;  // rows start 16-byte aligned; a piece is all in or all out
#pragma unroll 4
  for (int r = threadIdx.x / kChunksPerRow; r < kBM; r += kRowsPerPass) {
    const int m = m0 + r;
    if (m >= M || n >= N) continue;
    const u32x4 v = *(const lds_u32x4*)(sm + r * kPitch + c * 16);
    OutT* const o = out + static_cast<size_t>(m) * N + n;
    if (whole) {
      *reinterpret_cast<u32x4*>(o) = v;
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
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int per_xcd = static_cast<int>((tiles + 7) / 8);
  const dim3 grid(static_cast<uint32_t>(8 * per_xcd)), block(256);
  if (y != nullptr)
    return launch_kernel(w8a8_gemm_kernel<true>, grid, block, 0, stream, xq, s_tok, wq, s_ch, y,
                         static_cast<int32_t*>(nullptr), m, n, k, tiles_m, tiles_n, per_xcd);
  return launch_kernel(w8a8_gemm_kernel<false>, grid, block, 0, stream, xq, s_tok, wq, s_ch,
                       static_cast<uint16_t*>(nullptr), acc, m, n, k, tiles_m, tiles_n, per_xcd);
}

}  // namespace mq
