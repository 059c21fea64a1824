// W8A8 int8 GEMM with int32 accumulation and a per-token x per-channel
// scale epilogue, for gfx950.
//
// Source: pymllm Setup and Usage, Overview (int8 activations and weights on
// INT8 matrix units) and section "W8A8 first-run JIT compilation" (int8
// scaled matmul). acc[m,n] = sum_k xq[m,k] * wq[n,k] (exact int32);
// y[m,n] = fp16(fl32(fl32(acc) * s_tok[m]) * s_ch[n]).
//
// Both operands are K-contiguous ([M,K] and [N,K]), which is the layout the
// int8 MFMA wants for A and B alike: lane (r = lane%16, h = lane/16) of
// v_mfma_i32_16x16x64_i8 supplies 16 consecutive k of row r. A workgroup of
// four wavefronts computes a 128x128 tile; each wavefront owns 64x64 (4x4
// MFMA tiles, int32 accumulators in registers). K advances 64 at a time
// through double-buffered LDS tiles padded to an 80-byte row pitch so that
// the 16-byte fragment reads of 16 consecutive rows hit distinct banks.
#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 16;  // LDS row pitch in bytes

template <bool kScaled>
__global__ __launch_bounds__(256) void w8a8_gemm_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ s_tok,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ s_ch,
                                                        uint16_t* __restrict__ y,
                                                        int32_t* __restrict__ acc_out,
                                                        int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = static_cast<int>(blockIdx.x / tiles_n) * BM;
  const int n0 = static_cast<int>(blockIdx.x % tiles_n) * BN;

  // Global -> LDS mapping: a tile is 128 rows x 4 chunks of 16 bytes; thread
  // t moves chunks t and t + 256.
  int ld_row[2], ld_chk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    ld_row[i] = idx >> 2;
    ld_chk[i] = idx & 3;
  }
  u32x4 ra[2], rb[2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = kt * BK + ld_chk[i] * 16;
      const int am = m0 + ld_row[i], bn = n0 + ld_row[i];
      ra[i] = (am < M && k < K) ? *reinterpret_cast<const u32x4*>(xq + static_cast<size_t>(am) * K + k)
                                : u32x4{0u, 0u, 0u, 0u};
      rb[i] = (bn < N && k < K) ? *reinterpret_cast<const u32x4*>(wq + static_cast<size_t>(bn) * K + k)
                                : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][ld_row[i] * LDK + ld_chk[i] * 16]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][ld_row[i] * LDK + ld_chk[i] * 16]) = rb[i];
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  const int nkt = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 16;
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    i32x4 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = *reinterpret_cast<const i32x4*>(&As[cur][(wm * 64 + t * 16 + frag_row) * LDK + frag_k]);
      b[t] = *reinterpret_cast<const i32x4*>(&Bs[cur][(wn * 64 + t * 16 + frag_row) * LDK + frag_k]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nkt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Accumulator layout of a 16x16 tile: lane (j = lane%16, h = lane/16),
  // register r holds row 4h + r, column j.
  const int col_in = lane & 15;
  const int row_in = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + col_in;
    if (n >= N) continue;
    float sc = 0.f;
    if constexpr (kScaled) sc = s_ch[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + row_in + r;
        if (m >= M) continue;
        if constexpr (kScaled) {
          const float v = (static_cast<float>(acc[i][j][r]) * s_tok[m]) * sc;
          y[static_cast<size_t>(m) * N + n] = __builtin_bit_cast(uint16_t, static_cast<f16>(v));
        } else {
          acc_out[static_cast<size_t>(m) * N + n] = acc[i][j][r];
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
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid(static_cast<uint32_t>(tiles)), block(256);
  if (y != nullptr)
    return launch_kernel(w8a8_gemm_kernel<true>, grid, block, 0, stream, xq, s_tok, wq, s_ch, y,
                         static_cast<int32_t*>(nullptr), m, n, k);
  return launch_kernel(w8a8_gemm_kernel<false>, grid, block, 0, stream, xq, s_tok, wq, s_ch,
                       static_cast<uint16_t*>(nullptr), acc, m, n, k);
}

}  // namespace mq
