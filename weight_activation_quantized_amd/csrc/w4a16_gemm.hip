// W4A16 GEMM for prefill-shaped M on gfx950.
//
// Source: LMDeploy toolkit overview, section 2.5 (AWQ 4-bit weights, group
// size 128) and LMDeploy 4-bit deployment guide, sections 2.2-2.3 (scales
// and weights consumed inside the matmul kernel; a real low-bit kernel rather
// than fake quantization). y[m,n] = sum_k x[m,k] * fp16((q - z) * s).
//
// Design: a workgroup of four wavefronts (2 x 2) computes a 128 x 256 tile
// with v_mfma_f32_16x16x32_f16 and fp32 accumulators; a wavefront owns 64 x
// 128 (4 token tiles x 8 field tiles). Activation tiles (128 x 32 fp16) go
// through double-buffered LDS. Each wavefront reads its own packed weights
// straight from global memory (word j of rows 8h..8h+7 per lane, prefetched
// one step ahead) and unpacks them in registers into fp16 B fragments of
// (q - z) * s, so no dequantized weight ever touches memory.
#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"

namespace mq {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int LDA = BK + 8;  // LDS row pitch in fp16 elements (80 bytes)

struct GroupParams {
  uint32_t negz[8];
  uint32_t sc2[8];
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
                                                         uint16_t* __restrict__ y, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = static_cast<int>(blockIdx.x / tiles_n) * BM;
  const int n0 = static_cast<int>(blockIdx.x % tiles_n) * BN;
  const int NP = N >> 3;
  const int j = lane & 15;
  const int h = lane >> 4;
  const int c = (n0 >> 3) + wn * 16 + j;
  const bool cvalid = c < NP;
  const uint32_t* wcol = qw + static_cast<size_t>(8 * h) * NP + (cvalid ? c : 0);

  // Activation tile: 128 rows x 4 chunks of 8 fp16; thread t moves chunks t, t + 256.
  int ld_row[2], ld_chk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    ld_row[i] = idx >> 2;
    ld_chk[i] = idx & 3;
  }
  u32x4 ra[2];
  auto load_a = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mrow = m0 + ld_row[i];
      ra[i] = mrow < M ? *reinterpret_cast<const u32x4*>(x + static_cast<size_t>(mrow) * K + ks * BK +
                                                          ld_chk[i] * 8)
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][ld_row[i] * LDA + ld_chk[i] * 8]) = ra[i];
  };
  uint32_t wcur[8], wnext[8];
  auto load_w = [&](int ks, uint32_t (&w)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = cvalid ? wcol[static_cast<size_t>(ks * BK + e) * NP] : 0u;
  };
  uint32_t zw_next = 0u;
  u32x4 sv_next = u32x4{0u, 0u, 0u, 0u};
  auto load_group = [&](int g) {
    if (cvalid) {
      zw_next = qz[static_cast<size_t>(g) * NP + c];
      sv_next = *reinterpret_cast<const u32x4*>(scales + static_cast<size_t>(g) * N + 8 * c);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int p = 0; p < 8; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / BK;
  constexpr int kStepsPerGroup = kGroup / BK;
  load_a(0);
  load_w(0, wcur);
  load_group(0);
  store_a(0);
  GroupParams gp;
  make_group_params(zw_next, sv_next, gp);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 8;
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    const bool new_group = more && ((ks + 1) % kStepsPerGroup == 0);
    if (more) {
      load_a(ks + 1);
      load_w(ks + 1, wnext);
      if (new_group) load_group((ks + 1) / kStepsPerGroup);
    }
    f16x8 b[8];
    unpack_step_scaled(wcur, gp.negz, gp.sc2, b);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(&As[cur][(wm * 64 + t * 16 + frag_row) * LDA + frag_k]);
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[t][p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[p], acc[t][p], 0, 0, 0);
    }
    if (more) {
      store_a(cur ^ 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) wcur[e] = wnext[e];
      if (new_group) make_group_params(zw_next, sv_next, gp);
    }
    __syncthreads();
  }

  if (!cvalid) return;
  // Accumulator layout: lane (j, h), register r -> row 4h + r of the token
  // tile, column j; field tile p covers output 8c + p, so the lane writes
  // 8 consecutive outputs per row.
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + t * 16 + 4 * h + r;
      if (m >= M) continue;
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x2 pr;
        pr[0] = static_cast<f16>(acc[t][2 * q][r]);
        pr[1] = static_cast<f16>(acc[t][2 * q + 1][r]);
        out[q] = as_u32(pr);
      }
      *reinterpret_cast<u32x4*>(y + static_cast<size_t>(m) * N + 8 * c) = out;
    }
  }
}

}  // namespace

hipError_t launch_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch_kernel(w4a16_gemm_kernel, dim3(static_cast<uint32_t>(tiles)), dim3(256), 0, stream, x,
                       reinterpret_cast<const uint32_t*>(qweight), scales,
                       reinterpret_cast<const uint32_t*>(qzeros), y, static_cast<int>(M),
                       static_cast<int>(N), static_cast<int>(K));
}

}  // namespace mq
