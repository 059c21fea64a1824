// W4A16 GEMV for decode (M <= 16) on gfx950.
//
// Source: LMDeploy toolkit overview, section 2.5 (AWQ 4-bit weights, group
// size 128, 4-bit inference speedup from the smaller weight stream) and
// LMDeploy 4-bit deployment guide, section 2.2 (scale and weight consumed in
// one kernel). y[m,n] = sum_k x[m,k] * (q[k,n] - z[k/128,n]) * s[k/128,n].
//
// Decode reads every weight once and does little arithmetic per weight, so
// the kernel is bound by the HBM weight stream. Design:
//  * the M <= 16 tokens ride on the 16-row side of v_mfma_f32_16x16x32_f16
//    (rows >= M are zero), so a weight costs only its unpack on the vector
//    ALU, not M multiply-adds;
//  * a workgroup owns a strip of 16 packed columns (128 outputs); lane
//    (j = lane%16, h = lane/16) reads word j of rows 8h..8h+7 of each 32-row
//    step, so one wavefront load covers 4 rows x 64 contiguous bytes;
//  * each group's sum of x * (q - z) is formed exactly (fp16 fragments of
//    q - z, fp32 MFMA accumulation) and scaled in fp32 once per group;
//  * the wavefronts of a workgroup take interleaved groups of the
//    workgroup's K slice and are summed through LDS in a fixed order; when K
//    is also split across workgroups, fp32 partials go to the workspace and
//    a second kernel sums them in split order. Results are deterministic.
#include "device_common.h"
#include "launch.h"
#include "w4a16_common.h"

namespace mq {
namespace {

constexpr int kStrip = 16;  // packed columns per workgroup (128 outputs)

template <int NW>
__global__ __launch_bounds__(NW * 64) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qz,
    uint16_t* __restrict__ y, float* __restrict__ partial, int M, int N, int K, int splits) {
  __shared__ float red[NW > 1 ? NW - 1 : 1][32][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int h = lane >> 4;
  const int NP = N >> 3;
  const int c = blockIdx.x * kStrip + j;
  const bool cvalid = c < NP;
  const int split = blockIdx.y;
  const int G = K / kGroup;
  const int g_begin = static_cast<int>(static_cast<int64_t>(split) * G / splits);
  const int g_end = static_cast<int>(static_cast<int64_t>(split + 1) * G / splits);

  // A operand: lane (i = lane%16, h) carries token i, k-slots 8h..8h+7.
  const bool xvalid = j < M;
  const uint16_t* xrow = x + static_cast<size_t>(xvalid ? j : 0) * K + 8 * h;
  const uint32_t* wcol = qw + static_cast<size_t>(8 * h) * NP + (cvalid ? c : 0);

  float tot[8][4];
#pragma unroll
  for (int p = 0; p < 8; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) tot[p][r] = 0.f;

  for (int g = g_begin + wave; g < g_end; g += NW) {
    uint32_t zw = 0u;
    u32x4 sv = u32x4{0u, 0u, 0u, 0u};
    if (cvalid) {
      zw = qz[static_cast<size_t>(g) * NP + c];
      sv = *reinterpret_cast<const u32x4*>(scales + static_cast<size_t>(g) * N + 8 * c);
    }
    uint32_t negz[8];
    zero_bias(zw, negz);

    f32x4 acc[8];
#pragma unroll
    for (int ks = 0; ks < kGroup / 32; ++ks) {
      const int k0 = g * kGroup + ks * 32;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = cvalid ? wcol[static_cast<size_t>(k0 + e) * NP] : 0u;
      f16x8 a;
      if (xvalid) {
        a = *reinterpret_cast<const f16x8*>(xrow + k0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = static_cast<f16>(0.f);
      }
      f16x8 b[8];
      unpack_step(w, negz, b);
#pragma unroll
      for (int p = 0; p < 8; ++p)
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[p], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[p],
                                                       0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 s2 = as_f16x2(sv[p >> 1]);
      const float sc = static_cast<float>(s2[p & 1]) * ((p & 1) ? 0.0625f : 1.0f);
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[p][r] = fmaf(acc[p][r], sc, tot[p][r]);
    }
  }

  if constexpr (NW > 1) {
    if (wave > 0) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 1][p * 4 + r][lane] = tot[p][r];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[p][r] += red[w][p * 4 + r][lane];
  }
  if (!cvalid) return;

  // Accumulator layout: lane (j, h), register r -> token 4h + r, column j of
  // the tile; tile p is field p, so the lane owns outputs 8c .. 8c+7.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * h + r;
    if (m >= M) continue;
    if (splits == 1) {
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x2 pr;
        pr[0] = static_cast<f16>(tot[2 * q][r]);
        pr[1] = static_cast<f16>(tot[2 * q + 1][r]);
        out[q] = as_u32(pr);
      }
      *reinterpret_cast<u32x4*>(y + static_cast<size_t>(m) * N + 8 * c) = out;
    } else {
      float* dst = partial + (static_cast<size_t>(split) * M + m) * N + 8 * c;
      *reinterpret_cast<f32x4*>(dst) = f32x4{tot[0][r], tot[1][r], tot[2][r], tot[3][r]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{tot[4][r], tot[5][r], tot[6][r], tot[7][r]};
    }
  }
}

// y = fp16(sum over splits of partial[split]), summed in split order; one
// thread per 8 consecutive outputs.
__global__ __launch_bounds__(256) void w4a16_gemv_reduce(const float* __restrict__ partial,
                                                         uint16_t* __restrict__ y, int M, int N,
                                                         int splits) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = static_cast<size_t>(M) * N / 8;
  if (idx >= total) return;
  const size_t off = idx * 8;
  const size_t stride = static_cast<size_t>(M) * N;
  f32x4 lo = *reinterpret_cast<const f32x4*>(partial + off);
  f32x4 hi = *reinterpret_cast<const f32x4*>(partial + off + 4);
  for (int s = 1; s < splits; ++s) {
    lo += *reinterpret_cast<const f32x4*>(partial + s * stride + off);
    hi += *reinterpret_cast<const f32x4*>(partial + s * stride + off + 4);
  }
  u32x4 out;
  f16x2 pr;
  pr[0] = static_cast<f16>(lo[0]); pr[1] = static_cast<f16>(lo[1]); out[0] = as_u32(pr);
  pr[0] = static_cast<f16>(lo[2]); pr[1] = static_cast<f16>(lo[3]); out[1] = as_u32(pr);
  pr[0] = static_cast<f16>(hi[0]); pr[1] = static_cast<f16>(hi[1]); out[2] = as_u32(pr);
  pr[0] = static_cast<f16>(hi[2]); pr[1] = static_cast<f16>(hi[3]); out[3] = as_u32(pr);
  *reinterpret_cast<u32x4*>(y + off) = out;
}

}  // namespace

GemvPlan plan_w4a16_gemv(int64_t M, int64_t N, int64_t K) {
  GemvPlan plan{1, 1, 0};
  const int64_t strips = (N / 8 + kStrip - 1) / kStrip;
  const int64_t G = K / kGroup;
  // Smallest divisor of the group count that gives at least one workgroup
  // per compute unit (256), so that no split is left with an uneven share.
  int64_t splits = 1;
#ifdef MQ_GEMV_FORCE_SPLITS
  splits = MQ_GEMV_FORCE_SPLITS;
  if (splits > G) splits = G;
  while (G % splits) --splits;
#else
  while (strips * splits < 256 && splits < G) {
    ++splits;
    while (G % splits) ++splits;
  }
#endif
  const int64_t per_split = G / splits;
  int waves = 1;
  while (waves < 4 && per_split % (2 * waves) == 0) waves *= 2;
#ifdef MQ_GEMV_FORCE_WAVES
  waves = MQ_GEMV_FORCE_WAVES;
#endif
  plan.splits = static_cast<int>(splits);
  plan.waves = waves;
  plan.workspace_bytes = splits > 1 ? static_cast<size_t>(splits) * M * N * sizeof(float) : 0;
  return plan;
}

hipError_t launch_w4a16_gemv(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, const GemvPlan& plan,
                             void* workspace, hipStream_t stream) {
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const int strips = static_cast<int>((N / 8 + kStrip - 1) / kStrip);
  const dim3 grid(strips, plan.splits);
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  float* part = static_cast<float*>(workspace);
  hipError_t err;
  switch (plan.waves) {
    case 1:
      err = launch_kernel(w4a16_gemv_kernel<1>, grid, dim3(64), 0, stream, x, qw, scales, qz, y, part, m, n, k,
                          plan.splits);
      break;
    case 2:
      err = launch_kernel(w4a16_gemv_kernel<2>, grid, dim3(128), 0, stream, x, qw, scales, qz, y, part, m, n,
                          k, plan.splits);
      break;
    case 4:
      err = launch_kernel(w4a16_gemv_kernel<4>, grid, dim3(256), 0, stream, x, qw, scales, qz, y, part, m, n,
                          k, plan.splits);
      break;
    default:
      err = launch_kernel(w4a16_gemv_kernel<8>, grid, dim3(512), 0, stream, x, qw, scales, qz, y, part, m, n,
                          k, plan.splits);
      break;
  }
  if (err != hipSuccess || plan.splits == 1) return err;
  const size_t total = static_cast<size_t>(M) * N / 8;
  const dim3 rgrid(static_cast<uint32_t>((total + 255) / 256));
  return launch_kernel(w4a16_gemv_reduce, rgrid, dim3(256), 0, stream, part, y, m, n, plan.splits);
}

}  // namespace mq
