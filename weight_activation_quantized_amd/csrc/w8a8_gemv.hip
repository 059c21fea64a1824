// W8A8 int8 GEMM for decode-shaped M (M <= 64) on gfx950.
//
// Source: pymllm Setup and Usage, Overview (int8 activations and weights on
// INT8 matrix units) and section "W8A8 first-run JIT compilation" (int8
// scaled matmul). acc[m,n] = sum_k xq[m,k] * wq[n,k] (exact int32);
// y[m,n] = fp16(fl32(fl32(acc) * s_tok[m]) * s_ch[n]).
//
// With few tokens the layer is bound by the weight stream (N*K bytes), so
// this kernel reads every weight byte once with as many bytes in flight as
// possible:
// - A workgroup owns 16 (or, for more tokens and large N, 32) output
//   channels; its four wavefronts split K into four contiguous quarters, so
//   each wavefront streams 16 or 32 weight rows of K/4 contiguous bytes. The int32 partial sums of the four quarters are
//   added in LDS (integer addition: exact, order-free).
// - v_mfma_i32_16x16x64_i8 with the weight rows as the A operand (lane
//   (i = lane%16, h = lane/16) takes 16 consecutive k of row i, one 16-byte
//   load) and up to four 16-token tiles of xq as B operands. Every
//   workgroup reads all of xq (from L2); past 16 tokens these re-reads,
//   not HBM, limit the kernel.
// - Two register sets of k-steps alternate: the loads of one are issued
//   before the MFMAs of the other, so about 4-8 KB of weights per
//   wavefront stay in flight. Buffer loads past a descriptor's
//   size return zero (rows past N, tokens past M); k-chunks past the
//   wavefront's quarter are sent past the end too.
#include "device_common.h"
#include "launch.h"

namespace mq {
namespace {

constexpr int kQuarters = 4;              // wavefronts, one K quarter each
constexpr uint32_t kOob = 0x80000000u;    // a buffer offset past every tile: the load returns 0
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3 (raw 32-bit data)

// 64-byte k-steps per register set: two sets alternate, so one set's loads
// are in flight while the other's MFMAs run. With kLoads 16-byte loads per
// lane and k-step, about 16 loads per set keeps both sets in the register
// file (140-150 VGPRs).
template <int kLoads>
constexpr int steps_per_set() {
  return 16 / kLoads < 2 ? 2 : (16 / kLoads > 8 ? 8 : 16 / kLoads);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n), kBufferFlags);
}

// One register set: kU k-steps of kA 16-byte weight chunks (one per 16
// channels) and kT 16-byte activation chunks (one per 16 tokens) per lane.
template <int kU, int kA, int kT>
struct Frags {
  i32x4 w[kU][kA];
  i32x4 x[kU][kT];
};

// The wavefront's K range [k_begin, k_end) in 64-byte steps j = 0 .. n64-1;
// lane group h takes bytes 16 h .. 16 h + 15 of a step. Steps at or past
// n64, and the lanes of a ragged last step that fall past k_end, load zeros.
struct Walk {
  int k_begin, k_end, n64;
  __device__ __forceinline__ int chunk(int j, int h) const {
    const int kc = k_begin + 64 * j + 16 * h;
    return (j < n64 && kc < k_end) ? kc : -1;
  }
};

template <int kU, int kA, int kT>
__device__ __forceinline__ void issue(Frags<kU, kA, kT>& f, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                      int i, int h, int K, const Walk& wk, int j0) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int kc = wk.chunk(j0 + u, h);
#pragma unroll
    for (int a = 0; a < kA; ++a)
      f.w[u][a] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kc >= 0 ? static_cast<uint32_t>((16 * a + i) * K + kc) : kOob, 0, 0));
#pragma unroll
    for (int t = 0; t < kT; ++t)
      f.x[u][t] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, kc >= 0 ? static_cast<uint32_t>((16 * t + i) * K + kc) : kOob, 0, 0));
  }
}

template <int kU, int kA, int kT>
__device__ __forceinline__ void mfmas(const Frags<kU, kA, kT>& f, i32x4 (&acc)[kA][kT]) {
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int a = 0; a < kA; ++a)
#pragma unroll
      for (int t = 0; t < kT; ++t)
        acc[a][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[u][a], f.x[u][t], acc[a][t], 0, 0, 0);
}

// A workgroup owns 16 kA output channels and all M <= 16 kT tokens.
template <bool kScaled, int kA, int kT, bool kBf16>
__global__ __launch_bounds__(256) void w8a8_gemv_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ s_tok,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ s_ch,
                                                        uint16_t* __restrict__ y,
                                                        int32_t* __restrict__ acc_out, int M, int N, int K) {
  constexpr int kCh = 16 * kA;
  __shared__ int32_t part[kQuarters][kCh][16 * kT];

  const int n0 = static_cast<int>(blockIdx.x) * kCh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, h = lane >> 4;

  // This wavefront's K quarter, in whole 64-byte steps.
  Walk wk;
  const int kq = (K / kQuarters + 63) / 64 * 64;
  wk.k_begin = wave * kq;
  wk.k_end = min(K, wk.k_begin + kq);
  wk.n64 = (wk.k_end - wk.k_begin + 63) / 64;  // <= 0 when the quarter is empty

  // Weights: rows n0 .. n0 + kCh - 1 (rows past N read zero).
  const __amdgpu_buffer_rsrc_t rw = rsrc(wq + static_cast<size_t>(n0) * K, static_cast<int64_t>(min(kCh, N - n0)) * K);
  const __amdgpu_buffer_rsrc_t rx = rsrc(xq, static_cast<int64_t>(M) * K);

  i32x4 acc[kA][kT];
#pragma unroll
  for (int a = 0; a < kA; ++a)
#pragma unroll
    for (int t = 0; t < kT; ++t) acc[a][t] = i32x4{0, 0, 0, 0};

  constexpr int kU = steps_per_set<kA + kT>();
  const int sets = (wk.n64 + kU - 1) / kU;
  Frags<kU, kA, kT> fa, fb;
  issue(fa, rw, rx, i, h, K, wk, 0);
  // No early exit between the halves: a branch there lets the compiler sink
  // the loads of the second set below the first set's MFMAs. A set past the
  // end loads zeros.
  for (int s = 0; s < sets; s += 2) {
    issue(fb, rw, rx, i, h, K, wk, (s + 1) * kU);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa, acc);
    __builtin_amdgcn_sched_barrier(0);
    issue(fa, rw, rx, i, h, K, wk, (s + 2) * kU);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fb, acc);
    __builtin_amdgcn_sched_barrier(0);
  }

  // D[n][m] of a 16x16 tile: lane (j, hh) register r holds channel 4 hh + r
  // of token j.
#pragma unroll
  for (int a = 0; a < kA; ++a)
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][16 * a + 4 * h + r][16 * t + i] = acc[a][t][r];
  __syncthreads();

  for (int e = threadIdx.x; e < kCh * 16 * kT; e += blockDim.x) {
    const int nl = e % kCh, m = e / kCh;
    const int n = n0 + nl;
    if (m >= M || n >= N) continue;
    const int32_t v = part[0][nl][m] + part[1][nl][m] + part[2][nl][m] + part[3][nl][m];
    const size_t o = static_cast<size_t>(m) * N + n;
    if constexpr (kScaled) {
      const float f = (static_cast<float>(v) * s_tok[m]) * s_ch[n];
      y[o] = half_bits<kBf16>(f);
    } else {
      acc_out[o] = v;
    }
  }
}

// Workgroups of the capped-grid kernels below: a grid of at most this many
// walks the 16-channel tiles (measured, 24576 x 4096: one token 28.5 us
// with a workgroup per tile, 23.6 us with 1024).
constexpr int64_t kFusedGridCap = 1024;

// Up to 16 tokens with codes already formed, where they fit LDS: a
// workgroup moves the M rows of xq into LDS by DMA once (right behind its
// first weight set) and a capped grid walks the 16-channel tiles, so the
// codes are read from L2 once per workgroup rather than at every k-step of
// every tile. Otherwise as w8a8_gemv_kernel (same sums, same epilogue).
template <bool kScaled, bool kBf16>
__global__ __launch_bounds__(256) void w8a8_gemv_staged_kernel(const int8_t* __restrict__ xq,
                                                               const float* __restrict__ s_tok,
                                                               const int8_t* __restrict__ wq,
                                                               const float* __restrict__ s_ch,
                                                               uint16_t* __restrict__ y,
                                                               int32_t* __restrict__ acc_out, int M, int N, int K) {
  __shared__ int32_t part[kQuarters][16][16];
  extern __shared__ __attribute__((aligned(16))) int8_t codes[];  // M * (K + 16) bytes (launch)
  const int pitch = K + 16;  // token rows of codes fall on different bank groups

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, h = lane >> 4;
  const int tiles = (N + 15) / 16;

  Walk wk;
  const int kq = (K / kQuarters + 63) / 64 * 64;
  wk.k_begin = wave * kq;
  wk.k_end = min(K, wk.k_begin + kq);
  wk.n64 = (wk.k_end - wk.k_begin + 63) / 64;
  constexpr int kU = 8;
  const int sets = (wk.n64 + kU - 1) / kU;

  int tile = static_cast<int>(blockIdx.x);  // < tiles: the grid is at most the tile count
  __amdgpu_buffer_rsrc_t rw;
  auto set_tile = [&](int t) {
    rw = rsrc(wq + static_cast<size_t>(t) * 16 * K, static_cast<int64_t>(min(16, N - 16 * t)) * K);
  };
  i32x4 wa[kU], wb[kU];
  i32x4 acc;
  auto issue_w = [&](i32x4 (&w)[kU], int j0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kc = wk.chunk(j0 + u, h);
      w[u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kc >= 0 ? static_cast<uint32_t>(i * K + kc) : kOob, 0, 0));
    }
  };
  auto mma = [&](const i32x4 (&w)[kU], int j0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kc = wk.chunk(j0 + u, h);
      i32x4 b = i32x4{0, 0, 0, 0};
      if (i < M && kc >= 0) b = *reinterpret_cast<const i32x4*>(&codes[i * pitch + kc]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], b, acc, 0, 0, 0);
    }
  };

  set_tile(tile);
  issue_w(wa, 0);
  __builtin_amdgcn_sched_barrier(0);
  {
    // 1 KB per load: row m, bytes 1024 v .. (K % 1024 == 0, host)
    const __amdgpu_buffer_rsrc_t rx = rsrc(xq, static_cast<int64_t>(M) * K);
    const int per = K / 1024;
    for (int q = wave; q < M * per; q += kQuarters) {
      const int m = q / per, v = q % per;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(codes + m * pitch + 1024 * v), 16,
                                               static_cast<uint32_t>(m * K + 1024 * v + 16 * lane), 0, 0, 0);
    }
  }
  wait_counts<0, 15>();  // the codes (and the first weight set, needed next anyway)
  __syncthreads();

  for (;;) {
    const int n0 = tile * 16;
    acc = i32x4{0, 0, 0, 0};
    for (int st = 0; st < sets; st += 2) {
      issue_w(wb, (st + 1) * kU);
      __builtin_amdgcn_sched_barrier(0);
      mma(wa, st * kU);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(wa, (st + 2) * kU);
      __builtin_amdgcn_sched_barrier(0);
      mma(wb, (st + 1) * kU);
      __builtin_amdgcn_sched_barrier(0);
    }
    // D[n][m]: lane (j, hh) register r holds channel 4 hh + r of token j.
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * h + r][i] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * M; e += 256) {
      const int nl = e % 16, m = e / 16, n = n0 + nl;
      if (n >= N) continue;
      const int32_t v = part[0][nl][m] + part[1][nl][m] + part[2][nl][m] + part[3][nl][m];
      const size_t o = static_cast<size_t>(m) * N + n;
      if constexpr (kScaled) {
        const float f = (static_cast<float>(v) * s_tok[m]) * s_ch[n];
        y[o] = half_bits<kBf16>(f);
      } else {
        acc_out[o] = v;
      }
    }
    __syncthreads();  // the next tile rewrites part
    tile += static_cast<int>(gridDim.x);
    if (tile >= tiles) break;
    set_tile(tile);
    issue_w(wa, 0);
  }
}

// Staged codes: M rows of K + 16 bytes within this much LDS (two or more
// workgroups per CU; 16 tokens at K = 4096 take 66 KB: gate_up 32.5 ->
// 27.7 us against the L2 reads of the codes at every k-step).
constexpr int64_t kStagedLds = 80 * 1024;

// ---------------------------------------------------------------------------
// Fused decode layer for one to four tokens: per-token quantization folded
// into the weight-streaming kernel (pymllm Setup and Usage, "W8A8 first-run
// JIT compilation": the quantizer feeds the scaled matmul). Every workgroup
// forms s[m] = fl32(absmax(x[m,:]) / 127) for the M rows (x is small and
// L2-resident at these M) and the codes q = clamp(rne(fl32(x / s)), -127,
// 127) with the IEEE binary32 quotient, s = 0 giving q = 0. Codes, scales,
// accumulators and outputs are therefore bit-identical to
// mq_quant_per_token_int8 followed by mq_w8a8_scaled_mm.
// ---------------------------------------------------------------------------

// Codes of the IEEE binary32 quotient v / s rounded half to even, for s > 0:
// the product with r = rcp(s) decides every element farther than 2^-12 from
// a half-integer (its error is below 3.1e-5 for quotients up to 127.5, the
// correctly rounded quotient's below 3.9e-6), the IEEE division the rest.
__device__ __forceinline__ float fused_code(float v, float s, float r) {
  const float p = v * r;
  const float t = rintf(p);
  if (!(0.5f - fabsf(p - t) >= 1.0f / 4096.0f)) return rintf(v / s);  // non-finite p: divide
  return t;
}

// Up to four tokens (kM rows, M rounded up to 1, 2 or 4) and the 16-channel
// tiles blockIdx.x, blockIdx.x + gridDim.x, ... per workgroup. The token
// rows of x are loaded into registers (kXR 16-byte chunks per thread and
// row: K <= 2048 kXR) and the first tile's first weight set is requested
// right behind them, so the weight stream starts while the workgroup forms
// the scales (maxima over the workgroup) and the codes (into LDS) from
// those registers (8B layers at one token, against a prologue that read x
// twice before the first weight request and two kernels for the narrow
// layers: gate_up 23.1 -> 20.1 us, qkv 11.7 -> 8.2, o_proj 8.7 -> 6.2, down
// 15.2 -> 13.5; at two tokens against two kernels: gate_up 25.2 -> 19.7,
// qkv 11.6 -> 8.8, o_proj 8.6 -> 7.1). Per tile: as
// w8a8_gemv_kernel, with the B fragments read from LDS. The grid is capped,
// so a wide layer's workgroups walk several tiles and form the codes once
// for all of them.
constexpr int kFusedMaxXR = 6;

template <int kM, int kXR, bool kBf16>
__global__ __launch_bounds__(256) void w8a8_gemv_fused_kernel(const uint16_t* __restrict__ x,
                                                              const int8_t* __restrict__ wq,
                                                              const float* __restrict__ s_ch,
                                                              uint16_t* __restrict__ y, int M, int N, int K) {
  __shared__ int32_t part[kQuarters][16][16];
  __shared__ float s_wave[kQuarters][kM];
  extern __shared__ __attribute__((aligned(16))) int8_t codes[];  // kM * (K + 16) bytes (launch)
  const int pitch = K + 16;  // token rows of codes fall on different bank groups

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, h = lane >> 4;
  const int tiles = (N + 15) / 16;

  Walk wk;
  const int kq = (K / kQuarters + 63) / 64 * 64;
  wk.k_begin = wave * kq;
  wk.k_end = min(K, wk.k_begin + kq);
  wk.n64 = (wk.k_end - wk.k_begin + 63) / 64;
  constexpr int kU = 8;
  const int sets = (wk.n64 + kU - 1) / kU;

  int tile = static_cast<int>(blockIdx.x);  // < tiles: the grid is at most the tile count
  __amdgpu_buffer_rsrc_t rw;
  auto set_tile = [&](int t) {
    rw = rsrc(wq + static_cast<size_t>(t) * 16 * K, static_cast<int64_t>(min(16, N - 16 * t)) * K);
  };
  i32x4 wa[kU], wb[kU];
  i32x4 acc;
  auto issue_w = [&](i32x4 (&w)[kU], int j0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kc = wk.chunk(j0 + u, h);
      w[u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kc >= 0 ? static_cast<uint32_t>(i * K + kc) : kOob, 0, 0));
    }
  };
  auto mma = [&](const i32x4 (&w)[kU], int j0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kc = wk.chunk(j0 + u, h);
      i32x4 b = i32x4{0, 0, 0, 0};
      if (i < kM && kc >= 0) b = *reinterpret_cast<const i32x4*>(&codes[i * pitch + kc]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], b, acc, 0, 0, 0);
    }
  };

  // The token rows in registers (rows M .. kM - 1 are zero: scale 0, codes
  // 0, never stored), then the first tile's first weight set.
  const int nc = K / 8;
  u32x4 xv[kM][kXR];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const u32x4* const row = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(m < M ? m : 0) * K);
#pragma unroll
    for (int r = 0; r < kXR; ++r) {
      const int c = threadIdx.x + 256 * r;
      xv[m][r] = (m < M && c < nc) ? row[c] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  set_tile(tile);
  issue_w(wa, 0);
  __builtin_amdgcn_sched_barrier(0);
  // s = fl32(absmax(x) / 127) per row (max is exact and order-free), then
  // the codes
  float sm[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < kXR; ++r)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float lo, hi;
        word_to_floats<kBf16>(xv[m][r][w], lo, hi);
        amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
      }
    amax = wave_max(amax);
    if (lane == 0) s_wave[wave][m] = amax;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    sm[m] = fmaxf(fmaxf(s_wave[0][m], s_wave[1][m]), fmaxf(s_wave[2][m], s_wave[3][m])) / 127.0f;  // IEEE division
    // a binary32-subnormal scale: infinite reciprocal, so fused_code divides
    const float rc = sm[m] < 1.17549435e-38f ? __builtin_inff() : __builtin_amdgcn_rcpf(sm[m]);
#pragma unroll
    for (int r = 0; r < kXR; ++r) {
      const int c = threadIdx.x + 256 * r;
      if (c >= nc) continue;
      uint32_t packed[2] = {0u, 0u};
      if (sm[m] > 0.f) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float lo, hi;
          word_to_floats<kBf16>(xv[m][r][w], lo, hi);
          const float q0 = fminf(fmaxf(fused_code(lo, sm[m], rc), -127.f), 127.f);
          const float q1 = fminf(fmaxf(fused_code(hi, sm[m], rc), -127.f), 127.f);
          const uint32_t b = (static_cast<uint32_t>(static_cast<int32_t>(q0)) & 0xFFu) |
                             ((static_cast<uint32_t>(static_cast<int32_t>(q1)) & 0xFFu) << 8);
          packed[w >> 1] |= b << (16 * (w & 1));
        }
      }
      *reinterpret_cast<u32x2*>(&codes[m * pitch + 8 * c]) = u32x2{packed[0], packed[1]};
    }
  }
  __syncthreads();

  for (;;) {
    const int n0 = tile * 16;
    acc = i32x4{0, 0, 0, 0};
    for (int st = 0; st < sets; st += 2) {
      issue_w(wb, (st + 1) * kU);
      __builtin_amdgcn_sched_barrier(0);
      mma(wa, st * kU);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(wa, (st + 2) * kU);
      __builtin_amdgcn_sched_barrier(0);
      mma(wb, (st + 1) * kU);
      __builtin_amdgcn_sched_barrier(0);
    }

    // D[n][m]: lane (j, hh) register r holds channel 4 hh + r of token j.
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * h + r][i] = acc[r];
    __syncthreads();
    if (threadIdx.x < 16 * kM) {
      const int nl = threadIdx.x % 16, m = threadIdx.x / 16, n = n0 + nl;
      if (m < M && n < N) {
        const int32_t v = part[0][nl][m] + part[1][nl][m] + part[2][nl][m] + part[3][nl][m];
        const float f = (static_cast<float>(v) * sm[m]) * s_ch[n];
        y[static_cast<size_t>(m) * N + n] = half_bits<kBf16>(f);
      }
    }
    __syncthreads();  // the next tile rewrites part
    tile += static_cast<int>(gridDim.x);
    if (tile >= tiles) break;
    set_tile(tile);
    issue_w(wa, 0);
  }
}

template <bool kScaled, int kA, int kT, bool kBf16>
hipError_t launch_one(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch, uint16_t* y,
                      int32_t* acc, int M, int N, int K, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((N + 16 * kA - 1) / (16 * kA))), block(256);
  return launch_kernel(w8a8_gemv_kernel<kScaled, kA, kT, kBf16>, grid, block, 0, stream, xq, s_tok, wq, s_ch, y, acc,
                       M, N, K);
}

template <bool kScaled, bool kBf16>
hipError_t launch_tiles(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch, uint16_t* y,
                        int32_t* acc, int M, int N, int K, hipStream_t stream) {
  // Every workgroup reads all of xq, so xq is read N / (16 kA) times over
  // (from L2): 32 channels per workgroup halves that, but only pays while
  // the grid still has about 192 or more workgroups.
  const bool wide = N >= 32 * 192;
  // Staged codes where they measured faster (8B layers at 3-16 tokens): on
  // layers of 6144+ channels (gate_up at 8 tokens 27.6 -> 24.3 us, qkv
  // 12.8 -> 12.2); on 4096-channel layers 0.4-0.5 us slower.
  if (M <= 16 && N >= 6144 && K % 1024 == 0 && static_cast<int64_t>(M) * (K + 16) <= kStagedLds) {
    const int64_t tiles = (N + 15) / 16;
    const dim3 grid(static_cast<uint32_t>(tiles < kFusedGridCap ? tiles : kFusedGridCap)), block(256);
    return launch_kernel(w8a8_gemv_staged_kernel<kScaled, kBf16>, grid, block, static_cast<size_t>(M) * (K + 16),
                         stream, xq, s_tok, wq, s_ch, y, acc, M, N, K);
  }
  if (M <= 16) return launch_one<kScaled, 1, 1, kBf16>(xq, s_tok, wq, s_ch, y, acc, M, N, K, stream);
  if (M <= 32)
    return wide ? launch_one<kScaled, 2, 2, kBf16>(xq, s_tok, wq, s_ch, y, acc, M, N, K, stream)
                : launch_one<kScaled, 1, 2, kBf16>(xq, s_tok, wq, s_ch, y, acc, M, N, K, stream);
  return wide ? launch_one<kScaled, 2, 4, kBf16>(xq, s_tok, wq, s_ch, y, acc, M, N, K, stream)
              : launch_one<kScaled, 1, 4, kBf16>(xq, s_tok, wq, s_ch, y, acc, M, N, K, stream);
}

}  // namespace

bool w8a8_use_gemv(int64_t M, int64_t N) {
  // Measured crossover against the tiled GEMM: up to 32 tokens always; 33-64
  // tokens unless N is so large that the GEMM's 128-channel tiles already
  // fill the chip and its smaller activation re-read wins.
  if (M <= 32) return true;
  return M <= kW8A8GemvMaxM && N < 16384;
}

bool w8a8_use_fused(int64_t M, int64_t N, int64_t K) {
  // Where the fused form measured faster than the quantizer and the decode
  // kernel (8B layers at 1-4 tokens): one or two tokens on every layer whose
  // rows fit the registers; three or four only on layers of 6144 or more
  // channels (o_proj, 4096, at four tokens 8.9 -> 9.3 us fused).
  return N >= 1 && ((M == 1 && K <= 256 * 8 * kFusedMaxXR) || (M == 2 && K <= 256 * 8 * 4) ||
                    (M >= 3 && M <= 4 && K <= 256 * 8 * 2 && N >= 6144));
}

hipError_t launch_w8a8_gemv_fused(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y,
                                  int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream) {
  if (!w8a8_use_fused(M, N, K)) return hipErrorInvalidValue;
  const int64_t tiles = (N + 15) / 16;
  const int64_t cap = kFusedGridCap;
  const dim3 grid(static_cast<uint32_t>(tiles < cap ? tiles : cap)), block(256);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  // kM token rows (M rounded up to 1, 2 or 4) of 2, 4 or 6 16-byte chunks
  // per thread in registers, their codes in LDS
  auto go = [&](auto kernel, int kM) {
    return launch_kernel(kernel, grid, block, static_cast<size_t>(kM) * (K + 16), stream, x, wq, s_ch, y, m, n, k);
  };
  if (M > 2)  // 3 or 4 tokens, K <= 4096
    return bf16 ? go(w8a8_gemv_fused_kernel<4, 2, true>, 4) : go(w8a8_gemv_fused_kernel<4, 2, false>, 4);
  if (M == 2) {
    if (K <= 2048 * 2)
      return bf16 ? go(w8a8_gemv_fused_kernel<2, 2, true>, 2) : go(w8a8_gemv_fused_kernel<2, 2, false>, 2);
    return bf16 ? go(w8a8_gemv_fused_kernel<2, 4, true>, 2) : go(w8a8_gemv_fused_kernel<2, 4, false>, 2);
  }
  if (K <= 2048 * 2)
    return bf16 ? go(w8a8_gemv_fused_kernel<1, 2, true>, 1) : go(w8a8_gemv_fused_kernel<1, 2, false>, 1);
  if (K <= 2048 * 4)
    return bf16 ? go(w8a8_gemv_fused_kernel<1, 4, true>, 1) : go(w8a8_gemv_fused_kernel<1, 4, false>, 1);
  return bf16 ? go(w8a8_gemv_fused_kernel<1, kFusedMaxXR, true>, 1)
              : go(w8a8_gemv_fused_kernel<1, kFusedMaxXR, false>, 1);
}

hipError_t launch_w8a8_gemv(const int8_t* xq, const float* s_tok, const int8_t* wq,
                            const float* s_ch, uint16_t* y, int32_t* acc,
                            int64_t M, int64_t N, int64_t K, bool bf16, hipStream_t stream) {
  if (M > kW8A8GemvMaxM) return hipErrorInvalidValue;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  if (y != nullptr && bf16) return launch_tiles<true, true>(xq, s_tok, wq, s_ch, y, nullptr, m, n, k, stream);
  if (y != nullptr) return launch_tiles<true, false>(xq, s_tok, wq, s_ch, y, nullptr, m, n, k, stream);
  return launch_tiles<false, false>(xq, nullptr, wq, nullptr, nullptr, acc, m, n, k, stream);
}

}  // namespace mq
