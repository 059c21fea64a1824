// C ABI of libmq: argument validation (host only, before any HIP call),
// status strings, thread-local error detail, and dispatch to the kernels.
// The operations and their sources are documented in include/mq.h.
#include "mq.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

mq_status fail(mq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

mq_status ok() {
  g_last_error[0] = '\0';
  return MQ_OK;
}

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxK = int64_t{1} << 20;
constexpr int64_t kMaxKInt8 = 133136;            // largest multiple of 16 with 127 * 127 * K < 2^31
constexpr int64_t kMaxElems = int64_t{1} << 40;  // bound on M*N, M*K, K*N
constexpr int64_t kMaxN4 = int64_t{1} << 27;     // W4A16 N (32-bit lane offsets)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output must be disjoint from every input and from the other outputs.
template <size_t NI, size_t NO>
mq_status check_alias(const Range (&in)[NI], const Range (&out)[NO]) {
  for (size_t o = 0; o < NO; ++o) {
    for (size_t i = 0; i < NI; ++i)
      if (overlap(out[o], in[i]))
        return fail(MQ_ERR_ALIAS, "output %s overlaps input %s", out[o].name, in[i].name);
    for (size_t p = o + 1; p < NO; ++p)
      if (overlap(out[o], out[p]))
        return fail(MQ_ERR_ALIAS, "output %s overlaps output %s", out[o].name, out[p].name);
  }
  return MQ_OK;
}

mq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MQ_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// A tensor pointer may be NULL only when the tensor has no elements (an
// empty torch tensor reports a NULL data pointer).
mq_status need(const void* p, int64_t elems, const char* name) {
  if (p == nullptr && elems > 0) return fail(MQ_ERR_NULL, "%s is NULL", name);
  return MQ_OK;
}

#define MQ_TRY(expr)                  \
  do {                                \
    const mq_status st_ = (expr);     \
    if (st_ != MQ_OK) return st_;     \
  } while (0)

mq_status check_mk(int64_t M, int64_t K, int64_t k_min, int64_t k_max, int64_t k_mult) {
  if (M < 0 || M > kMaxDim) return fail(MQ_ERR_SHAPE, "M=%lld out of range", (long long)M);
  if (K < k_min || K > k_max) return fail(MQ_ERR_SHAPE, "K=%lld out of [%lld, %lld]", (long long)K,
                                          (long long)k_min, (long long)k_max);
  if (K % k_mult) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of %lld", (long long)K, (long long)k_mult);
  if (M * K > kMaxElems) return fail(MQ_ERR_SHAPE, "M*K too large");
  return MQ_OK;
}

// group -1: one scale and zero point per output column over all of K
// (per-channel); the kernels run it as groups of 128 rows that all read the
// one parameter row.
bool w4a16_group_ok(int64_t group) { return group == 32 || group == 64 || group == 128 || group == -1; }
int64_t kernel_group(int64_t group) { return group == -1 ? 128 : group; }
size_t group_rows(int64_t K, int64_t group) { return group == -1 ? 1 : static_cast<size_t>(K / group); }

mq_status check_w4a16(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                      const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t group) {
  if (!w4a16_group_ok(group))
    return fail(MQ_ERR_UNSUPPORTED, "group=%lld (32, 64, 128 and -1 = per-channel are provided)", (long long)group);
  MQ_TRY(check_mk(M, K, 128, kMaxK, 128));
  if (N < 8 || N > kMaxN4 || N % 8)
    return fail(MQ_ERR_SHAPE, "N=%lld must be a multiple of 8 in [8, 2^27]", (long long)N);
  if (M * N > kMaxElems || K * N > kMaxElems) return fail(MQ_ERR_SHAPE, "problem too large");
  MQ_TRY(need(x, M * K, "x"));
  MQ_TRY(need(qweight, K * N, "qweight"));
  MQ_TRY(need(scales, N, "scales"));
  MQ_TRY(need(qzeros, N, "qzeros"));
  MQ_TRY(need(y, M * N, "y"));
  if (!aligned(x, 16) || !aligned(scales, 16) || !aligned(y, 16))
    return fail(MQ_ERR_ALIGN, "x, scales and y must be 16-byte aligned");
  if (!aligned(qweight, 4) || !aligned(qzeros, 4))
    return fail(MQ_ERR_ALIGN, "qweight and qzeros must be 4-byte aligned");
  const size_t G = group_rows(K, group);
  const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"},
                      {qweight, static_cast<size_t>(K * (N / 8)) * 4, "qweight"},
                      {scales, G * static_cast<size_t>(N) * 2, "scales"},
                      {qzeros, G * static_cast<size_t>(N / 8) * 4, "qzeros"}};
  const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"}};
  return check_alias(in, out);
}

mq_status check_w8a8(const int8_t* xq, const int8_t* wq, const void* out, size_t out_elem,
                     int64_t M, int64_t N, int64_t K) {
  mq_status s = check_mk(M, K, 16, kMaxKInt8, 16);
  if (s != MQ_OK) return s;
  if (N < 0 || N > kMaxDim) return fail(MQ_ERR_SHAPE, "N=%lld out of range", (long long)N);
  if (M * N > kMaxElems || K * N > kMaxElems) return fail(MQ_ERR_SHAPE, "problem too large");
  MQ_TRY(need(xq, M * K, "xq"));
  MQ_TRY(need(wq, N * K, "wq"));
  MQ_TRY(need(out, M * N, "the output"));
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(out, 16))
    return fail(MQ_ERR_ALIGN, "xq, wq and the output must be 16-byte aligned");
  (void)out_elem;
  return MQ_OK;
}

}  // namespace

extern "C" {

int mq_abi_version(void) { return MQ_ABI_VERSION; }

const char* mq_status_string(mq_status s) {
  // A C caller may pass any int (a C enum is an int); in C++ a value outside
  // the enumerators' range must not be read as mq_status, so the argument's
  // bytes are read as an int first.
  int v;
  static_assert(sizeof(v) == sizeof(s), "mq_status is passed as an int");
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_NULL: return "MQ_ERR_NULL";
    case MQ_ERR_SHAPE: return "MQ_ERR_SHAPE";
    case MQ_ERR_ALIGN: return "MQ_ERR_ALIGN";
    case MQ_ERR_UNSUPPORTED: return "MQ_ERR_UNSUPPORTED";
    case MQ_ERR_WORKSPACE: return "MQ_ERR_WORKSPACE";
    case MQ_ERR_ALIAS: return "MQ_ERR_ALIAS";
    case MQ_ERR_HIP: return "MQ_ERR_HIP";
  }
  return "MQ_ERR_UNKNOWN";
}

const char* mq_last_error(void) { return g_last_error; }

static mq_status quant_impl(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K, bool bf16,
                            void* stream) {
  mq_status s = check_mk(M, K, 16, kMaxK, 16);
  if (s != MQ_OK) return s;
  MQ_TRY(need(x, M * K, "x"));
  MQ_TRY(need(xq, M * K, "xq"));
  MQ_TRY(need(s_tok, M, "s_tok"));
  if (!aligned(x, 16) || !aligned(xq, 16)) return fail(MQ_ERR_ALIGN, "x and xq must be 16-byte aligned");
  if (!aligned(s_tok, 4)) return fail(MQ_ERR_ALIGN, "s_tok must be 4-byte aligned");
  const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"}};
  const Range out[] = {{xq, static_cast<size_t>(M * K), "xq"}, {s_tok, static_cast<size_t>(M) * 4, "s_tok"}};
  s = check_alias(in, out);
  if (s != MQ_OK) return s;
  if (M == 0) return ok();
  return hip_status(mq::launch_quant_per_token_int8(x, xq, s_tok, M, K, bf16, as_stream(stream)),
                    "quant_per_token_int8 launch");
}

mq_status mq_quant_per_token_int8(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K, void* stream) {
  return quant_impl(x, xq, s_tok, M, K, false, stream);
}

mq_status mq_quant_per_token_int8_bf16(const uint16_t* x, int8_t* xq, float* s_tok, int64_t M, int64_t K,
                                       void* stream) {
  return quant_impl(x, xq, s_tok, M, K, true, stream);
}

static mq_status scaled_mm_impl(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, bool bf16, void* stream) {
  mq_status s = check_w8a8(xq, wq, y, 2, M, N, K);
  if (s != MQ_OK) return s;
  MQ_TRY(need(s_tok, M, "s_tok"));
  MQ_TRY(need(s_ch, N, "s_ch"));
  if (!aligned(s_tok, 4) || !aligned(s_ch, 4)) return fail(MQ_ERR_ALIGN, "s_tok and s_ch must be 4-byte aligned");
  const Range in[] = {{xq, static_cast<size_t>(M * K), "xq"},
                      {s_tok, static_cast<size_t>(M) * 4, "s_tok"},
                      {wq, static_cast<size_t>(N * K), "wq"},
                      {s_ch, static_cast<size_t>(N) * 4, "s_ch"}};
  const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"}};
  s = check_alias(in, out);
  if (s != MQ_OK) return s;
  if (M == 0 || N == 0) return ok();
  return hip_status(mq::launch_w8a8_gemm(xq, s_tok, wq, s_ch, y, nullptr, M, N, K, bf16, as_stream(stream)),
                    "w8a8_scaled_mm launch");
}

mq_status mq_w8a8_scaled_mm(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, void* stream) {
  return scaled_mm_impl(xq, s_tok, wq, s_ch, y, M, N, K, false, stream);
}

mq_status mq_w8a8_scaled_mm_bf16(const int8_t* xq, const float* s_tok, const int8_t* wq, const float* s_ch,
                                 uint16_t* y, int64_t M, int64_t N, int64_t K, void* stream) {
  return scaled_mm_impl(xq, s_tok, wq, s_ch, y, M, N, K, true, stream);
}

mq_status mq_w8a8_mm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc,
                         int64_t M, int64_t N, int64_t K, void* stream) {
  mq_status s = check_w8a8(xq, wq, acc, 4, M, N, K);
  if (s != MQ_OK) return s;
  const Range in[] = {{xq, static_cast<size_t>(M * K), "xq"}, {wq, static_cast<size_t>(N * K), "wq"}};
  const Range out[] = {{acc, static_cast<size_t>(M * N) * 4, "acc"}};
  s = check_alias(in, out);
  if (s != MQ_OK) return s;
  if (M == 0 || N == 0) return ok();
  return hip_status(mq::launch_w8a8_gemm(xq, nullptr, wq, nullptr, nullptr, acc, M, N, K, false, as_stream(stream)),
                    "w8a8_mm_i32 launch");
}

size_t mq_w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (!w4a16_group_ok(group) || M < 1 || M > kMaxDim || N < 8 || N % 8 || N > kMaxN4 ||
      K < 128 || K > kMaxK || K % 128 || M * N > kMaxElems)
    return 0;
  return mq::w4a16_gemm_workspace(M, N, K);
}

static mq_status w4a16_gemm_impl(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                                   const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                   int64_t group, void* workspace, size_t workspace_bytes, bool bf16, void* stream) {
  mq_status s = check_w4a16(x, qweight, scales, qzeros, y, M, N, K, group);
  if (s != MQ_OK) return s;
  if (M == 0) return ok();
  // A workspace is optional: given (large enough for the split plan), K may
  // be split for small tile grids; NULL never splits.
  void* ws = nullptr;
  if (workspace != nullptr) {
    const size_t need = mq::w4a16_gemm_workspace(M, N, K);
    if (need > 0) {
      if (workspace_bytes < need)
        return fail(MQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
      if (!aligned(workspace, 16)) return fail(MQ_ERR_ALIGN, "workspace must be 16-byte aligned");
      const size_t G = group_rows(K, group);
      const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"},
                          {qweight, static_cast<size_t>(K * (N / 8)) * 4, "qweight"},
                          {scales, G * static_cast<size_t>(N) * 2, "scales"},
                          {qzeros, G * static_cast<size_t>(N / 8) * 4, "qzeros"}};
      const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"}, {workspace, need, "workspace"}};
      s = check_alias(in, out);
      if (s != MQ_OK) return s;
      ws = workspace;
    }
  }
  return hip_status(mq::launch_w4a16_gemm(x, qweight, scales, qzeros, y, M, N, K, kernel_group(group), group == -1,
                                          ws, bf16, as_stream(stream)),
                    "w4a16_gemm launch");
}

size_t mq_w4a16_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (!w4a16_group_ok(group) || M < 1 || M > mq::kGemvMaxM || N < 8 || N % 8 ||
      N > kMaxN4 || K < 128 || K > kMaxK || K % 128)
    return 0;
  return mq::plan_w4a16_gemv(M, N, K, kernel_group(group)).workspace_bytes;
}

static mq_status w4a16_gemv_impl(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                                   const int32_t* qzeros, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                   int64_t group, void* workspace, size_t workspace_bytes, bool bf16, void* stream) {
  mq_status s = check_w4a16(x, qweight, scales, qzeros, y, M, N, K, group);
  if (s != MQ_OK) return s;
  if (M > mq::kGemvMaxM)
    return fail(MQ_ERR_UNSUPPORTED, "GEMV needs M <= %lld (got %lld); use mq_w4a16_gemm",
                (long long)mq::kGemvMaxM, (long long)M);
  if (M == 0) return ok();
  mq::GemvPlan plan = mq::plan_w4a16_gemv(M, N, K, kernel_group(group));
  plan.per_channel = group == -1;
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes)
      return fail(MQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.workspace_bytes,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t G = group_rows(K, group);
    const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"},
                        {qweight, static_cast<size_t>(K * (N / 8)) * 4, "qweight"},
                        {scales, G * static_cast<size_t>(N) * 2, "scales"},
                        {qzeros, G * static_cast<size_t>(N / 8) * 4, "qzeros"}};
    const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"}, {workspace, plan.workspace_bytes, "workspace"}};
    s = check_alias(in, out);
    if (s != MQ_OK) return s;
  }
  return hip_status(mq::launch_w4a16_gemv(x, qweight, scales, qzeros, y, M, N, K, plan,
                                          plan.workspace_bytes ? workspace : nullptr, bf16, as_stream(stream)),
                    "w4a16_gemv launch");
}

static mq_status kv_quant_impl(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                               int32_t bits, bool bf16, void* stream) {
  if (bits != 8 && bits != 4) return fail(MQ_ERR_UNSUPPORTED, "bits=%d (8 and 4 are provided)", (int)bits);
  if (head_dim < 8 || head_dim > 512 || (head_dim & (head_dim - 1)))
    return fail(MQ_ERR_SHAPE, "head_dim=%lld must be a power of two in [8, 512]", (long long)head_dim);
  if (rows < 0 || rows > kMaxDim) return fail(MQ_ERR_SHAPE, "rows=%lld out of range", (long long)rows);
  // one lane per 8 values: the launch holds rows * head_dim / 8 < 2^32 work-items
  if (rows * head_dim >= (int64_t{1} << 35))
    return fail(MQ_ERR_SHAPE, "rows * head_dim = %lld must be below 2^35", (long long)(rows * head_dim));
  MQ_TRY(need(x, rows * head_dim, "x"));
  MQ_TRY(need(codes, rows * head_dim, "codes"));
  MQ_TRY(need(params, rows, "params"));
  if (!aligned(x, 16)) return fail(MQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(codes, bits == 8 ? 8 : 4)) return fail(MQ_ERR_ALIGN, "codes must be %d-byte aligned", bits == 8 ? 8 : 4);
  if (!aligned(params, 8)) return fail(MQ_ERR_ALIGN, "params must be 8-byte aligned");
  const Range in[] = {{x, static_cast<size_t>(rows * head_dim) * 2, "x"}};
  const Range out[] = {{codes, static_cast<size_t>(rows * head_dim) * bits / 8, "codes"},
                       {params, static_cast<size_t>(rows) * 8, "params"}};
  MQ_TRY(check_alias(in, out));
  if (rows == 0) return ok();
  return hip_status(mq::launch_kv_quant(x, codes, params, rows, head_dim, bits, bf16, as_stream(stream)),
                    "kv_quant launch");
}

mq_status mq_kv_quant(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                      int32_t bits, void* stream) {
  return kv_quant_impl(x, codes, params, rows, head_dim, bits, false, stream);
}

mq_status mq_kv_quant_bf16(const uint16_t* x, uint8_t* codes, float* params, int64_t rows, int64_t head_dim,
                           int32_t bits, void* stream) {
  return kv_quant_impl(x, codes, params, rows, head_dim, bits, true, stream);
}

namespace {

// A field order: NULL means the library's own (field j = element j);
// otherwise a permutation of 0..7.
mq_status field_order(const uint8_t* order, uint8_t (&out)[8]) {
  for (int j = 0; j < 8; ++j) out[j] = static_cast<uint8_t>(j);
  if (order == nullptr) return MQ_OK;
  unsigned seen = 0;
  for (int j = 0; j < 8; ++j) {
    if (order[j] > 7 || (seen >> order[j]) & 1u)
      return fail(MQ_ERR_UNSUPPORTED, "field_order must be a permutation of 0..7");
    seen |= 1u << order[j];
    out[j] = order[j];
  }
  return MQ_OK;
}

}  // namespace

mq_status mq_int4_reorder(const int32_t* src, int32_t* dst, int64_t words, const uint8_t* order, void* stream) {
  uint8_t ord[8];
  MQ_TRY(field_order(order, ord));
  if (words < 0 || words >= (int64_t{1} << 34))
    return fail(MQ_ERR_SHAPE, "words=%lld out of range", (long long)words);
  MQ_TRY(need(src, words, "src"));
  MQ_TRY(need(dst, words, "dst"));
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(MQ_ERR_ALIGN, "src and dst must be 16-byte aligned");
  const Range in[] = {{src, static_cast<size_t>(words) * 4, "src"}};
  const Range out[] = {{dst, static_cast<size_t>(words) * 4, "dst"}};
  MQ_TRY(check_alias(in, out));
  if (words == 0) return ok();
  return hip_status(mq::launch_int4_reorder(src, dst, words, ord, as_stream(stream)), "int4_reorder launch");
}

mq_status mq_int4_transpose(const int32_t* src, int32_t* dst, int64_t A, int64_t B, const uint8_t* order,
                            void* stream) {
  uint8_t ord[8];
  MQ_TRY(field_order(order, ord));
  if (A < 0 || B < 0 || A % 8 || B % 8)
    return fail(MQ_ERR_SHAPE, "A=%lld and B=%lld must be non-negative multiples of 8", (long long)A, (long long)B);
  if (A > mq::kInt4TransposeMaxA || B > kMaxDim || A * B > kMaxElems)
    return fail(MQ_ERR_SHAPE, "A=%lld, B=%lld too large", (long long)A, (long long)B);
  MQ_TRY(need(src, A * B, "src"));
  MQ_TRY(need(dst, A * B, "dst"));
  if (!aligned(src, 4) || !aligned(dst, 4)) return fail(MQ_ERR_ALIGN, "src and dst must be 4-byte aligned");
  const Range in[] = {{src, static_cast<size_t>(A * B) / 2, "src"}};
  const Range out[] = {{dst, static_cast<size_t>(A * B) / 2, "dst"}};
  MQ_TRY(check_alias(in, out));
  if (A == 0 || B == 0) return ok();
  return hip_status(mq::launch_int4_transpose(src, dst, A, B, ord, as_stream(stream)), "int4_transpose launch");
}

mq_status mq_u16_transpose(const uint16_t* src, uint16_t* dst, int64_t A, int64_t B, void* stream) {
  if (A < 0 || B < 0 || A > mq::kU16TransposeMaxA || B > mq::kU16TransposeMaxB || A * B > kMaxElems)
    return fail(MQ_ERR_SHAPE, "A=%lld, B=%lld out of range", (long long)A, (long long)B);
  MQ_TRY(need(src, A * B, "src"));
  MQ_TRY(need(dst, A * B, "dst"));
  if (!aligned(src, 2) || !aligned(dst, 2)) return fail(MQ_ERR_ALIGN, "src and dst must be 2-byte aligned");
  const Range in[] = {{src, static_cast<size_t>(A * B) * 2, "src"}};
  const Range out[] = {{dst, static_cast<size_t>(A * B) * 2, "dst"}};
  MQ_TRY(check_alias(in, out));
  if (A == 0 || B == 0) return ok();
  return hip_status(mq::launch_u16_transpose(src, dst, A, B, as_stream(stream)), "u16_transpose launch");
}

// The workspace does not depend on N: it is sized for the two-kernel path,
// which every M can take (the one-kernel path for 1-4 tokens leaves it
// unused).
size_t mq_w8a8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || M > kMaxDim || K < 16 || K > kMaxKInt8 || K % 16 || M * K > kMaxElems || M == 0) return 0;
  return (static_cast<size_t>(M * K) + 255) / 256 * 256 + static_cast<size_t>(M) * 4;
}

static_assert(mq::kNoallocScratchBytes == MQ_NOALLOC_SCRATCH_BYTES, "scratch size in mq.h");

// noalloc: the workspace is the library's scratch array, looked up after
// every argument check passed (the only HIP call before the launches).
static mq_status linear_impl(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, void* workspace, size_t workspace_bytes, bool bf16, void* stream,
                             bool noalloc = false) {
  mq_status s = check_mk(M, K, 16, kMaxKInt8, 16);
  if (s != MQ_OK) return s;
  if (N < 0 || N > kMaxDim) return fail(MQ_ERR_SHAPE, "N=%lld out of range", (long long)N);
  if (M * N > kMaxElems || K * N > kMaxElems) return fail(MQ_ERR_SHAPE, "problem too large");
  MQ_TRY(need(x, M * K, "x"));
  MQ_TRY(need(wq, N * K, "wq"));
  MQ_TRY(need(s_ch, N, "s_ch"));
  MQ_TRY(need(y, M * N, "y"));
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(MQ_ERR_ALIGN, "x, wq and y must be 16-byte aligned");
  if (!aligned(s_ch, 4)) return fail(MQ_ERR_ALIGN, "s_ch must be 4-byte aligned");
  const bool fused = mq::w8a8_use_fused(M, N, K);
  const size_t ws = fused ? 0 : mq_w8a8_linear_workspace_bytes(M, K);
  if (noalloc) {
    if (ws > MQ_NOALLOC_SCRATCH_BYTES)
      return fail(MQ_ERR_WORKSPACE, "M*K=%lld needs %zu bytes of scratch; the allocation-free entry holds %zu",
                  (long long)(M * K), ws, static_cast<size_t>(MQ_NOALLOC_SCRATCH_BYTES));
  } else if (ws > 0) {
    if (!workspace || workspace_bytes < ws)
      return fail(MQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"},
                      {wq, static_cast<size_t>(N * K), "wq"},
                      {s_ch, static_cast<size_t>(N) * 4, "s_ch"}};
  // (the library's scratch cannot overlap a caller's buffer)
  const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"},
                       {ws && !noalloc ? workspace : nullptr, noalloc ? 0 : ws, "workspace"}};
  s = check_alias(in, out);
  if (s != MQ_OK) return s;
  if (M == 0 || N == 0) return ok();
  if (noalloc && ws > 0) {
    MQ_TRY(hip_status(mq::noalloc_scratch(&workspace), "w8a8_linear_noalloc scratch lookup"));
    workspace_bytes = MQ_NOALLOC_SCRATCH_BYTES;
  }
  if (fused)
    return hip_status(mq::launch_w8a8_gemv_fused(x, wq, s_ch, y, M, N, K, bf16, as_stream(stream)),
                      "w8a8_linear launch");
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* s_tok = reinterpret_cast<float*>(static_cast<char*>(workspace) + (static_cast<size_t>(M * K) + 255) / 256 * 256);
  s = hip_status(mq::launch_quant_per_token_int8(x, xq, s_tok, M, K, bf16, as_stream(stream)),
                 "w8a8_linear quant launch");
  if (s != MQ_OK) return s;
  return hip_status(mq::launch_w8a8_gemm(xq, s_tok, wq, s_ch, y, nullptr, M, N, K, bf16, as_stream(stream)),
                    "w8a8_linear gemm launch");
}

mq_status mq_w8a8_linear(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M, int64_t N,
                         int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(x, wq, s_ch, y, M, N, K, workspace, workspace_bytes, false, stream);
}

mq_status mq_w8a8_linear_bf16(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(x, wq, s_ch, y, M, N, K, workspace, workspace_bytes, true, stream);
}

mq_status mq_w8a8_linear_noalloc(const uint16_t* x, const int8_t* wq, const float* s_ch, uint16_t* y, int64_t M,
                                 int64_t N, int64_t K, void* stream) {
  return linear_impl(x, wq, s_ch, y, M, N, K, nullptr, 0, false, stream, true);
}

mq_status mq_w4a16_block_weights(const int32_t* qweight, int32_t* qweight_blocked, int64_t N, int64_t K,
                                 void* stream) {
  if (N < 0 || N > kMaxN4 || N % 32)
    return fail(MQ_ERR_SHAPE, "N=%lld must be a multiple of 32 in [0, 2^27]", (long long)N);
  if (K < 0 || K > kMaxK || K % 128)
    return fail(MQ_ERR_SHAPE, "K=%lld must be a multiple of 128 in [0, 2^20]", (long long)K);
  if (K * N > kMaxElems) return fail(MQ_ERR_SHAPE, "problem too large");
  MQ_TRY(need(qweight, K * N, "qweight"));
  MQ_TRY(need(qweight_blocked, K * N, "qweight_blocked"));
  if (!aligned(qweight, 4)) return fail(MQ_ERR_ALIGN, "qweight must be 4-byte aligned");
  if (!aligned(qweight_blocked, 16)) return fail(MQ_ERR_ALIGN, "qweight_blocked must be 16-byte aligned");
  const size_t bytes = static_cast<size_t>(K * (N / 8)) * 4;
  const Range in[] = {{qweight, bytes, "qweight"}};
  const Range out[] = {{qweight_blocked, bytes, "qweight_blocked"}};
  MQ_TRY(check_alias(in, out));
  if (K == 0 || N == 0) return ok();
  return hip_status(mq::launch_w4a16_block_weights(qweight, qweight_blocked, N, K, as_stream(stream)),
                    "w4a16_block_weights launch");
}

// The decode-layout kernels address the scale and zero-point tables with
// 32-bit buffer offsets.
constexpr size_t kMaxScaleBytes = (size_t{1} << 31) - 1;
static bool blocked_scales_fit(int64_t N, int64_t K, int64_t group) {
  return group_rows(K, group) * static_cast<size_t>(N) * 2 <= kMaxScaleBytes;
}

size_t mq_w4a16_gemv_blocked_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (!w4a16_group_ok(group) || M < 1 || M > mq::kGemvMaxM || N < 32 || N % 32 ||
      N > kMaxN4 || K < 128 || K > kMaxK || K % 128 || !blocked_scales_fit(N, K, group))
    return 0;
  return mq::w4a16_gemv_blocked_workspace(M, N, K, kernel_group(group));
}

static mq_status w4a16_gemv_blocked_impl(const uint16_t* x, const int32_t* qweight_blocked,
                                         const uint16_t* scales, const int32_t* qzeros, uint16_t* y, int64_t M,
                                         int64_t N, int64_t K, int64_t group, void* workspace,
                                         size_t workspace_bytes, bool bf16, void* stream) {
  mq_status s = check_w4a16(x, qweight_blocked, scales, qzeros, y, M, N, K, group);
  if (s != MQ_OK) return s;
  if (N % 32) return fail(MQ_ERR_SHAPE, "the blocked layout needs N %% 32 == 0 (got N=%lld)", (long long)N);
  if (!blocked_scales_fit(N, K, group))
    return fail(MQ_ERR_SHAPE, "scales of %zu bytes: the decode-layout GEMV takes at most 2^31 - 1",
                group_rows(K, group) * static_cast<size_t>(N) * 2);
  if (!aligned(qweight_blocked, 16)) return fail(MQ_ERR_ALIGN, "qweight_blocked must be 16-byte aligned");
  if (M > mq::kGemvMaxM)
    return fail(MQ_ERR_UNSUPPORTED, "GEMV needs M <= %lld (got %lld); use mq_w4a16_gemm",
                (long long)mq::kGemvMaxM, (long long)M);
  if (M == 0) return ok();
  const size_t need_ws = mq::w4a16_gemv_blocked_workspace(M, N, K, kernel_group(group));
  if (need_ws > 0) {
    if (!workspace || workspace_bytes < need_ws)
      return fail(MQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need_ws,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t G = group_rows(K, group);
    const Range in[] = {{x, static_cast<size_t>(M * K) * 2, "x"},
                        {qweight_blocked, static_cast<size_t>(K * (N / 8)) * 4, "qweight_blocked"},
                        {scales, G * static_cast<size_t>(N) * 2, "scales"},
                        {qzeros, G * static_cast<size_t>(N / 8) * 4, "qzeros"}};
    const Range out[] = {{y, static_cast<size_t>(M * N) * 2, "y"}, {workspace, need_ws, "workspace"}};
    s = check_alias(in, out);
    if (s != MQ_OK) return s;
  }
  mq::GemvPlan plan = mq::plan_w4a16_gemv_blocked(M, N, K, kernel_group(group));
  plan.per_channel = group == -1;
  return hip_status(mq::launch_w4a16_gemv_blocked(x, qweight_blocked, scales, qzeros, y, M, N, K, plan,
                                                  need_ws ? workspace : nullptr, bf16, as_stream(stream)),
                    "w4a16_gemv_blocked launch");
}

#define MQ_W4A16_ENTRY(NAME, IMPL, BF, WNAME)                                                                  \
  mq_status NAME(const uint16_t* x, const int32_t* WNAME, const uint16_t* scales, const int32_t* qzeros,       \
                 uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t group, void* workspace,                  \
                 size_t workspace_bytes, void* stream) {                                                        \
    return IMPL(x, WNAME, scales, qzeros, y, M, N, K, group, workspace, workspace_bytes, BF, stream);         \
  }
MQ_W4A16_ENTRY(mq_w4a16_gemm, w4a16_gemm_impl, false, qweight)
MQ_W4A16_ENTRY(mq_w4a16_gemm_bf16, w4a16_gemm_impl, true, qweight)
MQ_W4A16_ENTRY(mq_w4a16_gemv, w4a16_gemv_impl, false, qweight)
MQ_W4A16_ENTRY(mq_w4a16_gemv_bf16, w4a16_gemv_impl, true, qweight)
MQ_W4A16_ENTRY(mq_w4a16_gemv_blocked, w4a16_gemv_blocked_impl, false, qweight_blocked)
MQ_W4A16_ENTRY(mq_w4a16_gemv_blocked_bf16, w4a16_gemv_blocked_impl, true, qweight_blocked)
#undef MQ_W4A16_ENTRY

}  // extern "C"
