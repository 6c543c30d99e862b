// C-ABI layer: argument validation, diagnostics and dispatch to the kernels.
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing and touches no output.
#include "tiled_attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

attn_status ok() {
  g_last_error.clear();
  return ATTN_OK;
}

struct Range {
  const char* name;
  uintptr_t lo;
  uintptr_t hi;  // exclusive
};

// Empty ranges overlap nothing.
bool overlaps(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Sizes shared by both entry points. Fills `elems` (elements per tensor)
// and `rows` (B*H*N) when the shape is valid.
attn_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype dtype,
                        int64_t* elems, int64_t* rows) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (B < 0 || H < 0 || N < 0 || d < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "negative size (B=%lld H=%lld N=%lld d=%lld)",
                (long long)B, (long long)H, (long long)N, (long long)d);
  if (d != 64 && d != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%lld is not supported (64 or 128)",
                (long long)d);
  // One head's [N, d] slice is addressed with 32-bit byte offsets.
  if (N > INT32_MAX / (d * 4))
    return fail(ATTN_ERR_UNSUPPORTED, "sequence length N=%lld too large for d=%lld (N*d*4 must be < 2^31)",
                (long long)N, (long long)d);
  if (B > (int64_t(1) << 30) || H > (int64_t(1) << 30) || (B && H && B * H > (int64_t(1) << 31)))
    return fail(ATTN_ERR_UNSUPPORTED, "B*H too large (B=%lld H=%lld)", (long long)B, (long long)H);
  const int64_t bh = B * H;
  if (bh && N && bh > (INT64_MAX / 8) / N / d)
    return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
  *rows = bh * N;
  *elems = *rows * d;
  return ATTN_OK;
}

attn_status check_ptr(const void* p, const char* name, uintptr_t align) {
  if (!p) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if ((uintptr_t)p % align)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "%s=%p is not %zu-byte aligned", name, p, (size_t)align);
  return ATTN_OK;
}

attn_status check_scale(float scale) {
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0 (got %g)", (double)scale);
  return ATTN_OK;
}

// Compute units of the current device, cached per device id.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

attn_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return ATTN_OK;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return ATTN_OK;
}

int env_int(const char* name, std::initializer_list<int> allowed) {
  const char* s = std::getenv(name);
  if (!s) return 0;
  const int w = std::atoi(s);
  for (int a : allowed)
    if (w == a) return w;
  return 0;
}

int env_waves() {
  const char* s = std::getenv("TILED_ATTN_FWD_WAVES");
  if (!s) return 0;
  const int w = std::atoi(s);
  return (w == 2 || w == 4 || w == 8) ? w : 0;
}

// TILED_ATTN_FWD_KSPLIT=1 (never) or 2 (where allowed) overrides the
// choice of splitting a workgroup's keys between its waves.
int env_ksplit() {
  const char* s = std::getenv("TILED_ATTN_FWD_KSPLIT");
  if (!s) return 0;
  const int k = std::atoi(s);
  return (k == 1 || k == 2) ? k : 0;
}

// TILED_ATTN_FWD_F32_BM=16 or 32 fixes the query tile of the fp32 key-split
// kernel at d = 64 (16: the 16x16x4 MFMA kernel for the smallest grids).
int env_f32_bm() {
  const char* s = std::getenv("TILED_ATTN_FWD_F32_BM");
  if (!s) return 0;
  const int b = std::atoi(s);
  return (b == 16 || b == 32) ? b : 0;
}

// TILED_ATTN_BWD_DKDV_WAVES=4 or 8 fixes the waves per workgroup of the
// dK/dV sweep (128 or 256 keys per workgroup).
int env_dkdv_waves() { return env_int("TILED_ATTN_BWD_DKDV_WAVES", {4, 8}); }

// TILED_ATTN_BWD_DQ_WAVES=4 or 8 fixes the waves per workgroup of the dQ
// sweep (4: 128 queries, lock-step; 8: 256 queries).
int env_dq_waves() { return env_int("TILED_ATTN_BWD_DQ_WAVES", {4, 8}); }

// TILED_ATTN_FWD_KSPLIT_BN=64 or 128 fixes the key tile of the bf16
// key-split kernel at d = 64.
int env_ksplit_bn() { return env_int("TILED_ATTN_FWD_KSPLIT_BN", {64, 128}); }

// TILED_ATTN_FWD_DECODE=1 keeps bf16 launches with one query per head on
// the tiled kernels instead of the one-query kernel.
int env_decode() {
  const char* s = std::getenv("TILED_ATTN_FWD_DECODE");
  return (s && std::atoi(s) == 1) ? 1 : 0;
}

}  // namespace

extern "C" {

int attn_version(void) { return 3; }

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARGUMENT: return "ATTN_ERR_INVALID_ARGUMENT";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_STATUS_UNKNOWN";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Bytes of the split-key workspace: fp32 O parts [S, B*H, Nq, d] and LSE
// parts [S, B*H, Nq].
size_t split_workspace_bytes(int64_t rows, int64_t d, int64_t splits) {
  return splits > 1 ? (size_t)splits * (size_t)rows * (size_t)(d + 1) * sizeof(float) : 0;
}

attn_status fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                       int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int mask,
                       int64_t num_splits, void* workspace, size_t workspace_bytes,
                       attn_dtype dtype, void* stream, void* ev_start = nullptr, void* ev_stop = nullptr) {
  int64_t q_elems = 0, q_rows = 0, k_elems = 0, k_rows = 0;
  attn_status s = check_shape(B, H, Nq, d, dtype, &q_elems, &q_rows);
  if (s != ATTN_OK) return s;
  if ((s = check_shape(B, H, Nk, d, dtype, &k_elems, &k_rows)) != ATTN_OK) return s;
  if ((s = check_scale(scale)) != ATTN_OK) return s;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown mask %d", mask);
  if (num_splits < 0 || num_splits > tattn::kMaxSplits)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "num_splits=%lld out of range (0 .. %d)",
                (long long)num_splits, tattn::kMaxSplits);
  if (q_rows == 0) return ok();
  if ((s = check_ptr(q, "q", 16)) != ATTN_OK || (s = check_ptr(o, "o", 16)) != ATTN_OK ||
      (s = check_ptr(lse, "lse", 16)) != ATTN_OK)
    return s;
  if (k_rows > 0 && ((s = check_ptr(k, "k", 16)) != ATTN_OK || (s = check_ptr(v, "v", 16)) != ATTN_OK))
    return s;

  int cus = 0;
  if (num_splits == 0 && (s = device_cus(&cus)) != ATTN_OK) return s;
  const int64_t bh = B * H;
  int64_t splits = num_splits == 0 ? tattn::fwd_auto_splits(bh, Nq, Nk, dtype == ATTN_FP32, cus) : num_splits;
  if (k_rows == 0) splits = 1;
  tattn::FwdTailPlan tail{0, 0};
  const bool use_tail = num_splits == 0 && splits == 1 && k_rows > 0 &&
                        tattn::fwd_tail_plan(bh, Nq, Nk, dtype == ATTN_FP32, mask == ATTN_MASK_CAUSAL, cus, &tail);
  const size_t need = use_tail ? split_workspace_bytes((bh - tail.head_split) * Nq, d, tail.tail_splits)
                               : split_workspace_bytes(q_rows, d, splits);
  if (need > 0) {
    if ((s = check_ptr(workspace, "workspace", 16)) != ATTN_OK) return s;
    if (workspace_bytes < need)
      return fail(ATTN_ERR_INVALID_ARGUMENT, "workspace too small for %lld key splits: %zu bytes given, %zu needed",
                  (long long)splits, workspace_bytes, need);
  }

  const uintptr_t e = dtype == ATTN_FP32 ? 4 : 2;
  const Range in[3] = {{"q", (uintptr_t)q, (uintptr_t)q + (uintptr_t)q_elems * e},
                 {"k", (uintptr_t)k, (uintptr_t)k + (uintptr_t)k_elems * e},
                 {"v", (uintptr_t)v, (uintptr_t)v + (uintptr_t)k_elems * e}};
  const Range out[3] = {{"o", (uintptr_t)o, (uintptr_t)o + (uintptr_t)q_elems * e},
                        {"lse", (uintptr_t)lse, (uintptr_t)lse + (uintptr_t)q_rows * 4},
                        {"workspace", (uintptr_t)workspace, (uintptr_t)workspace + need}};
  for (int i = 0; i < 3; ++i) {
    for (const Range& b : in)
      if (overlaps(out[i], b))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", out[i].name, b.name);
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(out[i], out[j]))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs %s and %s overlap", out[i].name, out[j].name);
  }

  if (cus == 0 && (s = device_cus(&cus)) != ATTN_OK) return s;
  tattn::FwdArgs a{q, k, v, o, lse, bh, Nq, Nk, d, scale, dtype == ATTN_FP32,
                   mask == ATTN_MASK_CAUSAL, (int)splits, (float*)workspace, stream, cus, env_waves(),
                   env_ksplit(), env_decode(), env_f32_bm()};
  a.ksplit_bn = env_ksplit_bn();
  if (use_tail) {
    a.tail_heads = bh - tail.head_split;
    a.tail_splits = tail.tail_splits;
  }
  a.ev_start = ev_start;
  a.ev_stop = ev_stop;
  const hipError_t he = tattn::launch_attn_fwd(a);
  if (he != hipSuccess) return fail(ATTN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(he));
  return ok();
}

}  // namespace

extern "C" {

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, float scale, attn_dtype dtype,
                     void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, N, N, d, scale, ATTN_MASK_NONE, 1, nullptr, 0, dtype,
                    stream);
}

size_t attn_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                   int64_t num_splits, attn_dtype dtype) {
  int64_t elems = 0, rows = 0, ke = 0, kr = 0;
  if (check_shape(B, H, Nq, d, dtype, &elems, &rows) != ATTN_OK) return 0;
  if (check_shape(B, H, Nk, d, dtype, &ke, &kr) != ATTN_OK) return 0;
  if (num_splits < 0 || num_splits > tattn::kMaxSplits) return 0;
  if (num_splits == 0 && rows > 0 && kr > 0) {
    // The library's own choice on the current device.
    int cus = 0;
    if (device_cus(&cus) != ATTN_OK) return 0;
    const bool fp32 = dtype == ATTN_FP32;
    const int64_t bh = B * H;
    tattn::FwdTailPlan tail{0, 0};
    const int64_t splits = tattn::fwd_auto_splits(bh, Nq, Nk, fp32, cus);
    if (splits == 1 && tattn::fwd_tail_plan(bh, Nq, Nk, fp32, false, cus, &tail))
      return split_workspace_bytes((bh - tail.head_split) * Nq, d, tail.tail_splits);
    return split_workspace_bytes(rows, d, splits);
  }
  return split_workspace_bytes(rows, d, num_splits);
}

int64_t attn_fwd_ex_auto_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                attn_dtype dtype) {
  int64_t elems = 0, rows = 0, ke = 0, kr = 0;
  if (check_shape(B, H, Nq, d, dtype, &elems, &rows) != ATTN_OK) return 0;
  if (check_shape(B, H, Nk, d, dtype, &ke, &kr) != ATTN_OK) return 0;
  if (rows == 0 || kr == 0) return 1;
  int cus = 0;
  if (device_cus(&cus) != ATTN_OK) return 0;
  return tattn::fwd_auto_splits(B * H, Nq, Nk, dtype == ATTN_FP32, cus);
}

attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                        attn_mask mask, int64_t num_splits, void* workspace,
                        size_t workspace_bytes, attn_dtype dtype, void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, (int)mask, num_splits, workspace,
                    workspace_bytes, dtype, stream);
}

attn_status attn_fwd_ex_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                              attn_mask mask, int64_t num_splits, void* workspace,
                              size_t workspace_bytes, attn_dtype dtype, void* stream,
                              void* start_event, void* stop_event) {
  return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, (int)mask, num_splits, workspace,
                    workspace_bytes, dtype, stream, start_event, stop_event);
}

attn_status attn_matmul_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                           attn_dtype dtype, void* stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the matrix product is implemented for bf16 only");
  if (M < 0 || N < 0 || K < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 8 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "K=%lld must be a multiple of 8 (16-byte rows)", (long long)K);
  // Each operand is addressed with 32-bit byte offsets.
  if ((M && K && M > (INT32_MAX / 2) / K) || (N && K && N > (INT32_MAX / 2) / K))
    return fail(ATTN_ERR_UNSUPPORTED, "operand too large (M*K*2 and N*K*2 must be < 2^31)");
  if (M > INT32_MAX || N > INT32_MAX || (M && N && M > INT64_MAX / 2 / N))
    return fail(ATTN_ERR_UNSUPPORTED, "result too large");
  if (M == 0 || N == 0) return ok();
  attn_status s;
  if ((s = check_ptr(c, "c", 16)) != ATTN_OK) return s;
  if (K > 0 && ((s = check_ptr(a, "a", 16)) != ATTN_OK || (s = check_ptr(b, "b", 16)) != ATTN_OK))
    return s;
  const Range in[2] = {{"a", (uintptr_t)a, (uintptr_t)a + (uintptr_t)(M * K) * 2},
                       {"b", (uintptr_t)b, (uintptr_t)b + (uintptr_t)(N * K) * 2}};
  const Range out = {"c", (uintptr_t)c, (uintptr_t)c + (uintptr_t)(M * N) * 2};
  for (const Range& x : in)
    if (overlaps(out, x)) return fail(ATTN_ERR_INVALID_ARGUMENT, "output c overlaps input %s", x.name);
  const hipError_t he = tattn::launch_matmul_nt(a, b, c, M, N, K, stream);
  if (he != hipSuccess) return fail(ATTN_ERR_HIP, "matmul launch failed: %s", hipGetErrorString(he));
  return ok();
}

attn_status attn_quantize_mxfp8(const void* x, int64_t batch, int64_t rows, int64_t cols, int transpose,
                                void* q, void* scales, attn_dtype dtype, void* stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "MXFP8 quantization takes bf16 input only");
  if (batch < 0 || rows < 0 || cols < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "negative size (batch=%lld rows=%lld cols=%lld)", (long long)batch,
                (long long)rows, (long long)cols);
  if (transpose != 0 && transpose != 1)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1 (got %d)", transpose);
  const int64_t blocked = transpose ? rows : cols;
  if (blocked % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "the blocked dimension (%s=%lld) must be a multiple of 32",
                transpose ? "rows" : "cols", (long long)blocked);
  if (rows > INT32_MAX || cols > INT32_MAX || (rows && cols && batch > (INT64_MAX / 4) / rows / cols))
    return fail(ATTN_ERR_UNSUPPORTED, "input too large");
  const int64_t elems = batch * rows * cols;
  if (elems == 0) return ok();
  attn_status s;
  if ((s = check_ptr(x, "x", 16)) != ATTN_OK || (s = check_ptr(q, "q", 16)) != ATTN_OK ||
      (s = check_ptr(scales, "scales", 1)) != ATTN_OK)
    return s;
  const Range in = {"x", (uintptr_t)x, (uintptr_t)x + (uintptr_t)elems * 2};
  const Range out[2] = {{"q", (uintptr_t)q, (uintptr_t)q + (uintptr_t)elems},
                        {"scales", (uintptr_t)scales, (uintptr_t)scales + (uintptr_t)(elems / 32)}};
  for (const Range& o : out)
    if (overlaps(o, in)) return fail(ATTN_ERR_INVALID_ARGUMENT, "output %s overlaps input x", o.name);
  if (overlaps(out[0], out[1])) return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs q and scales overlap");
  const hipError_t he = tattn::launch_mx_quantize(x, batch, rows, cols, transpose == 1, q, scales, stream);
  if (he != hipSuccess) return fail(ATTN_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(he));
  return ok();
}

attn_status attn_fwd_mxfp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales,
                           const void* vt8, const void* vt_scales, void* o, float* lse, int64_t B,
                           int64_t H, int64_t N, int64_t d, float scale, void* stream) {
  int64_t elems = 0, rows = 0;
  attn_status s = check_shape(B, H, N, d, ATTN_BF16, &elems, &rows);
  if (s != ATTN_OK) return s;
  if ((s = check_scale(scale)) != ATTN_OK) return s;
  if (N % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "N=%lld must be a multiple of 32 (the 32-key scale blocks of V^T)",
                (long long)N);
  if (rows == 0) return ok();
  const struct { const void* p; const char* n; uintptr_t align, bytes; } ins[] = {
      {q8, "q8", 16, (uintptr_t)elems}, {q_scales, "q_scales", 4, (uintptr_t)elems / 32},
      {k8, "k8", 16, (uintptr_t)elems}, {k_scales, "k_scales", 4, (uintptr_t)elems / 32},
      {vt8, "vt8", 16, (uintptr_t)elems}, {vt_scales, "vt_scales", 4, (uintptr_t)elems / 32}};
  for (auto& x : ins)
    if ((s = check_ptr(x.p, x.n, x.align)) != ATTN_OK) return s;
  if ((s = check_ptr(o, "o", 16)) != ATTN_OK || (s = check_ptr(lse, "lse", 16)) != ATTN_OK) return s;
  const Range out[2] = {{"o", (uintptr_t)o, (uintptr_t)o + (uintptr_t)elems * 2},
                        {"lse", (uintptr_t)lse, (uintptr_t)lse + (uintptr_t)rows * 4}};
  for (const Range& r : out)
    for (auto& x : ins)
      if (overlaps(r, Range{x.n, (uintptr_t)x.p, (uintptr_t)x.p + x.bytes}))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", r.name, x.n);
  if (overlaps(out[0], out[1])) return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs o and lse overlap");
  tattn::Fp8Args a{q8, q_scales, k8, k_scales, vt8, vt_scales, o, lse, B * H, N, d, scale, stream};
  const hipError_t he = tattn::launch_attn_fwd_mxfp8(a);
  if (he != hipSuccess) return fail(ATTN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(he));
  return ok();
}

attn_status attn_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t B,
                       int64_t H, int64_t N, int64_t d, void* o, float* lse, attn_dtype dtype,
                       void* stream) {
  int64_t elems = 0, rows = 0;
  attn_status s = check_shape(B, H, N, d, dtype, &elems, &rows);
  if (s != ATTN_OK) return s;
  if (num_parts < 1 || num_parts > (int64_t(1) << 20))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "num_parts=%lld out of range (1 .. 2^20)", (long long)num_parts);
  if (rows == 0) return ok();
  if ((s = check_ptr(o_parts, "o_parts", 16)) != ATTN_OK || (s = check_ptr(lse_parts, "lse_parts", 4)) != ATTN_OK ||
      (s = check_ptr(o, "o", 16)) != ATTN_OK || (s = check_ptr(lse, "lse", 4)) != ATTN_OK)
    return s;
  if ((uint64_t)num_parts * (uint64_t)elems > (uint64_t)INT64_MAX / 8)
    return fail(ATTN_ERR_UNSUPPORTED, "partial results too large");
  const uintptr_t e = dtype == ATTN_FP32 ? 4 : 2;
  const Range in[2] = {{"o_parts", (uintptr_t)o_parts, (uintptr_t)o_parts + (uintptr_t)(num_parts * elems) * 4},
                       {"lse_parts", (uintptr_t)lse_parts, (uintptr_t)lse_parts + (uintptr_t)(num_parts * rows) * 4}};
  const Range out[2] = {{"o", (uintptr_t)o, (uintptr_t)o + (uintptr_t)elems * e},
                        {"lse", (uintptr_t)lse, (uintptr_t)lse + (uintptr_t)rows * 4}};
  for (const Range& a : out)
    for (const Range& b : in)
      if (overlaps(a, b)) return fail(ATTN_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", a.name, b.name);
  if (overlaps(out[0], out[1])) return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs o and lse overlap");
  const hipError_t he = tattn::launch_attn_merge(o_parts, lse_parts, (int)num_parts, rows, d, o, lse,
                                                 dtype == ATTN_FP32, stream);
  if (he != hipSuccess) return fail(ATTN_ERR_HIP, "merge launch failed: %s", hipGetErrorString(he));
  return ok();
}

}  // extern "C"

namespace {

// noalloc: the allocation-free variant (no workspace argument; the row terms
// go to the library's fixed per-device array, which bounds B * H * Nq).
attn_status bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                       int64_t d, float scale, int mask, attn_dtype dtype, void* stream,
                       bool noalloc = false) {
  int64_t q_elems = 0, q_rows = 0, k_elems = 0, k_rows = 0;
  attn_status s = check_shape(B, H, Nq, d, dtype, &q_elems, &q_rows);
  if (s != ATTN_OK) return s;
  if ((s = check_shape(B, H, Nk, d, dtype, &k_elems, &k_rows)) != ATTN_OK) return s;
  if (dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "the backward pass is implemented for bf16 only");
  if ((s = check_scale(scale)) != ATTN_OK) return s;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown mask %d", mask);
  if (noalloc && q_rows > tattn::kNoAllocRows)
    return fail(ATTN_ERR_UNSUPPORTED,
                "B*H*Nq = %lld query rows exceed the allocation-free backward's scratch (%lld rows)",
                (long long)q_rows, (long long)tattn::kNoAllocRows);
  if (q_rows == 0 && k_rows == 0) return ok();
  // Tensors of zero rows may be NULL; the others must be valid.
  const int64_t ws_rows = noalloc ? 0 : q_rows;
  const struct { const void* p; const char* n; int64_t rows; } ins[] = {
      {q, "q", q_rows}, {k, "k", k_rows}, {v, "v", k_rows}, {o, "o", q_rows},
      {dout, "dout", q_rows}, {lse, "lse", q_rows}};
  const struct { const void* p; const char* n; int64_t rows; } outs[] = {
      {dq, "dq", q_rows}, {dk, "dk", k_rows}, {dv, "dv", k_rows}, {workspace, "workspace", ws_rows}};
  for (auto& x : ins)
    if (x.rows > 0 && (s = check_ptr(x.p, x.n, 16)) != ATTN_OK) return s;
  for (auto& x : outs)
    if (x.rows > 0 && (s = check_ptr(x.p, x.n, 16)) != ATTN_OK) return s;
  const size_t need = (size_t)ws_rows * sizeof(float);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  Range rin[6], rout[4];
  for (int i = 0; i < 6; ++i) {
    const uintptr_t bytes = i == 5 ? (uintptr_t)ins[i].rows * 4 : (uintptr_t)ins[i].rows * d * 2;
    rin[i] = {ins[i].n, (uintptr_t)ins[i].p, (uintptr_t)ins[i].p + bytes};
  }
  for (int i = 0; i < 4; ++i) {
    const uintptr_t bytes = i == 3 ? need : (uintptr_t)outs[i].rows * d * 2;
    rout[i] = {outs[i].n, (uintptr_t)outs[i].p, (uintptr_t)outs[i].p + bytes};
  }
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(rout[i], rin[j]))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", rout[i].name, rin[j].name);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(rout[i], rout[j]))
        return fail(ATTN_ERR_INVALID_ARGUMENT, "outputs %s and %s overlap", rout[i].name, rout[j].name);
  }
  int cus = 0;
  if ((s = device_cus(&cus)) != ATTN_OK) return s;
  tattn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B * H, Nq, Nk, d, scale,
                   mask == ATTN_MASK_CAUSAL, stream, cus};
  a.dkdv_waves = env_dkdv_waves();
  a.dq_waves = env_dq_waves();
  const hipError_t e = noalloc ? tattn::launch_attn_bwd_noalloc(a) : tattn::launch_attn_bwd(a);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype dtype) {
  int64_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, dtype, &elems, &rows) != ATTN_OK) return 0;
  return (size_t)rows * sizeof(float);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                     float scale, attn_dtype dtype, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, N, d,
                    scale, ATTN_MASK_NONE, dtype, stream);
}

attn_status attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, float scale, attn_mask mask, attn_dtype dtype,
                        void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, d,
                    scale, (int)mask, dtype, stream);
}

attn_status attn_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                attn_mask mask, attn_dtype dtype, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, H, Nq, Nk, d, scale, (int)mask,
                    dtype, stream, true);
}

}  // extern "C"
