// ptg_api.cpp - the C ABI: argument validation, error reporting and dispatch to the
// pipelined kernels.  Nothing here touches the GPU before every host-checkable
// precondition has passed, so invalid calls fail the same way with or without a device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <algorithm>
#include <atomic>
#include <memory>
#include <mutex>
#include <vector>

#include "ptg.h"

#include <cmath>
#include "ptg_launch.h"

namespace {

thread_local char g_err[512] = "";

ptg_status fail(ptg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ptg_status hip_fail(hipError_t e, const char* what) {
  return fail(PTG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bad_dim(int64_t x) { return x < 0; }

#define PTG_TRY(body)                                                  \
  try {                                                                \
    body                                                               \
  } catch (const std::exception& ex) {                                 \
    return fail(PTG_ERR_HIP, "internal error: %s", ex.what());         \
  } catch (...) {                                                      \
    return fail(PTG_ERR_HIP, "internal error");                        \
  }

// Debug switches, read from the environment at every call (set and not "0": on).
//   PTG_LOG    each launch prints its entry point, shape and tile configuration to stderr.
//   PTG_CHECK  entry points whose inputs include device-resident bookkeeping (group or user
//              offsets, user indices) first run that bookkeeping's device check, which
//              synchronises the stream, and return its error instead of launching.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

void log_launch(const char* fmt, ...) {
  if (!env_on("PTG_LOG")) return;
  char line[384];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[ptg] %s\n", line);
}

bool valid_epi(int e) { return e >= PTG_EPI_NONE && e <= PTG_EPI_BIAS_SILU; }
bool needs_bias(int e) { return e == PTG_EPI_BIAS || e == PTG_EPI_BIAS_SILU; }

// Checks shared by every operand pair: sizes, multiples of 8, alignment, 31-bit offsets.
ptg_status check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K))
    return fail(PTG_ERR_INVALID_ARG, "%s: negative size (M=%lld N=%lld K=%lld)", fn, (long long)M,
                (long long)N, (long long)K);
  if (K == 0) return fail(PTG_ERR_UNSUPPORTED, "%s: K = 0 is not supported", fn);
  if (K % 8 || N % 8)
    return fail(PTG_ERR_UNSUPPORTED, "%s: N and K must be multiples of 8 (N=%lld K=%lld)", fn,
                (long long)N, (long long)K);
  if (M > ptg::kMaxDim || N > ptg::kMaxDim || K > ptg::kMaxDim)
    return fail(PTG_ERR_UNSUPPORTED, "%s: a dimension exceeds 2^30", fn);
  return PTG_OK;
}

// The kernels address one tile of each operand with 31-bit byte offsets.
bool fits31(int64_t rows, int64_t ld, int64_t cols) {
  const int64_t bytes = ((rows > 0 ? rows - 1 : 0) * ld + cols) * 2;
  return bytes < ((int64_t)1 << 31);
}

// The epilogue addresses an output tile of up to 256 rows and 256 columns (elements of
// `osz` bytes, row stride ldc) with 31-bit byte offsets, and takes ldc as a 32-bit value.
bool out_fits(int64_t ldc, int64_t osz) {
  return ldc < ((int64_t)1 << 31) && (255 * ldc + 256) * osz < ((int64_t)1 << 31);
}

// After a synchronising check: a set watchdog word (a kernel of an earlier launch tripped a
// bounded wait or a range check, and its output is incomplete) is reported as a failed check.
ptg_status watchdog_status(const char* fn) {
  uint32_t gemm = 0, attention = 0;
  uint32_t onerole = 0;
  hipError_t e = ptg::read_watchdog(&gemm, 0);
  if (e == hipSuccess) e = ptg::read_attention_watchdog(&attention, 0);
  if (e == hipSuccess) e = ptg::read_onerole_watchdog(&onerole, 0);
  gemm |= onerole;
  if (e != hipSuccess) return hip_fail(e, fn);
  if (gemm | attention)
    return fail(PTG_ERR_DEVICE_CHECK, "%s: the device's watchdog word is 0x%x (an earlier launch stopped early)",
                fn, gemm | attention);
  return PTG_OK;
}

}  // namespace

extern "C" {

const char* ptg_status_string(ptg_status s) {
  switch (s) {
    case PTG_OK: return "PTG_OK";
    case PTG_ERR_INVALID_ARG: return "PTG_ERR_INVALID_ARG";
    case PTG_ERR_UNSUPPORTED: return "PTG_ERR_UNSUPPORTED";
    case PTG_ERR_WORKSPACE: return "PTG_ERR_WORKSPACE";
    case PTG_ERR_HIP: return "PTG_ERR_HIP";
    case PTG_ERR_DEVICE_CHECK: return "PTG_ERR_DEVICE_CHECK";
  }
  return "PTG_ERR_UNKNOWN";
}

const char* ptg_last_error(void) { return g_err; }

int32_t ptg_version(void) { return 1; }

ptg_status ptg_describe_config(int64_t M, int64_t N, int64_t K, ptg_layout b_layout, int32_t cfg[6]) {
  if (!cfg) return fail(PTG_ERR_INVALID_ARG, "ptg_describe_config: cfg is NULL");
  ptg::dense_config(M, N, K, b_layout == PTG_B_KN, cfg);
  return PTG_OK;
}

ptg_status ptg_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, ptg_layout b_layout, void* C, int64_t ldc, ptg_dtype c_dtype,
                    const float* bias, ptg_epilogue epi, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_gemm";
    ptg_status st = check_mnk(fn, M, N, K);
    if (st) return st;
    if (b_layout != PTG_B_KN && b_layout != PTG_B_NK) return fail(PTG_ERR_UNSUPPORTED, "%s: bad layout", fn);
    if (c_dtype != PTG_BF16 && c_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!valid_epi(epi)) return fail(PTG_ERR_UNSUPPORTED, "%s: bad epilogue", fn);
    if (M == 0 || N == 0) return PTG_OK;
    if (!A || !B || !C) return fail(PTG_ERR_INVALID_ARG, "%s: null operand", fn);
    if (needs_bias(epi) && !bias) return fail(PTG_ERR_INVALID_ARG, "%s: epilogue needs a bias", fn);
    const int64_t b_row = b_layout == PTG_B_KN ? N : K;
    if (lda < K || ldb < b_row || ldc < N) return fail(PTG_ERR_INVALID_ARG, "%s: leading dimension too small", fn);
    if (lda % 8 || ldb % 8 || (c_dtype == PTG_BF16 ? ldc % 8 : ldc % 4))
      return fail(PTG_ERR_UNSUPPORTED, "%s: leading dimensions must be multiples of 16 bytes", fn);
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (bias && !aligned16(bias)))
      return fail(PTG_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned", fn);
    const bool kn = b_layout == PTG_B_KN;
    if (!fits31(256, lda, K) || !(kn ? fits31(K, ldb, 256) : fits31(256, ldb, K)) ||
        !out_fits(ldc, c_dtype == PTG_F32 ? 4 : 2))
      return fail(PTG_ERR_UNSUPPORTED, "%s: operand or output tile exceeds 2 GiB of addressing", fn);
    ptg::DenseLaunch d{};
    d.A = A; d.B = B; d.C = C; d.bias = needs_bias(epi) ? bias : nullptr;
    d.lda = lda; d.ldb = ldb; d.ldc = ldc;
    d.M = M; d.N = N; d.K = K;
    d.b_kn = kn; d.epi = epi; d.out_f32 = c_dtype == PTG_F32;
    int32_t cfg[6];
    ptg::dense_config(M, N, K, kn, cfg);
    if (cfg[5] == 0)
      log_launch("%s M=%lld N=%lld K=%lld %s %s: tile %dx%dx%d, %d slots, %d waves each copying and computing", fn,
                 (long long)M, (long long)N, (long long)K, kn ? "KN" : "NK", d.out_f32 ? "fp32" : "bf16", cfg[0],
                 cfg[1], cfg[2], cfg[3], cfg[4]);
    else
      log_launch("%s M=%lld N=%lld K=%lld %s %s: tile %dx%dx%d, %d slots, %d consumer and %d producer waves", fn,
                 (long long)M, (long long)N, (long long)K, kn ? "KN" : "NK", d.out_f32 ? "fp32" : "bf16", cfg[0],
                 cfg[1], cfg[2], cfg[3], cfg[4], cfg[5]);
    hipError_t e = ptg::launch_dense(d, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

}  // extern "C"

namespace {

std::atomic<uint32_t> g_epoch{0};

// A value that no earlier launch of this process used (skipping 0, the value of zeroed memory).
uint32_t next_epoch() {
  uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

ptg_status grouped_call(const char* fn, int32_t G, int64_t M_total, int64_t N, int64_t K, const void* X,
                        const void* W, ptg_layout w_layout, const int32_t* group_offsets, void* Y,
                        ptg_dtype y_dtype, const float* bias, ptg_epilogue epi, void* workspace, size_t ws_bytes,
                        bool with_ws, void* stream) {
  PTG_TRY({
    if (G <= 0) return fail(PTG_ERR_INVALID_ARG, "%s: G must be positive", fn);
    if (G > ptg::kMaxGroups) return fail(PTG_ERR_UNSUPPORTED, "%s: G exceeds %d", fn, ptg::kMaxGroups);
    ptg_status st = check_mnk(fn, M_total, N, K);
    if (st) return st;
    if (w_layout != PTG_B_KN && w_layout != PTG_B_NK) return fail(PTG_ERR_UNSUPPORTED, "%s: bad layout", fn);
    if (y_dtype != PTG_BF16 && y_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!valid_epi(epi)) return fail(PTG_ERR_UNSUPPORTED, "%s: bad epilogue", fn);
    if (M_total == 0 || N == 0) return PTG_OK;
    if (!X || !W || !Y || !group_offsets) return fail(PTG_ERR_INVALID_ARG, "%s: null operand", fn);
    if (needs_bias(epi) && !bias) return fail(PTG_ERR_INVALID_ARG, "%s: epilogue needs a bias", fn);
    if (M_total >= ((int64_t)1 << 31)) return fail(PTG_ERR_UNSUPPORTED, "%s: M_total must fit int32 offsets", fn);
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || (bias && !aligned16(bias)) ||
        (reinterpret_cast<uintptr_t>(group_offsets) & 3u))
      return fail(PTG_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (offsets 4-byte)", fn);
    const bool kn = w_layout == PTG_B_KN;
    if (!fits31(256, K, K) || !(kn ? fits31(K, N, 256) : fits31(256, K, K)) ||
        !out_fits(N, y_dtype == PTG_F32 ? 4 : 2))
      return fail(PTG_ERR_UNSUPPORTED, "%s: operand or output tile exceeds 2 GiB of addressing", fn);
    ptg::GroupedLaunch g{};
    if (with_ws) {
      if (!workspace) return fail(PTG_ERR_WORKSPACE, "%s: workspace is NULL", fn);
      if (!aligned16(workspace)) return fail(PTG_ERR_UNSUPPORTED, "%s: workspace must be 16-byte aligned", fn);
      const size_t need = ptg::grouped_split_workspace_bytes(ptg::device_compute_units());
      if (ws_bytes < need)
        return fail(PTG_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
      g.workspace = workspace;
      g.ws_bytes = ws_bytes;
      g.epoch = next_epoch();
    }
    g.X = X; g.W = W; g.Y = Y; g.bias = needs_bias(epi) ? bias : nullptr; g.offsets = group_offsets;
    g.M_total = M_total; g.N = N; g.K = K; g.G = G;
    g.b_kn = kn; g.epi = epi; g.out_f32 = y_dtype == PTG_F32;
    if (env_on("PTG_CHECK")) {
      st = ptg_grouped_gemm_check(G, M_total, group_offsets, stream);
      if (st) return st;
    }
    log_launch("%s G=%d M_total=%lld N=%lld K=%lld %s %s: tile 256x256x64, 2 slots, 8 consumer and 4 producer waves%s",
               fn, G, (long long)M_total, (long long)N, (long long)K, kn ? "KN" : "NK", g.out_f32 ? "fp32" : "bf16",
               with_ws ? ", last round split through the workspace" : "");
    hipError_t e = ptg::launch_grouped(g, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

}  // namespace

extern "C" {

ptg_status ptg_grouped_gemm(int32_t G, int64_t M_total, int64_t N, int64_t K, const void* X,
                            const void* W, ptg_layout w_layout, const int32_t* group_offsets,
                            void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                            void* stream) {
  return grouped_call("ptg_grouped_gemm", G, M_total, N, K, X, W, w_layout, group_offsets, Y, y_dtype, bias, epi,
                      nullptr, 0, false, stream);
}

size_t ptg_grouped_gemm_split_workspace(void) {
  const int cus = ptg::device_compute_units();
  return cus > 0 ? ptg::grouped_split_workspace_bytes(cus) : 0;
}

ptg_status ptg_grouped_gemm_split(int32_t G, int64_t M_total, int64_t N, int64_t K, const void* X,
                                  const void* W, ptg_layout w_layout, const int32_t* group_offsets,
                                  void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                                  void* workspace, size_t ws_bytes, void* stream) {
  return grouped_call("ptg_grouped_gemm_split", G, M_total, N, K, X, W, w_layout, group_offsets, Y, y_dtype, bias,
                      epi, workspace, ws_bytes, true, stream);
}

size_t ptg_grouped_gemm_wgrad_workspace(void) { return ptg::kWgradWorkspace; }

ptg_status ptg_grouped_gemm_wgrad(int32_t G, int64_t M_total, int64_t K, int64_t N, const void* X,
                                  const void* dY, const int32_t* group_offsets, void* dW,
                                  ptg_dtype dw_dtype, void* workspace, size_t ws_bytes, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_grouped_gemm_wgrad";
    if (G <= 0) return fail(PTG_ERR_INVALID_ARG, "%s: G must be positive", fn);
    if (G > ptg::kMaxGroups) return fail(PTG_ERR_UNSUPPORTED, "%s: G exceeds %d", fn, ptg::kMaxGroups);
    if (bad_dim(M_total) || bad_dim(K) || bad_dim(N))
      return fail(PTG_ERR_INVALID_ARG, "%s: negative size (M_total=%lld K=%lld N=%lld)", fn,
                  (long long)M_total, (long long)K, (long long)N);
    if (K % 8 || N % 8)
      return fail(PTG_ERR_UNSUPPORTED, "%s: K and N must be multiples of 8 (K=%lld N=%lld)", fn, (long long)K,
                  (long long)N);
    if (K > ptg::kMaxDim || N > ptg::kMaxDim) return fail(PTG_ERR_UNSUPPORTED, "%s: dimension too large", fn);
    if (M_total >= ((int64_t)1 << 31)) return fail(PTG_ERR_UNSUPPORTED, "%s: M_total must fit int32 offsets", fn);
    if (dw_dtype != PTG_BF16 && dw_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (K == 0 || N == 0) return PTG_OK;
    if (!dW || !group_offsets || (M_total > 0 && (!X || !dY)))
      return fail(PTG_ERR_INVALID_ARG, "%s: null operand", fn);
    if (!workspace || ws_bytes < ptg::kWgradWorkspace)
      return fail(PTG_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, ptg::kWgradWorkspace, ws_bytes);
    if ((X && !aligned16(X)) || (dY && !aligned16(dY)) || !aligned16(dW) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(group_offsets) & 3u))
      return fail(PTG_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (offsets 4-byte)", fn);
    // one tile's operand descriptors span up to an expert's whole row range of X and dY
    if (!fits31(M_total, K, K) || !fits31(M_total, N, N) || !fits31(512, N, 2 * N))
      return fail(PTG_ERR_UNSUPPORTED, "%s: operand exceeds 2 GiB of addressing", fn);
    ptg::WgradLaunch w{};
    w.X = X; w.dY = dY; w.dW = dW; w.offsets = group_offsets; w.workspace = workspace;
    w.M_total = M_total; w.K = K; w.N = N; w.G = G;
    w.out_f32 = dw_dtype == PTG_F32;
    if (env_on("PTG_CHECK")) {
      const ptg_status st = ptg_grouped_gemm_check(G, M_total, group_offsets, stream);
      if (st) return st;
    }
    log_launch("%s G=%d M_total=%lld K=%lld N=%lld %s: tile 256x256x64 (A staged K x M), 2 slots, 8 consumer and 4 "
               "producer waves, tiles from per-XCD queues", fn, G, (long long)M_total, (long long)K, (long long)N,
               w.out_f32 ? "fp32" : "bf16");
    hipError_t e = ptg::launch_grouped_wgrad(w, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

ptg_status ptg_ikbo_attention(int64_t U, int64_t Mc, int64_t H, int64_t D, int64_t L, float scale,
                              const void* Q, const void* K, const void* V, const int32_t* user_offsets,
                              void* O, ptg_dtype o_dtype, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_ikbo_attention";
    if (U <= 0 || Mc < 0 || H <= 0 || D <= 0 || L <= 0)
      return fail(PTG_ERR_INVALID_ARG, "%s: U, H, D, L must be positive and Mc >= 0", fn);
    if (U > ptg::kMaxGroups) return fail(PTG_ERR_UNSUPPORTED, "%s: U exceeds %d", fn, ptg::kMaxGroups);
    if (D != ptg::kAttnHeadDim) return fail(PTG_ERR_UNSUPPORTED, "%s: head dimension must be %d", fn, ptg::kAttnHeadDim);
    if (L % 64) return fail(PTG_ERR_UNSUPPORTED, "%s: L must be a multiple of 64 (L=%lld)", fn, (long long)L);
    if (o_dtype != PTG_BF16 && o_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
      return fail(PTG_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (Mc == 0) return PTG_OK;
    if (!Q || !K || !V || !O || !user_offsets) return fail(PTG_ERR_INVALID_ARG, "%s: null operand", fn);
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
        (reinterpret_cast<uintptr_t>(user_offsets) & 3u))
      return fail(PTG_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (offsets 4-byte)", fn);
    // 32-bit buffer offsets: all of Q or O, and one user's and head's rows of K or V
    const int64_t row_elems = H * D;
    if (Mc >= ((int64_t)1 << 31) || Mc * row_elems * 4 >= ((int64_t)1 << 31) || L * row_elems * 2 >= ((int64_t)1 << 31))
      return fail(PTG_ERR_UNSUPPORTED, "%s: operand exceeds 2 GiB of addressing", fn);
    ptg::AttentionLaunch a{};
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.offsets = user_offsets;
    a.U = U; a.Mc = Mc; a.H = H; a.L = L; a.scale = scale; a.out_f32 = o_dtype == PTG_F32;
    if (env_on("PTG_CHECK")) {
      const ptg_status st = ptg_grouped_gemm_check((int32_t)U, Mc, user_offsets, stream);
      if (st) return st;
    }
    log_launch("%s U=%lld Mc=%lld H=%lld D=%lld L=%lld %s: 128 candidates per tile, 64-key blocks in 4 slots", fn,
               (long long)U, (long long)Mc, (long long)H, (long long)D, (long long)L, a.out_f32 ? "fp32" : "bf16");
    hipError_t e = ptg::launch_attention(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

ptg_status ptg_grouped_gemm_check(int32_t G, int64_t M_total, const int32_t* group_offsets, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_grouped_gemm_check";
    if (G <= 0 || M_total < 0 || !group_offsets) return fail(PTG_ERR_INVALID_ARG, "%s: bad arguments", fn);
    int bad = 0;
    int busy = 0;
    hipError_t e = ptg::check_offsets(group_offsets, G, M_total, reinterpret_cast<hipStream_t>(stream), &bad, &busy);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (busy) return fail(PTG_ERR_UNSUPPORTED, "%s: %d checks already in flight", fn, ptg::kCheckWords);
    if (bad) return fail(PTG_ERR_DEVICE_CHECK, "%s: group offsets violate the precondition", fn);
    return watchdog_status(fn);
  })
}

ptg_status ptg_broadcast_gemm_check(int64_t U, int64_t Mc, const int32_t* user_idx, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_broadcast_gemm_check";
    if (U <= 0 || Mc < 0 || (Mc > 0 && !user_idx)) return fail(PTG_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (Mc == 0) return watchdog_status(fn);
    int bad = 0;
    int busy = 0;
    hipError_t e = ptg::check_index(user_idx, Mc, U, reinterpret_cast<hipStream_t>(stream), &bad, &busy);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (busy) return fail(PTG_ERR_UNSUPPORTED, "%s: %d checks already in flight", fn, ptg::kCheckWords);
    if (bad) return fail(PTG_ERR_DEVICE_CHECK, "%s: a user index is outside [0, U)", fn);
    return watchdog_status(fn);
  })
}

size_t ptg_grouped_gemm_ptr_array_workspace(int32_t count) {
  if (count <= 0) return 0;
  return ptg::batch_workspace_bytes(count);
}

}  // extern "C"

namespace {

ptg_status validate_problem(const char* fn, int32_t p, const ptg_problem& q, ptg_dtype c_dtype, ptg_epilogue epi) {
  if (q.M < 0 || q.N < 0 || q.K < 0) return fail(PTG_ERR_INVALID_ARG, "%s: problem %d: negative size", fn, p);
  if (q.K == 0) return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: K = 0", fn, p);
  if (q.K % 8 || q.N % 8) return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: N and K must be multiples of 8", fn, p);
  if (q.M >= ((int64_t)1 << 30) || q.N >= ((int64_t)1 << 30) || q.K >= ((int64_t)1 << 30))
    return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: dimension too large", fn, p);
  if (q.M == 0 || q.N == 0) return PTG_OK;
  if (!q.A || !q.B || !q.C) return fail(PTG_ERR_INVALID_ARG, "%s: problem %d: null operand", fn, p);
  if (needs_bias(epi) && !q.bias) return fail(PTG_ERR_INVALID_ARG, "%s: problem %d: epilogue needs a bias", fn, p);
  if (q.lda < q.K || q.ldb < q.N || q.ldc < q.N) return fail(PTG_ERR_INVALID_ARG, "%s: problem %d: leading dimension too small", fn, p);
  if (q.lda % 8 || q.ldb % 8 || q.ldc % 8) return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: leading dimensions must be multiples of 8", fn, p);
  if (!aligned16(q.A) || !aligned16(q.B) || !aligned16(q.C) || (q.bias && !aligned16(q.bias)))
    return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: pointers must be 16-byte aligned", fn, p);
  if (!fits31(256, q.lda, q.K) || !fits31(q.K, q.ldb, 256) || !out_fits(q.ldc, c_dtype == PTG_F32 ? 4 : 2))
    return fail(PTG_ERR_UNSUPPORTED, "%s: problem %d: operand or output tile exceeds 2 GiB of addressing", fn, p);
  return PTG_OK;
}

// Pinned host buffers that stage a problem table on its way to the device, per device.  A
// buffer is handed out again once the copy that read it has completed (its event), so a
// call returns as soon as the copy is enqueued and the caller's array may be freed at once.
struct StagingBuffer {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;   // recorded on the stream after the copy
};
struct StagingPool {
  std::mutex mu;
  std::vector<StagingBuffer> bufs;
  size_t next = 0;             // the buffer waited for when all are in flight (round robin)
};
constexpr size_t kStagingBuffers = 8;

StagingPool& staging_pool(int dev) {
  static std::mutex mu;
  static std::vector<std::unique_ptr<StagingPool>> pools;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)pools.size() <= dev) pools.resize(dev + 1);
  if (!pools[dev]) pools[dev].reset(new StagingPool);
  return *pools[dev];
}

// Copies `bytes` from `fill` (a function writing the table into a host buffer) to the device
// pointer `dst` on `stream` through a pinned staging buffer.
template <class Fill>
hipError_t staged_copy(void* dst, size_t bytes, hipStream_t stream, Fill fill) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  StagingPool& pool = staging_pool(dev);
  std::lock_guard<std::mutex> lock(pool.mu);
  StagingBuffer* b = nullptr;
  for (StagingBuffer& c : pool.bufs) {
    if (c.cap >= bytes && hipEventQuery(c.done) == hipSuccess) {
      b = &c;
      break;
    }
  }
  if (!b && pool.bufs.size() < kStagingBuffers) {
    pool.bufs.emplace_back();
    b = &pool.bufs.back();
    e = hipEventCreateWithFlags(&b->done, hipEventDisableTiming);
    if (e != hipSuccess) {
      pool.bufs.pop_back();
      return e;
    }
  }
  if (!b) {
    // every buffer is in flight (or too small): wait for the oldest one handed out
    b = &pool.bufs[pool.next % pool.bufs.size()];
    pool.next++;
    e = hipEventSynchronize(b->done);
    if (e != hipSuccess) return e;
  }
  if (b->cap < bytes) {
    if (b->host) {
      e = hipEventSynchronize(b->done);
      if (e != hipSuccess) return e;
      (void)hipHostFree(b->host);
      b->host = nullptr;
      b->cap = 0;
    }
    const size_t cap = std::max<size_t>(bytes, 64 << 10);
    e = hipHostMalloc(&b->host, cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      b->host = nullptr;
      return e;
    }
    b->cap = cap;
  }
  fill(static_cast<char*>(b->host));
  e = hipMemcpyAsync(dst, b->host, bytes, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipEventRecord(b->done, stream);
  return e;
}

}  // namespace

extern "C" {

ptg_status ptg_grouped_gemm_ptr_array_prepare(int32_t count, const ptg_problem* problems, ptg_dtype c_dtype,
                                              ptg_epilogue epi, void* workspace, size_t ws_bytes, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_grouped_gemm_ptr_array_prepare";
    if (count <= 0 || !problems) return fail(PTG_ERR_INVALID_ARG, "%s: count must be positive and problems non-null", fn);
    if (count > ptg::kMaxBatch) return fail(PTG_ERR_UNSUPPORTED, "%s: count exceeds %d", fn, ptg::kMaxBatch);
    if (c_dtype != PTG_BF16 && c_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!valid_epi(epi)) return fail(PTG_ERR_UNSUPPORTED, "%s: bad epilogue", fn);
    const size_t need = ptg::batch_workspace_bytes(count);
    if (!workspace || ws_bytes < need)
      return fail(PTG_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (!aligned16(workspace)) return fail(PTG_ERR_UNSUPPORTED, "%s: workspace must be 16-byte aligned", fn);
    for (int32_t p = 0; p < count; ++p) {
      ptg_status st = validate_problem(fn, p, problems[p], c_dtype, epi);
      if (st) return st;
    }
    const int64_t osz = c_dtype == PTG_F32 ? 4 : 2;
    // Table order = tile order of the launch, whose workgroups take tiles round-robin: the
    // problems with the most k-steps per tile go first (stable, so equal costs keep the
    // caller's order), and the cheapest tiles are the last round's, which then ends evenly.
    // Every problem writes only its own output, so the order changes no result.
    std::vector<int32_t> order(count);
    for (int32_t p = 0; p < count; ++p) order[p] = p;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      return (problems[x].K + 63) / 64 > (problems[y].K + 63) / 64;
    });
    int64_t total = 0;
    for (int32_t p = 0; p < count; ++p) {
      const ptg_problem& q = problems[p];
      if (q.M > 0 && q.N > 0) total += ((q.M + ptg::kBatchBM - 1) / ptg::kBatchBM) * ((q.N + ptg::kBatchBN - 1) / ptg::kBatchBN);
    }
    if (total >= ((int64_t)1 << 31)) return fail(PTG_ERR_UNSUPPORTED, "%s: too many tiles", fn);
    auto fill = [&](char* host) {
      std::memset(host, 0, need);
      auto* hdr = reinterpret_cast<ptg::BatchHeader*>(host);
      auto* pre = reinterpret_cast<int32_t*>(host + sizeof(ptg::BatchHeader));
      auto* rec = reinterpret_cast<ptg::BatchProblem*>(host + sizeof(ptg::BatchHeader) + ptg::batch_prefix_bytes(count));
      ptg::Guards& gu = hdr->guard;
      gu.a_lo = gu.b_lo = gu.c_lo = gu.bias_lo = UINT64_MAX;
      gu.a_hi = gu.b_hi = gu.c_hi = gu.bias_hi = 0;
      auto widen = [](uint64_t& lo, uint64_t& hi, const void* ptr, uint64_t bytes) {
        const uint64_t a = reinterpret_cast<uint64_t>(ptr);
        if (a < lo) lo = a;
        if (a + bytes > hi) hi = a + bytes;
      };
      int64_t run = 0;
      for (int32_t p = 0; p < count; ++p) {
        const ptg_problem& q = problems[order[p]];
        ptg::BatchProblem& r = rec[p];
        r.A = q.A; r.B = q.B; r.C = q.C; r.bias = needs_bias(epi) ? q.bias : nullptr;
        r.lda = q.lda; r.ldb = q.ldb; r.ldc = q.ldc;
        r.M = (int32_t)q.M; r.N = (int32_t)q.N; r.K = (int32_t)q.K;
        const bool empty = q.M == 0 || q.N == 0;
        r.tiles_m = empty ? 0 : (int32_t)((q.M + ptg::kBatchBM - 1) / ptg::kBatchBM);
        r.tiles_n = empty ? 0 : (int32_t)((q.N + ptg::kBatchBN - 1) / ptg::kBatchBN);
        if (!empty) {
          widen(gu.a_lo, gu.a_hi, q.A, (uint64_t)(((q.M - 1) * q.lda + q.K) * 2));
          widen(gu.b_lo, gu.b_hi, q.B, (uint64_t)(((q.K - 1) * q.ldb + q.N) * 2));
          widen(gu.c_lo, gu.c_hi, q.C, (uint64_t)(((q.M - 1) * q.ldc + q.N) * osz));
          if (r.bias) widen(gu.bias_lo, gu.bias_hi, r.bias, (uint64_t)q.N * 4);
        }
        pre[p] = (int32_t)run;
        run += (int64_t)r.tiles_m * r.tiles_n;
      }
      pre[count] = (int32_t)run;
      if (gu.a_lo > gu.a_hi) gu.a_lo = gu.a_hi = 0;
      if (gu.b_lo > gu.b_hi) gu.b_lo = gu.b_hi = 0;
      if (gu.c_lo > gu.c_hi) gu.c_lo = gu.c_hi = 0;
      if (gu.bias_lo > gu.bias_hi) gu.bias_lo = gu.bias_hi = 0;
      hdr->magic = ptg::kBatchMagic;
      hdr->count = count;
      hdr->total_tiles = (int32_t)run;
      hdr->bm = ptg::kBatchBM;
      hdr->bn = ptg::kBatchBN;
      hdr->epi = epi;
      hdr->out_f32 = c_dtype == PTG_F32;
    };
    hipError_t e = staged_copy(workspace, need, reinterpret_cast<hipStream_t>(stream), fill);
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

ptg_status ptg_grouped_gemm_ptr_array_run(int32_t count, const void* workspace, size_t ws_bytes, ptg_dtype c_dtype,
                                          ptg_epilogue epi, void* stream) {
  PTG_TRY({
    const char* fn = "ptg_grouped_gemm_ptr_array_run";
    if (count <= 0) return fail(PTG_ERR_INVALID_ARG, "%s: count must be positive", fn);
    if (count > ptg::kMaxBatch) return fail(PTG_ERR_UNSUPPORTED, "%s: count exceeds %d", fn, ptg::kMaxBatch);
    if (c_dtype != PTG_BF16 && c_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!valid_epi(epi)) return fail(PTG_ERR_UNSUPPORTED, "%s: bad epilogue", fn);
    const size_t need = ptg::batch_workspace_bytes(count);
    if (!workspace || ws_bytes < need)
      return fail(PTG_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (!aligned16(workspace)) return fail(PTG_ERR_UNSUPPORTED, "%s: workspace must be 16-byte aligned", fn);
    ptg::BatchLaunch b{};
    b.workspace = workspace; b.count = count; b.epi = epi; b.out_f32 = c_dtype == PTG_F32;
    log_launch("%s count=%d %s: tile 128x128x64, 4 slots, 2 groups of 4 consumer waves, 2 producer waves", fn, count,
               b.out_f32 ? "fp32" : "bf16");
    hipError_t e = ptg::launch_batch(b, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}

ptg_status ptg_grouped_gemm_ptr_array(int32_t count, const ptg_problem* problems, ptg_dtype c_dtype,
                                      ptg_epilogue epi, void* workspace, size_t ws_bytes, void* stream) {
  ptg_status st = ptg_grouped_gemm_ptr_array_prepare(count, problems, c_dtype, epi, workspace, ws_bytes, stream);
  if (st) return st;
  return ptg_grouped_gemm_ptr_array_run(count, workspace, ws_bytes, c_dtype, epi, stream);
}

size_t ptg_broadcast_gemm_workspace(int64_t U, int64_t N) {
  if (U <= 0 || N <= 0) return 0;
  const int32_t splits = ptg::broadcast_user_splits(U, N);
  // P, then one partial product per split when the user phase splits K
  return (size_t)U * (size_t)N * sizeof(float) * (splits > 1 ? 1 + (size_t)splits : 1);
}

size_t ptg_broadcast_gemm_fused_workspace(int64_t U, int64_t N) {
  if (U <= 0 || N <= 0) return 0;
  // the sync words, P, then up to 32 partial products
  return ptg::broadcast_sync_bytes(N, ptg::kBroadcastMaxSlices) +
         (size_t)U * (size_t)N * sizeof(float) * (1 + (size_t)ptg::kBroadcastMaxSlices);
}

}  // extern "C"

namespace {
// The broadcast GEMM behind the entry points.  `scratch(need, &ws, &bytes)` supplies the
// workspace once every host-checkable argument has passed (the caller's, or the library's
// static array), or returns an error status.  `fused`: one persistent launch.
template <class Scratch>
ptg_status broadcast_call(const char* fn, int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N, const void* Xu,
                          const void* Xc, const int32_t* user_idx, const void* W, ptg_layout w_layout,
                          void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                          Scratch scratch, void* stream, bool fused = false) {
  PTG_TRY({
    ptg_status st = PTG_OK;
    if (U <= 0 || Mc < 0 || Ku < 0 || Kc < 0 || N < 0)
      return fail(PTG_ERR_INVALID_ARG, "%s: bad sizes (U must be positive)", fn);
    if (Ku == 0 || Kc == 0) return fail(PTG_ERR_UNSUPPORTED, "%s: Ku and Kc must be positive", fn);
    if (Ku % 8 || Kc % 8 || N % 8) return fail(PTG_ERR_UNSUPPORTED, "%s: Ku, Kc and N must be multiples of 8", fn);
    if (U > ptg::kMaxDim || Mc > ptg::kMaxDim || Ku + Kc > ptg::kMaxDim || N > ptg::kMaxDim)
      return fail(PTG_ERR_UNSUPPORTED, "%s: a dimension exceeds 2^30", fn);
    if (w_layout != PTG_B_KN && w_layout != PTG_B_NK) return fail(PTG_ERR_UNSUPPORTED, "%s: bad layout", fn);
    if (y_dtype != PTG_BF16 && y_dtype != PTG_F32) return fail(PTG_ERR_UNSUPPORTED, "%s: bad output dtype", fn);
    if (!valid_epi(epi)) return fail(PTG_ERR_UNSUPPORTED, "%s: bad epilogue", fn);
    if (Mc == 0 || N == 0) return PTG_OK;
    if (!Xu || !Xc || !user_idx || !W || !Y) return fail(PTG_ERR_INVALID_ARG, "%s: null operand", fn);
    if (needs_bias(epi) && !bias) return fail(PTG_ERR_INVALID_ARG, "%s: epilogue needs a bias", fn);
    if (!aligned16(Xu) || !aligned16(Xc) || !aligned16(W) || !aligned16(Y) ||
        (bias && !aligned16(bias)) || (reinterpret_cast<uintptr_t>(user_idx) & 3u))
      return fail(PTG_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (indices 4-byte)", fn);
    const int64_t Kt = Ku + Kc;
    const bool kn = w_layout == PTG_B_KN;
    if (!fits31(256, Ku, Ku) || !fits31(256, Kc, Kc) || !(kn ? fits31(Kt, N, 256) : fits31(256, Kt, Kt)) ||
        !out_fits(N, y_dtype == PTG_F32 ? 4 : 2))
      return fail(PTG_ERR_UNSUPPORTED, "%s: operand or output tile exceeds 2 GiB of addressing", fn);
    if (U * N * 4 >= ((int64_t)1 << 31))
      return fail(PTG_ERR_UNSUPPORTED, "%s: P (U x N fp32) exceeds 2 GiB of addressing", fn);
    // the one-launch form: at most 256 users (one m-tile), at least two 64-deep slices of Ku,
    // the sync words of every column block in their 4 KB block, and a workspace under 2 GiB
    // (its reduction units address it with 31-bit offsets)
    const int64_t max_splits1 = ptg::kBroadcastMaxSlices;
    const int64_t unit_steps = std::max<int64_t>(1, (Kc + 63) / 64 / 2);
    int64_t chunk1 = std::min<int64_t>(unit_steps * 64, (Ku + 127) / 128 * 64);
    if ((Ku + chunk1 - 1) / chunk1 > max_splits1) chunk1 = ((Ku + max_splits1 - 1) / max_splits1 + 63) / 64 * 64;
    const int32_t splits1 = (int32_t)((Ku + chunk1 - 1) / chunk1);
    if (fused && (!ptg::broadcast_single_launch_fits(U, N, splits1) ||
                  ptg_broadcast_gemm_fused_workspace(U, N) >= ((size_t)1 << 31)))
      return fail(PTG_ERR_UNSUPPORTED,
                  "%s: one launch needs U <= 256, Ku > 64, N <= %lld and a workspace under 2 GiB", fn,
                  (long long)((ptg::broadcast_flags_offset() / 8 - 1) * 256));
    void* workspace = nullptr;
    size_t ws_bytes = 0;
    const size_t need = fused ? ptg_broadcast_gemm_fused_workspace(U, N) : ptg_broadcast_gemm_workspace(U, N);
    st = scratch(need, &workspace, &ws_bytes);
    if (st) return st;
    if (!workspace || ws_bytes < need)
      return fail(PTG_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (!aligned16(workspace)) return fail(PTG_ERR_UNSUPPORTED, "%s: workspace must be 16-byte aligned", fn);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (env_on("PTG_CHECK")) {
      st = ptg_broadcast_gemm_check(U, Mc, user_idx, stream);
      if (st) return st;
    }
    if (fused) {
      // User units (slice s of Ku for one 256-column block, its fp32 partial product to the
      // workspace), reduction units (rows of P summed from the partials once all have
      // arrived) and candidate tiles (started from P once their column block is ready) in
      // one persistent launch.  Each user unit takes about half a candidate tile's k-steps.
      ptg::BroadcastLaunch b{};
      b.Xu = Xu; b.Xc = Xc; b.idx = user_idx; b.W = W; b.Y = Y;
      b.bias = needs_bias(epi) ? bias : nullptr;
      b.workspace = workspace;
      b.U = U; b.Mc = Mc; b.Ku = Ku; b.Kc = Kc; b.N = N;
      b.S = splits1; b.k_chunk = chunk1;
      b.sync_bytes = ptg::broadcast_sync_bytes(N, ptg::kBroadcastMaxSlices);
      b.b_kn = kn; b.epi = epi; b.out_f32 = y_dtype == PTG_F32;
      b.epoch = next_epoch();
      log_launch("%s U=%lld Mc=%lld Ku=%lld Kc=%lld N=%lld: one launch, %d user slices of %lld, tile 256x256x64", fn,
                 (long long)U, (long long)Mc, (long long)Ku, (long long)Kc, (long long)N, splits1, (long long)chunk1);
      const hipError_t e = ptg::launch_broadcast_single(b, s);
      if (e != hipSuccess) return hip_fail(e, fn);
      return PTG_OK;
    }
    float* P = reinterpret_cast<float*>(workspace);
    // Matmul decomposition: the user half of W meets each user's features once ...
    ptg::DenseLaunch u{};
    u.A = Xu; u.lda = Ku;
    u.B = W; u.ldb = kn ? N : Kt;
    u.C = P; u.ldc = N;
    u.M = U; u.N = N; u.K = Ku;
    u.b_kn = kn; u.out_f32 = 1;
    // The user product is small (U rows): split K so that it spreads over the chip, each
    // split writing a partial product after P, then sum the partials in split order (the
    // result does not depend on timing) and add the bias, which rides along with P.
    const int32_t max_splits = ptg::broadcast_user_splits(U, N);
    const int64_t chunk = ((Ku + max_splits - 1) / max_splits + 63) / 64 * 64;  // whole k-steps
    const int32_t splits = (int32_t)((Ku + chunk - 1) / chunk);
    {
      int32_t cu[6];
      int32_t cc[6];
      ptg::dense_config(U, N, Ku, kn, cu);
      ptg::dense_config(Mc, N, Kc, kn, cc);
      log_launch("%s U=%lld Mc=%lld Ku=%lld Kc=%lld N=%lld: user phase tile %dx%dx%d in %d slices of %lld%s, "
                 "candidate phase tile %dx%dx%d", fn, (long long)U, (long long)Mc, (long long)Ku, (long long)Kc,
                 (long long)N, cu[0], cu[1], cu[2], splits, (long long)chunk, splits > 1 ? " + ordered reduction" : "",
                 cc[0], cc[1], cc[2]);
    }
    hipError_t e;
    if (splits > 1) {
      u.C = P + U * N;
      u.splits = splits; u.k_chunk = chunk; u.c_split = U * N;
      u.epi = PTG_EPI_NONE;
      e = ptg::launch_dense(u, s);
      if (e != hipSuccess) return hip_fail(e, fn);
      e = ptg::launch_reduce_splits(P, P + U * N, U * N, splits, needs_bias(epi) ? bias : nullptr, N, s);
    } else {
      u.bias = needs_bias(epi) ? bias : nullptr;
      u.epi = needs_bias(epi) ? PTG_EPI_BIAS : PTG_EPI_NONE;
      e = ptg::launch_dense(u, s);
    }
    if (e != hipSuccess) return hip_fail(e, fn);
    // ... and the candidate half runs per candidate, starting from P[user_idx[r]].
    ptg::DenseLaunch c{};
    c.A = Xc; c.lda = Kc;
    c.B = kn ? static_cast<const void*>(static_cast<const char*>(W) + Ku * N * 2)
             : static_cast<const void*>(static_cast<const char*>(W) + Ku * 2);
    c.ldb = kn ? N : Kt;
    c.C = Y; c.ldc = N;
    c.bias = nullptr;
    c.gidx = user_idx; c.P = P; c.ldp = N; c.p_rows = U;
    c.M = Mc; c.N = N; c.K = Kc;
    c.b_kn = kn; c.out_f32 = y_dtype == PTG_F32;
    c.epi = (epi == PTG_EPI_SILU || epi == PTG_EPI_BIAS_SILU) ? PTG_EPI_SILU : PTG_EPI_NONE;
    e = ptg::launch_dense(c, s);
    if (e != hipSuccess) return hip_fail(e, fn);
    return PTG_OK;
  })
}


// Scratch of ptg_broadcast_gemm_noalloc: one array per GPU, held until the process ends.  In
// host code `g_noalloc_scratch` names a host-side stand-in; the device address of each GPU's
// copy comes from hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
__device__ __attribute__((aligned(256))) char g_noalloc_scratch[kNoAllocScratchBytes];

ptg_status noalloc_scratch(const char* fn, void** ptr) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch));
    if (e != hipSuccess) return hip_fail(e, fn);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return PTG_OK;
}

}  // namespace

extern "C" {

ptg_status ptg_broadcast_gemm(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N, const void* Xu,
                              const void* Xc, const int32_t* user_idx, const void* W, ptg_layout w_layout,
                              void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                              void* workspace, size_t ws_bytes, void* stream) {
  return broadcast_call("ptg_broadcast_gemm", U, Mc, Ku, Kc, N, Xu, Xc, user_idx, W, w_layout, Y, y_dtype, bias,
                        epi, [&](size_t, void** ws, size_t* bytes) {
                          *ws = workspace;
                          *bytes = ws_bytes;
                          return PTG_OK;
                        }, stream);
}

ptg_status ptg_broadcast_gemm_fused(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N, const void* Xu,
                                    const void* Xc, const int32_t* user_idx, const void* W, ptg_layout w_layout,
                                    void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return broadcast_call("ptg_broadcast_gemm_fused", U, Mc, Ku, Kc, N, Xu, Xc, user_idx, W, w_layout, Y, y_dtype,
                        bias, epi, [&](size_t, void** ws, size_t* bytes) {
                          *ws = workspace;
                          *bytes = ws_bytes;
                          return PTG_OK;
                        }, stream, true);
}

ptg_status ptg_broadcast_gemm_noalloc(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N, const void* Xu,
                                      const void* Xc, const int32_t* user_idx, const void* W, ptg_layout w_layout,
                                      void* Y, ptg_dtype y_dtype, const float* bias, ptg_epilogue epi,
                                      void* stream) {
  const char* fn = "ptg_broadcast_gemm_noalloc";
  return broadcast_call(fn, U, Mc, Ku, Kc, N, Xu, Xc, user_idx, W, w_layout, Y, y_dtype, bias, epi,
                        [&](size_t need, void** ws, size_t* bytes) {
                          if (need > kNoAllocScratchBytes)
                            return fail(PTG_ERR_UNSUPPORTED, "%s: %zu bytes of scratch needed, at most %zu available",
                                        fn, need, kNoAllocScratchBytes);
                          *bytes = kNoAllocScratchBytes;
                          return noalloc_scratch(fn, ws);
                        }, stream);
}

ptg_status ptg_watchdog(uint32_t* value, int32_t clear) {
  PTG_TRY({
    if (!value) return fail(PTG_ERR_INVALID_ARG, "ptg_watchdog: value is NULL");
    uint32_t gemm = 0;
    uint32_t attention = 0;
    uint32_t onerole = 0;
    hipError_t e = ptg::read_watchdog(&gemm, clear);
    if (e == hipSuccess) e = ptg::read_attention_watchdog(&attention, clear);
    if (e == hipSuccess) e = ptg::read_onerole_watchdog(&onerole, clear);
    if (e != hipSuccess) return hip_fail(e, "ptg_watchdog");
    *value = gemm | attention | onerole;
    return PTG_OK;
  })
}

}  // extern "C"
