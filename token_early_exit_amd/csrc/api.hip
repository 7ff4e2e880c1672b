// C interface of the river library: argument validation, error reporting
// and dispatch to the kernel launchers. Every function here is extern "C";
// nothing throws across the interface.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "common.h"

namespace river_host {

static thread_local char g_err[512] = "";
// test hooks (process-wide; read by every launch, so atomics)
static std::atomic<int> g_compact_path{0};
static std::atomic<int> g_gemm_path{0};
static std::atomic<int> g_decode_path{0};
static std::atomic<int> g_fill_fuse{0};

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

river_status fail(river_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

river_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RIVER_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return RIVER_OK;
}

int compact_path_override() { return g_compact_path.load(std::memory_order_relaxed); }
int gemm_path_override() { return g_gemm_path.load(std::memory_order_relaxed); }
int decode_path_override() { return g_decode_path.load(std::memory_order_relaxed); }
int fill_fuse_override() { return g_fill_fuse.load(std::memory_order_relaxed); }

// event records of river_debug_time_kernels: a fixed table (nothing here
// allocates beyond the events themselves, created on first use and reused)
namespace {
struct TimedLaunch {
  hipEvent_t a = nullptr, b = nullptr;
  int dev = -1, kind = 0;
  bool used = false, ended = false;
};
constexpr int TIMED_MAX = 1024;
std::atomic<int> g_time_on{0};
std::mutex g_time_mu;
TimedLaunch g_timed[TIMED_MAX];
}  // namespace

int debug_timer_begin(hipStream_t s, int kind) {
  if (!g_time_on.load(std::memory_order_relaxed)) return -1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  int dev = -1;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone ||
      hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();   // leave no error behind for the launch checks
    return -1;
  }
  std::lock_guard<std::mutex> lk(g_time_mu);
  int idx = -1;
  for (int i = 0; i < TIMED_MAX && idx < 0; ++i)
    if (!g_timed[i].used && g_timed[i].dev == dev) idx = i;
  for (int i = 0; i < TIMED_MAX && idx < 0; ++i)
    if (g_timed[i].dev < 0) idx = i;
  if (idx < 0) return -1;
  TimedLaunch& t = g_timed[idx];
  if (t.dev < 0) {
    if (hipEventCreate(&t.a) != hipSuccess || hipEventCreate(&t.b) != hipSuccess) {
      if (t.a) (void)hipEventDestroy(t.a);
      t.a = nullptr;
      (void)hipGetLastError();
      return -1;
    }
    t.dev = dev;
  }
  if (hipEventRecord(t.a, s) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  t.kind = kind;
  t.used = true;
  t.ended = false;
  return idx;
}

void debug_timer_end(hipStream_t s, int rec) {
  if (rec < 0 || rec >= TIMED_MAX) return;
  std::lock_guard<std::mutex> lk(g_time_mu);
  TimedLaunch& t = g_timed[rec];
  if (hipEventRecord(t.b, s) == hipSuccess) t.ended = true;
  else (void)hipGetLastError();
}

static bool dt_ok(river_dtype dt) { return dt == RIVER_F32 || dt == RIVER_BF16; }

// leading dimension: >= d and a multiple of 16 bytes
static bool ld_ok(int64_t ld, int d, river_dtype dt) {
  return ld >= d && ((ld * (int64_t)esize(dt)) % 16) == 0;
}

}  // namespace river_host

using namespace river_host;

extern "C" {

const char* river_last_error(void) { return g_err; }

const char* river_version(void) { return "river 0.1.0 (gfx950)"; }

river_status river_debug_set_compact_path(int path) {
  if (path < 0 || path > 4) return fail(RIVER_ERR_ARG, "compact path must be 0..4, got %d", path);
  g_compact_path.store(path, std::memory_order_relaxed);
  return RIVER_OK;
}

river_status river_debug_set_gemm_path(int path) {
  if (path < 0 || path > 3) return fail(RIVER_ERR_ARG, "gemm path must be 0..3, got %d", path);
  g_gemm_path.store(path, std::memory_order_relaxed);
  return RIVER_OK;
}

river_status river_debug_set_decode_path(int path) {
  if (path < 0 || path > 1) return fail(RIVER_ERR_ARG, "decode path must be 0..1, got %d", path);
  g_decode_path.store(path, std::memory_order_relaxed);
  return RIVER_OK;
}

river_status river_debug_set_fill_fuse(int mode) {
  if (mode < 0 || mode > 2) return fail(RIVER_ERR_ARG, "fill fuse mode must be 0..2, got %d", mode);
  g_fill_fuse.store(mode, std::memory_order_relaxed);
  return RIVER_OK;
}

river_status river_debug_time_kernels(int on) {
  g_time_on.store(on != 0, std::memory_order_relaxed);
  return RIVER_OK;
}

river_status river_debug_kernel_times(int kind, double* total_ms, int* launches) {
  g_err[0] = 0;
  if (kind != RIVER_TIMED_FILL_PROJECTION && kind != RIVER_TIMED_FILL_PRODUCT)
    return fail(RIVER_ERR_ARG, "kernel_times: unknown launch kind %d", kind);
  if (!total_ms || !launches) return fail(RIVER_ERR_ARG, "kernel_times: null output");
  std::lock_guard<std::mutex> lk(g_time_mu);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(RIVER_ERR_HIP, "kernel_times: hipGetDevice failed");
  double sum = 0.0;
  int n = 0;
  river_status st = RIVER_OK;
  for (int i = 0; i < TIMED_MAX; ++i) {
    TimedLaunch& t = g_timed[i];
    if (!t.used || t.kind != kind) continue;
    t.used = false;
    if (!t.ended || st != RIVER_OK) continue;
    float ms = 0.f;
    hipError_t e = t.dev == cur ? hipSuccess : hipSetDevice(t.dev);
    if (e == hipSuccess) e = hipEventSynchronize(t.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
    if (e != hipSuccess) {
      st = fail(RIVER_ERR_HIP, "kernel_times: %s", hipGetErrorString(e));
      continue;
    }
    sum += ms;
    ++n;
  }
  if (hipSetDevice(cur) != hipSuccess && st == RIVER_OK)
    st = fail(RIVER_ERR_HIP, "kernel_times: restoring the device failed");
  *total_ms = sum;
  *launches = n;
  return st;
}

river_status river_debug_kv_fill_plan(int m_max, int dev_count, int d, int n_out, int n_layers,
                                      size_t ws_bytes, int* chunk, int* path, int* parts) {
  g_err[0] = 0;
  if (m_max < 1 || d < 256 || d % 256 || n_out < 64 || n_out % 64 || n_layers < 1 || !chunk || !path || !parts)
    return fail(RIVER_ERR_ARG, "kv_fill_plan: the plain MFMA fill's shape is needed");
  if (ws_bytes < kv_fill_workspace(m_max, d, 1, RIVER_BF16))
    return fail(RIVER_ERR_WORKSPACE, "kv_fill_plan: less than one layer of x_hat");
  kv_fill_plan(m_max, dev_count != 0, d, n_out, n_layers, ws_bytes, chunk, path, parts);
  return RIVER_OK;
}

size_t river_workspace_size(int op, int n, int d, int d_out, int n_targets, int n_layers) {
  (void)n_targets;
  switch (op) {
    case RIVER_OP_ROUTE: return 0;
    case RIVER_OP_COMPACT: return n > 0 ? compact_workspace(n) : 0;
    case RIVER_OP_KV_FILL:
      if (n <= 0 || d <= 0 || n_layers <= 0) return 0;
      return kv_fill_workspace(n, d, n_layers, RIVER_BF16) + kv_fill_proj_workspace(n, d, d_out, n_layers);
    case RIVER_OP_KV_FILL_LAYER:
      if (n <= 0 || d <= 0 || n_layers <= 0) return 0;
      return kv_fill_layer_workspace(n, d, n_layers);
    case RIVER_OP_DECODE_STEP:
      if (n <= 0 || d <= 0) return 0;
      return decode_fixed_workspace(n, d, RIVER_F32, n_layers) + (n_layers > 1 ? kv_fill_workspace(n, d, n_layers - 1, RIVER_BF16) : 0) +
             decode_proj_workspace(n, d, d_out, n_layers);
    case RIVER_OP_ROUTER_FIT:
      if (n <= 0 || d <= 0 || d_out <= 0 || n_targets <= 0 || n_layers <= 0) return 0;
      return calib_workspace(n, d, d_out, n_targets, n_layers);
    case RIVER_OP_KV_FOLD:
      if (d <= 0 || d_out <= 0 || n_layers <= 0) return 0;
      return kv_fold_workspace(d, d_out, n_layers, true);
    case RIVER_OP_RIDGE_FIT:
      if (n <= 0 || d <= 0 || d_out <= 0) return 0;
      return ridge_workspace(n, d, d_out, n_layers == RIVER_F32 ? RIVER_F32 : RIVER_BF16);
    default: return 0;
  }
}

river_status river_route(int n, int d, river_dtype dt, const void* h_prev, int64_t ld_prev,
                         const void* h_cur, int64_t ld_cur, const void* gamma, float eps,
                         const void* w_down, const void* w_up, int b, float tau, float theta,
                         river_rule rule, float* cos_out, float* prob_out, uint8_t* mask_out,
                         int32_t* all_exit_out, hipStream_t s) {
  g_err[0] = 0;
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "route: dtype %d is not RIVER_F32 or RIVER_BF16", (int)dt);
  if (n < 0) return fail(RIVER_ERR_ARG, "route: n = %d < 0", n);
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "route: d = %d must be a positive multiple of 8", d);
  if (rule != RIVER_RULE_TOKEN && rule != RIVER_RULE_BATCH_MIN)
    return fail(RIVER_ERR_ARG, "route: unknown rule %d", (int)rule);
  if (isnan(tau) || isnan(theta)) return fail(RIVER_ERR_ARG, "route: tau and theta must not be NaN");
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RIVER_ERR_ARG, "route: eps must be finite and >= 0");
  if (w_down) {
    if (b < 1 || b > 512) return fail(RIVER_ERR_ARG, "route: router width b = %d must be in [1, 512]", b);
    if (!w_up) return fail(RIVER_ERR_ARG, "route: w_up is NULL while w_down is set");
    if (!aligned16(w_down) || !aligned16(w_up)) return fail(RIVER_ERR_ALIGN, "route: router weights must be 16-byte aligned");
  }
  if (gamma && !aligned16(gamma)) return fail(RIVER_ERR_ALIGN, "route: gamma must be 16-byte aligned");
  if (n == 0) {
    if (all_exit_out) return launch_route(0, d, dt, nullptr, d, nullptr, d, nullptr, eps, nullptr,
                                          nullptr, b, tau, theta, rule, nullptr, nullptr, nullptr,
                                          all_exit_out, nullptr, s);
    return RIVER_OK;
  }
  if (!h_prev || !h_cur || !mask_out) return fail(RIVER_ERR_ARG, "route: h_prev, h_cur and mask_out are required");
  if (!ld_ok(ld_prev, d, dt) || !ld_ok(ld_cur, d, dt))
    return fail(RIVER_ERR_ALIGN, "route: leading dims must be >= d and a multiple of 16 bytes");
  if (!aligned16(h_prev) || !aligned16(h_cur)) return fail(RIVER_ERR_ALIGN, "route: hidden states must be 16-byte aligned");
  return launch_route(n, d, dt, h_prev, ld_prev, h_cur, ld_cur, gamma, eps, w_down, w_up, b, tau,
                      theta, rule, cos_out, prob_out, mask_out, all_exit_out, nullptr, s);
}

river_status river_compact(int n, int d, river_dtype dt, const uint8_t* mask, const void* h,
                           int64_t ld_h, const int32_t* row_ids, int32_t* cont_idx,
                           int32_t* exit_idx, int32_t* counts, void* h_cont, int64_t ld_cont,
                           int32_t* row_ids_cont, void* out, int64_t ld_out, int64_t n_out_rows,
                           void* workspace, size_t ws_bytes, hipStream_t s) {
  g_err[0] = 0;
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "compact: dtype %d is not RIVER_F32 or RIVER_BF16", (int)dt);
  if (n < 0) return fail(RIVER_ERR_ARG, "compact: n = %d < 0", n);
  if (!counts) return fail(RIVER_ERR_ARG, "compact: counts is required");
  if (n > 0 && (!mask || !cont_idx || !exit_idx)) return fail(RIVER_ERR_ARG, "compact: mask, cont_idx and exit_idx are required");
  if (n > 0 && !aligned16(mask)) return fail(RIVER_ERR_ALIGN, "compact: mask must be 16-byte aligned");
  bool rows = (h_cont || out);
  if (rows) {
    if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "compact: d = %d must be a positive multiple of 8", d);
    if (n > 0 && !h) return fail(RIVER_ERR_ARG, "compact: h is required when h_cont or out is given");
    if (n > 0 && (!ld_ok(ld_h, d, dt) || !aligned16(h))) return fail(RIVER_ERR_ALIGN, "compact: h misaligned or ld_h invalid");
    if (h_cont && (!ld_ok(ld_cont, d, dt) || !aligned16(h_cont))) return fail(RIVER_ERR_ALIGN, "compact: h_cont misaligned or ld_cont invalid");
    if (out && (!ld_ok(ld_out, d, dt) || !aligned16(out))) return fail(RIVER_ERR_ALIGN, "compact: out misaligned or ld_out invalid");
    if (out && n_out_rows < 0) return fail(RIVER_ERR_ARG, "compact: n_out_rows < 0");
  }
  size_t need = n > 0 ? compact_workspace(n) : 0;
  if (need && (!workspace || ws_bytes < need))
    return fail(RIVER_ERR_WORKSPACE, "compact: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (workspace && !aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "compact: workspace must be 16-byte aligned");
  int p = compact_path_override();
  if (p == 1 && n > 64) return fail(RIVER_ERR_UNSUPPORTED, "compact: forced wave path needs n <= 64");
  return launch_compact(n, d, dt, mask, h, ld_h, row_ids, cont_idx, exit_idx, counts, h_cont,
                        ld_cont, row_ids_cont, out, ld_out, n_out_rows, workspace, ws_bytes, s);
}

river_status river_exit_projection(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                   const void* h, int64_t ld_h, int n_rows,
                                   const int32_t* row_idx, const int32_t* row_ids,
                                   const void* gamma, float eps, void* out, int64_t ld_out,
                                   int64_t n_out_rows, hipStream_t s) {
  g_err[0] = 0;
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "exit_projection: dtype %d is not RIVER_F32 or RIVER_BF16", (int)dt);
  if (m_max < 0 || n_rows < 0 || n_out_rows < 0) return fail(RIVER_ERR_ARG, "exit_projection: negative size");
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "exit_projection: d = %d must be a positive multiple of 8", d);
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RIVER_ERR_ARG, "exit_projection: eps must be finite and >= 0");
  if (m_max == 0) return RIVER_OK;
  if (!h || !out) return fail(RIVER_ERR_ARG, "exit_projection: h and out are required");
  if (!row_idx && m_max > n_rows)
    return fail(RIVER_ERR_ARG, "exit_projection: m_max = %d > n_rows = %d without row_idx", m_max, n_rows);
  if (!ld_ok(ld_h, d, dt) || !aligned16(h)) return fail(RIVER_ERR_ALIGN, "exit_projection: h misaligned or ld_h invalid");
  if (!ld_ok(ld_out, d, dt) || !aligned16(out)) return fail(RIVER_ERR_ALIGN, "exit_projection: out misaligned or ld_out invalid");
  if (gamma && !aligned16(gamma)) return fail(RIVER_ERR_ALIGN, "exit_projection: gamma must be 16-byte aligned");
  return launch_exit_projection(m_max, m_dev, d, dt, h, ld_h, n_rows, row_idx, row_ids, gamma, eps,
                                out, ld_out, n_out_rows, s);
}

// argument checks of a fill (RIVER_OK when the call may go ahead; an empty
// call is valid)
static river_status kv_fill_validate(const char* who, int m_max, int d, river_dtype dt, const void* h,
                                     int64_t ld_h, int n_rows, const int32_t* row_idx,
                                     const int32_t* slot, int n_layers, const void* maps,
                                     const river_w4* wk, const river_w4* wv, const river_layer* L,
                                     int n_kv_heads, int head_dim, void* k_cache, void* v_cache,
                                     int64_t n_slots, void* workspace, size_t ws_bytes) {
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "%s: dtype %d is not RIVER_F32 or RIVER_BF16", who, (int)dt);
  if (m_max < 0 || n_layers < 0 || n_rows < 0) return fail(RIVER_ERR_ARG, "%s: negative size", who);
  if (m_max == 0 || n_layers == 0) return RIVER_OK;
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "%s: d = %d must be a positive multiple of 8", who, d);
  if (n_kv_heads < 1 || head_dim < 1) return fail(RIVER_ERR_ARG, "%s: n_kv_heads and head_dim must be >= 1", who);
  if (!h || !slot || !wk || !wv || !k_cache || !v_cache) return fail(RIVER_ERR_ARG, "%s: a required pointer is NULL", who);
  if (!row_idx && m_max > n_rows) return fail(RIVER_ERR_ARG, "%s: m_max = %d > n_rows = %d without row_idx", who, m_max, n_rows);
  if (n_slots < 1) return fail(RIVER_ERR_ARG, "%s: n_slots must be >= 1", who);
  if (!ld_ok(ld_h, d, dt) || !aligned16(h)) return fail(RIVER_ERR_ALIGN, "%s: h misaligned or ld_h invalid", who);
  for (const river_w4* w : {wk, wv}) {
    if (!w->q || !w->scale || !w->zero) return fail(RIVER_ERR_ARG, "%s: int4 descriptor has a NULL pointer", who);
    if (!dt_ok(w->sz_dtype)) return fail(RIVER_ERR_DTYPE, "%s: scale/zero dtype %d unsupported", who, (int)w->sz_dtype);
    if (w->group < 2 || d % w->group || w->group % 2) return fail(RIVER_ERR_ARG, "%s: group %d must be even and divide d", who, w->group);
    if (!aligned16(w->q)) return fail(RIVER_ERR_ALIGN, "%s: int4 weights must be 16-byte aligned", who);
  }
  if ((int64_t)n_kv_heads * head_dim > (1 << 24)) return fail(RIVER_ERR_ARG, "%s: n_kv_heads * head_dim too large", who);
  if (n_layers > 65535) return fail(RIVER_ERR_UNSUPPORTED, "%s: at most 65535 layers per call", who);
  if (!aligned16(k_cache) || !aligned16(v_cache) || (maps && !aligned16(maps)))
    return fail(RIVER_ERR_ALIGN, "%s: caches and maps must be 16-byte aligned", who);
  const bool norm = L && L->norm_gamma;
  if (L) {
    if (norm && (!(L->norm_eps >= 0.0f) || isinf(L->norm_eps)))
      return fail(RIVER_ERR_ARG, "%s: norm_eps must be finite and >= 0", who);
    if ((L->norm_gamma && !aligned16(L->norm_gamma)) || (L->k_bias && !aligned16(L->k_bias)) ||
        (L->v_bias && !aligned16(L->v_bias)))
      return fail(RIVER_ERR_ALIGN, "%s: norm weight and biases must be 16-byte aligned", who);
    if (L->pos) {
      if (!L->rope_cos || !L->rope_sin || L->n_pos < 1)
        return fail(RIVER_ERR_ARG, "%s: rotation needs rope_cos, rope_sin and n_pos >= 1", who);
      if (head_dim % 2) return fail(RIVER_ERR_ARG, "%s: rotation needs an even head_dim", who);
      if (!aligned16(L->rope_cos) || !aligned16(L->rope_sin))
        return fail(RIVER_ERR_ALIGN, "%s: rotary tables must be 16-byte aligned", who);
    }
  }
  if (maps || norm) {
    const size_t need = L ? kv_fill_layer_workspace(m_max, d, 1) : kv_fill_workspace(m_max, d, 1, dt);
    if (!workspace || ws_bytes < need)
      return fail(RIVER_ERR_WORKSPACE, "%s: at least %zu workspace bytes needed, %zu given", who, need, ws_bytes);
    if (!aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  }
  return RIVER_OK;
}

static river_status kv_fill_checked(const char* who, int m_max, const int32_t* m_dev, int d,
                                    river_dtype dt, const void* h, int64_t ld_h, int n_rows,
                                    const int32_t* row_idx, const int32_t* slot, int n_layers,
                                    const void* maps, const river_w4* wk, const river_w4* wv,
                                    const river_layer* L, int n_kv_heads, int head_dim,
                                    void* k_cache, void* v_cache, int64_t n_slots, void* workspace,
                                    size_t ws_bytes, hipStream_t s) {
  g_err[0] = 0;
  river_status st = kv_fill_validate(who, m_max, d, dt, h, ld_h, n_rows, row_idx, slot, n_layers, maps,
                                     wk, wv, L, n_kv_heads, head_dim, k_cache, v_cache, n_slots,
                                     workspace, ws_bytes);
  if (st != RIVER_OK || m_max == 0 || n_layers == 0) return st;
  return launch_kv_fill(m_max, m_dev, d, dt, h, ld_h, n_rows, row_idx, slot, n_layers, maps, wk, wv,
                        L, n_kv_heads, head_dim, k_cache, v_cache, n_slots, workspace, ws_bytes, s);
}

river_status river_kv_fill(int m_max, const int32_t* m_dev, int d, river_dtype dt, const void* h,
                           int64_t ld_h, int n_rows, const int32_t* row_idx, const int32_t* slot,
                           int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                           int n_kv_heads, int head_dim, void* k_cache, void* v_cache,
                           int64_t n_slots, void* workspace, size_t ws_bytes, hipStream_t s) {
  return kv_fill_checked("kv_fill", m_max, m_dev, d, dt, h, ld_h, n_rows, row_idx, slot, n_layers,
                         maps, wk, wv, nullptr, n_kv_heads, head_dim, k_cache, v_cache, n_slots,
                         workspace, ws_bytes, s);
}

river_status river_kv_fill_layer(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                 const void* h, int64_t ld_h, int n_rows, const int32_t* row_idx,
                                 const int32_t* slot, int n_layers, const void* maps,
                                 const river_w4* wk, const river_w4* wv, const river_layer* layer,
                                 int n_kv_heads, int head_dim, void* k_cache, void* v_cache,
                                 int64_t n_slots, void* workspace, size_t ws_bytes, hipStream_t s) {
  return kv_fill_checked("kv_fill_layer", m_max, m_dev, d, dt, h, ld_h, n_rows, row_idx, slot,
                         n_layers, maps, wk, wv, layer, n_kv_heads, head_dim, k_cache, v_cache,
                         n_slots, workspace, ws_bytes, s);
}

river_status river_kv_fold(int d, int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                           int n_kv_heads, int head_dim, void* F, void* workspace, size_t ws_bytes,
                           hipStream_t s) {
  g_err[0] = 0;
  if (d < 0 || n_layers < 0) return fail(RIVER_ERR_ARG, "kv_fold: negative size");
  if (d == 0 || n_layers == 0) return RIVER_OK;
  if (n_kv_heads < 1 || head_dim < 1) return fail(RIVER_ERR_ARG, "kv_fold: n_kv_heads and head_dim must be >= 1");
  if (!wk || !wv || !F) return fail(RIVER_ERR_ARG, "kv_fold: a required pointer is NULL");
  for (const river_w4* w : {wk, wv}) {
    if (!w->q || !w->scale || !w->zero) return fail(RIVER_ERR_ARG, "kv_fold: int4 descriptor has a NULL pointer");
    if (!dt_ok(w->sz_dtype)) return fail(RIVER_ERR_DTYPE, "kv_fold: scale/zero dtype %d unsupported", (int)w->sz_dtype);
    if (w->group < 2 || d % w->group || w->group % 2) return fail(RIVER_ERR_ARG, "kv_fold: group %d must be even and divide d", w->group);
    if (!aligned16(w->q)) return fail(RIVER_ERR_ALIGN, "kv_fold: int4 weights must be 16-byte aligned");
  }
  if ((int64_t)n_kv_heads * head_dim > (1 << 24)) return fail(RIVER_ERR_ARG, "kv_fold: n_kv_heads * head_dim too large");
  const int nh = n_kv_heads * head_dim;
  if (!kv_fold_ok(d, nh, wk, wv))
    return fail(RIVER_ERR_UNSUPPORTED, "kv_fold: needs d %% 256 == 0, n_out %% 64 == 0 and groups of 64k (d = %d, n_out = %d)", d, nh);
  if (n_layers > 65535) return fail(RIVER_ERR_UNSUPPORTED, "kv_fold: at most 65535 layers per call");
  if (!aligned16(F) || (maps && !aligned16(maps))) return fail(RIVER_ERR_ALIGN, "kv_fold: F and maps must be 16-byte aligned");
  if (maps) {
    const size_t need = kv_fold_workspace(d, nh, 1, true);
    if (!workspace || ws_bytes < need)
      return fail(RIVER_ERR_WORKSPACE, "kv_fold: at least %zu workspace bytes needed, %zu given", need, ws_bytes);
    if (!aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "kv_fold: workspace must be 16-byte aligned");
  }
  return launch_kv_fold(d, n_layers, maps, wk, wv, nh, F, workspace, ws_bytes, s);
}

river_status river_kv_fill_folded(int m_max, const int32_t* m_dev, int d, const void* h, int64_t ld_h,
                                  int n_rows, const int32_t* row_idx, const int32_t* slot, int n_layers,
                                  const void* F, int n_kv_heads, int head_dim, void* k_cache,
                                  void* v_cache, int64_t n_slots, hipStream_t s) {
  g_err[0] = 0;
  if (m_max < 0 || n_layers < 0 || n_rows < 0) return fail(RIVER_ERR_ARG, "kv_fill_folded: negative size");
  if (m_max == 0 || n_layers == 0) return RIVER_OK;
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "kv_fill_folded: d = %d must be a positive multiple of 8", d);
  if (n_kv_heads < 1 || head_dim < 1) return fail(RIVER_ERR_ARG, "kv_fill_folded: n_kv_heads and head_dim must be >= 1");
  if (!h || !slot || !F || !k_cache || !v_cache) return fail(RIVER_ERR_ARG, "kv_fill_folded: a required pointer is NULL");
  if (!row_idx && m_max > n_rows) return fail(RIVER_ERR_ARG, "kv_fill_folded: m_max = %d > n_rows = %d without row_idx", m_max, n_rows);
  if (n_slots < 1) return fail(RIVER_ERR_ARG, "kv_fill_folded: n_slots must be >= 1");
  if (!ld_ok(ld_h, d, RIVER_BF16) || !aligned16(h)) return fail(RIVER_ERR_ALIGN, "kv_fill_folded: h misaligned or ld_h invalid");
  if ((int64_t)n_kv_heads * head_dim > (1 << 24)) return fail(RIVER_ERR_ARG, "kv_fill_folded: n_kv_heads * head_dim too large");
  const int64_t nh = (int64_t)n_kv_heads * head_dim;
  if (d % 256 || nh % 64) return fail(RIVER_ERR_UNSUPPORTED, "kv_fill_folded: needs d %% 256 == 0 and n_out %% 64 == 0");
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)n_rows * ld_h * 2 >= lim || 4 * nh * d >= lim)
    return fail(RIVER_ERR_UNSUPPORTED, "kv_fill_folded: an operand spans 2^31 bytes or more");
  if (n_layers > 65535) return fail(RIVER_ERR_UNSUPPORTED, "kv_fill_folded: at most 65535 layers per call");
  if (!aligned16(F) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(RIVER_ERR_ALIGN, "kv_fill_folded: F and the caches must be 16-byte aligned");
  return launch_kv_fill_folded(m_max, m_dev, d, h, ld_h, n_rows, row_idx, slot, n_layers, F, (int)nh,
                               k_cache, v_cache, n_slots, s);
}

// fork_ok: the step may run one checkpoint's fill on a second stream (made
// on first use); the allocation-free entry point never does
static river_status decode_step(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                                const river_checkpoint* ck, int n_layers, const void* gamma,
                                float eps, int b, river_rule rule, const river_w4* wk,
                                const river_w4* wv, int n_kv_heads, int head_dim,
                                const int32_t* slot, void* k_cache, void* v_cache, int64_t n_slots,
                                int32_t* exit_layer, void* workspace, size_t ws_bytes,
                                hipStream_t s, bool fork_ok) {
  g_err[0] = 0;
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "decode_step: dtype %d is not RIVER_F32 or RIVER_BF16", (int)dt);
  if (n < 0 || n_ck < 0) return fail(RIVER_ERR_ARG, "decode_step: negative size");
  if (n == 0) return RIVER_OK;
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "decode_step: d = %d must be a positive multiple of 8", d);
  if (n_layers < 2) return fail(RIVER_ERR_ARG, "decode_step: n_layers = %d must be >= 2", n_layers);
  if (!exit_layer || (n_ck > 0 && !ck)) return fail(RIVER_ERR_ARG, "decode_step: exit_layer and the checkpoints are required");
  if (!ld_ok(ld, d, dt)) return fail(RIVER_ERR_ALIGN, "decode_step: ld must be >= d and a multiple of 16 bytes");
  if (rule != RIVER_RULE_TOKEN && rule != RIVER_RULE_BATCH_MIN) return fail(RIVER_ERR_ARG, "decode_step: unknown rule %d", (int)rule);
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RIVER_ERR_ARG, "decode_step: eps must be finite and >= 0");
  if (gamma && !aligned16(gamma)) return fail(RIVER_ERR_ALIGN, "decode_step: gamma must be 16-byte aligned");
  bool any_maps = false;
  for (int c = 0; c < n_ck; ++c) {
    const river_checkpoint& k = ck[c];
    if (k.layer < 1 || k.layer >= n_layers || (c > 0 && k.layer <= ck[c - 1].layer))
      return fail(RIVER_ERR_ARG, "decode_step: checkpoint %d: layers must increase within [1, n_layers)", c);
    if (!k.h_prev || !k.h_cur) return fail(RIVER_ERR_ARG, "decode_step: checkpoint %d: states are required", c);
    if (!aligned16(k.h_prev) || !aligned16(k.h_cur)) return fail(RIVER_ERR_ALIGN, "decode_step: checkpoint %d: states must be 16-byte aligned", c);
    if (isnan(k.tau) || isnan(k.theta)) return fail(RIVER_ERR_ARG, "decode_step: checkpoint %d: NaN threshold", c);
    if (k.w_down) {
      if (b < 1 || b > 512) return fail(RIVER_ERR_ARG, "decode_step: router width b = %d must be in [1, 512]", b);
      if (!k.w_up) return fail(RIVER_ERR_ARG, "decode_step: checkpoint %d: w_up is NULL while w_down is set", c);
      if (!aligned16(k.w_down) || !aligned16(k.w_up)) return fail(RIVER_ERR_ALIGN, "decode_step: router weights must be 16-byte aligned");
    }
    if (k.folded) {
      if (dt != RIVER_BF16) return fail(RIVER_ERR_DTYPE, "decode_step: checkpoint %d: folded products need bf16", c);
      if (!aligned16(k.folded)) return fail(RIVER_ERR_ALIGN, "decode_step: checkpoint %d: folded products must be 16-byte aligned", c);
      if (d % 256 || ((int64_t)n_kv_heads * head_dim) % 64 || (int64_t)4 * n_kv_heads * head_dim * d >= ((int64_t)1 << 31))
        return fail(RIVER_ERR_UNSUPPORTED, "decode_step: checkpoint %d: folded products need d %% 256 == 0 and n_out %% 64 == 0", c);
    }
    any_maps |= k.maps != nullptr && !k.folded;
  }
  const size_t fixed = decode_fixed_workspace(n, d, dt, n_layers);
  const size_t need = fixed + (any_maps ? kv_fill_workspace(n, d, 1, dt) : 0);
  if (!workspace || ws_bytes < need)
    return fail(RIVER_ERR_WORKSPACE, "decode_step: workspace of at least %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "decode_step: workspace must be 16-byte aligned");
  // the fill of each checkpoint: blocks e+1..L from its exit state
  for (int c = 0; c < n_ck; ++c) {
    const int e = ck[c].layer;
    river_w4 k4, v4;
    decode_layer_offset(*wk, e, n_kv_heads * head_dim, d, &k4);
    decode_layer_offset(*wv, e, n_kv_heads * head_dim, d, &v4);
    river_status st = kv_fill_validate("decode_step", n, d, dt, ck[c].h_cur, ld, n, nullptr, slot,
                                       n_layers - e, ck[c].folded ? nullptr : ck[c].maps, &k4, &v4, nullptr, n_kv_heads,
                                       head_dim, k_cache, v_cache, n_slots,
                                       (char*)workspace + fixed, ws_bytes - fixed);
    if (st != RIVER_OK) return st;
  }
  return launch_decode_step(n, d, dt, ld, n_ck, ck, n_layers, gamma, eps, b, rule, wk, wv, n_kv_heads,
                            head_dim, slot, k_cache, v_cache, n_slots, exit_layer, workspace, ws_bytes, s,
                            fork_ok);
}

river_status river_decode_step(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                               const river_checkpoint* ck, int n_layers, const void* gamma,
                               float eps, int b, river_rule rule, const river_w4* wk,
                               const river_w4* wv, int n_kv_heads, int head_dim,
                               const int32_t* slot, void* k_cache, void* v_cache, int64_t n_slots,
                               int32_t* exit_layer, void* workspace, size_t ws_bytes,
                               hipStream_t s) {
  return decode_step(n, d, dt, ld, n_ck, ck, n_layers, gamma, eps, b, rule, wk, wv, n_kv_heads, head_dim, slot,
                     k_cache, v_cache, n_slots, exit_layer, workspace, ws_bytes, s, true);
}

river_status river_decode_step_static(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                                      const river_checkpoint* ck, int n_layers, const void* gamma,
                                      float eps, int b, river_rule rule, const river_w4* wk,
                                      const river_w4* wv, int n_kv_heads, int head_dim,
                                      const int32_t* slot, void* k_cache, void* v_cache,
                                      int64_t n_slots, int32_t* exit_layer, hipStream_t s) {
  g_err[0] = 0;
  if (n <= 0 || d < 8 || n_layers < 2 || n_ck < 0 || n_kv_heads < 1 || head_dim < 1 || (n_ck > 0 && !ck))
    return decode_step(n, d, dt, ld, n_ck, ck, n_layers, gamma, eps, b, rule, wk, wv, n_kv_heads, head_dim,
                       slot, k_cache, v_cache, n_slots, exit_layer, nullptr, 0, s, false);
  void* p = nullptr;
  size_t cap = 0;
  river_status st = decode_static_scratch(&p, &cap);
  if (st != RIVER_OK) return st;
  bool any_maps = false;
  for (int c = 0; c < n_ck; ++c) any_maps |= ck[c].maps != nullptr && !ck[c].folded;
  // the least river_decode_step takes, and the size that fills every
  // checkpoint in one pass with room for the split reductions
  const size_t need = decode_fixed_workspace(n, d, dt, n_layers) + (any_maps ? kv_fill_workspace(n, d, 1, dt) : 0);
  if (need > cap)
    return fail(RIVER_ERR_WORKSPACE,
                "decode_step_static: %zu bytes of scratch needed (n = %d, d = %d, %d blocks), the static "
                "scratch holds %zu", need, n, d, n_layers, cap);
  const size_t want = decode_fixed_workspace(n, d, dt, n_layers) + kv_fill_workspace(n, d, n_layers - 1, RIVER_BF16) +
                      decode_proj_workspace(n, d, n_kv_heads * head_dim, n_layers);
  return decode_step(n, d, dt, ld, n_ck, ck, n_layers, gamma, eps, b, rule, wk, wv, n_kv_heads, head_dim, slot,
                     k_cache, v_cache, n_slots, exit_layer, p, want < cap ? want : cap, s, false);
}

river_status river_router_fit(int n, int d, river_dtype dt, const void* h, int64_t ld_h,
                              const uint8_t* labels, const void* gamma, float eps, int b,
                              float* w_down, float* w_up, int epochs, int batch,
                              const int32_t* order, float lr, float beta1, float beta2,
                              float adam_eps, float* loss_out, void* workspace, size_t ws_bytes,
                              hipStream_t s) {
  g_err[0] = 0;
  if (!dt_ok(dt)) return fail(RIVER_ERR_DTYPE, "router_fit: dtype %d is not RIVER_F32 or RIVER_BF16", (int)dt);
  if (n < 1 || epochs < 1) return fail(RIVER_ERR_ARG, "router_fit: n and epochs must be >= 1");
  if (d < 8 || d % 8) return fail(RIVER_ERR_ARG, "router_fit: d = %d must be a positive multiple of 8", d);
  if (b < 1 || b > 512) return fail(RIVER_ERR_ARG, "router_fit: b = %d must be in [1, 512]", b);
  if (batch < 1 || batch > 1000) return fail(RIVER_ERR_ARG, "router_fit: batch = %d must be in [1, 1000]", batch);
  if (!(lr > 0.0f) || isinf(lr)) return fail(RIVER_ERR_ARG, "router_fit: lr must be finite and > 0");
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(RIVER_ERR_ARG, "router_fit: beta1 and beta2 must be in [0, 1)");
  if (!(adam_eps > 0.0f) || isinf(adam_eps)) return fail(RIVER_ERR_ARG, "router_fit: adam_eps must be finite and > 0");
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RIVER_ERR_ARG, "router_fit: eps must be finite and >= 0");
  if (!h || !labels || !w_down || !w_up) return fail(RIVER_ERR_ARG, "router_fit: h, labels, w_down and w_up are required");
  if (!ld_ok(ld_h, d, dt) || !aligned16(h)) return fail(RIVER_ERR_ALIGN, "router_fit: h misaligned or ld_h invalid");
  if (gamma && !aligned16(gamma)) return fail(RIVER_ERR_ALIGN, "router_fit: gamma must be 16-byte aligned");
  if ((int64_t)n * epochs > ((int64_t)1 << 31)) return fail(RIVER_ERR_UNSUPPORTED, "router_fit: n * epochs must stay below 2^31");
  const size_t need = calib_workspace(n, d, b, batch, epochs);
  if (!workspace || ws_bytes < need)
    return fail(RIVER_ERR_WORKSPACE, "router_fit: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "router_fit: workspace must be 16-byte aligned");
  return launch_router_fit(n, d, dt, h, ld_h, labels, gamma, eps, b, w_down, w_up, epochs, batch, order,
                           lr, beta1, beta2, adam_eps, loss_out, workspace, s);
}

river_status river_ridge_fit(int n, int d_in, int d_out, int n_targets, const void* X,
                             river_dtype xdt, const void* Y, river_dtype ydt, float lambda,
                             void* W, river_dtype wdt, void* workspace, size_t ws_bytes,
                             hipStream_t s) {
  g_err[0] = 0;
  if (!dt_ok(xdt) || !dt_ok(ydt) || !dt_ok(wdt)) return fail(RIVER_ERR_DTYPE, "ridge_fit: unsupported dtype");
  if (xdt != ydt) return fail(RIVER_ERR_DTYPE, "ridge_fit: X and Y must have the same dtype");
  if (n < 1 || d_in < 1 || d_out < 1 || n_targets < 0) return fail(RIVER_ERR_ARG, "ridge_fit: invalid sizes");
  if (!(lambda >= 0.0f) || isinf(lambda)) return fail(RIVER_ERR_ARG, "ridge_fit: lambda must be finite and >= 0");
  if (n_targets == 0) return RIVER_OK;
  if (!X || !Y || !W) return fail(RIVER_ERR_ARG, "ridge_fit: X, Y and W are required");
  if (!aligned16(X) || !aligned16(Y) || !aligned16(W)) return fail(RIVER_ERR_ALIGN, "ridge_fit: X, Y, W must be 16-byte aligned");
  if (xdt == RIVER_BF16 && (d_in % 64 || d_out % 64 || n % 64))
    return fail(RIVER_ERR_UNSUPPORTED, "ridge_fit: bf16 path needs n, d_in, d_out multiples of 64");
  if (xdt == RIVER_F32 && (d_in % 4 || d_out % 4)) return fail(RIVER_ERR_UNSUPPORTED, "ridge_fit: fp32 path needs d_in, d_out multiples of 4");
  if (xdt == RIVER_BF16) {
    // the MFMA GEMMs address each operand (X^T and Y_t^T over the padded
    // calibration count, and the split factors over 3 d_in) with 31-bit
    // byte offsets
    const int64_t np = ((int64_t)n + 255) / 256 * 256, k3 = (3 * (int64_t)d_in + 255) / 256 * 256;
    const int64_t lim = (int64_t)1 << 31, dmax = d_in > d_out ? d_in : d_out;
    if (dmax * np * 2 >= lim || dmax * k3 * 2 >= lim)
      return fail(RIVER_ERR_UNSUPPORTED, "ridge_fit: an operand of %lld x %lld bf16 exceeds 2^31 bytes",
                  (long long)dmax, (long long)(np > k3 ? np : k3));
  }
  size_t need = ridge_workspace(n, d_in, d_out, xdt);
  if (!workspace || ws_bytes < need)
    return fail(RIVER_ERR_WORKSPACE, "ridge_fit: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned16(workspace)) return fail(RIVER_ERR_ALIGN, "ridge_fit: workspace must be 16-byte aligned");
  return launch_ridge_fit(n, d_in, d_out, n_targets, X, xdt, Y, lambda, W, wdt, workspace, ws_bytes, s);
}

}  // extern "C"
