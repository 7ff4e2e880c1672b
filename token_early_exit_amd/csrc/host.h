// Host side of the library: error reporting, small helpers and the
// launchers the kernel files implement (argument checks are done by
// api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "river.h"

namespace river_host {

void set_error(const char* fmt, ...);
river_status fail(river_status st, const char* fmt, ...);
river_status check_launch(const char* what);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t esize(river_dtype dt) { return dt == RIVER_BF16 ? 2 : 4; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int compact_path_override();
int gemm_path_override();
int decode_path_override();
int fill_fuse_override();
// event marks around a launch (river_debug_time_kernels): the begin mark
// returns a record, or -1 when timing is off, the stream is capturing or
// the records are full; the end mark closes that record
int debug_timer_begin(hipStream_t s, int kind);
void debug_timer_end(hipStream_t s, int rec);

// launchers implemented by the kernel files; argument checks are done by
// the caller (api.hip)

// the running-token state of the generation loop (river_decode_step)
struct RouteLive {
  const uint8_t* alive_in; uint8_t* alive_out; int32_t* exit_layer; int exit_value;
};
river_status launch_route(int n, int d, river_dtype dt, const void* h_prev, int64_t ld_prev,
                          const void* h_cur, int64_t ld_cur, const void* gamma, float eps,
                          const void* w_down, const void* w_up, int b, float tau, float theta,
                          river_rule rule, float* cos_out, float* prob_out, uint8_t* mask_out,
                          int32_t* all_exit_out, const RouteLive* live, hipStream_t s);

size_t compact_workspace(int n);
river_status launch_compact(int n, int d, river_dtype dt, const uint8_t* mask, const void* h,
                            int64_t ld_h, const int32_t* row_ids, int32_t* cont_idx,
                            int32_t* exit_idx, int32_t* counts, void* h_cont, int64_t ld_cont,
                            int32_t* row_ids_cont, void* out, int64_t ld_out, int64_t n_out_rows,
                            void* workspace, size_t ws_bytes, hipStream_t s);

river_status launch_exit_projection(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                    const void* h, int64_t ld_h, int n_rows,
                                    const int32_t* row_idx, const int32_t* row_ids,
                                    const void* gamma, float eps, void* out, int64_t ld_out,
                                    int64_t n_out_rows, hipStream_t s);

size_t kv_fill_workspace(int m_max, int d, int n_layers, river_dtype dt);
size_t kv_fill_layer_workspace(int m_max, int d, int n_layers);
size_t kv_fill_proj_workspace(int m_max, int d, int n_out, int n_layers);
size_t decode_proj_workspace(int n, int d, int n_out, int n_layers);
size_t kv_fill_full_workspace(int m_max, int d, int n_out, int nl, bool maps);
void kv_fill_plan(int m_max, bool dev_count, int d, int nh, int n_layers, size_t ws_bytes, int* chunk,
                  int* path, int* ks);
river_status launch_kv_fill(int m_max, const int32_t* m_dev, int d, river_dtype dt, const void* h,
                            int64_t ld_h, int n_rows, const int32_t* row_idx, const int32_t* slot,
                            int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                            const river_layer* layer, int n_kv_heads, int head_dim, void* k_cache,
                            void* v_cache, int64_t n_slots, void* workspace, size_t ws_bytes,
                            hipStream_t s, const int32_t* m_dev_layer = nullptr);
// m_dev_layer: rows of layer j = clamp(m_dev_layer[j], 0, m_max) instead of
// one count (the plain MFMA path only: no maps, no layer parts)
bool kv_fill_plain_mfma(int m_max, int d, river_dtype dt, int n_rows, int64_t ld_h, const river_w4* wk,
                        const river_w4* wv, int nh);
// folded products F[l] = deq([Wk[l]; Wv[l]]) . maps[l] and the fill through them
size_t kv_fold_workspace(int d, int n_out, int chunk, bool maps);
bool kv_fold_ok(int d, int nh, const river_w4* wk, const river_w4* wv);
river_status launch_kv_fold(int d, int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                            int nh, void* F, void* workspace, size_t ws_bytes, hipStream_t s);
river_status launch_kv_fill_folded(int m_max, const int32_t* m_dev, int d, const void* h, int64_t ld_h,
                                   int n_rows, const int32_t* row_idx, const int32_t* slot, int n_layers,
                                   const void* F, int nh, void* k_cache, void* v_cache, int64_t n_slots,
                                   hipStream_t s);

// cosine and router probability of every token at every checkpoint (all
// with a router) in one launch, [n_ck][n] each; mask_scratch [n_ck][n]
bool route_scores_ok(int n, int d, river_dtype dt, int b, int64_t ld, int n_ck);
// halves: room for route_halves_bytes(n, n_ck) (the reduction over d in two
// workgroups per token group where d % 512 == 0), or NULL
river_status launch_route_scores(int n, int d, river_dtype dt, int64_t ld, int n_ck, const river_checkpoint* ck,
                                 const void* gamma, float eps, int b, float* cos_out, float* prob_out,
                                 uint8_t* mask_scratch, void* halves, hipStream_t s);
size_t route_halves_bytes(int n, int n_ck);

size_t decode_fixed_workspace(int n, int d, river_dtype dt, int n_layers);
river_status decode_static_scratch(void** ptr, size_t* bytes);
void decode_layer_offset(const river_w4& w, int e, int n_out, int d, river_w4* out);
river_status launch_decode_step(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                                const river_checkpoint* ck, int n_layers, const void* gamma,
                                float eps, int b, river_rule rule, const river_w4* wk,
                                const river_w4* wv, int n_kv_heads, int head_dim,
                                const int32_t* slot, void* k_cache, void* v_cache, int64_t n_slots,
                                int32_t* exit_layer, void* workspace, size_t ws_bytes,
                                hipStream_t s, bool fork_ok);

size_t calib_workspace(int n, int d, int b, int batch, int epochs);
river_status launch_router_fit(int n, int d, river_dtype dt, const void* h, int64_t ld_h,
                               const uint8_t* labels, const void* gamma, float eps, int b,
                               float* w_down, float* w_up, int epochs, int batch,
                               const int32_t* order, float lr, float beta1, float beta2,
                               float adam_eps, float* loss_out, void* workspace, hipStream_t s);

size_t ridge_workspace(int n, int d_in, int d_out, river_dtype dt);
river_status launch_ridge_fit(int n, int d_in, int d_out, int n_targets, const void* X,
                              river_dtype xdt, const void* Y, float lambda, void* W,
                              river_dtype wdt, void* workspace, size_t ws_bytes, hipStream_t s);

}  // namespace river_host
