// One generation step of the token-level exit loop (river_decode_step).
//
// River-LLM, "方法步骤详情" step 3: while a token's state climbs the blocks,
// the state-transition similarity after each checked block decides whether
// it switches to the exit path, which writes the K/V of every remaining
// block at the token's slot (step 1). With a router (TIDE formula 3) the
// decision also needs the router's probability; River's batch rule exits
// only when every running token passes.
//
// The step is an ordered sequence of launches on one stream: an init
// kernel, then per checkpoint route (over all n rows, with the running
// flags of the previous checkpoint), compact (the exiting rows in order)
// and the fill of blocks e+1..L for those rows, whose count stays on the
// device. Nothing waits on the host, allocates or sets memory through the
// runtime, so the whole step can be captured once into a HIP graph and
// replayed for every generated token.
#include "common.h"

namespace river {

// every token running, no exit yet
__global__ __launch_bounds__(256) void decode_init_kernel(int n, uint8_t* alive, int32_t* exit_layer,
                                                          int n_layers) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    alive[i] = 1;
    exit_layer[i] = n_layers;
  }
}

}  // namespace river

namespace river_host {
using namespace river;

// workspace: running flags [2][n], mask [n], exit and continuing indices
// [n] each, counts [2], then compact's own scratch; the fill's x_hat
// scratch follows (with maps)
static size_t a256(size_t x) { return align_up(x, 256); }

size_t decode_fixed_workspace(int n) {
  return a256(2 * (size_t)n) + a256((size_t)n) + 2 * a256(4 * (size_t)n) + 256 + compact_workspace(n);
}

// descriptor of blocks e+1..L inside one that covers blocks 1..L
void decode_layer_offset(const river_w4& w, int e, int n_out, int d, river_w4* out) {
  *out = w;
  const int64_t per_layer_sz = (int64_t)n_out * (d / w.group) * (int64_t)esize(w.sz_dtype);
  out->q = w.q + (int64_t)e * n_out * (d / 2);
  out->scale = (const char*)w.scale + e * per_layer_sz;
  out->zero = (const char*)w.zero + e * per_layer_sz;
}

river_status launch_decode_step(int n, int d, river_dtype dt, int64_t ld, int n_ck,
                                const river_checkpoint* ck, int n_layers, const void* gamma,
                                float eps, int b, river_rule rule, const river_w4* wk,
                                const river_w4* wv, int n_kv_heads, int head_dim,
                                const int32_t* slot, void* k_cache, void* v_cache, int64_t n_slots,
                                int32_t* exit_layer, void* workspace, size_t ws_bytes,
                                hipStream_t s) {
  char* w = (char*)workspace;
  uint8_t* alive = (uint8_t*)w;
  w += a256(2 * (size_t)n);
  uint8_t* mask = (uint8_t*)w;
  w += a256((size_t)n);
  int32_t* exit_idx = (int32_t*)w;
  w += a256(4 * (size_t)n);
  int32_t* cont_idx = (int32_t*)w;
  w += a256(4 * (size_t)n);
  int32_t* counts = (int32_t*)w;
  w += 256;
  void* cws = w;
  const size_t cws_bytes = compact_workspace(n);
  w += cws_bytes;
  void* fws = w;
  const size_t fixed = (size_t)(w - (char*)workspace);
  const size_t fws_bytes = ws_bytes - fixed;

  decode_init_kernel<<<(n + 255) / 256, 256, 0, s>>>(n, alive, exit_layer, n_layers);
  river_status st = check_launch("decode_step init");
  if (st != RIVER_OK) return st;
  const int n_out = n_kv_heads * head_dim;
  const int64_t cache_layer = n_slots * n_out * (int64_t)esize(dt);   // bytes per cache layer
  for (int c = 0; c < n_ck; ++c) {
    const river_checkpoint& k = ck[c];
    const int e = k.layer;
    RouteLive live{alive + (c & 1) * n, alive + ((c + 1) & 1) * n, exit_layer, e};
    st = launch_route(n, d, dt, k.h_prev, ld, k.h_cur, ld, gamma, eps, k.w_down, k.w_up, b, k.tau,
                      k.theta, rule, nullptr, nullptr, mask, nullptr, &live, s);
    if (st != RIVER_OK) return st;
    st = launch_compact(n, d, dt, mask, nullptr, 0, nullptr, cont_idx, exit_idx, counts, nullptr, 0,
                        nullptr, nullptr, 0, 0, cws, cws_bytes, s);
    if (st != RIVER_OK) return st;
    river_w4 k4, v4;
    decode_layer_offset(*wk, e, n_out, d, &k4);
    decode_layer_offset(*wv, e, n_out, d, &v4);
    st = launch_kv_fill(n, counts + 1, d, dt, k.h_cur, ld, n, exit_idx, slot, n_layers - e, k.maps,
                        &k4, &v4, nullptr, n_kv_heads, head_dim, (char*)k_cache + e * cache_layer,
                        (char*)v_cache + e * cache_layer, n_slots, fws, fws_bytes, s);
    if (st != RIVER_OK) return st;
  }
  return RIVER_OK;
}

}  // namespace river_host
