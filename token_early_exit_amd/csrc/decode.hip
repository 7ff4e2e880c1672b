// One generation step of the token-level exit loop (river_decode_step).
//
// River-LLM, "方法步骤详情" step 3: while a token's state climbs the blocks,
// the state-transition similarity after each checked block decides whether
// it switches to the exit path, which writes the K/V of every remaining
// block at the token's slot (step 1). With a router (TIDE formula 3) the
// decision also needs the router's probability; River's batch rule exits
// only when every running token passes.
//
// The step is an ordered sequence of launches on one stream. With a router
// at any checkpoint (or more than 1024 tokens): an init kernel, then per
// checkpoint route (over all n rows, with the running flags of the
// previous checkpoint), compact (the exiting rows in order) and the fill
// of blocks e+1..L for those rows, whose count stays on the device. With
// the routers off, the decisions of all checkpoints take two launches
// instead of 3 per checkpoint: the cosines of every (checkpoint, token)
// pair, then one workgroup that walks the checkpoints in order (running
// flags, token or batch rule, the exiting rows of each checkpoint in token
// order); the fills follow. Both give bit-identical results (same cosine
// code, same decisions). Nothing waits on the host, allocates or sets
// memory through the runtime, so the whole step can be captured once into
// a HIP graph and replayed for every generated token.
#include "common.h"
#include "cosine.h"

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

// ------------------------------------------------- all checkpoints at once
constexpr int DC_MAX = 32;       // checkpoints of the two-launch path
constexpr int DC_TOKENS = 1024;  // tokens of the two-launch path (one workgroup)

struct DecodeCos {
  int n, d;
  int64_t ld;                     // elements
  const void* hp[DC_MAX];
  const void* hc[DC_MAX];
  float* cos;                     // [n_ck][n]
};

// cos[c][i]: one wave per token, four tokens per workgroup, blockIdx.y = c
template <bool BF16, int KPL>
__global__ __launch_bounds__(256) void decode_cos_kernel(DecodeCos a) {
  const int c = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  const int i = blockIdx.x * 4 + wave;
  if (i >= a.n) return;
  constexpr int ES = BF16 ? 2 : 4;
  const int64_t off = (int64_t)i * a.ld * ES;
  const float v = token_cosine<BF16, KPL>((const char*)a.hp[c] + off, (const char*)a.hc[c] + off, a.d, lane);
  if (lane == 0) a.cos[(int64_t)c * a.n + i] = v;
}

struct DecodePlan {
  int n, n_ck, batch_min, n_layers;
  const float* cos;               // [n_ck][n]
  float tau[DC_MAX];
  int layer[DC_MAX];
  int32_t* exit_idx;              // [n_ck][idx_stride]: the exiting rows of checkpoint c in order
  int idx_stride;
  int32_t* counts;                // [n_ck][64]: {running or done before, exiting} (compact's layout)
  int32_t* exit_layer;            // [n]
};

// One workgroup, token i in thread i: the checkpoints in order. Under the
// token rule a running token exits where its cosine passes tau; under the
// batch rule every running token exits where all of them pass (and at
// least one runs). Each checkpoint's exits are listed in token order from
// a ballot per wave and the wave totals.
__global__ __launch_bounds__(DC_TOKENS) void decode_plan_kernel(DecodePlan p) {
  __shared__ int wsum[DC_TOKENS / WAVE];
  const int i = threadIdx.x, lane = i % WAVE, wave = i / WAVE;
  const int n = p.n;
  bool alive = i < n;
  int el = p.n_layers;
  for (int c = 0; c < p.n_ck; ++c) {
    bool e = alive && p.cos[(int64_t)c * n + (i < n ? i : 0)] > p.tau[c];
    if (p.batch_min) {
      const int all = __syncthreads_and(!alive || e);
      const int any = __syncthreads_or(alive);
      e = alive && all && any;
    }
    if (e) el = p.layer[c];
    const uint64_t b = __ballot(e);
    if (lane == 0) wsum[wave] = __popcll(b);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < DC_TOKENS / WAVE; ++w) {
      const int v = wsum[w];
      before += w < wave ? v : 0;
      total += v;
    }
    if (e) {
      const int r = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
      p.exit_idx[(int64_t)c * p.idx_stride + r] = i;
    }
    if (i == 0) {
      p.counts[c * 64] = n - total;
      p.counts[c * 64 + 1] = total;
    }
    __syncthreads();                          // wsum is rewritten next round
    alive = alive && !e;
  }
  if (i < n) p.exit_layer[i] = el;
}

}  // namespace river

namespace river_host {
using namespace river;

// workspace: running flags [2][n], mask [n], exit and continuing indices
// [n] each, counts [2], then compact's own scratch; the fill's x_hat
// scratch follows (with maps)
static size_t a256(size_t x) { return align_up(x, 256); }

// the two-launch path: per checkpoint (at most n_layers - 1) the cosines,
// the exiting rows and the counts
static size_t plan_ck_bytes(int n) { return 2 * a256(4 * (size_t)n) + 256; }

size_t decode_fixed_workspace(int n, int n_layers) {
  return a256(2 * (size_t)n) + a256((size_t)n) + 2 * a256(4 * (size_t)n) + 256 + compact_workspace(n) +
         (size_t)(n_layers > 1 ? n_layers - 1 : 0) * plan_ck_bytes(n);
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
  char* plan = w;                                   // [n_ck] x (cos, exit rows, counts)
  w += (size_t)(n_layers - 1) * plan_ck_bytes(n);
  void* fws = w;
  const size_t fixed = (size_t)(w - (char*)workspace);
  const size_t fws_bytes = ws_bytes - fixed;

  const int n_out = n_kv_heads * head_dim;
  const int64_t cache_layer = n_slots * n_out * (int64_t)esize(dt);   // bytes per cache layer
  bool two_launch = n <= DC_TOKENS && n_ck <= DC_MAX && decode_path_override() == 0;
  for (int c = 0; c < n_ck; ++c) two_launch = two_launch && !ck[c].w_down;
  if (two_launch) {
    // plan area: cosines [n_ck][n], then the exit rows of each checkpoint
    // (CO bytes apart), then its counts (256 bytes apart)
    const size_t CO = a256(4 * (size_t)n);
    river_status st = RIVER_OK;
    if (n_ck > 0) {
      DecodeCos a{};
      a.n = n; a.d = d; a.ld = ld;
      for (int c = 0; c < n_ck; ++c) { a.hp[c] = ck[c].h_prev; a.hc[c] = ck[c].h_cur; }
      a.cos = (float*)plan;
      const dim3 grid((unsigned)((n + 3) / 4), (unsigned)n_ck);
      auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a); };
      const int kpl = cosine_kpl(d, dt == RIVER_BF16);
      if (dt == RIVER_BF16) {
        if (kpl == 1) go(decode_cos_kernel<true, 1>); else if (kpl == 2) go(decode_cos_kernel<true, 2>);
        else if (kpl == 4) go(decode_cos_kernel<true, 4>); else if (kpl == 8) go(decode_cos_kernel<true, 8>);
        else go(decode_cos_kernel<true, 0>);
      } else {
        if (kpl == 1) go(decode_cos_kernel<false, 1>); else if (kpl == 2) go(decode_cos_kernel<false, 2>);
        else if (kpl == 4) go(decode_cos_kernel<false, 4>); else if (kpl == 8) go(decode_cos_kernel<false, 8>);
        else go(decode_cos_kernel<false, 0>);
      }
      st = check_launch("decode_step cosines");
      if (st != RIVER_OK) return st;
    }
    DecodePlan q{};
    q.n = n; q.n_ck = n_ck; q.batch_min = rule == RIVER_RULE_BATCH_MIN; q.n_layers = n_layers;
    q.cos = (const float*)plan;
    for (int c = 0; c < n_ck; ++c) { q.tau[c] = ck[c].tau; q.layer[c] = ck[c].layer; }
    char* rec = plan + (size_t)n_ck * CO;
    q.exit_idx = (int32_t*)rec;
    q.idx_stride = (int)(CO / 4);
    q.counts = (int32_t*)(rec + (size_t)n_ck * CO);
    q.exit_layer = exit_layer;
    decode_plan_kernel<<<1, DC_TOKENS, 0, s>>>(q);
    st = check_launch("decode_step plan");
    if (st != RIVER_OK) return st;
    for (int c = 0; c < n_ck; ++c) {
      const river_checkpoint& k = ck[c];
      const int e = k.layer;
      river_w4 k4, v4;
      decode_layer_offset(*wk, e, n_out, d, &k4);
      decode_layer_offset(*wv, e, n_out, d, &v4);
      st = launch_kv_fill(n, q.counts + c * 64 + 1, d, dt, k.h_cur, ld, n, q.exit_idx + (size_t)c * q.idx_stride,
                          slot, n_layers - e, k.maps, &k4, &v4, nullptr, n_kv_heads, head_dim,
                          (char*)k_cache + e * cache_layer, (char*)v_cache + e * cache_layer, n_slots, fws,
                          fws_bytes, s);
      if (st != RIVER_OK) return st;
    }
    return RIVER_OK;
  }

  decode_init_kernel<<<(n + 255) / 256, 256, 0, s>>>(n, alive, exit_layer, n_layers);
  river_status st = check_launch("decode_step init");
  if (st != RIVER_OK) return st;
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
