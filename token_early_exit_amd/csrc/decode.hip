// One generation step of the token-level exit loop (river_decode_step).
//
// River-LLM, "方法步骤详情" step 3: while a token's state climbs the blocks,
// the state-transition similarity after each checked block decides whether
// it switches to the exit path, which writes the K/V of every remaining
// block at the token's slot (step 1). With a router (TIDE formula 3) the
// decision also needs the router's probability; River's batch rule exits
// only when every running token passes.
//
// The step is an ordered sequence of launches on one stream. In general
// (more than 1024 tokens, routers at some checkpoints only, or router
// shapes off the streaming route): an init kernel, then per checkpoint
// route (over all n rows, with the running flags of the previous
// checkpoint), compact (the exiting rows in order) and the fill of blocks
// e+1..L for those rows, whose count stays on the device. Otherwise the
// decisions of all checkpoints take two launches instead of 3 per
// checkpoint: the cosines (and, with routers, the probabilities) of every
// (checkpoint, token) pair, by the same kernel code as the per-checkpoint
// route, then one workgroup that walks the checkpoints in order (running
// flags, token or batch rule, the exiting rows of each checkpoint in token
// order): the same decisions. Without
// maps the fills of all checkpoints then become one: block e + 1 needs the
// exits of every checkpoint before it, which (listed checkpoint by
// checkpoint) form a prefix of one exit order, so after a gather of each
// exiting token's state one projection over blocks e_0 + 1..L, with a row
// count per block, writes them all. It computes every (token, block) value
// as the per-checkpoint fill does when both split the reduction over d
// into the same parts (bit-identical then; to rounding otherwise).
// Nothing waits on the host, allocates or sets memory through the runtime,
// so the whole step can be captured once into a HIP graph and replayed for
// every generated token.
#include <mutex>

#include "common.h"
#include "cosine.h"
#include "gemm.h"

namespace river {

// The scratch of river_decode_step_static: a file-scope device array that
// each GPU the library runs on holds from the code object's load until the
// process ends. Host code never passes the array's name to a kernel (on
// the host it only stands for the symbol); it passes the device address
// hipGetSymbolAddress returned for the current device.
constexpr size_t DECODE_STATIC_SCRATCH = (size_t)64 << 20;
static __device__ __align__(256) char scratch[DECODE_STATIC_SCRATCH];

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
constexpr int RM_HALVES = 16;    // checkpoints whose route halves the workspace holds
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
  const float* prob;              // [n_ck][n] router probabilities (NULL: routers off)
  float tau[DC_MAX];
  float theta[DC_MAX];
  int layer[DC_MAX];
  int32_t* exit_idx;              // [n_ck][idx_stride]: the exiting rows of checkpoint c in order
  int idx_stride;
  int32_t* counts;                // [n_ck][64]: {running or done before, exiting} (compact's layout)
  int32_t* exit_layer;            // [n]
  // one fill for the checkpoints of single_mask (bit c: checkpoint c; NULL
  // arrays: not wanted): their exits in checkpoint order, the checkpoint of
  // each token's exit among them (-1: none or another checkpoint) and, for
  // block first + j (first = 1 + the layer of the lowest checkpoint of the
  // mask), the number of their exits before it (a prefix of ord)
  int32_t* ord;                   // [n]
  int32_t* ck_of;                 // [n]
  int32_t* m_layer;               // [n_layers + 1 - first]
  uint32_t single_mask;
};

// One workgroup, token i in thread i: the checkpoints in order. Under the
// token rule a running token exits where its cosine passes tau (and, with
// routers, its probability theta); under the
// batch rule every running token exits where all of them pass (and at
// least one runs). Each checkpoint's exits are listed in token order from
// a ballot per wave and the wave totals.
// The workgroup has as many waves as the tokens need (its barriers and the
// wave totals' reads scale with them).
__global__ __launch_bounds__(DC_TOKENS) void decode_plan_kernel(DecodePlan p) {
  __shared__ int wsum[DC_TOKENS / WAVE];
  const int nw = blockDim.x / WAVE;
  __shared__ int tot[DC_MAX];
  const int i = threadIdx.x, lane = i % WAVE, wave = i / WAVE;
  const int n = p.n;
  bool alive = i < n;
  int el = p.n_layers, my_ck = -1;
  int off = 0;                                // exits of the single fill's checkpoints before c
  // the scores of PF checkpoints are loaded together, so their latencies
  // overlap instead of adding up checkpoint by checkpoint
  constexpr int PF = 8;
  for (int c0 = 0; c0 < p.n_ck; c0 += PF) {
    float cv[PF], pv[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int64_t at = (int64_t)(c0 + k < p.n_ck ? c0 + k : 0) * n + (i < n ? i : 0);
      cv[k] = p.cos[at];
      pv[k] = p.prob ? p.prob[at] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int c = c0 + k;
      if (c >= p.n_ck) break;                   // uniform
      const bool sf = (p.single_mask >> c) & 1u;
      // the route's decision: cos > tau, and p > theta with a router
      bool e = alive && cv[k] > p.tau[c] && (!p.prob || pv[k] > p.theta[c]);
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
      for (int w = 0; w < nw; ++w) {
        const int v = wsum[w];
        before += w < wave ? v : 0;
        total += v;
      }
      if (e) {
        const int r = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        p.exit_idx[(int64_t)c * p.idx_stride + r] = i;
        if (p.ord && sf) p.ord[off + r] = i;
        if (sf) my_ck = c;
      }
      if (i == 0) {
        p.counts[c * 64] = n - total;
        p.counts[c * 64 + 1] = total;
        tot[c] = total;
      }
      off += sf ? total : 0;
      __syncthreads();                          // wsum is rewritten next round
      alive = alive && !e;
    }
  }
  if (i < n) {
    p.exit_layer[i] = el;
    if (p.ck_of) p.ck_of[i] = my_ck;
  }
  if (p.m_layer && p.single_mask) {
    const int first = p.layer[__builtin_ctz(p.single_mask)] + 1;   // first filled block
    for (int j = i; j < p.n_layers + 1 - first; j += blockDim.x) {
      int m = 0;
      for (int c = 0; c < p.n_ck; ++c)
        m += ((p.single_mask >> c) & 1u) && p.layer[c] < first + j ? tot[c] : 0;
      p.m_layer[j] = m;
    }
  }
}

struct DecodeGather {
  int n, row_bytes;               // row_bytes a multiple of 16
  int64_t ld_bytes;               // source leading dimension in bytes
  const void* hc[DC_MAX];
  const int32_t* ck_of;
  char* x;                        // [n][row_bytes]
};

// x[i] = the state of token i at its exit checkpoint (workgroup i, 64 lanes;
// up to four 16-byte pieces per lane in flight)
__global__ __launch_bounds__(64) void decode_gather_kernel(DecodeGather a) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const int c = a.ck_of[i];
  if (c < 0) return;
  const u32x4* src = (const u32x4*)((const char*)a.hc[c] + (int64_t)i * a.ld_bytes);
  u32x4* dst = (u32x4*)(a.x + (int64_t)i * a.row_bytes);
  const int nch = a.row_bytes >> 4;
  for (int c0 = 0; c0 < nch; c0 += 4 * WAVE) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = c0 + lane + WAVE * k;
      v[k] = src[q < nch ? q : nch - 1];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = c0 + lane + WAVE * k;
      if (q < nch) dst[q] = v[k];
    }
  }
}

}  // namespace river

namespace river_host {
using namespace river;

// workspace: running flags [2][n], mask [n], exit and continuing indices
// [n] each, counts [2], then compact's own scratch; the fill's x_hat
// scratch follows (with maps)
static size_t a256(size_t x) { return align_up(x, 256); }

// the two-launch path: per checkpoint (at most n_layers - 1) the cosines,
// the exiting rows, the counts, the router probabilities and the route's
// (unused) masks; then for the single fill the exit
// states [n][d] (sized for fp32), the exit order, the exit checkpoints and
// the per-block row counts
static size_t plan_ck_bytes(int n) { return 3 * a256(4 * (size_t)n) + a256((size_t)n) + 256; }
static size_t plan_fill_bytes(int n, int d, int n_layers) {
  return a256((size_t)n * d * 4) + 2 * a256(4 * (size_t)n) + a256(4 * (size_t)n_layers);
}

// Device address of the static scratch on the current device (looked up
// once per device, on its first use, with that device current).
river_status decode_static_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[256] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RIVER_ERR_HIP, "decode_step_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 256) return fail(RIVER_ERR_UNSUPPORTED, "decode_step_static: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RIVER_ERR_HIP, "decode_step_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = DECODE_STATIC_SCRATCH;
  return RIVER_OK;
}

// The second stream of a decode step on each device, with the events of
// its fork and join, made on the device's first step that forks (default
// priority, non-blocking) and kept until the process ends. The mutex keeps
// the fork-to-join launches of two host threads from interleaving.
// DECODE_SIDE_CUS: the second stream's CU budget; at the 8B decode shape
// (the first fill streams 21 maps of 4096^2, the others need one map and
// one block) 176 and 192 measured 241 and 243 us per graph-replayed step,
// 208 and 224 (the others then take longer than the first) 279 and 297.
constexpr int DECODE_SIDE_CUS = 176;
struct DecodeSide {
  std::mutex mu;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

static river_status decode_side(DecodeSide** out) {
  static std::mutex mu;
  static DecodeSide sides[256];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RIVER_ERR_HIP, "decode_step: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 256) return fail(RIVER_ERR_UNSUPPORTED, "decode_step: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  DecodeSide& sd = sides[dev];
  if (!sd.stream) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) return fail(RIVER_ERR_HIP, "decode_step: second stream: %s", hipGetErrorString(e));
    sd.fork = f;
    sd.join = j;
    sd.stream = st;
  }
  *out = &sd;
  return RIVER_OK;
}

size_t decode_fixed_workspace(int n, int d, river_dtype dt, int n_layers) {
  (void)dt;
  return a256(2 * (size_t)n) + a256((size_t)n) + 2 * a256(4 * (size_t)n) + 256 + compact_workspace(n) +
         (size_t)(n_layers > 1 ? n_layers - 1 : 0) * plan_ck_bytes(n) + plan_fill_bytes(n, d, n_layers) +
         (n <= DC_TOKENS ? route_halves_bytes(n, n_layers - 1 < RM_HALVES ? n_layers - 1 : RM_HALVES) : 0);
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
                                hipStream_t s, bool fork_ok) {
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
  char* xs = w;                                     // exit states of the single fill
  w += a256((size_t)n * d * 4);
  int32_t* ord = (int32_t*)w;
  w += a256(4 * (size_t)n);
  int32_t* ck_of = (int32_t*)w;
  w += a256(4 * (size_t)n);
  int32_t* m_layer = (int32_t*)w;
  w += a256(4 * (size_t)n_layers);
  // the route's halves (two-launch path with routers)
  void* halves = n <= DC_TOKENS ? (void*)w : nullptr;
  w += n <= DC_TOKENS ? route_halves_bytes(n, n_layers - 1 < RM_HALVES ? n_layers - 1 : RM_HALVES) : 0;
  void* fws = w;
  const size_t fixed = (size_t)(w - (char*)workspace);
  const size_t fws_bytes = ws_bytes - fixed;

  const int n_out = n_kv_heads * head_dim;
  const int64_t cache_layer = n_slots * n_out * (int64_t)esize(dt);   // bytes per cache layer
  bool routers_off = true, routers_on = n_ck > 0;
  for (int c = 0; c < n_ck; ++c) {
    routers_off = routers_off && !ck[c].w_down;
    routers_on = routers_on && ck[c].w_down;
  }
  routers_on = routers_on && route_scores_ok(n, d, dt, b, ld, n_ck);
  const bool two_launch = n <= DC_TOKENS && n_ck <= DC_MAX && decode_path_override() == 0 &&
                          (routers_off || routers_on);
  if (two_launch) {
    // plan area: cosines [n_ck][n], then the exit rows of each checkpoint
    // (CO bytes apart), then its counts (256 bytes apart), then the router
    // probabilities [n_ck][n] and the route's masks (n bytes apart)
    const size_t CO = a256(4 * (size_t)n);
    float* prob = (float*)(plan + (size_t)n_ck * (2 * CO + 256));
    uint8_t* masks = (uint8_t*)(plan + (size_t)n_ck * (3 * CO + 256));
    river_status st = RIVER_OK;
    if (routers_on) {
      st = launch_route_scores(n, d, dt, ld, n_ck, ck, gamma, eps, b, (float*)plan, prob, masks,
                               n_ck <= RM_HALVES ? halves : nullptr, s);
      if (st != RIVER_OK) return st;
    } else if (n_ck > 0) {
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
    // one fill for the checkpoints without maps (all of them, or at least
    // two beside checkpoints with maps) when the plain MFMA projection
    // takes the shape: block e_0 + 1 + j (e_0 the first such checkpoint)
    // projects the first m_layer[j] rows of their exit order, gathered from
    // each token's exit checkpoint; checkpoints with maps fill on their own
    river_w4 k0, v0;
    uint32_t mask = 0;
    for (int c = 0; c < n_ck; ++c)
      if (!ck[c].maps && !ck[c].folded) mask |= 1u << c;
    bool single = mask != 0 && (__builtin_popcount(mask) >= 2 || mask == (n_ck == 32 ? ~0u : (1u << n_ck) - 1));
    const int c0 = single ? __builtin_ctz(mask) : 0;
    if (single) {
      decode_layer_offset(*wk, ck[c0].layer, n_out, d, &k0);
      decode_layer_offset(*wv, ck[c0].layer, n_out, d, &v0);
      single = kv_fill_plain_mfma(n, d, dt, n, d, &k0, &v0, n_out);
    }
    DecodePlan q{};
    q.n = n; q.n_ck = n_ck; q.batch_min = rule == RIVER_RULE_BATCH_MIN; q.n_layers = n_layers;
    if (single) { q.ord = ord; q.ck_of = ck_of; q.m_layer = m_layer; q.single_mask = mask; }
    q.cos = (const float*)plan;
    q.prob = routers_on ? prob : nullptr;
    for (int c = 0; c < n_ck; ++c) { q.tau[c] = ck[c].tau; q.theta[c] = ck[c].theta; q.layer[c] = ck[c].layer; }
    char* rec = plan + (size_t)n_ck * CO;
    q.exit_idx = (int32_t*)rec;
    q.idx_stride = (int)(CO / 4);
    q.counts = (int32_t*)(rec + (size_t)n_ck * CO);
    q.exit_layer = exit_layer;
    decode_plan_kernel<<<1, (n + WAVE - 1) / WAVE * WAVE, 0, s>>>(q);
    st = check_launch("decode_step plan");
    if (st != RIVER_OK) return st;
    // The fills left: the single fill, and one per other checkpoint. When
    // there are at least two and the workspace holds, besides what the
    // others take, everything the first checkpoint's fill (the most blocks,
    // with maps its GEMM streams the most maps) would take with unlimited
    // room, that fill runs on a second stream on DECODE_SIDE_CUS of the
    // CUs while the rest run on s on the others: the two share no data
    // (each token exits once) and their kernels make the same choices as
    // in sequence, so the results are the same.
    int side_c = -1, n_fills = single ? 1 : 0;
    for (int c = 0; c < n_ck; ++c) {
      if (single && ((mask >> c) & 1u)) continue;
      if (side_c < 0) side_c = c;
      ++n_fills;
    }
    size_t side_bytes = 0;
    bool use_side = false;
    // a checkpoint with folded products fills without workspace
    auto ck_maps = [&](int c) { return ck[c].maps != nullptr && !ck[c].folded; };
    if (fork_ok && side_c >= 0 && n_fills >= 2 && decode_path_override() == 0) {
      const size_t need_side =
          ck[side_c].folded ? 0 : kv_fill_full_workspace(n, d, n_out, n_layers - ck[side_c].layer, ck_maps(side_c));
      size_t need_rest = single ? kv_fill_full_workspace(n, d, n_out, n_layers - ck[c0].layer, false) : 0;
      for (int c = side_c + 1; c < n_ck; ++c) {
        if (single && ((mask >> c) & 1u)) continue;
        const size_t b = ck[c].folded ? 0 : kv_fill_full_workspace(n, d, n_out, n_layers - ck[c].layer, ck_maps(c));
        need_rest = b > need_rest ? b : need_rest;
      }
      if (need_side + need_rest <= fws_bytes) {
        side_bytes = align_up(need_side, 256);
        use_side = true;
      }
    }
    DecodeSide* side = nullptr;
    std::unique_lock<std::mutex> side_lock;
    if (use_side) {
      st = decode_side(&side);
      if (st != RIVER_OK) return st;
      side_lock = std::unique_lock<std::mutex>(side->mu);
      hipError_t e = hipEventRecord(side->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
      if (e != hipSuccess) return fail(RIVER_ERR_HIP, "decode_step: fork: %s", hipGetErrorString(e));
    }
    auto fill_ck = [&](int c, void* ws, size_t wsb, hipStream_t on) -> river_status {
      const river_checkpoint& k = ck[c];
      const int e = k.layer;
      if (k.folded)
        return launch_kv_fill_folded(n, q.counts + c * 64 + 1, d, k.h_cur, ld, n,
                                     q.exit_idx + (size_t)c * q.idx_stride, slot, n_layers - e, k.folded, n_out,
                                     (char*)k_cache + e * cache_layer, (char*)v_cache + e * cache_layer,
                                     n_slots, on);
      river_w4 k4, v4;
      decode_layer_offset(*wk, e, n_out, d, &k4);
      decode_layer_offset(*wv, e, n_out, d, &v4);
      return launch_kv_fill(n, q.counts + c * 64 + 1, d, dt, k.h_cur, ld, n, q.exit_idx + (size_t)c * q.idx_stride,
                            slot, n_layers - e, k.maps, &k4, &v4, nullptr, n_kv_heads, head_dim,
                            (char*)k_cache + e * cache_layer, (char*)v_cache + e * cache_layer, n_slots, ws,
                            wsb, on);
    };
    if (use_side) {
      CuBudget budget(DECODE_SIDE_CUS);
      st = fill_ck(side_c, fws, side_bytes, side->stream);
    }
    void* rws = (char*)fws + side_bytes;
    const size_t rws_bytes = fws_bytes - side_bytes;
    if (st == RIVER_OK) {
      CuBudget budget(use_side ? N_CU - DECODE_SIDE_CUS : N_CU);
      if (single) {
        DecodeGather gq{};
        gq.n = n; gq.row_bytes = (int)(d * esize(dt)); gq.ld_bytes = ld * (int64_t)esize(dt);
        for (int c = 0; c < n_ck; ++c) gq.hc[c] = ck[c].h_cur;
        gq.ck_of = ck_of; gq.x = xs;
        decode_gather_kernel<<<n, WAVE, 0, s>>>(gq);
        st = check_launch("decode_step gather");
        if (st == RIVER_OK) {
          const int e0 = ck[c0].layer;
          st = launch_kv_fill(n, nullptr, d, dt, xs, d, n, ord, slot, n_layers - e0, nullptr, &k0, &v0, nullptr,
                              n_kv_heads, head_dim, (char*)k_cache + e0 * cache_layer,
                              (char*)v_cache + e0 * cache_layer, n_slots, rws, rws_bytes, s, m_layer);
        }
      }
      for (int c = 0; c < n_ck && st == RIVER_OK; ++c) {
        if ((single && ((mask >> c) & 1u)) || (use_side && c == side_c)) continue;
        st = fill_ck(c, rws, rws_bytes, s);
      }
    }
    if (use_side) {
      // join, also after a failed launch, so that a capture of s stays whole
      hipError_t e = hipEventRecord(side->join, side->stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
      if (e != hipSuccess && st == RIVER_OK) st = fail(RIVER_ERR_HIP, "decode_step: join: %s", hipGetErrorString(e));
    }
    return st;
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
    if (k.folded) {
      st = launch_kv_fill_folded(n, counts + 1, d, k.h_cur, ld, n, exit_idx, slot, n_layers - e, k.folded, n_out,
                                 (char*)k_cache + e * cache_layer, (char*)v_cache + e * cache_layer, n_slots, s);
      if (st != RIVER_OK) return st;
      continue;
    }
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
