// kv_fill: K/V of every skipped layer, written into each exited token's
// own cache slot.
//
// River-LLM, 方法步骤详情 step 1 / 技术新颖性: the exit path writes K/V at
// the backbone's own addresses (position, head split, dimension layout).
// RidgeFill, 思路源头: each skipped layer's input is predicted from the
// exit state by a fitted linear map and the layer's own projection writes
// the cache. With no map this is River-LLM's State Propagation.
//
// bf16 path, two grouped GEMM phases per chunk of layers:
//   1. x_hat[l] = X . maps[l]^T       (bf16 MFMA, fp32 acc, rounded to bf16
//                                      into the workspace); skipped when the
//                                      map is the identity
//   2. [K|V][l] = x_hat[l] . [Wk[l]; Wv[l]]^T   (int4 dequantized in
//                                      registers, bf16 MFMA) with the cache
//                                      scatter as the epilogue
// Layers are the grid's z dimension, so one launch covers a whole chunk.
//
// Both phases are linear in the exit state, so at row counts well above the
// projection's outputs (given on the host) the fill instead forms, per
// chunk of layers, F[l] = deq([Wk[l]; Wv[l]]) . maps[l] (2 n_out x d, bf16:
// 2 n_out d^2 flops per layer instead of 2 m d^2) and projects the exit
// states through it: [K|V][l] = X . F[l]^T. The same K and V up to
// rounding (one bf16 rounding of F instead of one of x_hat).
//
// Generic path (fp32, or shapes the MFMA tiles do not take): one workgroup
// per (token, layer), fp32 throughout.
//
// river_kv_fill_layer adds the rest of the skipped layer's K/V path: its
// input RMSNorm (gamma_l), K/V biases and the rotary embedding of K. On the
// MFMA path the map GEMM multiplies x_hat by gamma_l before rounding it and
// leaves per-row partial sums of squares (or, without maps, a row kernel
// writes gamma_l * h and the row sums); the projection's epilogue applies the
// row scale, the bias and the rotation to its fp32 accumulators.
#include "common.h"
#include "gemm.h"
#include "gemm_big.h"
#include "gemm_quad.h"
#include "gemm_narrow.h"
#include "w4gemm.h"
#include "w4deep.h"

namespace river {

struct FillGeneric {
  int m_max; const int32_t* m_dev; int d;
  const void* h; int64_t ld_h; int n_rows;
  const int32_t* row_idx; const int32_t* slot;
  const void* maps;
  const uint8_t* q[2]; const void* s[2]; const void* zp[2]; int group[2]; int sz_bf16[2];
  int nh; int64_t n_slots;
  void* kc; void* vc;
  // the layer's K/V path (all optional)
  const void* gamma; float eps;              // dt [n_layers][d]
  const void* bias[2];                       // dt [n_layers][nh]
  const int32_t* pos; const float* rcos; const float* rsin; int64_t n_pos; int head_dim;
};

template <bool BF16>
__global__ __launch_bounds__(256) void kv_fill_generic_kernel(FillGeneric a) {
  extern __shared__ float sm[];   // x [d], x_hat [d], outputs [2 nh], partial sums [4]
  float* x = sm;
  float* xh = sm + a.d;
  float* ko = sm + 2 * a.d;
  float* red = ko + 2 * a.nh;
  int m = a.m_max;
  if (a.m_dev) {
    const int md = *a.m_dev;
    m = md < 0 ? 0 : (md < a.m_max ? md : a.m_max);
  }
  const int t = blockIdx.x, l = blockIdx.y;
  if (t >= m) return;
  const int r = a.row_idx ? a.row_idx[t] : t;
  if (r < 0 || r >= a.n_rows) return;
  const int sl = a.slot[r];
  if (sl < 0 || sl >= a.n_slots) return;
  const int p = a.pos ? a.pos[r] : 0;
  if (a.pos && (p < 0 || p >= a.n_pos)) return;
  const int d = a.d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) x[k] = load_elem<BF16>(a.h, (int64_t)r * a.ld_h + k);
  __syncthreads();
  if (a.maps) {
    const int64_t mo = (int64_t)l * d * d;
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(load_elem<BF16>(a.maps, mo + (int64_t)j * d + k), x[k], acc);
      xh[j] = acc;
    }
  } else {
    for (int k = threadIdx.x; k < d; k += blockDim.x) xh[k] = x[k];
  }
  __syncthreads();
  if (a.gamma) {   // the layer's input RMSNorm
    float ss = 0.f;
    for (int k = threadIdx.x; k < d; k += blockDim.x) ss = fmaf(xh[k], xh[k], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + a.eps);
    for (int k = threadIdx.x; k < d; k += blockDim.x)
      xh[k] = xh[k] * rs * load_elem<BF16>(a.gamma, (int64_t)l * d + k);
    __syncthreads();
  }
  for (int o = threadIdx.x; o < 2 * a.nh; o += blockDim.x) {
    const int which = o >= a.nh ? 1 : 0;
    const int row = o - which * a.nh;
    const int grp = a.group[which];
    const uint8_t* q = a.q[which] + ((int64_t)l * a.nh + row) * (d / 2);
    const int64_t sz0 = ((int64_t)l * a.nh + row) * (d / grp);
    float acc = 0.f;
    for (int k = 0; k < d; k += 2) {
      const uint8_t byte = q[k >> 1];
      const int64_t gi = sz0 + k / grp;
      const float sc = load_sz(a.s[which], gi, a.sz_bf16[which]);
      const float ze = load_sz(a.zp[which], gi, a.sz_bf16[which]);
      acc = fmaf(((float)(byte & 15) - ze) * sc, xh[k], acc);
      acc = fmaf(((float)(byte >> 4) - ze) * sc, xh[k + 1], acc);
    }
    if (a.bias[which]) acc += load_elem<BF16>(a.bias[which], (int64_t)l * a.nh + row);
    ko[o] = acc;
  }
  __syncthreads();
  for (int o = threadIdx.x; o < 2 * a.nh; o += blockDim.x) {
    const int which = o >= a.nh ? 1 : 0;
    const int row = o - which * a.nh;
    float v = ko[o];
    if (a.pos && which == 0) {   // rotary embedding of K, half-split pairs per head
      const int hd = a.head_dim, half = hd >> 1;
      const int i = row % hd;
      const int f = i < half ? i : i - half;
      const float c = a.rcos[(int64_t)p * half + f], sn = a.rsin[(int64_t)p * half + f];
      v = i < half ? ko[o] * c - ko[o + half] * sn : ko[o - half] * sn + ko[o] * c;
    }
    const int64_t off = ((int64_t)l * a.n_slots + sl) * a.nh + row;
    if (BF16) ((uint16_t*)(which ? a.vc : a.kc))[off] = f32_to_bf16(v);
    else ((float*)(which ? a.vc : a.kc))[off] = v;
  }
}

// gamma_l * h[row] for every layer of a chunk (bf16) and the row's sum of
// squares (as four partial sums, the last three zero): the input of the
// projection when the map is the identity and the layer has an input
// RMSNorm. One wave per (row t < m, layer): grid (ceil(m_max / 4), layers);
// the row is read once per layer (from L2 after the first), 16 bytes per
// lane, and layer 0 also writes the row's sum.
__global__ __launch_bounds__(256) void norm_rows_kernel(int m_max, const int32_t* __restrict__ m_dev, int d,
                                                        const uint16_t* __restrict__ h, int64_t ld_h,
                                                        int n_rows, const int32_t* __restrict__ row_idx,
                                                        const uint16_t* __restrict__ gamma,
                                                        uint16_t* __restrict__ xh, int64_t xh_bstride,
                                                        float* __restrict__ ss) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  const int z = blockIdx.y;
  if (t >= m_max) return;
  const int m_in = m_dev ? *m_dev : m_max;
  const int r = row_idx ? row_idx[t] : (int)t;
  if (t >= min(max(m_in, 0), m_max) || r < 0 || r >= n_rows) return;
  const int nch = d / 8;
  const u32x4* src = (const u32x4*)(h + (int64_t)r * ld_h);
  const u32x4* gz = (const u32x4*)(gamma + (int64_t)z * d);
  u32x4* dst = (u32x4*)(xh + (int64_t)z * xh_bstride + t * d);
  float a = 0.f;
  for (int c = lane; c < nch; c += WAVE) {
    const u32x4 v = src[c], gw = gz[c];
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_lo(v[i]), hi = bf16_hi(v[i]);
      a = fmaf(lo, lo, a);
      a = fmaf(hi, hi, a);
      o[i] = pack_bf16x2(lo * bf16_lo(gw[i]), hi * bf16_hi(gw[i]));
    }
    dst[c] = o;
  }
  if (z == 0) {
    a = wave_sum(a);
    if (lane == 0) *(f32x4*)(ss + 4 * t) = f32x4{a, 0.f, 0.f, 0.f};   // four partials, as the map GEMM leaves
  }
}

// The parts of the map GEMM's split reduction (EPI_PART) added in order,
// rounded to bf16 into C: thread (z, row, 8-column piece).
__global__ __launch_bounds__(256) void gemm_part_finish_kernel(GemmArgs g, int batch) {
  const int N = g.N, per = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int p = (int)(idx % per);
  const int t = (int)((idx / per) % g.M_max);
  const int z = (int)(idx / ((int64_t)per * g.M_max));
  if (z >= batch) return;
  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  if (t >= M) return;
  const int col = 8 * p;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < g.ksplit; ++ks) {
    const float* src = g.part + (((int64_t)ks * batch + z) * g.M_max + t) * N + col;
    const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[i];
      v[4 + i] += b[i];
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *(u32x4*)((uint16_t*)g.C + (int64_t)z * g.c_bstride + (int64_t)t * g.ldc + col) = o;
}

// bf16 copies of a chunk's int4 K/V weights, [nl][2 nh][K]: the values the
// W4 kernel forms in registers (dequant8, the same scale and -zero * scale),
// one thread per 32 weights (16 bytes in, 64 bytes out; K % 32 == 0 and the
// group a multiple of 32, so one scale and zero per thread); 32-bit indices
// (nl * 2 nh * K / 32 < 2^31, checked by the launcher)
__global__ __launch_bounds__(256) void w4_dequant_kernel(GemmArgs g, int nl, uint16_t* out) {
  const int K = g.K, nh = g.nh, N = 2 * nh;
  const int per_row = K / 32;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nl * N * per_row) return;
  const int row = idx / per_row, k32 = idx - row * per_row;
  const int z = row / N, col = row - z * N;
  const int which = col >= nh ? 1 : 0, hc = col - which * nh;
  const u32x4 w = *(const u32x4*)(g.q[which] + z * g.q_bstride + (int64_t)hc * (K / 2) + k32 * 16);
  const int gpr = K / g.group[which];
  const int64_t si = z * g.sz_bstride[which] + (int64_t)hc * gpr + (k32 * 32) / g.group[which];
  const float sc = load_sz(g.s[which], si, g.sz_bf16[which]);
  const float ze = load_sz(g.zp[which], si, g.sz_bf16[which]);
  u32x4* o = (u32x4*)(out + (int64_t)row * K + k32 * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v[4];
    dequant8(w[i], sc, -ze * sc, v);
    o[i] = u32x4{v[0], v[1], v[2], v[3]};
  }
}

// out[z] = in[z]^T for d x d bf16 matrices (d % 64 == 0): 64 x 64 tiles,
// 16-byte loads along the rows of in and 16-byte stores along the rows of
// out, the tile transposed through LDS (rows padded by 16 bytes)
__global__ __launch_bounds__(256) void transpose_maps_kernel(const uint16_t* in, uint16_t* out, int d) {
  __shared__ uint16_t t[64][72];
  const int64_t zo = (int64_t)blockIdx.z * d * d;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, ch = i & 7;
    *(u32x4*)&t[r][ch * 8] = *(const u32x4*)(in + zo + (int64_t)(r0 + r) * d + c0 + ch * 8);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int c = i >> 3, ch = i & 7;          // row c of out, its rows ch * 8 .. + 7 of in
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)t[ch * 8 + 2 * e][c] | ((uint32_t)t[ch * 8 + 2 * e + 1][c] << 16);
    *(u32x4*)(out + zo + (int64_t)(c0 + c) * d + r0 + ch * 8) = v;
  }
}

}  // namespace river

namespace river_host {

using namespace river;

// launch of w4_dequant_kernel over nl layers of 2 nh rows of K weights
static river_status w4_dequant_launch(const GemmArgs& q, int nl, uint16_t* out, hipStream_t s) {
  const int64_t threads = (int64_t)nl * 2 * q.nh * (q.K / 32);
  if (q.K % 32 || q.group[0] % 32 || q.group[1] % 32 || threads >= ((int64_t)1 << 31))
    return fail(RIVER_ERR_UNSUPPORTED, "kv_fill: weight dequantisation needs K and the groups in multiples of 32");
  w4_dequant_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(q, nl, out);
  return check_launch("kv_fill weight dequantisation");
}

// The MFMA path: K-slabs in groups of four (d % 256), 64-column blocks inside
// the K or the V half (nh % 64), one quantization group per slab or more
// (group % 64, the same for K and V), an even number of groups per row for
// bf16 scale/zero (read as aligned 4-byte words), and every operand's byte
// span addressable with 31-bit offsets.
static bool fill_mfma_ok(int d, river_dtype dt, int nh, const river_w4* wk, const river_w4* wv,
                         int64_t a_span, int64_t ws_span) {
  const bool even = wk->sz_dtype == RIVER_F32 || (d / wk->group) % 2 == 0;
  const int64_t lim = (int64_t)1 << 31;
  return dt == RIVER_BF16 && d % 256 == 0 && nh % 64 == 0 && wk->group % 64 == 0 &&
         wk->group == wv->group && wk->sz_dtype == wv->sz_dtype && even &&
         a_span < lim && ws_span < lim && (int64_t)4 * nh * d < lim && (int64_t)d * d * 2 < lim;
}

bool kv_fill_plain_mfma(int m_max, int d, river_dtype dt, int n_rows, int64_t ld_h, const river_w4* wk,
                        const river_w4* wv, int nh) {
  return fill_mfma_ok(d, dt, nh, wk, wv, (int64_t)n_rows * ld_h * 2, (int64_t)m_max * d * 2);
}

size_t kv_fill_workspace(int m_max, int d, int n_layers, river_dtype dt) {
  return align_up((size_t)n_layers * (size_t)m_max * (size_t)d * esize(dt), 256);
}

// per layer of a chunk: x_hat (bf16 [m_max][d]) and, with an input norm, the
// partial sums of squares (fp32 [d / 64][m_max])
static size_t layer_xhat_bytes(int m_max, int d) { return align_up((size_t)m_max * d * 2, 256); }
static size_t layer_ss_bytes(int m_max, int d) { return align_up((size_t)(d / 64 > 4 ? d / 64 : 4) * m_max * 4, 256); }

// Parts of the reduction for a projection of at most 256 rows (64-row
// tiles): enough workgroups to fill the CUs, each part a multiple of 256
// input channels, the fp32 partial sums within the space left in the
// workspace. Only a projection with few tiles is split (ks * tiles <= half
// the CUs): at 256 rows, up to 4 layers of 2048 outputs.
static int choose_ksplit(int m_max, int N, int K, int nl, size_t avail) {
  if (m_max > 256) return 1;
  const int tiles = ((N + 255) / 256) * ((m_max + 63) / 64) * nl;
  const int kt = K / 64;
  int ks = 1;
  while (ks < 8 && ks * 2 * tiles <= N_CU && kt % (ks * 2 * 4) == 0 &&
         (size_t)(ks * 2) * nl * m_max * N * 4 <= avail)
    ks *= 2;
  return ks;
}

// Parts of the reduction for the map GEMM (d x d per layer) with few tiles,
// chosen like the projection's: at most one tile per CU, each part a
// multiple of 256 input channels, the partial sums within avail bytes.
static int choose_map_ksplit(int m_max, int d, int nl, size_t avail) {
  const int bm = m_max <= 64 ? 64 : 128;
  const int64_t tiles = (int64_t)((d + 127) / 128) * ((m_max + bm - 1) / bm) * nl;
  const int kt = d / 64;
  int ks = 1;
  while (ks < 8 && ks * 2 * tiles <= N_CU && kt % (ks * 2 * 4) == 0 &&
         (size_t)(ks * 2) * nl * m_max * d * 4 <= avail)
    ks *= 2;
  return ks;
}

// At large row counts the projection runs as the 256x256 bf16 GEMM on
// weights dequantised into the workspace beforehand: each weight is then
// dequantised once per call instead of once per row tile, and the GEMM
// reads 0.75 KB of LDS per MFMA instead of about 1.1. The dequantisation
// costs (1/2 + 2) bytes of traffic per weight, against 2 m flops per weight
// for m rows: from 2048 rows on it is a few percent of the GEMM (at 410
// rows and 21 layers it made the projection slower). At least half a tile
// per CU.
static bool dequant_wanted(int m_max, int N, int nl) {
  return m_max >= 2048 && (int64_t)((N + 255) / 256) * ((m_max + 255) / 256) * nl >= N_CU / 2;
}

// the projection's own workspace: fp32 partial sums of up to 8 parts, K and
// V, for at most 64 rows, and of the parts chosen for 65 to 256 rows; the
// bf16 weights of n_layers layers where they are dequantised beforehand;
// nothing otherwise
size_t kv_fill_proj_workspace(int m_max, int d, int n_out, int n_layers) {
  if (n_out <= 0 || n_layers <= 0 || m_max <= 0) return 0;
  if (m_max <= 64) return align_up((size_t)8 * n_layers * m_max * 2 * n_out * 4, 256);
  if (m_max <= 256) {
    const int ks = choose_ksplit(m_max, 2 * n_out, d, n_layers, SIZE_MAX);
    if (ks > 1) return align_up((size_t)ks * n_layers * m_max * 2 * n_out * 4, 256);
  }
  if (dequant_wanted(m_max, 2 * n_out, n_layers)) return align_up((size_t)n_layers * 2 * n_out * d * 2, 256);
  return 0;
}

// The plain projection's path for nl layers with avail workspace bytes
// (the automatic choice, or the one the gemm-path hook forces):
// PROJ_DEQUANT, the 256 x 256 bf16 GEMM on weights dequantised into the
// workspace; PROJ_SPLIT, the reduction over d in *ks parts whose fp32 sums
// a second kernel adds; PROJ_REGS, the int4 kernel dequantising in
// registers. dev_count: the row count lives on the device (m_max may bound
// far fewer rows, so no automatic dequantisation); per_layer_rows: a row
// count per layer (the decode step's single fill).
enum { PROJ_REGS = 0, PROJ_SPLIT = 1, PROJ_DEQUANT = 2 };
static int proj_path(int m_max, bool dev_count, bool per_layer_rows, int d, int N, int nl, size_t avail,
                     int* ks) {
  const int path = gemm_path_override();
  *ks = 1;
  if (path != 1 && m_max > 64 && !per_layer_rows &&
      (path >= 2 || (!dev_count && dequant_wanted(m_max, N, nl))) && avail >= (size_t)nl * N * d * 2)
    return PROJ_DEQUANT;
  *ks = choose_ksplit(m_max, N, d, nl, avail);
  return *ks > 1 ? PROJ_SPLIT : PROJ_REGS;
}

// Decode-sized projections (a row bound of at most 256 with one count on
// the device) take the deep pipeline (w4deep.h) when it takes the shape and
// its tiles for the count fit one round on the CUs. At the 8B decode shape
// (d = 4096, 2 x 1024 outputs) it measured 41 us against 50 for 13 rows x
// 21 blocks and 24 against 57 (28 split) for 243 rows x 1 block, but 80
// against 65 for 64 rows x 21 blocks (336 tiles): every 32-row tile
// dequantises its weights again.
static bool deep_wanted(int m_max, bool dev_count, const GemmArgs& q) {
  return gemm_path_override() == 0 && dev_count && m_max <= 256 && w4_deep_ok(q);
}

// the workspace bytes of the dequantised weights of nl layers when the
// automatic path projects on them (large row counts), else 0
static size_t dequant_room(int m_max, bool dev_count, int d, int nh, int nl) {
  int ks;
  const int p = proj_path(m_max, dev_count, false, d, 2 * nh, nl, SIZE_MAX, &ks);
  return p == PROJ_DEQUANT ? align_up((size_t)nl * 2 * nh * d * 2, 256) : 0;
}

// The product path (F[l] = deq(W[l]) . maps[l], then X . F[l]^T): for a
// plain fill with maps and the row count on the host, from 2 (2 n_out) rows
// on (F's 2 (2 n_out) d^2 flops at most half the map GEMM's 2 m d^2, which
// leaves room for the maps' transposition), when the 256 x 256 tiles take
// both GEMMs (d % 128 == 0). Per layer the workspace holds the dequantised
// weights, the transposed map and F. The fill-fuse hook: 1 never, 2 from
// one row on.
static size_t fused_layer_bytes(int d, int nh) {
  return 2 * align_up((size_t)2 * nh * d * 2, 256) + align_up((size_t)d * d * 2, 256);
}
static bool fused_wanted(int m_max, bool dev_count, int d, int nh, size_t ws_bytes) {
  const int mode = fill_fuse_override();
  if (mode == 1 || dev_count || d % 128 || gemm_path_override() == 1 || gemm_path_override() == 3) return false;
  if (ws_bytes < fused_layer_bytes(d, nh)) return false;
  return mode == 2 || m_max >= 4 * nh;
}

// Layers per chunk of a fill that keeps x_hat (and, with an input norm, the
// row sums) in the workspace, per_layer bytes per layer. At large row
// counts, as many as fit after the chunk's dequantised weights, so that a
// workspace sized for fewer layers than the call has still projects on
// them; when not even one layer leaves that room, as many layers as fit
// (the projection then dequantises in registers). Otherwise as many as fit;
// what is left holds the partial sums of a split reduction, if any.
static int fill_chunk(int m_max, bool dev_count, int d, int nh, int n_layers, size_t per_layer,
                      size_t ws_bytes, bool plain) {
  const size_t fit = ws_bytes / per_layer;
  const int chunk = fit < (size_t)n_layers ? (int)fit : n_layers;
  if (!plain) return chunk;
  for (int c = chunk; c >= 1; --c)
    if ((size_t)c * per_layer + dequant_room(m_max, dev_count, d, nh, c) <= ws_bytes) return c;
  return chunk;
}

// The workspace from which a fill whose row count lives on the device (a
// decode step's) makes the choices it would make with unlimited room: the
// maps' outputs of all nl layers in one chunk, and the largest split
// reduction its map GEMM or projection would take.
size_t kv_fill_full_workspace(int m_max, int d, int n_out, int nl, bool maps) {
  if (m_max <= 0 || nl <= 0) return 0;
  const int kp = choose_ksplit(m_max, 2 * n_out, d, nl, SIZE_MAX);
  size_t split = kp > 1 ? (size_t)kp * nl * m_max * 2 * n_out * 4 : 0;
  // the deep projection's split keeps every part's 32-row tile on a CU of
  // its own: at most N_CU x 32 x 256 partial sums
  if (m_max <= 256 && split < (size_t)N_CU * 32 * 256 * 4) split = (size_t)N_CU * 32 * 256 * 4;
  if (!maps) return align_up(split, 256);
  // (the map GEMM splits only where the 32-row tiles do not take it)
  const int km = m_max <= 256 && d % 512 == 0 ? 1 : choose_map_ksplit(m_max, d, nl, SIZE_MAX);
  const size_t ms = km > 1 ? (size_t)km * nl * m_max * d * 4 : 0;
  return (size_t)nl * layer_xhat_bytes(m_max, d) + align_up(ms > split ? ms : split, 256);
}

// the split space any fill of a decode step may use: blocks e + 1 .. L for a
// checkpoint e, 1 to n_layers - 1 layers of at most n rows each
size_t decode_proj_workspace(int n, int d, int n_out, int n_layers) {
  if (n > 256) return 0;
  size_t m = 0;
  for (int nl = 1; nl < n_layers; ++nl) {
    const size_t b = kv_fill_proj_workspace(n, d, n_out, nl);
    if (b > m) m = b;
  }
  return m;
}

size_t kv_fill_layer_workspace(int m_max, int d, int n_layers) {
  return (size_t)n_layers * (layer_xhat_bytes(m_max, d) + layer_ss_bytes(m_max, d));
}

// The int4 fields of GemmArgs for the K/V weights of a fill (layer 0 of the
// descriptors at q[0], s[0], zp[0] for K and [1] for V).
static void set_w4(GemmArgs& g, int d, int nh, const river_w4* wk, const river_w4* wv) {
  g.q[0] = wk->q; g.q[1] = wv->q;
  g.s[0] = wk->scale; g.s[1] = wv->scale;
  g.zp[0] = wk->zero; g.zp[1] = wv->zero;
  g.group[0] = wk->group; g.group[1] = wv->group;
  g.sz_bf16[0] = wk->sz_dtype == RIVER_BF16; g.sz_bf16[1] = wv->sz_dtype == RIVER_BF16;
  g.nh = nh;
  g.q_bstride = (int64_t)nh * d / 2;
  g.sz_bstride[0] = (int64_t)nh * (d / wk->group);
  g.sz_bstride[1] = (int64_t)nh * (d / wv->group);
}

// F[l] = deq([Wk[l]; Wv[l]]) . maps[l] for layers l0 .. l0 + nl - 1 of the
// weights in g (set_w4): the weights dequantised as the int4 kernels form
// them, the maps transposed, then the product (rows: the 2 n_out outputs,
// reduction over the map's output index, a row of the transposed map),
// rounded to bf16 into F (layer stride f_bs elements). Without maps F is the
// dequantised weights. ws holds chunk layers of dequantised weights followed
// by chunk layers of transposed maps (nl <= chunk).
static river_status form_products(const GemmArgs& g, int d, int l0, int nl, const void* maps, uint16_t* F,
                                  int64_t f_bs, void* ws, int chunk, hipStream_t s) {
  const int nh = g.nh;
  const size_t wb = align_up((size_t)2 * nh * d * 2, 256);
  GemmArgs q = g;
  q.N = 2 * nh;
  q.q[0] = g.q[0] + (int64_t)l0 * q.q_bstride;
  q.q[1] = g.q[1] + (int64_t)l0 * q.q_bstride;
  q.s[0] = (const char*)g.s[0] + (int64_t)l0 * q.sz_bstride[0] * (g.sz_bf16[0] ? 2 : 4);
  q.zp[0] = (const char*)g.zp[0] + (int64_t)l0 * q.sz_bstride[0] * (g.sz_bf16[0] ? 2 : 4);
  q.s[1] = (const char*)g.s[1] + (int64_t)l0 * q.sz_bstride[1] * (g.sz_bf16[1] ? 2 : 4);
  q.zp[1] = (const char*)g.zp[1] + (int64_t)l0 * q.sz_bstride[1] * (g.sz_bf16[1] ? 2 : 4);
  if (!maps) {
    if (f_bs != (int64_t)q.N * d) return fail(RIVER_ERR_ARG, "kv_fold: identity needs a packed F");
    return w4_dequant_launch(q, nl, F, s);
  }
  uint16_t* dq = (uint16_t*)ws;
  uint16_t* tr = (uint16_t*)((char*)ws + (size_t)chunk * wb);
  river_status st = w4_dequant_launch(q, nl, dq, s);
  if (st != RIVER_OK) return st;
  transpose_maps_kernel<<<dim3((unsigned)(d / 64), (unsigned)(d / 64), (unsigned)nl), 256, 0, s>>>(
      (const uint16_t*)maps + (int64_t)l0 * d * d, tr, d);
  if ((st = check_launch("kv_fill map transposition")) != RIVER_OK) return st;
  GemmArgs f{};
  f.M_max = q.N; f.N = d; f.K = d;
  f.A = dq; f.lda = d; f.a_bstride = (int64_t)q.N * d; f.a_nrows = q.N;
  f.B = tr; f.ldb = d; f.b_bstride = (int64_t)d * d;
  f.C = F; f.ldc = d; f.c_bstride = f_bs;
  const int tf = debug_timer_begin(s, RIVER_TIMED_FILL_PRODUCT);
  gemm_bf16_auto<EPI_BF16>(f, nl, s);
  debug_timer_end(s, tf);
  return check_launch("kv_fill map-weight product");
}

river_status launch_kv_fill(int m_max, const int32_t* m_dev, int d, river_dtype dt, const void* h,
                            int64_t ld_h, int n_rows, const int32_t* row_idx, const int32_t* slot,
                            int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                            const river_layer* L, int n_kv_heads, int head_dim, void* k_cache,
                            void* v_cache, int64_t n_slots, void* workspace, size_t ws_bytes,
                            hipStream_t s, const int32_t* m_dev_layer) {
  const int nh = n_kv_heads * head_dim;
  const void* gamma = L ? L->norm_gamma : nullptr;
  const bool has_bias = L && (L->k_bias || L->v_bias);
  const bool rope = L && L->pos;
  const bool layer = gamma || has_bias || rope;
  const bool mfma = fill_mfma_ok(d, dt, nh, wk, wv, (int64_t)n_rows * ld_h * 2, (int64_t)m_max * d * 2) &&
                    (!rope || head_dim % 32 == 0) && (!gamma || d <= 8192);
  if (m_dev_layer && (!mfma || layer || maps))
    return fail(RIVER_ERR_UNSUPPORTED, "kv_fill: per-layer row counts need the plain MFMA path");
  if (!mfma) {
    const size_t lds = (2 * (size_t)d + 2 * (size_t)nh + 4) * sizeof(float);
    if (lds > 65536) return fail(RIVER_ERR_UNSUPPORTED, "kv_fill: d = %d, n_out = %d too large for the generic path", d, nh);
    FillGeneric a{m_max, m_dev, d, h, ld_h, n_rows, row_idx, slot, maps,
                  {wk->q, wv->q}, {wk->scale, wv->scale}, {wk->zero, wv->zero},
                  {wk->group, wv->group},
                  {wk->sz_dtype == RIVER_BF16, wv->sz_dtype == RIVER_BF16}, nh, n_slots,
                  k_cache, v_cache,
                  gamma, L ? L->norm_eps : 0.f,
                  {L ? L->k_bias : nullptr, L ? L->v_bias : nullptr},
                  rope ? L->pos : nullptr, rope ? L->rope_cos : nullptr,
                  rope ? L->rope_sin : nullptr, rope ? L->n_pos : 0, head_dim};
    dim3 grid(m_max, n_layers);
    if (dt == RIVER_BF16) kv_fill_generic_kernel<true><<<grid, 256, lds, s>>>(a);
    else kv_fill_generic_kernel<false><<<grid, 256, lds, s>>>(a);
    return check_launch("kv_fill generic");
  }

  GemmArgs g{};
  g.K = d;
  g.M_max = m_max;
  g.M_dev = m_dev;
  g.M_dev_z = m_dev_layer;
  set_w4(g, d, nh, wk, wv);
  g.slot = slot;
  g.n_slots = n_slots;
  g.e_nrows = n_rows;
  g.cache_bstride = n_slots * nh;
  if (rope) {
    g.pos = L->pos; g.rcos = L->rope_cos; g.rsin = L->rope_sin; g.n_pos = L->n_pos;
    g.head_dim = head_dim;
  }

  // ss: partial sums of squares of this chunk's rows (parts per row, layer
  // stride ss_bs; 0 when every layer shares one input)
  // part_ws: workspace left for the partial sums of a split reduction
  char* part_ws = nullptr;
  size_t part_bytes = 0;
  auto stage2 = [&](int l0, int nl, const uint16_t* A, int64_t lda, int64_t a_bs,
                    const int32_t* a_rows, int a_nrows, const float* ss, int64_t ss_bs,
                    int parts) -> river_status {
    GemmArgs q = g;
    q.N = 2 * nh;
    q.A = A; q.lda = lda; q.a_bstride = a_bs; q.a_rows = a_rows; q.a_nrows = a_nrows;
    q.q[0] = wk->q + (int64_t)l0 * q.q_bstride;
    q.q[1] = wv->q + (int64_t)l0 * q.q_bstride;
    q.s[0] = (const char*)wk->scale + (int64_t)l0 * q.sz_bstride[0] * esize(wk->sz_dtype);
    q.zp[0] = (const char*)wk->zero + (int64_t)l0 * q.sz_bstride[0] * esize(wk->sz_dtype);
    q.s[1] = (const char*)wv->scale + (int64_t)l0 * q.sz_bstride[1] * esize(wv->sz_dtype);
    q.zp[1] = (const char*)wv->zero + (int64_t)l0 * q.sz_bstride[1] * esize(wv->sz_dtype);
    q.e_rows = row_idx;
    q.kc = (uint16_t*)k_cache + (int64_t)l0 * q.cache_bstride;
    q.vc = (uint16_t*)v_cache + (int64_t)l0 * q.cache_bstride;
    if (!layer) {
      if (deep_wanted(m_max, m_dev != nullptr && q.M_dev_z == nullptr, q)) {
        // the deep pipeline when its 32-row tiles for the count on the
        // device fit one round on the CUs, with the workspace left for the
        // partial sums of a split it chooses on the device; otherwise the
        // path below (each launch does nothing for the other's counts).
        // Both choices take the whole chip's CUs, whatever the launch's
        // budget, so that the results do not depend on it.
        const int cus = N_CU;
        GemmArgs qd = q;
        qd.gate = 1;
        qd.gate_units = ((q.N + 255) / 256) * nl;
        qd.gate_cus = cus;
        // (a split needs fewer tiles than half the CUs: with more column
        // tiles than that none is possible, and no finish kernel runs)
        if (part_bytes >= (size_t)256 * q.N * 4 && 2 * qd.gate_units <= cus) {
          qd.part = (float*)part_ws;
          qd.part_cap = (int64_t)part_bytes;
        }
        const bool all_deep = (int64_t)((m_max + 31) / 32) * qd.gate_units <= cus;
        int ks;
        if (!all_deep && m_max > 64 &&
            proj_path(m_max, true, false, d, q.N, nl, part_bytes, &ks) == PROJ_REGS) {
          // the other counts on the 128-row kernel without a split: one
          // launch takes both
          w4_either_launch(qd, nl, s);
          return check_launch("kv_fill projection (deep or 128-row)");
        }
        w4_deep_launch(qd, nl, s);
        river_status st = check_launch("kv_fill projection (deep)");
        if (st != RIVER_OK || all_deep) return st;
        q.gate = -1;
        q.gate_units = qd.gate_units;
        q.gate_cus = cus;
      }
      int ks;
      const int pp = proj_path(m_max, m_dev != nullptr, q.M_dev_z != nullptr, d, q.N, nl, part_bytes, &ks);
      if (pp == PROJ_DEQUANT) {
        uint16_t* dq = (uint16_t*)part_ws;
        river_status st = w4_dequant_launch(q, nl, dq, s);
        if (st != RIVER_OK) return st;
        GemmArgs p = q;
        p.B = dq; p.ldb = d; p.b_bstride = (int64_t)q.N * d;
        const int tp = debug_timer_begin(s, RIVER_TIMED_FILL_PROJECTION);
        gemm_cache_launch(p, nl, s);
        debug_timer_end(s, tp);
        return check_launch("kv_fill projection (bf16)");
      }
      if (pp == PROJ_SPLIT) {
        q.ksplit = ks;
        q.part = (float*)part_ws;
        w4_gemm_launch<64, EPI_PART, false>(q, nl, s);
        river_status st = check_launch("kv_fill projection parts");
        if (st != RIVER_OK) return st;
        const int64_t threads = (int64_t)nl * m_max * (q.N / 8);
        w4_part_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(q, nl);
        return check_launch("kv_fill projection sum");
      }
      w4_gemm_auto<EPI_CACHE>(q, nl, s);
      return check_launch("kv_fill projection");
    }
    q.ss_in = ss; q.ss_in_bstride = ss_bs; q.ss_parts = parts; q.norm_eps = L->norm_eps;
    q.bias[0] = L->k_bias ? (const uint16_t*)L->k_bias + (int64_t)l0 * nh : nullptr;
    q.bias[1] = L->v_bias ? (const uint16_t*)L->v_bias + (int64_t)l0 * nh : nullptr;
    q.bias_bstride = nh;
    w4_gemm_auto<EPI_CACHE, true>(q, nl, s);
    return check_launch("kv_fill projection");
  };

  if (!maps && !gamma) {
    part_ws = (char*)workspace;
    part_bytes = workspace ? ws_bytes : 0;
    return stage2(0, n_layers, (const uint16_t*)h, ld_h, 0, row_idx, n_rows, nullptr, 0, 0);
  }

  if (maps && !layer && fused_wanted(m_max, m_dev != nullptr, d, nh, ws_bytes)) {
    // per chunk: F = deq(W) . maps in the workspace, then the exit states
    // through F
    const size_t wb = align_up((size_t)2 * nh * d * 2, 256);
    const int fchunk = ws_bytes / fused_layer_bytes(d, nh) < (size_t)n_layers
                           ? (int)(ws_bytes / fused_layer_bytes(d, nh)) : n_layers;
    uint16_t* fw = (uint16_t*)((char*)workspace + (size_t)fchunk * (fused_layer_bytes(d, nh) - wb));
    for (int l0 = 0; l0 < n_layers; l0 += fchunk) {
      const int nl = n_layers - l0 < fchunk ? n_layers - l0 : fchunk;
      river_status st = form_products(g, d, l0, nl, maps, fw, (int64_t)wb / 2, workspace, fchunk, s);
      if (st != RIVER_OK) return st;
      // [K|V][l] = X . F[l]^T into the cache
      GemmArgs pr = g;
      pr.N = 2 * nh;
      pr.A = (const uint16_t*)h; pr.lda = ld_h; pr.a_bstride = 0; pr.a_rows = row_idx; pr.a_nrows = n_rows;
      pr.B = fw; pr.ldb = d; pr.b_bstride = (int64_t)wb / 2;
      pr.e_rows = row_idx;
      pr.kc = (uint16_t*)k_cache + (int64_t)l0 * g.cache_bstride;
      pr.vc = (uint16_t*)v_cache + (int64_t)l0 * g.cache_bstride;
      const int tp = debug_timer_begin(s, RIVER_TIMED_FILL_PROJECTION);
      gemm_cache_launch(pr, nl, s);
      debug_timer_end(s, tp);
      if ((st = check_launch("kv_fill projection through the product")) != RIVER_OK) return st;
    }
    return RIVER_OK;
  }

  const size_t xb = layer_xhat_bytes(m_max, d), sb = gamma ? layer_ss_bytes(m_max, d) : 0;
  const int chunk = fill_chunk(m_max, m_dev != nullptr, d, nh, n_layers, xb + sb, ws_bytes, !layer);
  uint16_t* xh = (uint16_t*)workspace;
  float* ss = (float*)((char*)workspace + (size_t)chunk * xb);
  part_ws = (char*)workspace + (size_t)chunk * (xb + sb);
  part_bytes = ws_bytes - (size_t)chunk * (xb + sb);
  const int parts = maps ? d / 64 : 4;
  for (int l0 = 0; l0 < n_layers; l0 += chunk) {
    const int nl = n_layers - l0 < chunk ? n_layers - l0 : chunk;
    river_status st;
    if (maps) {
      GemmArgs p = g;
      p.N = d;
      p.A = (const uint16_t*)h; p.lda = ld_h; p.a_bstride = 0; p.a_rows = row_idx; p.a_nrows = n_rows;
      p.B = (const uint16_t*)maps + (int64_t)l0 * d * d; p.ldb = d; p.b_bstride = (int64_t)d * d;
      p.C = xh; p.ldc = d; p.c_bstride = xb / 2;
      // a decode-sized row bound with the count on the device: 32-row tiles
      // with eight slabs of maps in flight (at 243 rows x one block of
      // 4096^2: 19 us, against 23 + 5.5 for the split below)
      const bool narrow = !gamma && gemm_path_override() == 0 && m_dev && m_max <= 256 && gemm_narrow_ok(p);
      const int mks = gamma || narrow || gemm_path_override() != 0 ? 1 : choose_map_ksplit(m_max, d, nl, part_bytes);
      if (gamma) {
        p.gamma = (const uint16_t*)gamma + (int64_t)l0 * d; p.gamma_bstride = d;
        p.ss = ss; p.ss_bstride = sb / 4;
        gemm_bf16_auto<EPI_BF16N>(p, nl, s);
        st = check_launch("kv_fill map");
      } else if (mks > 1) {
        // few tiles (a decode-sized batch): the reduction over d in parts,
        // their fp32 sums in the space after the maps' outputs, added in order
        p.ksplit = mks;
        p.part = (float*)part_ws;
        if (m_max <= 64) gemm_launch<64, EPI_PART>(p, nl, s);
        else gemm_launch<128, EPI_PART>(p, nl, s);
        st = check_launch("kv_fill map parts");
        if (st == RIVER_OK) {
          const int64_t threads = (int64_t)nl * m_max * (d / 8);
          gemm_part_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(p, nl);
          st = check_launch("kv_fill map sum");
        }
      } else if (narrow && nl == 1 && launch_cu_budget() < 128) {
        // one map on few CUs (a decode step's later fill beside the first
        // one): the 128-row tiles, a quarter of the tiles with four times
        // the MFMA work per byte; bit-identical to the 32-row tiles over one
        // map
        gemm_launch<128, EPI_BF16>(p, nl, s);
        st = check_launch("kv_fill map");
      } else if (narrow || (gemm_path_override() == 0 && m_max <= 256 && gemm_narrow_ok(p))) {
        // decode-sized row bound: 32-row tiles with eight slabs of maps in flight
        gemm_narrow_launch(p, nl, s);
        st = check_launch("kv_fill map narrow");
      } else {
        gemm_bf16_auto<EPI_BF16>(p, nl, s);
        st = check_launch("kv_fill map");
      }
    } else {
      const dim3 grid((unsigned)(((int64_t)m_max + 3) / 4), (unsigned)nl);
      norm_rows_kernel<<<grid, 256, 0, s>>>(m_max, m_dev, d, (const uint16_t*)h, ld_h, n_rows, row_idx,
                                            (const uint16_t*)gamma + (int64_t)l0 * d, xh, xb / 2, ss);
      st = check_launch("kv_fill norm rows");
    }
    if (st != RIVER_OK) return st;
    st = stage2(l0, nl, xh, d, xb / 2, nullptr, m_max, gamma ? ss : nullptr,
                maps ? (int64_t)(sb / 4) : 0, parts);
    if (st != RIVER_OK) return st;
  }
  return RIVER_OK;
}

// workspace of river_kv_fold for chunk layers per pass: the dequantised
// weights and the transposed map of each (nothing without maps)
size_t kv_fold_workspace(int d, int n_out, int chunk, bool maps) {
  if (!maps || chunk <= 0) return 0;
  return (size_t)chunk * (fused_layer_bytes(d, n_out) - align_up((size_t)2 * n_out * d * 2, 256));
}

// the shapes the folded products take: bf16, d % 128 == 0 (the 256 x 256
// product and projection tiles), 2 n_out outputs in 64-column blocks
bool kv_fold_ok(int d, int nh, const river_w4* wk, const river_w4* wv) {
  return fill_mfma_ok(d, RIVER_BF16, nh, wk, wv, 0, 0) && d % 128 == 0 && nh % 8 == 0;
}

river_status launch_kv_fold(int d, int n_layers, const void* maps, const river_w4* wk, const river_w4* wv,
                            int nh, void* F, void* workspace, size_t ws_bytes, hipStream_t s) {
  GemmArgs g{};
  g.K = d;
  set_w4(g, d, nh, wk, wv);
  const int64_t f_bs = (int64_t)2 * nh * d;
  const size_t per = kv_fold_workspace(d, nh, 1, maps != nullptr);
  const int chunk = !maps ? n_layers : (ws_bytes / per < (size_t)n_layers ? (int)(ws_bytes / per) : n_layers);
  for (int l0 = 0; l0 < n_layers; l0 += chunk) {
    const int nl = n_layers - l0 < chunk ? n_layers - l0 : chunk;
    river_status st = form_products(g, d, l0, nl, maps, (uint16_t*)F + l0 * f_bs, f_bs, workspace, chunk, s);
    if (st != RIVER_OK) return st;
  }
  return RIVER_OK;
}

// [K|V][l] = X . F[l]^T into the cache: the 32 x 128 tiles with eight slabs
// of F in flight for a decode-sized row bound (at most 256 rows, d % 512),
// the 256 x 256 tiles otherwise; the row count on the host (m_max) or on the
// device (m_dev, at most m_max). No workspace.
river_status launch_kv_fill_folded(int m_max, const int32_t* m_dev, int d, const void* h, int64_t ld_h,
                                   int n_rows, const int32_t* row_idx, const int32_t* slot, int n_layers,
                                   const void* F, int nh, void* k_cache, void* v_cache, int64_t n_slots,
                                   hipStream_t s) {
  GemmArgs g{};
  g.M_max = m_max; g.M_dev = m_dev;
  g.N = 2 * nh; g.K = d; g.nh = nh;
  g.A = (const uint16_t*)h; g.lda = ld_h; g.a_bstride = 0; g.a_rows = row_idx; g.a_nrows = n_rows;
  g.B = (const uint16_t*)F; g.ldb = d; g.b_bstride = (int64_t)2 * nh * d;
  g.e_rows = row_idx; g.e_nrows = n_rows;
  g.slot = slot; g.n_slots = n_slots;
  g.cache_bstride = n_slots * nh;
  g.kc = k_cache; g.vc = v_cache;
  if (m_max <= 256 && gemm_narrow_ok(g) && gemm_path_override() == 0) {
    gemm_narrow_launch<EPI_CACHE>(g, n_layers, s);
    return check_launch("kv_fill folded (32-row tiles)");
  }
  const int tp = debug_timer_begin(s, RIVER_TIMED_FILL_PROJECTION);
  gemm_cache_launch(g, n_layers, s);
  debug_timer_end(s, tp);
  return check_launch("kv_fill folded");
}

// the plan of a plain bf16 fill with maps (the test hook
// river_debug_kv_fill_plan): layers per chunk, and the projection's path
// and parts for the first chunk
void kv_fill_plan(int m_max, bool dev_count, int d, int nh, int n_layers, size_t ws_bytes, int* chunk,
                  int* path, int* ks) {
  if (fused_wanted(m_max, dev_count, d, nh, ws_bytes)) {
    const size_t per = fused_layer_bytes(d, nh);
    *chunk = ws_bytes / per < (size_t)n_layers ? (int)(ws_bytes / per) : n_layers;
    *path = 3;
    *ks = 1;
    return;
  }
  const size_t xb = layer_xhat_bytes(m_max, d);
  *chunk = fill_chunk(m_max, dev_count, d, nh, n_layers, xb, ws_bytes, true);
  const size_t used = (size_t)*chunk * xb;
  *path = *chunk > 0 ? proj_path(m_max, dev_count, false, d, 2 * nh, *chunk, ws_bytes - used, ks) : PROJ_REGS;
  if (*chunk == 0) *ks = 1;
}

}  // namespace river_host
