// Router calibration: BCE + Adam training of one checkpoint's router.
//
// TIDE, "模块1: 离线校准": the router of formula 3,
//   p = sigmoid(w_up . SiLU(W_down . RMSNorm(h))),
// is trained on calibration states labelled by whether the token has
// converged (cosine to the final-layer state above 0.98), with binary
// cross-entropy and Adam (lr 1e-3) for 100 epochs.
//
// Training runs in fp32 throughout (the oracle is float64), with every
// reduction in a fixed order, so a fit is deterministic. Per mini-batch of
// B tokens two kernels run:
//   forward   one workgroup per 8 tokens: RMSNorm scale, u = W_down x
//             (thread j owns unit j; W_down is kept transposed, [d][b], so
//             the loads are coalesced), SiLU, z, p, the BCE terms, dL/du for
//             every unit, partial dL/dw_up of its tokens;
//   update    one workgroup per KC input channels: dL/dW_down for its
//             columns from dL/du and the normalised inputs, Adam on those
//             columns; workgroup 0 also sums the dL/dw_up partials in order
//             and updates w_up.
// Adam: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
//       p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
#include <type_traits>

#include "common.h"

namespace river {

constexpr int CB_THREADS = 256;
constexpr int CB_RB = 8;              // tokens per forward workgroup
constexpr int CB_KC = 16;             // input channels per update workgroup

struct CalibArgs {
  int n, d, b, B, s0;                 // tokens, features, units, batch size, first batch slot
  const void* h; int64_t ld_h; int bf16;
  const int32_t* order;               // this epoch's token order, or NULL
  const uint8_t* labels;
  const void* gamma; float eps;
  float* wt;                          // W_down transposed [d][b]
  float* wup;                         // [b]
  float* gu;                          // dL/du [B][b]
  float* rs;                          // RMSNorm scale of the batch's tokens [B]
  float* gw_part;                     // [forward workgroups][b]
  float* loss_part;                   // [forward workgroups] of this step
  int nwg1;
  float* mt; float* vt;               // Adam moments of W_down [d][b]
  float* mu; float* vu;               // Adam moments of w_up [b]
  float lr, b1, b2, aeps, bc1, bc2;   // bc = 1 - beta^t
};

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ int token_of(const CalibArgs& a, int i) {
  const int slot = a.s0 + i;
  return a.order ? a.order[slot] : slot;
}

__device__ __forceinline__ float load_x(const CalibArgs& a, int tok, int k) {
  return a.bf16 ? bf16_to_f32(((const uint16_t*)a.h)[(int64_t)tok * a.ld_h + k])
                : ((const float*)a.h)[(int64_t)tok * a.ld_h + k];
}

__device__ __forceinline__ float gam(const CalibArgs& a, int k) {
  if (!a.gamma) return 1.0f;
  return a.bf16 ? bf16_to_f32(((const uint16_t*)a.gamma)[k]) : ((const float*)a.gamma)[k];
}

// block-wide sum over 256 threads in a fixed order
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Forward and dL/du for CB_RB = 8 tokens of the batch, all b units.
// Thread t owns units j = t % 128 + 128 q (q < 4) for tokens 4 (t / 128) ..
// + 3. The features are walked in chunks of KC = 8192 / b128 (b128: b
// rounded up to a multiple of 128): W_down's chunk [KC][b] and gamma * x of
// the 8 tokens [8][KC] go through LDS, double-buffered, the next chunk's
// global loads issued before the current chunk's arithmetic.
constexpr int CB_WBUF = 8192;          // floats of W_down per LDS buffer
template <bool BF16, bool GAMMA, int UPT>   // UPT: groups of 128 units (b <= 128 UPT)
__global__ __launch_bounds__(CB_THREADS) void calib_forward_kernel(CalibArgs a) {
  using raw_t = uint32_t;               // a bf16 load zero-extended, or fp32 bits
  // (+512: the last unit group may read past b; those sums are never used)
  __shared__ __align__(16) float wsm[2][CB_WBUF + 512];
  __shared__ __align__(16) float xsm[2][64][CB_RB];     // [feature][token]
  __shared__ float red[CB_THREADS * 2];
  __shared__ float gwx[128 * 4];
  __shared__ float lossx[2];
  __shared__ float zrow[CB_RB], rrow[CB_RB];
  __shared__ int toks[CB_RB];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * CB_RB;
  const int nr = min(CB_RB, a.B - i0);
  const int d = a.d, b = a.b;
  const int b128 = (b + 127) & ~127;
  const int KC = CB_WBUF / b128;        // 64, 32 or 16
  const int wq = KC * b / 4;            // float4 of W_down per chunk
  if (tid < CB_RB) toks[tid] = tid < nr ? token_of(a, i0 + tid) : -1;
  __syncthreads();
  // x elements of a chunk this thread loads: e = tid + 256 i (i < 2), row
  // e / KC, feature e % KC (8 x KC <= 512 elements)
  const int xe = CB_RB * KC;
  float ssp[2] = {0.f, 0.f};
  int xrow[2], xcol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + CB_THREADS * i;
    xrow[i] = e < xe ? e / KC : 0;
    xcol[i] = e < xe ? e % KC : 0;
  }
  const f32x4* wsrc = (const f32x4*)a.wt;
  // the loads of a chunk only; the arithmetic on them waits until the
  // chunk is stored, so that the loads stay in flight during the compute
  auto load_chunk = [&](int k0, f32x4 (&wr)[8], raw_t (&xr)[2], raw_t (&gr)[2], bool (&ok)[2]) {
    const int kc = min(KC, d - k0);
    const int nq = kc * b / 4;          // b % 4 == 0 is not assumed: scalar tail below
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + CB_THREADS * i;
      wr[i] = wsrc[((int64_t)k0 * b) / 4 + (q < nq ? q : 0)];     // extra lanes reload the first
    }
    // unconditional loads from a valid address (token 0, feature 0 stands
    // in), masked when stored: a load inside a branch would be waited for
    // at the branch's end
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + CB_THREADS * i;
      ok[i] = e < xe && xrow[i] < nr && xcol[i] < kc;
      const int k = ok[i] ? k0 + xcol[i] : 0;
      const int64_t o = ok[i] ? (int64_t)toks[xrow[i]] * a.ld_h + k : 0;
      if constexpr (BF16) {
        xr[i] = ((const uint16_t*)a.h)[o];
        if constexpr (GAMMA) gr[i] = ((const uint16_t*)a.gamma)[k];
      } else {
        xr[i] = ((const uint32_t*)a.h)[o];
        if constexpr (GAMMA) gr[i] = ((const uint32_t*)a.gamma)[k];
      }
    }
  };
  auto store_chunk = [&](int buf, const f32x4 (&wr)[8], const raw_t (&xr)[2], const raw_t (&gr)[2],
                         const bool (&ok)[2]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + CB_THREADS * i;
      if (q < wq) *(f32x4*)&wsm[buf][4 * q] = wr[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + CB_THREADS * i;
      const float x = !ok[i] ? 0.f : BF16 ? __uint_as_float((uint32_t)xr[i] << 16) : __uint_as_float(xr[i]);
      const float g = !GAMMA ? 1.0f : BF16 ? __uint_as_float((uint32_t)gr[i] << 16) : __uint_as_float(gr[i]);
      ssp[i] = fmaf(x, x, ssp[i]);
      if (e < xe) xsm[buf][xcol[i]][xrow[i]] = x * g;
    }
  };
  const int rg = tid >> 7, ul = tid & 127;
  float acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[q][r] = 0.f;
  static_assert(UPT >= 1 && UPT <= 4, "b <= 512");
  f32x4 wr[8];
  raw_t xr[2], gr[2] = {0, 0};
  bool okx[2];
  load_chunk(0, wr, xr, gr, okx);
  store_chunk(0, wr, xr, gr, okx);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < d; k0 += KC) {
    const bool more = k0 + KC < d;
    // the next chunk's loads (after the last chunk: the last one again,
    // unused), unconditional so that nothing waits for them before the
    // arithmetic of this chunk
    load_chunk(more ? k0 + KC : k0, wr, xr, gr, okx);
    const int kc = min(KC, d - k0);         // a multiple of 8
#pragma unroll 8
    for (int c = 0; c < kc; ++c) {
      const f32x4 xv = *(const f32x4*)&xsm[buf][c][4 * rg];
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const float w = wsm[buf][c * b + ul + 128 * q];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(w, xv[r], acc[q][r]);
      }
    }
    if (more) {
      store_chunk(buf ^ 1, wr, xr, gr, okx);
      __syncthreads();
      buf ^= 1;
    }
  }
  // RMSNorm scale of each token: the partial sums of squares by row, in order
  red[2 * tid] = ssp[0];
  red[2 * tid + 1] = ssp[1];
  __syncthreads();
  if (tid < CB_RB) {
    // row tid's elements are e = tid KC .. tid KC + KC - 1, held by thread
    // e % 256 in its slot e / 256
    float ss = 0.f;
    for (int e = tid * KC; e < (tid + 1) * KC; ++e) ss += red[2 * (e & (CB_THREADS - 1)) + e / CB_THREADS];
    rrow[tid] = tid < nr ? rsqrtf(ss / (float)d + a.eps) : 0.f;
  }
  __syncthreads();
  // u, SiLU; z per token: this thread's units, then the 128 threads of the
  // row group (two waves) in a fixed order
  float u[4][4], sg[4][4], part[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    part[r] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = ul + 128 * q;
      u[q][r] = rrow[4 * rg + r] * acc[q][r];
      sg[q][r] = sigm(u[q][r]);
      if (j < b) part[r] = fmaf(a.wup[j], u[q][r] * sg[q][r], part[r]);
    }
    part[r] = wave_sum(part[r]);
  }
  __syncthreads();
  if ((tid & 63) == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(tid >> 6) * 4 + r] = part[r];
  }
  __syncthreads();
  if (tid < CB_RB) {
    const int g = tid >> 2, r = tid & 3;          // row group, row in group
    zrow[tid] = red[(2 * g) * 4 + r] + red[(2 * g + 1) * 4 + r];
  }
  __syncthreads();
  // BCE terms, dL/dz, dL/du, partial dL/dw_up (this thread's 4 tokens)
  float gw[4] = {0.f, 0.f, 0.f, 0.f};
  float loss = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * rg + r;
    if (row < nr) {
      const float z = zrow[row];
      const float y = a.labels[toks[row]] ? 1.0f : 0.0f;
      const float gz = (sigm(z) - y) / (float)a.B;
      // softplus(z) - y z, stable for either sign of z
      loss += fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))) - y * z;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = ul + 128 * q;
        if (j < b) {
          const float sv = sg[q][r], uu = u[q][r];
          gw[q] = fmaf(gz, uu * sv, gw[q]);
          a.gu[(int64_t)(i0 + row) * b + j] = gz * a.wup[j] * (sv * (1.0f + uu * (1.0f - sv)));
        }
      }
    }
  }
  // dL/dw_up partial of the workgroup: row group 0 then 1
  if (rg == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gwx[ul * 4 + q] = gw[q];
  }
  // loss of the workgroup's tokens: rows of group 0 then 1, one thread each
  if (ul == 0) lossx[rg] = loss;
  __syncthreads();
  if (rg == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = ul + 128 * q;
      if (j < b) a.gw_part[(int64_t)blockIdx.x * b + j] = gw[q] + gwx[ul * 4 + q];
    }
  }
  if (tid == 0) a.loss_part[blockIdx.x] = lossx[0] + lossx[1];
  if (tid < nr) a.rs[i0 + tid] = rrow[tid];
}

// dL/dW_down for CB_KC = 16 input channels and Adam on them; workgroup 0
// also updates w_up. Thread t owns units j = t % 128 + 128 q for channels
// 8 (t / 128) .. + 7. The normalised inputs of the channels for all B
// tokens sit in LDS; dL/du streams through LDS in blocks of rows,
// double-buffered.
constexpr int CB_BMAX = 1000;          // largest batch
template <int UPT>
__global__ __launch_bounds__(CB_THREADS) void calib_update_kernel(CalibArgs a) {
  __shared__ __align__(16) float xn[CB_BMAX * CB_KC];   // [B][16]
  __shared__ float gub[2 * 4096 + 512];                 // [2][RC * b] (+ reads past b, unused)
  const int tid = threadIdx.x;
  const int k0 = blockIdx.x * CB_KC;
  const int kc = min(CB_KC, a.d - k0);
  const int b = a.b, B = a.B;
  const int b128 = (b + 127) & ~127;
  const int RC = 4096 / b128;                         // rows per block: 32, 16 or 8
  for (int r = tid; r < B; r += CB_THREADS) {
    const int tok = token_of(a, r);
    const float rsr = a.rs[r];
#pragma unroll
    for (int c = 0; c < CB_KC; ++c)
      xn[r * CB_KC + c] = c < kc ? rsr * gam(a, k0 + c) * load_x(a, tok, k0 + c) : 0.f;
  }
  const int hc = tid >> 7, ul = tid & 127;
  float g[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 8; ++c) g[q][c] = 0.f;
  const int per = RC * b;                             // floats of dL/du per block (<= 4096)
  auto load_rows = [&](int r0, float (&v)[16]) {
    const int nrow = min(RC, B - r0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + CB_THREADS * i;
      v[i] = e < nrow * b ? a.gu[(int64_t)r0 * b + e] : 0.f;
    }
  };
  auto store_rows = [&](int bufi, const float (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + CB_THREADS * i;
      if (e < per) gub[bufi * 4096 + e] = v[i];
    }
  };
  float v[16];
  load_rows(0, v);
  store_rows(0, v);
  __syncthreads();
  int bufi = 0;
  for (int r0 = 0; r0 < B; r0 += RC) {
    const bool more = r0 + RC < B;
    if (more) load_rows(r0 + RC, v);
    const int nrow = min(RC, B - r0);
#pragma unroll 4
    for (int r = 0; r < nrow; ++r) {
      const f32x4 x0 = *(const f32x4*)&xn[(r0 + r) * CB_KC + 8 * hc];
      const f32x4 x1 = *(const f32x4*)&xn[(r0 + r) * CB_KC + 8 * hc + 4];
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const float gu = gub[bufi * 4096 + r * b + ul + 128 * q];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          g[q][c] = fmaf(gu, x0[c], g[q][c]);
          g[q][4 + c] = fmaf(gu, x1[c], g[q][4 + c]);
        }
      }
    }
    if (more) {
      store_rows(bufi ^ 1, v);
      __syncthreads();
      bufi ^= 1;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = ul + 128 * q;
    if (j >= b) continue;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int kk = 8 * hc + c;
      if (kk >= kc) continue;
      const int64_t o = (int64_t)(k0 + kk) * b + j;
      const float m = a.b1 * a.mt[o] + (1.0f - a.b1) * g[q][c];
      const float vv = a.b2 * a.vt[o] + (1.0f - a.b2) * g[q][c] * g[q][c];
      a.mt[o] = m;
      a.vt[o] = vv;
      a.wt[o] -= a.lr * (m / a.bc1) / (sqrtf(vv / a.bc2) + a.aeps);
    }
  }
  if (blockIdx.x == 0) {
    for (int j = tid; j < b; j += CB_THREADS) {
      float gw = 0.f;
      for (int w = 0; w < a.nwg1; ++w) gw += a.gw_part[(int64_t)w * b + j];
      const float m = a.b1 * a.mu[j] + (1.0f - a.b1) * gw;
      const float vv = a.b2 * a.vu[j] + (1.0f - a.b2) * gw * gw;
      a.mu[j] = m;
      a.vu[j] = vv;
      a.wup[j] -= a.lr * (m / a.bc1) / (sqrtf(vv / a.bc2) + a.aeps);
    }
  }
}

// W_down into its transposed working copy, moments to zero
__global__ __launch_bounds__(CB_THREADS) void calib_init_kernel(const float* w_down, float* wt, float* mt,
                                                                 float* vt, float* mu, float* vu, int b,
                                                                 int d) {
  const int64_t e = (int64_t)blockIdx.x * CB_THREADS + threadIdx.x;
  if (e < (int64_t)b * d) {
    const int k = (int)(e / b), j = (int)(e % b);
    wt[e] = w_down[(int64_t)j * d + k];
    mt[e] = 0.f;
    vt[e] = 0.f;
  }
  if (e < b) {
    mu[e] = 0.f;
    vu[e] = 0.f;
  }
}

__global__ __launch_bounds__(CB_THREADS) void calib_finish_kernel(const float* wt, float* w_down, int b,
                                                                   int d) {
  const int64_t e = (int64_t)blockIdx.x * CB_THREADS + threadIdx.x;
  if (e < (int64_t)b * d) {
    const int j = (int)(e / d), k = (int)(e % d);
    w_down[e] = wt[(int64_t)k * b + j];
  }
}

// mean loss per epoch: the partial sums of every step's forward workgroups,
// in order (a step of B_s tokens has ceil(B_s / CB_RB) of them)
__global__ __launch_bounds__(CB_THREADS) void calib_loss_kernel(const float* loss_part, int steps_per_epoch,
                                                                 int epochs, int nwg_max, int n, int B,
                                                                 float* loss_out) {
  const int e = blockIdx.x * CB_THREADS + threadIdx.x;
  if (e >= epochs) return;
  float t = 0.f;
  for (int s = 0; s < steps_per_epoch; ++s) {
    const int bs = min(B, n - s * B);
    const int nw = (bs + CB_RB - 1) / CB_RB;
    for (int w = 0; w < nw; ++w) t += loss_part[((int64_t)e * steps_per_epoch + s) * nwg_max + w];
  }
  loss_out[e] = t / (float)n;
}

}  // namespace river

namespace river_host {
using namespace river;

size_t calib_workspace(int n, int d, int b, int batch, int epochs) {
  const int B = batch < n ? batch : n;
  const int nwg1 = (B + CB_RB - 1) / CB_RB;
  const int steps = (n + B - 1) / B;
  return align_up(3 * (size_t)d * b * 4, 256) + align_up(2 * (size_t)b * 4, 256) +
         align_up((size_t)B * b * 4, 256) + align_up((size_t)B * 4, 256) +
         align_up((size_t)nwg1 * b * 4, 256) + align_up((size_t)epochs * steps * nwg1 * 4, 256);
}

template <bool BF16, bool G>
static void launch_forward_u(const CalibArgs& a, int upt, hipStream_t s) {
  switch (upt) {
    case 1: calib_forward_kernel<BF16, G, 1><<<a.nwg1, CB_THREADS, 0, s>>>(a); break;
    case 2: calib_forward_kernel<BF16, G, 2><<<a.nwg1, CB_THREADS, 0, s>>>(a); break;
    case 3: calib_forward_kernel<BF16, G, 3><<<a.nwg1, CB_THREADS, 0, s>>>(a); break;
    default: calib_forward_kernel<BF16, G, 4><<<a.nwg1, CB_THREADS, 0, s>>>(a); break;
  }
}

static void launch_forward(const CalibArgs& a, bool gamma, int upt, hipStream_t s) {
  if (a.bf16) {
    if (gamma) launch_forward_u<true, true>(a, upt, s);
    else launch_forward_u<true, false>(a, upt, s);
  } else {
    if (gamma) launch_forward_u<false, true>(a, upt, s);
    else launch_forward_u<false, false>(a, upt, s);
  }
}

river_status launch_router_fit(int n, int d, river_dtype dt, const void* h, int64_t ld_h,
                               const uint8_t* labels, const void* gamma, float eps, int b,
                               float* w_down, float* w_up, int epochs, int batch,
                               const int32_t* order, float lr, float beta1, float beta2,
                               float adam_eps, float* loss_out, void* workspace, hipStream_t s) {
  const int B = batch < n ? batch : n;
  const int nwg1 = (B + CB_RB - 1) / CB_RB;
  const int steps = (n + B - 1) / B;
  char* w = (char*)workspace;
  auto take = [&](size_t bytes) { char* p = w; w += align_up(bytes, 256); return p; };
  float* wt = (float*)take(3 * (size_t)d * b * 4);
  float* mt = wt + (size_t)d * b;
  float* vt = mt + (size_t)d * b;
  float* mu = (float*)take(2 * (size_t)b * 4);
  float* vu = mu + b;
  float* gu = (float*)take((size_t)B * b * 4);
  float* rs = (float*)take((size_t)B * 4);
  float* gw_part = (float*)take((size_t)nwg1 * b * 4);
  float* loss_part = (float*)take((size_t)epochs * steps * nwg1 * 4);

  const int64_t bd = (int64_t)b * d;
  calib_init_kernel<<<(unsigned)((bd + CB_THREADS - 1) / CB_THREADS), CB_THREADS, 0, s>>>(
      w_down, wt, mt, vt, mu, vu, b, d);
  river_status st = check_launch("router_fit init");
  if (st != RIVER_OK) return st;
  CalibArgs a{};
  a.n = n; a.d = d; a.b = b;
  a.h = h; a.ld_h = ld_h; a.bf16 = dt == RIVER_BF16;
  a.labels = labels; a.gamma = gamma; a.eps = eps;
  a.wt = wt; a.wup = w_up; a.gu = gu; a.rs = rs; a.gw_part = gw_part;
  a.mt = mt; a.vt = vt; a.mu = mu; a.vu = vu;
  a.lr = lr; a.b1 = beta1; a.b2 = beta2; a.aeps = adam_eps;
  int64_t t = 0;
  double p1 = 1.0, p2 = 1.0;
  for (int e = 0; e < epochs; ++e) {
    a.order = order ? order + (int64_t)e * n : nullptr;
    for (int st_i = 0; st_i < steps; ++st_i) {
      a.s0 = st_i * B;
      a.B = n - a.s0 < B ? n - a.s0 : B;
      a.nwg1 = (a.B + CB_RB - 1) / CB_RB;
      a.loss_part = loss_part + ((int64_t)e * steps + st_i) * nwg1;
      ++t;
      p1 *= beta1;
      p2 *= beta2;
      a.bc1 = (float)(1.0 - p1);
      a.bc2 = (float)(1.0 - p2);
      launch_forward(a, gamma != nullptr, (b + 127) / 128, s);
      const unsigned nwg2 = (unsigned)((d + CB_KC - 1) / CB_KC);
      switch ((b + 127) / 128) {
        case 1: calib_update_kernel<1><<<nwg2, CB_THREADS, 0, s>>>(a); break;
        case 2: calib_update_kernel<2><<<nwg2, CB_THREADS, 0, s>>>(a); break;
        case 3: calib_update_kernel<3><<<nwg2, CB_THREADS, 0, s>>>(a); break;
        default: calib_update_kernel<4><<<nwg2, CB_THREADS, 0, s>>>(a); break;
      }
    }
    st = check_launch("router_fit step");
    if (st != RIVER_OK) return st;
  }
  (void)t;
  calib_finish_kernel<<<(unsigned)((bd + CB_THREADS - 1) / CB_THREADS), CB_THREADS, 0, s>>>(wt, w_down, b, d);
  st = check_launch("router_fit finish");
  if (st != RIVER_OK) return st;
  if (loss_out) {
    calib_loss_kernel<<<(epochs + CB_THREADS - 1) / CB_THREADS, CB_THREADS, 0, s>>>(
        loss_part, steps, epochs, nwg1, n, B, loss_out);
    return check_launch("router_fit loss");
  }
  return RIVER_OK;
}

}  // namespace river_host
