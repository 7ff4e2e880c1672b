// ridge_fit: closed-form ridge maps W_t = (X^T X + lambda I)^-1 X^T Y_t
// (RidgeFill, closed-form ridge regression box), fitted once from one
// calibration pass; X holds split-layer states, Y_t a later layer's inputs.
//
// Steps (bf16 inputs):
//   1. Xt = X^T, Yt = Y_t^T  (LDS-tiled transposes, so every contraction
//      over the token dimension becomes a K-contiguous MFMA GEMM)
//   2. G = X^T X + lambda I   bf16 MFMA, fp32 accumulate (bf16 x bf16
//      products are exact in fp32)
//   3. G = L L^T              blocked fp32 Cholesky (64-wide panels): a
//      one-workgroup factor of the diagonal block, a triangular solve of
//      the panel below it, and a lower-triangular update of the trailing
//      matrix; a pivot that is not positive raises a device flag
//   4. G^-1 = L^-T L^-1       blocked fp32 triangular inverse, then X^T X
//   5. per target: C_t^T = Y_t^T X (MFMA), then W_t^T = C_t^T G^-1 with
//      both fp32 factors split into bf16 hi + lo parts:
//      C G ~= Chi Ghi + Chi Glo + Clo Ghi, one MFMA GEMM over a K axis of
//      3 d_in (relative error ~2^-16 per product instead of bf16's 2^-8).
// fp32 inputs take the same factorization with fp32 VALU GEMMs.
#include "common.h"
#include "gemm.h"

namespace river {

// ---------------------------------------------------- fp32 VALU GEMM
// C(m, n) = alpha * sum_k A(m, k) B(n, k) + beta * C(m, n) with arbitrary
// element strides: A(m, k) = A[m*sam + k*sak], B(n, k) = B[n*sbn + k*sbk],
// C(m, n) = C[m*ldc + n]; batch z adds a*_bs offsets. lower: skip tiles
// strictly above the diagonal.
struct VGemm {
  int M, N, K;
  const float* A; int64_t sam, sak, a_bs;
  const float* B; int64_t sbn, sbk, b_bs;
  void* C; int64_t ldc, c_bs;
  float alpha, beta;
  int lower;
};

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void vgemm_kernel(VGemm g) {
  constexpr int T = 64, BK = 16;
  __shared__ float As[BK][T + 4];
  __shared__ float Bs[BK][T + 4];
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T, z = blockIdx.z;
  if (g.lower && n0 > m0 + T - 1) return;
  const float* A = g.A + (int64_t)z * g.a_bs;
  const float* B = g.B + (int64_t)z * g.b_bs;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;
      // element e of the 64 x 16 tile: the row index varies fastest when the
      // row stride is 1, the k index otherwise (coalescing)
      int r, k;
      if (g.sam == 1) { r = e & 63; k = e >> 6; } else { k = e & 15; r = e >> 4; }
      const int gm = m0 + r, gk = k0 + k;
      As[k][r] = (gm < g.M && gk < g.K) ? A[gm * g.sam + gk * g.sak] : 0.f;
      if (g.sbn == 1) { r = e & 63; k = e >> 6; } else { k = e & 15; r = e >> 4; }
      const int gn = n0 + r, gk2 = k0 + k;
      Bs[k][r] = (gn < g.N && gk2 < g.K) ? B[gn * g.sbn + gk2 * g.sbk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[k][ty + 16 * i]; b[i] = Bs[k][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty + 16 * i;
    if (gm >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx + 16 * j;
      if (gn >= g.N) continue;
      const int64_t o = (int64_t)z * g.c_bs + (int64_t)gm * g.ldc + gn;
      if constexpr (OUT_BF16) {
        ((uint16_t*)g.C)[o] = f32_to_bf16(g.alpha * acc[i][j]);
      } else {
        float* c = (float*)g.C;
        const float prev = g.beta != 0.f ? g.beta * c[o] : 0.f;
        c[o] = fmaf(g.alpha, acc[i][j], prev);
      }
    }
  }
}

// ------------------------------------------------------ elementwise
// out[c][r] = in[r][c] for r < R; out[c][r] = 0 for R <= r < R_pad (the
// padding that makes the GEMM's reduction length a multiple of 256)
__global__ void transpose_bf16_kernel(const uint16_t* in, int R, int R_pad, int C, int64_t ld_in,
                                      uint16_t* out, int64_t ld_out) {
  __shared__ uint16_t t[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
    const int r = i >> 6, c = i & 63;
    t[r][c] = (r0 + r < R && c0 + c < C) ? in[(int64_t)(r0 + r) * ld_in + c0 + c] : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
    const int c = i >> 6, r = i & 63;
    if (c0 + c < C && r0 + r < R_pad) out[(int64_t)(c0 + c) * ld_out + r0 + r] = t[r][c];
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void add_diag_kernel(float* G, int d, float lam) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) G[(int64_t)i * d + i] += lam;
}

__global__ void zero_upper_kernel(float* G, int d) {
  const int64_t n = (int64_t)d * d;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    if ((i % d) > (i / d)) G[i] = 0.f;
}

// split fp32 rows into bf16 hi/lo parts laid out as three K-blocks, each
// row padded with zeros to ld_out columns:
// out[r][p*C + c] = part(p)(in[r][c]), part = hi when (pattern >> p) & 1 == 0
__global__ void split3_kernel(const float* in, int R, int C, uint16_t* out, int64_t ld_out, int pattern) {
  const int64_t n = (int64_t)R * ld_out;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ld_out, j = i % ld_out;
    const int p = (int)(j / C);
    uint16_t o = 0;
    if (p < 3) {
      const float v = in[r * C + j % C];
      const uint16_t hi = f32_to_bf16(v);
      o = ((pattern >> p) & 1) ? f32_to_bf16(v - bf16_to_f32(hi)) : hi;
    }
    out[i] = o;
  }
}

__global__ void f32_to_bf16_kernel(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = f32_to_bf16(in[i]);
}

// ------------------------------------------------------------ Cholesky
constexpr int NB = 64;

// factor the diagonal block at j0 (size nb <= 64) in place, lower
__global__ __launch_bounds__(256) void potrf_diag_kernel(float* G, int d, int j0, int nb, int* flag) {
  __shared__ float a[NB][NB + 1];
  for (int i = threadIdx.x; i < nb * nb; i += blockDim.x) {
    const int r = i / nb, c = i % nb;
    a[r][c] = G[(int64_t)(j0 + r) * d + j0 + c];
  }
  __syncthreads();
  for (int k = 0; k < nb; ++k) {
    if (threadIdx.x == 0) {
      float v = a[k][k];
      if (!(v > 0.f)) { *flag = 1; v = 1.f; }   // keep going with a harmless pivot
      a[k][k] = sqrtf(v);
    }
    __syncthreads();
    const float piv = a[k][k];
    for (int i = k + 1 + threadIdx.x; i < nb; i += blockDim.x) a[i][k] /= piv;
    __syncthreads();
    const int w = nb - k - 1;
    for (int e = threadIdx.x; e < w * w; e += blockDim.x) {
      const int i = k + 1 + e / w, j = k + 1 + e % w;
      if (j <= i) a[i][j] -= a[i][k] * a[j][k];
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < nb * nb; i += blockDim.x) {
    const int r = i / nb, c = i % nb;
    if (c <= r) G[(int64_t)(j0 + r) * d + j0 + c] = a[r][c];
  }
}

// rows i >= j0 + nb: L21[i] = A21[i] L11^-T (forward substitution per row)
__global__ __launch_bounds__(256) void trsm_panel_kernel(float* G, int d, int j0, int nb) {
  __shared__ float l[NB][NB + 1];
  for (int i = threadIdx.x; i < nb * nb; i += blockDim.x) {
    const int r = i / nb, c = i % nb;
    l[r][c] = G[(int64_t)(j0 + r) * d + j0 + c];
  }
  __syncthreads();
  const int row = j0 + nb + blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= d) return;
  float x[NB];
  float* g = G + (int64_t)row * d + j0;
#pragma unroll
  for (int k = 0; k < NB; ++k) x[k] = k < nb ? g[k] : 0.f;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (k < nb) {
      float v = x[k];
#pragma unroll
      for (int m = 0; m < k; ++m) v = fmaf(-x[m], l[k][m], v);
      x[k] = v / l[k][k];
    }
  }
#pragma unroll
  for (int k = 0; k < NB; ++k)
    if (k < nb) g[k] = x[k];
}

// inverse of each lower-triangular diagonal block of L, written into the
// matching block of X (one workgroup per block, one thread per column)
__global__ __launch_bounds__(64) void trinv_diag_kernel(const float* L, float* X, int d) {
  __shared__ float l[NB][NB + 1];
  __shared__ float x[NB][NB + 1];
  const int j0 = blockIdx.x * NB;
  const int nb = d - j0 < NB ? d - j0 : NB;
  for (int i = threadIdx.x; i < nb * nb; i += blockDim.x) {
    const int r = i / nb, c = i % nb;
    l[r][c] = L[(int64_t)(j0 + r) * d + j0 + c];
  }
  __syncthreads();
  const int j = threadIdx.x;
  if (j < nb) {
    for (int r = 0; r < nb; ++r) {
      if (r < j) { x[r][j] = 0.f; continue; }
      float v = r == j ? 1.f : 0.f;
      for (int m = j; m < r; ++m) v = fmaf(-l[r][m], x[m][j], v);
      x[r][j] = v / l[r][r];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb * nb; i += blockDim.x) {
    const int r = i / nb, c = i % nb;
    X[(int64_t)(j0 + r) * d + j0 + c] = x[r][c];
  }
}

}  // namespace river

namespace river_host {
using namespace river;

static river_status vgemm(const VGemm& g, int batch, bool out_bf16, hipStream_t s) {
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, batch);
  if (out_bf16) vgemm_kernel<true><<<grid, 256, 0, s>>>(g);
  else vgemm_kernel<false><<<grid, 256, 0, s>>>(g);
  return check_launch("ridge vgemm");
}

static int grid1d(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (int)(b > 65535 ? 65535 : (b < 1 ? 1 : b));
}

struct RidgeWs {
  uint16_t *Xt, *Yt, *Bcat, *Acat;
  float *G, *Xi, *Gi, *T, *Ct, *Wtmp;
  int* flag;
  size_t total;
};

// reduction lengths of the MFMA GEMMs: multiples of 256 (zero padded)
static int ridge_pad(int k) { return (k + 255) / 256 * 256; }

static RidgeWs ridge_layout(int n, int d_in, int d_out, river_dtype dt, char* base) {
  RidgeWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += align_up(bytes, 256); return p; };
  const size_t di = d_in, dd = d_out;
  w.flag = (int*)take(256);
  w.G = (float*)take(di * di * 4);
  w.Xi = (float*)take(di * di * 4);
  w.Gi = (float*)take(di * di * 4);
  w.T = (float*)take((size_t)NB * di * 4);
  w.Ct = (float*)take(dd * di * 4);
  if (dt == RIVER_BF16) {
    const size_t np = ridge_pad(n), k3 = ridge_pad(3 * d_in);
    w.Xt = (uint16_t*)take(di * np * 2);
    w.Yt = (uint16_t*)take(dd * np * 2);
    w.Bcat = (uint16_t*)take(di * k3 * 2);
    w.Acat = (uint16_t*)take(dd * k3 * 2);
  } else {
    w.Wtmp = (float*)take(dd * di * 4);
  }
  w.total = off;
  return w;
}

size_t ridge_workspace(int n, int d_in, int d_out, river_dtype dt) {
  return ridge_layout(n, d_in, d_out, dt, nullptr).total;
}

// Cholesky of G (fp32, d x d, in place, lower) and G^-1 into w.Gi
static river_status factor_and_invert(int d, RidgeWs& w, hipStream_t s) {
  river_status st;
  for (int j0 = 0; j0 < d; j0 += NB) {
    const int nb = d - j0 < NB ? d - j0 : NB;
    potrf_diag_kernel<<<1, 256, 0, s>>>(w.G, d, j0, nb, w.flag);
    if ((st = check_launch("ridge potrf")) != RIVER_OK) return st;
    const int rest = d - j0 - nb;
    if (rest <= 0) break;
    trsm_panel_kernel<<<(rest + 255) / 256, 256, 0, s>>>(w.G, d, j0, nb);
    if ((st = check_launch("ridge trsm")) != RIVER_OK) return st;
    // trailing update A22 -= L21 L21^T (lower tiles only)
    const float* L21 = w.G + (int64_t)(j0 + nb) * d + j0;
    VGemm u{rest, rest, nb, L21, d, 1, 0, L21, d, 1, 0,
            w.G + (int64_t)(j0 + nb) * d + (j0 + nb), d, 0, -1.f, 1.f, 1};
    if ((st = vgemm(u, 1, false, s)) != RIVER_OK) return st;
  }
  zero_upper_kernel<<<grid1d((int64_t)d * d), 256, 0, s>>>(w.G, d);
  // X = L^-1, block row by block row
  fill_f32_kernel<<<grid1d((int64_t)d * d), 256, 0, s>>>(w.Xi, (int64_t)d * d, 0.f);
  trinv_diag_kernel<<<(d + NB - 1) / NB, 64, 0, s>>>(w.G, w.Xi, d);
  if ((st = check_launch("ridge trinv")) != RIVER_OK) return st;
  for (int i0 = NB; i0 < d; i0 += NB) {
    const int nb = d - i0 < NB ? d - i0 : NB;
    // T = L[i][0:i] X[0:i][0:i]       (nb x i0)
    VGemm t{nb, i0, i0, w.G + (int64_t)i0 * d, d, 1, 0, w.Xi, 1, d, 0, w.T, i0, 0, 1.f, 0.f, 0};
    if ((st = vgemm(t, 1, false, s)) != RIVER_OK) return st;
    // X[i][0:i] = -X[i][i] T
    VGemm x{nb, i0, nb, w.Xi + (int64_t)i0 * d + i0, d, 1, 0, w.T, 1, i0, 0,
            w.Xi + (int64_t)i0 * d, d, 0, -1.f, 0.f, 0};
    if ((st = vgemm(x, 1, false, s)) != RIVER_OK) return st;
  }
  // G^-1 = X^T X
  VGemm gi{d, d, d, w.Xi, 1, d, 0, w.Xi, 1, d, 0, w.Gi, d, 0, 1.f, 0.f, 0};
  return vgemm(gi, 1, false, s);
}

river_status launch_ridge_fit(int n, int d_in, int d_out, int n_targets, const void* X,
                              river_dtype xdt, const void* Y, float lambda, void* W,
                              river_dtype wdt, void* workspace, size_t ws_bytes, hipStream_t s) {
  (void)ws_bytes;
  RidgeWs w = ridge_layout(n, d_in, d_out, xdt, (char*)workspace);
  river_status st;
  hipError_t he = hipMemsetAsync(w.flag, 0, sizeof(int), s);
  if (he != hipSuccess) return fail(RIVER_ERR_HIP, "ridge_fit: %s", hipGetErrorString(he));
  const int64_t wsz = (int64_t)d_out * d_in;
  const int np = ridge_pad(n), k3 = ridge_pad(3 * d_in);

  if (xdt == RIVER_BF16) {
    const uint16_t* Xb = (const uint16_t*)X;
    transpose_bf16_kernel<<<dim3((d_in + 63) / 64, np / 64), 256, 0, s>>>(Xb, n, np, d_in, d_in, w.Xt, np);
    if ((st = check_launch("ridge transpose X")) != RIVER_OK) return st;
    GemmArgs g{};
    g.M_max = d_in; g.N = d_in; g.K = np;
    g.A = w.Xt; g.lda = np; g.a_nrows = d_in;
    g.B = w.Xt; g.ldb = np;
    g.C = w.G; g.ldc = d_in; g.diag = lambda;
    gemm_auto<EPI_F32>(g, 1, s);
    if ((st = check_launch("ridge gram")) != RIVER_OK) return st;
  } else {
    const float* Xf = (const float*)X;
    VGemm g{d_in, d_in, n, Xf, 1, d_in, 0, Xf, 1, d_in, 0, w.G, d_in, 0, 1.f, 0.f, 0};
    if ((st = vgemm(g, 1, false, s)) != RIVER_OK) return st;
    add_diag_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(w.G, d_in, lambda);
  }
  if ((st = factor_and_invert(d_in, w, s)) != RIVER_OK) return st;

  if (xdt == RIVER_BF16) {
    split3_kernel<<<grid1d((int64_t)d_in * k3), 256, 0, s>>>(w.Gi, d_in, d_in, w.Bcat, k3, 0b010);
    for (int t = 0; t < n_targets; ++t) {
      const uint16_t* Yb = (const uint16_t*)Y + (int64_t)t * n * d_out;
      transpose_bf16_kernel<<<dim3((d_out + 63) / 64, np / 64), 256, 0, s>>>(Yb, n, np, d_out, d_out, w.Yt, np);
      GemmArgs c{};
      c.M_max = d_out; c.N = d_in; c.K = np;
      c.A = w.Yt; c.lda = np; c.a_nrows = d_out;
      c.B = w.Xt; c.ldb = np;
      c.C = w.Ct; c.ldc = d_in;
      gemm_auto<EPI_F32>(c, 1, s);
      split3_kernel<<<grid1d((int64_t)d_out * k3), 256, 0, s>>>(w.Ct, d_out, d_in, w.Acat, k3, 0b100);
      GemmArgs f{};
      f.M_max = d_out; f.N = d_in; f.K = k3;
      f.A = w.Acat; f.lda = k3; f.a_nrows = d_out;
      f.B = w.Bcat; f.ldb = k3;
      f.ldc = d_in;
      if (wdt == RIVER_BF16) {
        f.C = (uint16_t*)W + t * wsz;
        gemm_auto<EPI_BF16>(f, 1, s);
      } else {
        f.C = (float*)W + t * wsz;
        gemm_auto<EPI_F32>(f, 1, s);
      }
      if ((st = check_launch("ridge target")) != RIVER_OK) return st;
    }
  } else {
    for (int t = 0; t < n_targets; ++t) {
      const float* Yf = (const float*)Y + (int64_t)t * n * d_out;
      VGemm c{d_out, d_in, n, Yf, 1, d_out, 0, (const float*)X, 1, d_in, 0, w.Ct, d_in, 0, 1.f, 0.f, 0};
      if ((st = vgemm(c, 1, false, s)) != RIVER_OK) return st;
      VGemm f{d_out, d_in, d_in, w.Ct, d_in, 1, 0, w.Gi, d_in, 1, 0,
              wdt == RIVER_BF16 ? (void*)((uint16_t*)W + t * wsz) : (void*)((float*)W + t * wsz),
              d_in, 0, 1.f, 0.f, 0};
      if ((st = vgemm(f, 1, wdt == RIVER_BF16, s)) != RIVER_OK) return st;
    }
  }
  int flag = 0;
  he = hipMemcpyAsync(&flag, w.flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (he == hipSuccess) he = hipStreamSynchronize(s);
  if (he != hipSuccess) return fail(RIVER_ERR_HIP, "ridge_fit: %s", hipGetErrorString(he));
  if (flag) return fail(RIVER_ERR_NOT_SPD, "ridge_fit: X^T X + lambda I is not positive definite in fp32");
  return RIVER_OK;
}

}  // namespace river_host
