// Exit Projection: the final RMSNorm of each exited token's hidden state,
// written to the token's original row of the output buffer.
//
// TIDE, "模块4: 融合 CUDA 内核": Exit Projection fuses the RMSNorm with the
// scatter of exited tokens. "模块3: Post-Hoc Generation": an exited token's
// logits are the LM head applied to the RMSNorm of its state, so the row
// written here is what the LM head reads.
//
// One wave per row, four rows per 256-thread workgroup. The row is read
// once into registers (16-byte loads, KPL chunks per lane), its sum of
// squares reduced across the wave in fp32, then scaled by gamma and the
// reciprocal RMS and stored once. Each row costs 2 * d * element-size bytes
// of HBM traffic plus the two index reads; gamma stays in L2. Rows wider
// than 16 chunks per lane (d > 8192 bf16, d > 4096 fp32) take a two-pass
// variant that streams the row twice, the second pass mostly from L2.
#include "common.h"

namespace river {

constexpr int EP_ROWS = 4;   // waves (rows) per workgroup

template <bool BF16>
__device__ __forceinline__ void chunk_f32(const u32x4& v, float (&x)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(v[i]);
      x[2 * i + 1] = bf16_hi(v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
  }
}

template <bool BF16>
__device__ __forceinline__ float chunk_sumsq(const u32x4& v) {
  float x[BF16 ? 8 : 4];
  chunk_f32<BF16>(v, x);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < (BF16 ? 8 : 4); ++i) s = fmaf(x[i], x[i], s);
  return s;
}

// y = x * rs * gamma, rounded to the element type
template <bool BF16>
__device__ __forceinline__ u32x4 chunk_scale(const u32x4& v, const u32x4& g, bool has_gamma, float rs) {
  constexpr int E = BF16 ? 8 : 4;
  float x[E], w[E];
  chunk_f32<BF16>(v, x);
  chunk_f32<BF16>(g, w);
  u32x4 o;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = x[2 * i] * rs, b = x[2 * i + 1] * rs;
      if (has_gamma) { a *= w[2 * i]; b *= w[2 * i + 1]; }
      o[i] = pack_bf16x2(a, b);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = x[i] * rs;
      if (has_gamma) a *= w[i];
      o[i] = __float_as_uint(a);
    }
  }
  return o;
}

// KPL > 0: up to KPL 16-byte chunks per lane held in registers.
// KPL = 0: any width, the row is streamed twice.
template <bool BF16, int KPL>
__global__ __launch_bounds__(256) void exit_proj_kernel(
    int m_max, const int32_t* __restrict__ m_dev, int d, const uint8_t* __restrict__ h,
    int64_t ld_h_bytes, int n_rows, const int32_t* __restrict__ row_idx,
    const int32_t* __restrict__ row_ids, const u32x4* __restrict__ gamma, float eps,
    uint8_t* __restrict__ out, int64_t ld_out_bytes, int64_t n_out_rows) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  const int64_t t = (int64_t)blockIdx.x * EP_ROWS + wave;
  if (t >= m_max) return;
  // The count and the row index are independent loads (row_idx has m_max
  // entries), issued together; the row's own loads then overlap the read
  // of its destination, so a row costs two dependent memory latencies.
  const int m_in = m_dev ? *m_dev : m_max;
  const int r = row_idx ? row_idx[t] : (int)t;
  if (t >= min(max(m_in, 0), m_max)) return;
  if (r < 0 || r >= n_rows) return;

  constexpr int E = BF16 ? 8 : 4;
  const int nch = d / E;
  const u32x4* src = (const u32x4*)(h + (int64_t)r * ld_h_bytes);
  const bool has_gamma = gamma != nullptr;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  if constexpr (KPL > 0) {
    u32x4 v[KPL], g[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int c = lane + k * WAVE;
      v[k] = c < nch ? src[c] : zero;
    }
    const int64_t dst = row_ids ? (int64_t)row_ids[r] : (int64_t)r;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int c = lane + k * WAVE;
      g[k] = (has_gamma && c < nch) ? gamma[c] : zero;
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < KPL; ++k) ss += chunk_sumsq<BF16>(v[k]);
    ss = wave_sum(ss);
    const float rs = rsqrtf(ss / (float)d + eps);
    if (dst < 0 || dst >= n_out_rows) return;
    u32x4* dp = (u32x4*)(out + dst * ld_out_bytes);
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int c = lane + k * WAVE;
      if (c < nch) dp[c] = chunk_scale<BF16>(v[k], g[k], has_gamma, rs);
    }
  } else {
    const int64_t dst = row_ids ? (int64_t)row_ids[r] : (int64_t)r;
    if (dst < 0 || dst >= n_out_rows) return;
    u32x4* dp = (u32x4*)(out + dst * ld_out_bytes);
    float ss = 0.0f;
    for (int c = lane; c < nch; c += WAVE) ss += chunk_sumsq<BF16>(src[c]);
    ss = wave_sum(ss);
    const float rs = rsqrtf(ss / (float)d + eps);
    for (int c = lane; c < nch; c += WAVE)
      dp[c] = chunk_scale<BF16>(src[c], has_gamma ? gamma[c] : zero, has_gamma, rs);
  }
}

}  // namespace river

namespace river_host {

using namespace river;

template <bool BF16>
static river_status exit_proj_dispatch(int m_max, const int32_t* m_dev, int d, const void* h,
                                       int64_t ld_h, int n_rows, const int32_t* row_idx,
                                       const int32_t* row_ids, const void* gamma, float eps,
                                       void* out, int64_t ld_out, int64_t n_out_rows,
                                       hipStream_t s) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int64_t ES = BF16 ? 2 : 4;
  const int per_lane = (d / E + WAVE - 1) / WAVE;
  const dim3 grid((unsigned)(((int64_t)m_max + EP_ROWS - 1) / EP_ROWS)), block(EP_ROWS * WAVE);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, m_max, m_dev, d, (const uint8_t*)h, ld_h * ES,
                       n_rows, row_idx, row_ids, (const u32x4*)gamma, eps, (uint8_t*)out,
                       ld_out * ES, n_out_rows);
  };
  if (per_lane <= 1) go(exit_proj_kernel<BF16, 1>);
  else if (per_lane <= 2) go(exit_proj_kernel<BF16, 2>);
  else if (per_lane <= 4) go(exit_proj_kernel<BF16, 4>);
  else if (per_lane <= 8) go(exit_proj_kernel<BF16, 8>);
  else if (per_lane <= 16) go(exit_proj_kernel<BF16, 16>);
  else go(exit_proj_kernel<BF16, 0>);
  return check_launch("exit_projection");
}

river_status launch_exit_projection(int m_max, const int32_t* m_dev, int d, river_dtype dt,
                                    const void* h, int64_t ld_h, int n_rows,
                                    const int32_t* row_idx, const int32_t* row_ids,
                                    const void* gamma, float eps, void* out, int64_t ld_out,
                                    int64_t n_out_rows, hipStream_t s) {
  if (m_max == 0) return RIVER_OK;
  if (dt == RIVER_BF16)
    return exit_proj_dispatch<true>(m_max, m_dev, d, h, ld_h, n_rows, row_idx, row_ids, gamma,
                                    eps, out, ld_out, n_out_rows, s);
  return exit_proj_dispatch<false>(m_max, m_dev, d, h, ld_h, n_rows, row_idx, row_ids, gamma, eps,
                                   out, ld_out, n_out_rows, s);
}

}  // namespace river_host
