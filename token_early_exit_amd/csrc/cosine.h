// Cosine similarity of a token's states before and after a block, the
// exit signal of the token-level loop (TIDE, formula 1 / River-LLM's
// state-transition similarity): cos = <h_prev, h_cur> / (|h_prev| |h_cur|)
// in fp32. Shared by the router-off route and the decode step's all-
// checkpoint pass, which therefore take bit-identical decisions.
#pragma once

#include "common.h"

namespace river {

__device__ __forceinline__ float cosine_from(float dot, float na, float nb) {
  // NaN propagates (comparisons with NaN are false), zero norm gives 0
  if (isnan(dot) || isnan(na) || isnan(nb)) return __builtin_nanf("");
  if (!(na > 0.0f) || !(nb > 0.0f)) return 0.0f;
  float c = dot / (sqrtf(na) * sqrtf(nb));
  c = c > 1.0f ? 1.0f : c;
  c = c < -1.0f ? -1.0f : c;
  return c;
}

// the three products of one 16-byte chunk of each state (8 bf16 or 4 fp32)
template <bool BF16>
__device__ __forceinline__ void dot3(const u32x4& p, const u32x4& c, float& dot, float& na, float& nb) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = bf16_lo(p[i]), x1 = bf16_hi(p[i]), y0 = bf16_lo(c[i]), y1 = bf16_hi(c[i]);
      dot = fmaf(x0, y0, dot); dot = fmaf(x1, y1, dot);
      na = fmaf(x0, x0, na); na = fmaf(x1, x1, na);
      nb = fmaf(y0, y0, nb); nb = fmaf(y1, y1, nb);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = __uint_as_float(p[i]), y = __uint_as_float(c[i]);
      dot = fmaf(x, y, dot);
      na = fmaf(x, x, na);
      nb = fmaf(y, y, nb);
    }
  }
}

// One wave computes the cosine of one token's rows hp, hc (d elements,
// 16-byte aligned), left in every lane. Both rows are loaded whole into
// registers (KPL 16-byte chunks per lane, every load issued before the first
// product), so a token costs one memory latency; KPL = 0 streams any width.
template <bool BF16, int KPL>
__device__ __forceinline__ float token_cosine(const void* hp_row, const void* hc_row, int d, int lane) {
  constexpr int E = BF16 ? 8 : 4;
  const int nch = d / E;
  const u32x4* hp = (const u32x4*)hp_row;
  const u32x4* hc = (const u32x4*)hc_row;
  float dot = 0.f, na = 0.f, nb = 0.f;
  if constexpr (KPL > 0) {
    u32x4 p[KPL], c[KPL];
    const u32x4 z = {0u, 0u, 0u, 0u};
    // clamped addresses keep every load unconditional; chunks past the row
    // are zeroed after they land
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int ch = lane + WAVE * k;
      p[k] = hp[ch < nch ? ch : nch - 1];
      c[k] = hc[ch < nch ? ch : nch - 1];
    }
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const bool in = lane + WAVE * k < nch;
      dot3<BF16>(in ? p[k] : z, in ? c[k] : z, dot, na, nb);
    }
  } else {
    for (int ch = lane; ch < nch; ch += WAVE) dot3<BF16>(hp[ch], hc[ch], dot, na, nb);
  }
  dot = wave_sum(dot);
  na = wave_sum(na);
  nb = wave_sum(nb);
  return cosine_from(dot, na, nb);
}

// chunks per lane of the register-resident variant for width d (0: stream)
inline int cosine_kpl(int d, bool bf16) {
  const int per_lane = (d / (bf16 ? 8 : 4) + WAVE - 1) / WAVE;
  return per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 0;
}

}  // namespace river
