// route: per-token exit decision.
//
// River-LLM, 前置知识 / 方法步骤详情 step 3: the cosine between a block's
// input h_prev and output h_cur. TIDE, 关键公式 formula 3: the router
// sigmoid(w_up . SiLU(W_down . RMSNorm(h_cur))); formula 4: strict
// thresholds. TIDE 模块4 fuses RMSNorm and the router into one launch; here
// the cosine is fused in as well, so h_prev and h_cur are each read once.
//
// bf16 path: one workgroup = 8 waves = 16*RT tokens. The waves split the
// feature dimension into 32-wide slabs (4 groups) and the router units in
// two halves; each wave keeps partial norms in registers and runs the router
// down-projection on bf16 MFMA (16x16x32) with the RMSNorm scale applied
// afterwards in fp32:
//   u = r * (W_down . (gamma * h)),   r = 1 / sqrt(mean(h^2) + eps),
// which never rounds the normalised vector to bf16. gamma != 1 is fed as
// the exact fp32 product gamma*h split into two bf16 terms (hi + lo).
// The partial results of the waves are summed in LDS in a fixed order
// (deterministic), then the SiLU / w_up / sigmoid epilogue runs per token.
#include <type_traits>

#include "common.h"
#include "cosine.h"

namespace river {

struct RouteArgs {
  int n, d, b;
  const void* hp; int64_t ldp;
  const void* hc; int64_t ldc;
  const void* gamma; float eps;
  const void* wd; const void* wu;
  float tau, theta;
  float* cos_out; float* prob_out; uint8_t* mask_out;
  // generation loop (river_decode_step): only tokens with alive_in[i] != 0
  // take part; under the token rule the decision also writes alive_out and,
  // for an exiting token, exit_layer (under the batch rule the finish
  // kernel does, once the batch decision is known)
  const uint8_t* alive_in; uint8_t* alive_out; int32_t* exit_layer; int exit_value;
  int batch_min;
};


__device__ __forceinline__ void write_decision(const RouteArgs& a, int i, float c, float p,
                                               bool router) {
  bool e = router ? ((c > a.tau) && (p > a.theta)) : (c > a.tau);
  if (a.cos_out) a.cos_out[i] = c;
  if (a.prob_out) a.prob_out[i] = p;
  if (a.alive_in) {
    const bool al = a.alive_in[i] != 0;
    e = e && al;
    if (!a.batch_min) {
      a.alive_out[i] = (al && !e) ? 1 : 0;
      if (e) a.exit_layer[i] = a.exit_value;
    }
  }
  a.mask_out[i] = e ? 1 : 0;
}

// x * sigmoid(x) through the hardware base-2 exponential and reciprocal
// (about one ulp each; e^-x = 2^(-x log2 e))
__device__ __forceinline__ float silu_hw(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.44269504088896341f));
}

// --------------------------------------------------------- generic path
// One wave per token row. Used for fp32 and for shapes the MFMA path does
// not take. Dynamic LDS holds the normalised row (d floats) when the
// router is on.
template <bool BF16>
__global__ __launch_bounds__(64) void route_generic_kernel(RouteArgs a) {
  extern __shared__ float xs[];
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  const int d = a.d;
  float dot = 0.f, na = 0.f, nb = 0.f;
  const int64_t op = (int64_t)i * a.ldp, oc = (int64_t)i * a.ldc;
  for (int k = lane; k < d; k += WAVE) {
    float x = load_elem<BF16>(a.hp, op + k);
    float y = load_elem<BF16>(a.hc, oc + k);
    dot = fmaf(x, y, dot);
    na = fmaf(x, x, na);
    nb = fmaf(y, y, nb);
  }
  dot = wave_sum(dot);
  na = wave_sum(na);
  nb = wave_sum(nb);
  const float c = cosine_from(dot, na, nb);
  float p = 1.0f;
  const bool router = a.wd != nullptr;
  if (router) {
    const float r = 1.0f / sqrtf(nb / (float)d + a.eps);
    for (int k = lane; k < d; k += WAVE) {
      float g = a.gamma ? load_elem<BF16>(a.gamma, k) : 1.0f;
      xs[k] = load_elem<BF16>(a.hc, oc + k) * g;
    }
    __syncthreads();
    float zp = 0.f;
    for (int j = lane; j < a.b; j += WAVE) {
      float u = 0.f;
      const int64_t wo = (int64_t)j * d;
      for (int k = 0; k < d; ++k) u = fmaf(load_elem<BF16>(a.wd, wo + k), xs[k], u);
      u *= r;
      const float act = u * sigmoidf_(u);
      zp = fmaf(act, load_elem<BF16>(a.wu, j), zp);
    }
    p = sigmoidf_(wave_sum(zp));
  }
  if (lane == 0) write_decision(a, i, c, p, router);
}

// ------------------------------------------------------ cosine only
// The router switched off: one wave per token, four tokens per workgroup
// (token_cosine, cosine.h).
template <bool BF16, int KPL>
__global__ __launch_bounds__(256) void route_cos_kernel(RouteArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  const int i = blockIdx.x * 4 + wave;
  if (i >= a.n) return;
  constexpr int ES = BF16 ? 2 : 4;
  const float c = token_cosine<BF16, KPL>((const char*)a.hp + (int64_t)i * a.ldp * ES,
                                          (const char*)a.hc + (int64_t)i * a.ldc * ES, a.d, lane);
  if (lane == 0) write_decision(a, i, c, 1.0f, false);
}

// ------------------------------------------------------------ MFMA path
// 8 waves = KG K-groups x UG unit-groups. K-group kg streams the 32-wide
// feature slabs ks = kg + KG * j; unit-group ug owns router units
// [64 ug, 64 ug + 64). Each wave keeps its slabs of h_prev / h_cur for the
// 16 * RT token rows and its router-weight fragments in 4-deep register
// rings (three slabs in flight while one is used). Loads past the last slab
// re-read that slab (cache hits) so that every iteration issues the same
// loads and control flow stays uniform. Unit-group 0 also accumulates the
// cosine norms.
template <int RT>
struct HSlab {
  u32x4 c[RT], p[RT];
  u32x4 g;            // gamma chunk (when gamma is given)
};
template <int NT>
struct WSlab {
  u32x4 w[NT];
};

constexpr int R_KG = 4, R_UG = 2, R_NT = 4;   // 8 waves, 128 units

template <int RT, bool HAS_GAMMA, bool FULLB>
__global__ __launch_bounds__(512) void route_mfma_kernel(RouteArgs a) {
  constexpr int KG = R_KG, UG = R_UG, NT = R_NT;
  constexpr int T = 16 * RT;          // tokens per workgroup
  constexpr int BU = UG * NT * 16;    // router units per workgroup (128)
  constexpr int NTH = 64 * KG * UG;
  constexpr int TPR = NTH / T;        // epilogue threads per token
  __shared__ float red[KG][T][BU];    // per-K-group partial U
  __shared__ float nrm[KG][T][3];     // per-K-group partial dot, |a|^2, |b|^2

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave; say so, so that everything
  // derived from it (slab counts, offsets) lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave % KG, ug = wave / KG;
  const int row0 = blockIdx.x * T;
  const int d = a.d, b = a.b, n = a.n;
  const int fr = lane & 15;           // fragment row (token) / column (unit)
  const int fk = (lane >> 4) * 8;     // fragment k offset inside a 32-slab

  const uint16_t* hp = (const uint16_t*)a.hp;
  const uint16_t* hc = (const uint16_t*)a.hc;
  const uint16_t* wd = (const uint16_t*)a.wd;
  const uint16_t* gm = (const uint16_t*)a.gamma;

  const uint16_t* pc[RT];
  const uint16_t* pp[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + fr;
    const int rr = row < n ? row : n - 1;   // rows past n re-read the last row; dropped
    pc[rt] = hc + (int64_t)rr * a.ldc + fk;
    pp[rt] = hp + (int64_t)rr * a.ldp + fk;
  }
  const uint16_t* pw[NT];
  bool wv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = ug * NT * 16 + nt * 16 + fr;
    wv[nt] = FULLB || j < b;
    pw[nt] = wd + (int64_t)(j < b ? j : b - 1) * d + fk;   // units past b: zero below
  }
  const bool norms = ug == 0;

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dot[RT], na[RT], nb[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) dot[rt] = na[rt] = nb[rt] = 0.f;

  const int KS = d / 32;
  const int J = (KS - kg + KG - 1) / KG;   // this K-group's slabs (uniform)
  const int jl = J - 1;
  auto koff = [&](int j) { return (kg + KG * (j < jl ? j : jl)) * 32; };
  HSlab<RT> hr[4];
  WSlab<NT> wr[4];
  auto load = [&](HSlab<RT>& h, WSlab<NT>& w, int j) {
    const int k = koff(j);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      h.c[rt] = *(const u32x4*)(pc[rt] + k);
      if (norms) h.p[rt] = *(const u32x4*)(pp[rt] + k);
    }
    if constexpr (HAS_GAMMA) h.g = *(const u32x4*)(gm + k + fk);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) w.w[nt] = *(const u32x4*)(pw[nt] + k);
  };
  auto step = [&](const HSlab<RT>& h, const WSlab<NT>& w) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (norms) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float c0 = bf16_lo(h.c[rt][q]), c1 = bf16_hi(h.c[rt][q]);
          const float p0 = bf16_lo(h.p[rt][q]), p1 = bf16_hi(h.p[rt][q]);
          dot[rt] = fmaf(p0, c0, dot[rt]); dot[rt] = fmaf(p1, c1, dot[rt]);
          na[rt] = fmaf(p0, p0, na[rt]);   na[rt] = fmaf(p1, p1, na[rt]);
          nb[rt] = fmaf(c0, c0, nb[rt]);   nb[rt] = fmaf(c1, c1, nb[rt]);
        }
      }
      if constexpr (HAS_GAMMA) {
        u32x4 hi4, lo4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x0 = bf16_lo(h.c[rt][q]) * bf16_lo(h.g[q]);   // exact in fp32
          const float x1 = bf16_hi(h.c[rt][q]) * bf16_hi(h.g[q]);
          const uint32_t hh = pack_bf16x2(x0, x1);
          hi4[q] = hh;
          lo4[q] = pack_bf16x2(x0 - bf16_lo(hh), x1 - bf16_hi(hh));
        }
        const bf16x8 ah = __builtin_bit_cast(bf16x8, hi4);
        const bf16x8 al = __builtin_bit_cast(bf16x8, lo4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 bb = __builtin_bit_cast(bf16x8, wv[nt] ? w.w[nt] : u32x4{0u, 0u, 0u, 0u});
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, acc[rt][nt], 0, 0, 0);
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, acc[rt][nt], 0, 0, 0);
        }
      } else {
        const bf16x8 aa = __builtin_bit_cast(bf16x8, h.c[rt]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 bb = __builtin_bit_cast(bf16x8, wv[nt] ? w.w[nt] : u32x4{0u, 0u, 0u, 0u});
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, acc[rt][nt], 0, 0, 0);
        }
      }
    }
  };

  if (J > 0) {
    load(hr[0], wr[0], 0);
    load(hr[1], wr[1], 1);
    load(hr[2], wr[2], 2);
    int j = 0;
    for (; j + 4 <= J; j += 4) {     // whole groups of four slabs, uniform control flow
      load(hr[3], wr[3], j + 3); step(hr[0], wr[0]);
      load(hr[0], wr[0], j + 4); step(hr[1], wr[1]);
      load(hr[1], wr[1], j + 5); step(hr[2], wr[2]);
      load(hr[2], wr[2], j + 6); step(hr[3], wr[3]);
    }
    const int rem = J - j;            // 0..3 slabs left, in ring slots 0..2
    if (rem > 0) step(hr[0], wr[0]);
    if (rem > 1) step(hr[1], wr[1]);
    if (rem > 2) step(hr[2], wr[2]);
  }

  // lanes fr, fr+16, fr+32, fr+48 hold the same token row
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (norms) {
      dot[rt] += __shfl_xor(dot[rt], 16, WAVE); dot[rt] += __shfl_xor(dot[rt], 32, WAVE);
      na[rt] += __shfl_xor(na[rt], 16, WAVE);   na[rt] += __shfl_xor(na[rt], 32, WAVE);
      nb[rt] += __shfl_xor(nb[rt], 16, WAVE);   nb[rt] += __shfl_xor(nb[rt], 32, WAVE);
      if (lane < 16) {
        nrm[kg][rt * 16 + lane][0] = dot[rt];
        nrm[kg][rt * 16 + lane][1] = na[rt];
        nrm[kg][rt * 16 + lane][2] = nb[rt];
      }
    }
    // 16x16 accumulator layout: column = lane % 16, row = 4 * (lane / 16) + i
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[kg][rt * 16 + 4 * (lane >> 4) + i][ug * NT * 16 + nt * 16 + fr] = acc[rt][nt][i];
  }
  __syncthreads();

  const int row = tid / TPR, part = tid % TPR;
  const int gi = row0 + row;
  float sd = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
  for (int k = 0; k < KG; ++k) {      // fixed order: deterministic
    sd += nrm[k][row][0];
    sa += nrm[k][row][1];
    sb += nrm[k][row][2];
  }
  const float r = 1.0f / sqrtf(sb / (float)d + a.eps);
  float zp = 0.f;
  for (int u = part; u < b; u += TPR) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) s += red[k][row][u];
    const float x = s * r;
    const float act = x * sigmoidf_(x);
    zp = fmaf(act, load_elem<true>(a.wu, u), zp);
  }
  const float z = group_sum<TPR>(zp);
  if (part == 0 && gi < n) write_decision(a, gi, cosine_from(sd, sa, sb), sigmoidf_(z), true);
}

// The router epilogue of the streaming route, on the pre-activations of
// T = 16 RT tokens in the 16x16 MFMA layout (lane l of wave w holds unit
// UW w + 16 uf + l % 16 of tokens 16 rt + 4 (l / 16) + i) and the tokens'
// norms in nrm: RMSNorm scale, SiLU, w_up, the per-wave logits added in
// wave order, sigmoid, the decision. Every thread calls it.
template <int RT, int NW>
__device__ __forceinline__ void route_stream_epilogue(const RouteArgs& a, const f32x4 (&acc)[RT][8 / NW],
                                                      const float (&wup)[8 / NW], float (*red)[16 * RT],
                                                      float (*nrm)[3], int row0) {
  constexpr int T = 16 * RT, UF = 8 / NW, UW = 16 * UF;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d, b = a.b, n = a.n;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float zp[4] = {0.f, 0.f, 0.f, 0.f}, r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = 1.0f / sqrtf(nrm[rt * 16 + 4 * (lane >> 4) + i][2] / (float)d + a.eps);
#pragma unroll
    for (int uf = 0; uf < UF; ++uf) {
      const bool uok = wave * UW + uf * 16 + (lane & 15) < b;   // units past b do not exist
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = silu_hw(acc[rt][uf][i] * r[i]) * wup[uf];
        zp[i] += uok ? c : 0.f;   // a select: a missing unit adds nothing, whatever c is
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = row_sum<16>(zp[i]);
      if ((lane & 15) == 0) red[wave][rt * 16 + 4 * (lane >> 4) + i] = v;
    }
  }
  __syncthreads();
  if (tid < T) {
    const int gi = row0 + tid;
    float z = red[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) z += red[w][tid];   // fixed order
    if (gi < n) write_decision(a, gi, cosine_from(nrm[tid][0], nrm[tid][1], nrm[tid][2]), sigmoidf_(z), true);
  }
}

// The two halves of a route whose reduction over d is split (HALVES):
// per checkpoint and half, the pre-activations [half][token][128 units]
// and the norms [half][token][4] (dot, |h_prev|^2, |h_cur|^2, unused).
struct RouteHalves {
  float* u;                  // [n_ck][2][n][128]
  float* nrm;                // [n_ck][2][n][4]
};

// ------------------------------------------------------ streaming path
// d % 256 == 0, bf16, b <= 128: one workgroup = NW waves, T = 16 RT tokens.
// The feature dimension is walked in 64-wide slabs. Each slab of W_down
// (128 units x 64, 16 KB) and of the T rows of h_prev and h_cur goes through
// LDS by buffer loads (full 128-byte lines, three slabs ahead, rows past n
// and units past b read as zeros; every wave issues as many loads per slab,
// so a wave past the state blocks loads nothing into a spare block). Wave
// w owns units [UW w, UW w + UW), UW = 128 / NW, and runs
// u = W_down . (gamma * h_cur) on 16x16x32 bf16 MFMA over all slabs, so the
// pre-activations need no cross-wave sum; meanwhile 8 threads per token
// accumulate, in fp32, the three dot products over 8 features of each slab.
// The per-wave logits are added in wave order.
//
// HALVES (d % 512 == 0): the reduction over d in two halves of KT / 2
// slabs, each in an accumulator set of its own, added at the end (the
// pre-activations and the three norms). HALF < 0: one workgroup walks both
// and adds them; HALF = 0 or 1: the workgroup walks its half and writes the
// half's sums (hv) for route_halves_kernel, which adds them in the same
// order and runs the same epilogue. A decode step's route takes 16-token
// workgroups, 128 for 8 checkpoints of 256 tokens: each walks 64 slabs one
// barrier at a time, half the CUs idle; in halves, 256 workgroups walk 32.
// The results are the same bits either way.
template <int RT, bool HAS_GAMMA, int NW, bool HALVES = false>
__device__ __forceinline__ void route_stream_body(const RouteArgs& a, int half = -1,
                                                  RouteHalves hv = RouteHalves{}) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int T = 16 * RT;
  constexpr int UF = 8 / NW;             // 16-unit MFMA fragments per wave
  constexpr int UW = 16 * UF;            // units per wave
  constexpr int WB = 128 * 8;            // W slab: 128 units x 8 chunks of 16 bytes
  constexpr int WD = WB / (64 * NW);     // W DMAs per thread per slab
  constexpr int HB = T * 8;              // one state slab: T rows x 8 chunks
  constexpr int HBLK = 2 * HB / 64;      // state DMA blocks of 64 chunks
  constexpr int HD = (HBLK + NW - 1) / NW;   // state DMAs per thread per slab
  constexpr int DUMMY = HD * NW - HBLK;  // blocks past the states: zero-length loads
                                         // (every wave issues as many loads per slab)
  constexpr int SSZ = WB + 2 * HB + DUMMY * 64;   // W, then h_cur, then h_prev
  constexpr int PER_SLAB = WD + HD;      // buffer loads per thread per slab
  constexpr int DT = 8 * T;              // threads on the dot products: 8 per token,
                                         // one 16-byte chunk (8 features) each per slab
  __shared__ u32x4 S0[SSZ], S1[SSZ], S2[SSZ], S3[SSZ];
  __shared__ float red[NW][T];           // per-wave partial router logits
  __shared__ float nrm[T][3];            // dot, |h_prev|^2, |h_cur|^2
  __shared__ uint32_t gam[HAS_GAMMA ? 4096 : 1];   // gamma as bf16 pairs (d <= 8192)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * T;
  const int d = a.d, b = a.b, n = a.n;
  const int KT = d / 64;

  // w_up of this lane's units, fetched now for the epilogue (the first
  // slab wait covers these older loads)
  float wup[UF];
#pragma unroll
  for (int uf = 0; uf < UF; ++uf) {
    const int u = wave * UW + uf * 16 + (lane & 15);
    wup[uf] = u < b ? load_elem<true>(a.wu, u) : 0.f;
  }
  if constexpr (HAS_GAMMA) {
    for (int i = tid; i < d / 2; i += 64 * NW) gam[i] = ((const uint32_t*)a.gamma)[i];
    __syncthreads();
  }

  // buffer offsets: chunk p of a slab holds logical 16-byte chunk
  // (p % 8) ^ swz(p / 8) of row p / 8 (unit or token)
  const int w_bytes = b * d * 2;
  uint32_t w_off[WD];
#pragma unroll
  for (int i = 0; i < WD; ++i) {
    const int p = (i * NW + wave) * 64 + lane;
    const int u = p >> 3, c = (p & 7) ^ swz(u);
    w_off[i] = (uint32_t)(u * d * 2 + c * 16);
  }
  // state DMA i of this thread: block (i * NW + wave) of the 2 HB chunks
  // (h_cur first, then h_prev; a block past them loads nothing)
  uint32_t h_off[HD];
  int h_src[HD];                                     // 0: h_cur, 1: h_prev, 2: none
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    const int blk = i * NW + wave;                   // uniform
    const int p = blk * 64 + lane;                   // 0 .. 2 HB - 1 for a state block
    const bool pv = blk * 64 >= HB;
    const int q = pv ? p - HB : p;
    const int t = q >> 3, c = (q & 7) ^ swz(t);
    h_src[i] = blk >= HBLK ? 2 : (pv ? 1 : 0);
    h_off[i] = blk >= HBLK ? 0u : (uint32_t)((int64_t)(row0 + t) * (pv ? a.ldp : a.ldc) * 2 + c * 16);
  }
  const int hc_bytes = (int)((int64_t)n * a.ldc * 2), hp_bytes = (int)((int64_t)n * a.ldp * 2);
  auto stage = [&](auto st) -> u32x4* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return S0; else if constexpr (S == 1) return S1;
    else if constexpr (S == 2) return S2; else return S3;
  };
  auto issue = [&](auto st, int j) {
    u32x4* l = stage(st);
#pragma unroll
    for (int i = 0; i < WD; ++i) buf_lds<16>(a.wd, w_bytes, w_off[i], j * 128, l + (i * NW + wave) * 64);
#pragma unroll
    for (int i = 0; i < HD; ++i)   // one load per block; the source choice is uniform
      buf_lds<16>(h_src[i] == 1 ? a.hp : a.hc, h_src[i] == 2 ? 0 : (h_src[i] == 1 ? hp_bytes : hc_bytes),
                  h_off[i], j * 128, l + WB + (i * NW + wave) * 64);
  };

  struct Sums {
    f32x4 acc[RT][UF];
    float dot, na, nb;
  };
  auto zero = [&](Sums& s) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int uf = 0; uf < UF; ++uf) s.acc[rt][uf] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.dot = s.na = s.nb = 0.f;
  };
  Sums S0s, S1s;                                  // the halves' sums (the first only without HALVES)
  zero(S0s);
  if constexpr (HALVES) zero(S1s);
  const int my_t = tid >> 3, my_q = tid & 7;      // dot-product share: token, chunk

  auto compute = [&](const u32x4* l, int j, Sums& sm) {
    auto& acc = sm.acc;
    auto& dot = sm.dot;
    auto& na = sm.na;
    auto& nb = sm.nb;
    const u32x4* lw = l;
    const u32x4* lc = l + WB;
    const u32x4* lp = l + WB + HB;
    // dot products: chunk my_q (features 8 my_q .. 8 my_q + 7) of token my_t
    // (16-byte reads, which the compiler does not pair into a read2)
    if (DT == 64 * NW || tid < DT) {
      const int sw = my_q ^ swz(my_t);
      const u32x4 x = lp[my_t * 8 + sw], y = lc[my_t * 8 + sw];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = bf16_lo(x[e]), p1 = bf16_hi(x[e]), c0 = bf16_lo(y[e]), c1 = bf16_hi(y[e]);
        dot = fmaf(p0, c0, dot); dot = fmaf(p1, c1, dot);
        na = fmaf(p0, p0, na);   na = fmaf(p1, p1, na);
        nb = fmaf(c0, c0, nb);   nb = fmaf(c1, c1, nb);
      }
    }
    // router: two 32-wide k-steps; A = tokens (lane: row l % 16, chunk
    // 4 ks + l / 16), B = this wave's units
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + (lane >> 4);
      bf16x8 bw[UF];
#pragma unroll
      for (int uf = 0; uf < UF; ++uf) {
        const int u = wave * UW + uf * 16 + (lane & 15);
        bw[uf] = __builtin_bit_cast(bf16x8, lw[u * 8 + (c ^ swz(u))]);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int t = rt * 16 + (lane & 15);
        const u32x4 hx = lc[t * 8 + (c ^ swz(t))];
        if constexpr (HAS_GAMMA) {
          // gamma * h exactly in fp32, fed as hi + lo bf16 terms
          const int k0 = j * 64 + c * 8;
          u32x4 hi4, lo4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t gw = gam[(k0 >> 1) + e];
            const float x0 = bf16_lo(hx[e]) * bf16_lo(gw), x1 = bf16_hi(hx[e]) * bf16_hi(gw);
            const uint32_t hh = pack_bf16x2(x0, x1);
            hi4[e] = hh;
            lo4[e] = pack_bf16x2(x0 - bf16_lo(hh), x1 - bf16_hi(hh));
          }
#pragma unroll
          for (int uf = 0; uf < UF; ++uf) {
            acc[rt][uf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi4), bw[uf], acc[rt][uf], 0, 0, 0);
            acc[rt][uf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo4), bw[uf], acc[rt][uf], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int uf = 0; uf < UF; ++uf)
            acc[rt][uf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hx), bw[uf], acc[rt][uf], 0, 0, 0);
        }
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // slab j in stage j % 4; slab j + 3 is issued after the barrier of slab
  // j (its stage held slab j - 1, which every wave has finished with). The
  // slabs walked, [j0, j1), are a multiple of 4: the loop body has static
  // stages and no branches, and the last four slabs wait for exactly what
  // is still in flight. With HALVES and both halves in this workgroup the
  // sums switch sets at KT / 2 (a multiple of 4).
  const int j0 = HALVES && half == 1 ? KT / 2 : 0;
  const int j1 = HALVES && half == 0 ? KT / 2 : KT;
  issue(I0{}, j0);
  issue(I1{}, j0 + 1);
  issue(I2{}, j0 + 2);
  auto iter = [&](auto st, int j, auto w, auto iss, Sums& sm) {
    using NX = std::integral_constant<int, (decltype(st)::value + 3) & 3>;
    wait_barrier<decltype(w)::value, true>();   // slab j landed; its loads and older ones done
    if constexpr (decltype(iss)::value) issue(NX{}, j + 3);
    compute(stage(st), j, sm);
  };
  using W2 = std::integral_constant<int, 2 * PER_SLAB>;
  using W1 = std::integral_constant<int, PER_SLAB>;
  using W0 = std::integral_constant<int, 0>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto group = [&](int j, Sums& sm) {
    iter(I0{}, j, W2{}, T_{}, sm);
    iter(I1{}, j + 1, W2{}, T_{}, sm);
    iter(I2{}, j + 2, W2{}, T_{}, sm);
    iter(I3{}, j + 3, W2{}, T_{}, sm);
  };
  // the sums of slab j: the second set from KT / 2 on when one workgroup
  // walks both halves
  auto sums_of = [&](int j) -> Sums& {
    if constexpr (HALVES) {
      if (half < 0 && j >= KT / 2) return S1s;   // uniform
    }
    return S0s;
  };
  int j = j0;
  for (; j + 4 < j1; j += 4) group(j, sums_of(j));
  {
    Sums& sm = sums_of(j);
    iter(I0{}, j, W2{}, T_{}, sm);
    iter(I1{}, j + 1, W1{}, F_{}, sm);
    iter(I2{}, j + 2, W0{}, F_{}, sm);
    iter(I3{}, j + 3, W0{}, F_{}, sm);
  }

  // dot products: sum over the 8 threads of each token (fixed order); the
  // halves' sums added in order
  float dot = row_sum<8>(S0s.dot), na = row_sum<8>(S0s.na), nb = row_sum<8>(S0s.nb);
  f32x4 acc[RT][UF];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int uf = 0; uf < UF; ++uf) acc[rt][uf] = S0s.acc[rt][uf];
  if constexpr (HALVES) {
    if (half >= 0) {
      // this half's sums for route_halves_kernel: lane l of wave w holds
      // unit UW w + 16 uf + l % 16 of tokens 16 rt + 4 (l / 16) + i
      const int64_t base = (int64_t)half * n;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int uf = 0; uf < UF; ++uf)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = row0 + rt * 16 + 4 * (lane >> 4) + i;
            if (t < n) hv.u[(base + t) * 128 + wave * UW + uf * 16 + (lane & 15)] = acc[rt][uf][i];
          }
      if (my_q == 0 && tid < DT && row0 + my_t < n)
        *(f32x4*)(hv.nrm + (base + row0 + my_t) * 4) = f32x4{dot, na, nb, 0.f};
      return;
    }
    dot += row_sum<8>(S1s.dot);
    na += row_sum<8>(S1s.na);
    nb += row_sum<8>(S1s.nb);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int uf = 0; uf < UF; ++uf) acc[rt][uf] += S1s.acc[rt][uf];
  }
  if (my_q == 0 && tid < DT) { nrm[my_t][0] = dot; nrm[my_t][1] = na; nrm[my_t][2] = nb; }
  __syncthreads();
  route_stream_epilogue<RT, NW>(a, acc, wup, red, nrm, row0);
}

template <int RT, bool HAS_GAMMA, int NW, bool HALVES>
__global__ __launch_bounds__(64 * NW) void route_stream_kernel(RouteArgs a) {
  route_stream_body<RT, HAS_GAMMA, NW, HALVES>(a);
}

// The router checkpoints of a decode step in one launch: blockIdx.y picks
// the checkpoint (cosine and probability only; the decision is the
// caller's).
constexpr int RM_MAX = 16;
struct RouteMulti { RouteArgs a[RM_MAX]; };
static_assert(sizeof(RouteMulti) <= 4000, "kernel arguments are limited to 4 KB");

template <int RT, bool HAS_GAMMA, int NW, bool HALVES>
__global__ __launch_bounds__(64 * NW) void route_stream_multi_kernel(RouteMulti m) {
  route_stream_body<RT, HAS_GAMMA, NW, HALVES>(m.a[blockIdx.y]);
}

// The checkpoints' routes in halves: blockIdx.z picks the half, each
// writes its sums to hv (checkpoint blockIdx.y at its stride).
template <int RT, bool HAS_GAMMA, int NW>
__global__ __launch_bounds__(64 * NW) void route_stream_halves_kernel(RouteMulti m, RouteHalves hv) {
  const RouteArgs& a = m.a[blockIdx.y];
  RouteHalves h{hv.u + (int64_t)blockIdx.y * 2 * a.n * 128, hv.nrm + (int64_t)blockIdx.y * 2 * a.n * 4};
  route_stream_body<RT, HAS_GAMMA, NW, true>(a, blockIdx.z, h);
}

// The halves added (in the order of the one-workgroup route) and the
// streaming route's epilogue: the same cosines, probabilities and masks.
template <int RT, int NW>
__global__ __launch_bounds__(64 * NW) void route_halves_kernel(RouteMulti m, RouteHalves hv) {
  constexpr int T = 16 * RT, UF = 8 / NW, UW = 16 * UF;
  __shared__ float red[NW][T];
  __shared__ float nrm[T][3];
  const RouteArgs& a = m.a[blockIdx.y];
  const int n = a.n, b = a.b;
  const float* u = hv.u + (int64_t)blockIdx.y * 2 * n * 128;
  const float* nr = hv.nrm + (int64_t)blockIdx.y * 2 * n * 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * T;
  float wup[UF];
#pragma unroll
  for (int uf = 0; uf < UF; ++uf) {
    const int un = wave * UW + uf * 16 + (lane & 15);
    wup[uf] = un < b ? load_elem<true>(a.wu, un) : 0.f;
  }
  f32x4 acc[RT][UF];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int uf = 0; uf < UF; ++uf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = row0 + rt * 16 + 4 * (lane >> 4) + i;
        t = t < n ? t : n - 1;                    // rows past n: any values, not written
        const int64_t o = (int64_t)t * 128 + wave * UW + uf * 16 + (lane & 15);
        acc[rt][uf][i] = u[o] + u[(int64_t)n * 128 + o];
      }
  if (tid < T) {
    const int t = row0 + tid < n ? row0 + tid : n - 1;
    const f32x4 x = *(const f32x4*)(nr + (int64_t)t * 4), y = *(const f32x4*)(nr + ((int64_t)n + t) * 4);
    nrm[tid][0] = x[0] + y[0];
    nrm[tid][1] = x[1] + y[1];
    nrm[tid][2] = x[2] + y[2];
  }
  __syncthreads();
  route_stream_epilogue<RT, NW>(a, acc, wup, red, nrm, row0);
}

// ------------------------------------------------------------ batch rule
// AND of the per-token decisions; for the batch-min rule the AND is then
// broadcast to every token's mask (River-LLM 方法步骤详情 step 3, TIDE
// formula 4: exit only when every token of the batch passes).
// With alive_in (the generation loop) the AND runs over the running tokens
// only (0 when none runs), and the broadcast also writes alive_out and the
// exit layer of the tokens that exit.
__global__ __launch_bounds__(1024) void route_finish_kernel(int n, uint8_t* mask, int32_t* all_out,
                                                            int batch_min, const uint8_t* alive_in,
                                                            uint8_t* alive_out, int32_t* exit_layer,
                                                            int exit_value) {
  int all = 1, any = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const bool al = alive_in ? alive_in[i] != 0 : true;
    if (al) { all &= (mask[i] != 0); any = 1; }
  }
  all = __syncthreads_and(all);
  any = __syncthreads_or(any);
  if (!any) all = 0;
  if (threadIdx.x == 0 && all_out) *all_out = all;
  if (batch_min) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const bool al = alive_in ? alive_in[i] != 0 : true;
      const bool ex = al && all;
      mask[i] = ex ? 1 : 0;
      if (alive_in) {
        alive_out[i] = (al && !ex) ? 1 : 0;
        if (ex) exit_layer[i] = exit_value;
      }
    }
  }
}

}  // namespace river

namespace river_host {
using namespace river;

// waves per workgroup of the streaming route: eight issue the slab loads
// faster than four (measured, graph-timed: 7.25 against 7.49 µs for 4096
// tokens of d = 768, 21.6 against 24.4 µs for 256 tokens of d = 4096; the
// same at 8192 tokens)
constexpr int ROUTE_WAVES = 8;

// 32 tokens per workgroup (RT = 2) once 16-token workgroups would exceed
// one per CU: every workgroup reads the whole router (1 MB at b = 128,
// d = 4096) besides its tokens' states, so at 7782 tokens 487 workgroups of
// 16 (two per CU on most CUs) read 2.5 MB per CU where 244 of 32 read 1.5;
// up to 4096 tokens 16-token workgroups keep every CU busy with 1.25 MB.
static bool route_two(int n) { return n > 16 * 256; }   // 256 CUs

// the reduction over d in two halves (summed in a fixed order) where the
// slabs split into whole groups of four: d % 512 == 0
static bool route_halves(int d) { return d % 512 == 0; }

size_t route_halves_bytes(int n, int n_ck) {
  return align_up((size_t)n_ck * 2 * n * (128 + 4) * 4, 256);
}

// the streaming path's conditions (launch_route takes it whenever they hold)
static bool stream_ok(int n, int d, river_dtype dt, int b, int64_t ld_prev, int64_t ld_cur) {
  return dt == RIVER_BF16 && d % 256 == 0 && b <= 128 && (int64_t)n * ld_cur * 2 < ((int64_t)1 << 31) &&
         (int64_t)n * ld_prev * 2 < ((int64_t)1 << 31) && d <= 8192;
}

bool route_scores_ok(int n, int d, river_dtype dt, int b, int64_t ld, int n_ck) {
  return n_ck <= RM_MAX && stream_ok(n, d, dt, b, ld, ld);
}

river_status launch_route_scores(int n, int d, river_dtype dt, int64_t ld, int n_ck, const river_checkpoint* ck,
                                 const void* gamma, float eps, int b, float* cos_out, float* prob_out,
                                 uint8_t* mask_scratch, void* halves, hipStream_t s) {
  if (n <= 0 || n_ck <= 0) return RIVER_OK;
  if (!route_scores_ok(n, d, dt, b, ld, n_ck))
    return fail(RIVER_ERR_UNSUPPORTED, "route scores: shape outside the streaming path");
  RouteMulti m{};
  for (int c = 0; c < n_ck; ++c)
    m.a[c] = RouteArgs{n, d, b, ck[c].h_prev, ld, ck[c].h_cur, ld, gamma, eps, ck[c].w_down, ck[c].w_up,
                       __builtin_inff(), __builtin_inff(), cos_out + (int64_t)c * n, prob_out + (int64_t)c * n,
                       mask_scratch + (int64_t)c * n, nullptr, nullptr, nullptr, 0, 0};
  // the same tile as launch_route at this n, so the same values
  const bool two = route_two(n);
  const int T = two ? 32 : 16;
  const dim3 blk(64 * ROUTE_WAVES);
  if (halves && route_halves(d)) {
    // the reduction over d in two workgroups per token group, then their
    // sums added and the epilogue run (the same bits as launch_route's
    // one-workgroup halves)
    RouteHalves hv{(float*)halves, (float*)halves + (size_t)n_ck * 2 * n * 128};
    const dim3 grid((unsigned)((n + T - 1) / T), (unsigned)n_ck, 2);
    auto go = [&](auto rt, auto g) {
      constexpr int RT = decltype(rt)::value;
      route_stream_halves_kernel<RT, decltype(g)::value, ROUTE_WAVES><<<grid, blk, 0, s>>>(m, hv);
    };
    if (gamma) { if (two) go(std::integral_constant<int, 2>{}, std::true_type{}); else go(std::integral_constant<int, 1>{}, std::true_type{}); }
    else { if (two) go(std::integral_constant<int, 2>{}, std::false_type{}); else go(std::integral_constant<int, 1>{}, std::false_type{}); }
    river_status st = check_launch("route scores (halves)");
    if (st != RIVER_OK) return st;
    const dim3 g2((unsigned)((n + T - 1) / T), (unsigned)n_ck);
    if (two) route_halves_kernel<2, ROUTE_WAVES><<<g2, blk, 0, s>>>(m, hv);
    else route_halves_kernel<1, ROUTE_WAVES><<<g2, blk, 0, s>>>(m, hv);
    return check_launch("route scores (sum of halves)");
  }
  // (both halves in one workgroup where launch_route sums them so)
  const dim3 grid((unsigned)((n + T - 1) / T), (unsigned)n_ck);
  auto go = [&](auto rt, auto g, auto hl) {
    route_stream_multi_kernel<decltype(rt)::value, decltype(g)::value, ROUTE_WAVES, decltype(hl)::value>
        <<<grid, blk, 0, s>>>(m);
  };
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  auto pick = [&](auto g) {
    if (route_halves(d)) { if (two) go(R2{}, g, std::true_type{}); else go(R1{}, g, std::true_type{}); }
    else { if (two) go(R2{}, g, std::false_type{}); else go(R1{}, g, std::false_type{}); }
  };
  if (gamma) pick(std::true_type{});
  else pick(std::false_type{});
  return check_launch("route scores");
}

river_status launch_route(int n, int d, river_dtype dt, const void* h_prev, int64_t ld_prev,
                          const void* h_cur, int64_t ld_cur, const void* gamma, float eps,
                          const void* w_down, const void* w_up, int b, float tau, float theta,
                          river_rule rule, float* cos_out, float* prob_out, uint8_t* mask_out,
                          int32_t* all_exit_out, const RouteLive* live, hipStream_t s) {
  const int batch_min = rule == RIVER_RULE_BATCH_MIN;
  RouteArgs a{n, d, b, h_prev, ld_prev, h_cur, ld_cur, gamma, eps, w_down, w_up, tau, theta,
              cos_out, prob_out, mask_out,
              live ? live->alive_in : nullptr, live ? live->alive_out : nullptr,
              live ? live->exit_layer : nullptr, live ? live->exit_value : 0, batch_min};
  if (n > 0) {
    const bool mfma = dt == RIVER_BF16 && w_down && d % 32 == 0 && b % 16 == 0 && b <= 128;
    // streaming path: groups of four 64-wide slabs, byte offsets of both state arrays and
    // W_down within 31 bits, gamma (if any) within its LDS copy
    const bool stream = w_down && stream_ok(n, d, dt, b, ld_prev, ld_cur);
    if (stream) {
      const bool two = route_two(n);
      const int T = two ? 32 : 16;
      const dim3 grid((n + T - 1) / T);
      const dim3 blk(64 * ROUTE_WAVES);
      if (gamma) {
        if (route_halves(d)) {
          if (two) route_stream_kernel<2, true, ROUTE_WAVES, true><<<grid, blk, 0, s>>>(a);
          else route_stream_kernel<1, true, ROUTE_WAVES, true><<<grid, blk, 0, s>>>(a);
        } else {
          if (two) route_stream_kernel<2, true, ROUTE_WAVES, false><<<grid, blk, 0, s>>>(a);
          else route_stream_kernel<1, true, ROUTE_WAVES, false><<<grid, blk, 0, s>>>(a);
        }
      } else {
        if (route_halves(d)) {
          if (two) route_stream_kernel<2, false, ROUTE_WAVES, true><<<grid, blk, 0, s>>>(a);
          else route_stream_kernel<1, false, ROUTE_WAVES, true><<<grid, blk, 0, s>>>(a);
        } else {
          if (two) route_stream_kernel<2, false, ROUTE_WAVES, false><<<grid, blk, 0, s>>>(a);
          else route_stream_kernel<1, false, ROUTE_WAVES, false><<<grid, blk, 0, s>>>(a);
        }
      }
    } else if (mfma) {
      const bool two = n >= 8192;   // 32 tokens per workgroup once the grid is large
      const bool g = gamma != nullptr;
      const bool full = b == 128;
      auto go = [&](auto rt, auto gam, auto fb) {
        constexpr int RT = decltype(rt)::value;
        route_mfma_kernel<RT, decltype(gam)::value, decltype(fb)::value>
            <<<(n + 16 * RT - 1) / (16 * RT), 512, 0, s>>>(a);
      };
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using T = std::true_type;
      using F = std::false_type;
      if (two) {
        if (g) { if (full) go(I2{}, T{}, T{}); else go(I2{}, T{}, F{}); }
        else { if (full) go(I2{}, F{}, T{}); else go(I2{}, F{}, F{}); }
      } else {
        if (g) { if (full) go(I1{}, T{}, T{}); else go(I1{}, T{}, F{}); }
        else { if (full) go(I1{}, F{}, T{}); else go(I1{}, F{}, F{}); }
      }
    } else if (!w_down) {
      const int E = dt == RIVER_BF16 ? 8 : 4;
      const int per_lane = (d / E + WAVE - 1) / WAVE;
      const dim3 grid((unsigned)((n + 3) / 4));
      auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a); };
      if (dt == RIVER_BF16) {
        if (per_lane <= 1) go(route_cos_kernel<true, 1>);
        else if (per_lane <= 2) go(route_cos_kernel<true, 2>);
        else if (per_lane <= 4) go(route_cos_kernel<true, 4>);
        else if (per_lane <= 8) go(route_cos_kernel<true, 8>);
        else go(route_cos_kernel<true, 0>);
      } else {
        if (per_lane <= 1) go(route_cos_kernel<false, 1>);
        else if (per_lane <= 2) go(route_cos_kernel<false, 2>);
        else if (per_lane <= 4) go(route_cos_kernel<false, 4>);
        else if (per_lane <= 8) go(route_cos_kernel<false, 8>);
        else go(route_cos_kernel<false, 0>);
      }
    } else {
      const size_t lds = w_down ? (size_t)d * sizeof(float) : 0;
      if (lds > 65536) return fail(RIVER_ERR_UNSUPPORTED, "route: router with d = %d needs the bf16 path (d %% 32 == 0, b %% 16 == 0, b <= 128)", d);
      if (dt == RIVER_BF16) route_generic_kernel<true><<<n, 64, lds, s>>>(a);
      else route_generic_kernel<false><<<n, 64, lds, s>>>(a);
    }
    river_status st = check_launch("route");
    if (st != RIVER_OK) return st;
  }
  if (rule == RIVER_RULE_BATCH_MIN || all_exit_out) {
    route_finish_kernel<<<1, 1024, 0, s>>>(n, mask_out, all_exit_out, batch_min, a.alive_in,
                                           a.alive_out, a.exit_layer, a.exit_value);
    return check_launch("route finish");
  }
  return RIVER_OK;
}

}  // namespace river_host
