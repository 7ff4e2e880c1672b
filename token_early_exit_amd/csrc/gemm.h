// Tiled bf16 GEMM on gfx950 MFMA: C[z] = A[z] . B[z]^T with A [M][K] and
// B [N][K] both K-contiguous ("NT"), fp32 accumulation.
//
// Workgroup tile BM x 128 x 64 (K), 256 threads = 4 waves in a 2x2 grid;
// each wave owns a (BM/2) x 64 block of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16. Operand tiles are staged in LDS, double
// buffered, with 16-byte chunks XOR-swizzled by row (chunk ^ (row & 7)) so
// that the fragment reads (8 consecutive rows of one chunk per group of 8
// lanes) and the staging writes are bank-conflict free. Global loads of the
// next K-slab are issued before the MFMAs of the current one.
//
// A may be gathered through a row index (the exited tokens) and its row
// count may live in device memory (the compaction's count), so the grid is
// sized for M_max and surplus workgroups exit at once.
//
// B is either bf16 or group-quantized int4 ([Wk; Wv] stacked along N). The
// int4 path dequantizes in registers while staging to LDS:
//   w = (q - zero) * scale = fma(q, scale, -zero * scale)
// rounded to bf16 for the MFMA.
//
// Epilogues: bf16 store, fp32 store (+ a constant on the diagonal), or the
// K/V cache scatter: row t goes to slot[e_rows[t]] of layer z, columns
// [0, nh) to the K cache and [nh, 2 nh) to the V cache.
#pragma once

#include "common.h"

namespace river {

enum { EPI_BF16 = 0, EPI_F32 = 1, EPI_CACHE = 2 };

struct GemmArgs {
  int M_max;
  const int32_t* M_dev;      // rows = clamp(*M_dev, 0, M_max) when set
  int N, K;
  // A operand, bf16
  const uint16_t* A; int64_t lda; int64_t a_bstride;
  const int32_t* a_rows; int a_nrows;   // A row of output row t (NULL: t)
  // B operand, bf16
  const uint16_t* B; int64_t ldb; int64_t b_bstride;
  // B operand, int4: rows [0, nh) from descriptor 0, [nh, 2 nh) from 1
  const uint8_t* q[2]; const void* s[2]; const void* zp[2];
  int group[2]; int sz_bf16[2];
  int nh;
  int64_t q_bstride;         // bytes per layer  (nh * K / 2)
  int64_t sz_bstride[2];     // elements per layer (nh * K / group)
  // epilogue
  void* C; int64_t ldc; int64_t c_bstride; float diag;
  const int32_t* e_rows;     // slot row of output row t (NULL: t)
  const int32_t* slot; int64_t n_slots; int e_nrows;
  void* kc; void* vc; int64_t cache_bstride;   // elements per layer
};

__device__ __forceinline__ float load_sz(const void* p, int64_t i, int bf16) {
  return bf16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// 8 int4 weights (one dword, element k in nibble k) -> 8 bf16 in 4 dwords
__device__ __forceinline__ void dequant8(uint32_t w, float s, float c, uint32_t* out) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e0 = (float)((lo >> (8 * j)) & 0xFFu);
    const float e1 = (float)((hi >> (8 * j)) & 0xFFu);
    out[j] = pack_bf16x2(fmaf(e0, s, c), fmaf(e1, s, c));
  }
}

template <int BM, bool BQ4, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs g) {
  constexpr int BN = 128;
  constexpr int MI = BM / 64;          // 32-row fragments per wave
  constexpr int NI = BN / 64;          // 32-col fragments per wave
  constexpr int AL = BM / 32;          // 16-byte A chunks per thread per slab
  constexpr int BL = BN / 32;          // 16-byte B chunks per thread per slab (bf16 B)
  __shared__ u32x4 As[2][BM * 8];
  __shared__ u32x4 Bs[2][BN * 8];

  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int z = blockIdx.z;
  if (m0 >= M) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // ---- A loader setup
  const uint16_t* a_ptr[AL];
  bool a_ok[AL];
  int a_lds[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
    const int t = m0 + r;
    int src = t;
    bool ok = t < M;
    if (ok && g.a_rows) {
      src = g.a_rows[t];
      ok = src >= 0 && src < g.a_nrows;
    }
    a_ok[i] = ok;
    a_ptr[i] = g.A + (int64_t)z * g.a_bstride + (int64_t)(ok ? src : 0) * g.lda + ch * 8;
    a_lds[i] = r * 8 + (ch ^ (r & 7));
  }
  // ---- B loader setup
  const uint16_t* b_ptr[BL];
  int b_lds[BL];
  const uint8_t* q_ptr = nullptr;
  const void* s_ptr = nullptr;
  const void* z_ptr = nullptr;
  int q_row = 0, q_half = 0, q_grp = 0, q_szbf = 0;
  int64_t sz_row = 0;
  if constexpr (!BQ4) {
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int c = tid + 256 * i, r = c >> 3, ch = c & 7;
      const int nn = n0 + r < g.N ? n0 + r : 0;
      b_ptr[i] = g.B + (int64_t)z * g.b_bstride + (int64_t)nn * g.ldb + ch * 8;
      b_lds[i] = r * 8 + (ch ^ (r & 7));
    }
  } else {
    q_row = tid >> 1;
    q_half = tid & 1;
    int nn = n0 + q_row;
    if (nn >= 2 * g.nh) nn = 0;          // past the last tile's edge: any valid row
    const int which = nn >= g.nh ? 1 : 0;
    const int rr = nn - which * g.nh;
    q_grp = g.group[which];
    q_szbf = g.sz_bf16[which];
    q_ptr = g.q[which] + (int64_t)z * g.q_bstride + (int64_t)rr * (g.K / 2) + q_half * 16;
    s_ptr = g.s[which];
    z_ptr = g.zp[which];
    sz_row = (int64_t)z * g.sz_bstride[which] + (int64_t)rr * (g.K / q_grp);
  }

  u32x4 ra[AL], rb[BL];
  u32x4 rq;
  float rs = 0.f, rc = 0.f;

  auto load_slab = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = a_ok[i] ? *(const u32x4*)(a_ptr[i] + k0) : zero4;
    if constexpr (!BQ4) {
#pragma unroll
      for (int i = 0; i < BL; ++i) rb[i] = *(const u32x4*)(b_ptr[i] + k0);
    } else {
      rq = *(const u32x4*)(q_ptr + k0 / 2);
      const int64_t gi = sz_row + (k0 + 32 * q_half) / q_grp;
      const float sc = load_sz(s_ptr, gi, q_szbf);
      const float ze = load_sz(z_ptr, gi, q_szbf);
      rs = sc;
      rc = -ze * sc;
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) As[buf][a_lds[i]] = ra[i];
    if constexpr (!BQ4) {
#pragma unroll
      for (int i = 0; i < BL; ++i) Bs[buf][b_lds[i]] = rb[i];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v;
        uint32_t o[4];
        dequant8(rq[j], rs, rc, o);
        v[0] = o[0]; v[1] = o[1]; v[2] = o[2]; v[3] = o[3];
        const int ch = q_half * 4 + j;
        Bs[buf][q_row * 8 + (ch ^ (q_row & 7))] = v;
      }
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

  const int KT = g.K / 64;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_slab((kt + 1) * 64);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + (lane >> 5);
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * (BM / 2) + mi * 32 + (lane & 31);
        af[mi] = __builtin_bit_cast(bf16x8, As[buf][r * 8 + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * (BN / 2) + ni * 32 + (lane & 31);
        bfr[ni] = __builtin_bit_cast(bf16x8, Bs[buf][r * 8 + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) store_slab(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue. 32x32 accumulator layout: column = lane % 32,
  // row = 8 * (e / 4) + 4 * (lane / 32) + e % 4 for element e of 16.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = n0 + wn * (BN / 2) + ni * 32 + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * (BM / 2) + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= M) continue;
        const float v = acc[mi][ni][e];
        if constexpr (EPI == EPI_BF16) {
          ((uint16_t*)g.C)[(int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col] = f32_to_bf16(v);
        } else if constexpr (EPI == EPI_F32) {
          ((float*)g.C)[(int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col] = v + (row == col ? g.diag : 0.f);
        } else {
          const int er = g.e_rows ? g.e_rows[row] : row;
          if (er < 0 || er >= g.e_nrows) continue;
          const int sl = g.slot[er];
          if (sl < 0 || sl >= g.n_slots) continue;
          const bool isv = col >= g.nh;
          uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc);
          dst[(int64_t)z * g.cache_bstride + (int64_t)sl * g.nh + (isv ? col - g.nh : col)] = f32_to_bf16(v);
        }
      }
    }
  }
}

}  // namespace river
