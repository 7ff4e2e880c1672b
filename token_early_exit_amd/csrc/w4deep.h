// The W4A16 K/V projection for decode-sized row counts (the same operation
// as w4gemm.h, with the K/V cache scatter as its epilogue):
//   C[z] = A[z] . deq(W[z])^T,  deq(q) = (q - zero) * scale per group,
// rows [0, nh) of W from descriptor 0 (K), [nh, 2 nh) from descriptor 1 (V).
//
// At a decode step's row counts (tens of rows under a bound of 256) the
// 128-row tiles of w4gemm.h spend their time waiting: they keep the loads of
// about two 64-wide slabs in flight, and a load takes about 1.5 us to land
// under load, so each slab costs some 0.7 us whatever the rows (at the 8B
// shape, 21 blocks x 13 rows: 52 us, the same with every block's weights in
// L2). Here a tile is 32 rows x 256 columns and the pipeline moves in
// super-slabs of 256 input channels (four slabs) through a ring of three LDS
// stages of 52 KB: the A rows (32 x 512 B), the int4 weights (256 columns x
// 128 B, whole lines) and the scale / zero words of the super-slab; two
// super-slabs, eight slabs, are in flight while one is used, and one
// barrier serves four slabs.
//
// 8 waves, wave w owns columns [32 w, 32 w + 32): one 32x32 accumulator on
// v_mfma_f32_32x32x16_bf16, B first (lane l holds output row l % 32 and,
// per group of four registers, four consecutive columns). Slab s of a
// super-slab, sub-step u: lane half h = l / 32 contracts channels
// 64 s + 32 h + 8 u .. + 7, that is A chunk 8 s + 4 h + u of its row and
// dword u of the lane's 16 weight bytes of slab s, dequantised in registers
// with the code of w4gemm.h (dequant8): the same sums, in the same order,
// as w4_gemm_kernel, so the results are bit-identical to it.
//
// A few tiles leave most CUs idle (13 rows x 21 blocks: 168 tiles; one
// block of 243 rows: 64), and each CU streams its operands at a bounded
// rate (some 25 GB/s), so with room for partial sums (g.part, g.part_cap
// bytes) the kernel splits the reduction over d into P parts of whole
// super-slabs, P chosen on the device from the row count: as many as keep
// every part on a workgroup of its own, at most 8 and T, within the room
// (more parts than workgroups measured slower: each part pays the
// pipeline's start). The
// parts are written as fp32 and w4_deep_finish_kernel adds them in order
// (then the sums differ from w4_gemm_kernel's by rounding); with P = 1 the
// tile writes the cache itself and the finish kernel does nothing.
//
// Requirements (w4_deep_ok): d % 256 == 0, nh % 64 == 0, each super-slab's
// scales of a column in one aligned 4-byte word (bf16 with group 128 or
// 256, fp32 with group 256), the spans below 2^31 bytes.
#pragma once

#include "w4gemm.h"

namespace river {

// The parts of the deep projection's reduction: units is the tile count
// for the row count on the device, cus the CUs they are chosen for. The
// same function serves the projection and its finish kernel.
__device__ __forceinline__ int w4_deep_parts(const GemmArgs& g, int units, int rows, int batch, int cus) {
  if (!g.part || g.M_dev_z || units <= 0) return 1;
  const int T = g.K / 256;
  int p = cus / units;
  p = p < 8 ? p : 8;
  p = p < T ? p : T;
  const int64_t per = (int64_t)batch * rows * g.N * 4;   // bytes per part
  while (p > 1 && p * per > g.part_cap) --p;
  return p > 1 ? p : 1;
}

constexpr int W4_DEEP_LDS = 3 * (32 * 32 + 256 * 8 + 8 * 2 * 64 / 4);   // 16-byte units

// The deep projection's work on LDS (W4_DEEP_LDS of it) given by the
// caller; gated: honour the gate of a split launch.
template <bool SZ_BF16>
__device__ __forceinline__ void w4_deep_body(const GemmArgs& g, int tiles_n, int batch, u32x4* L, bool gated) {
  constexpr int BM = 32, BN = 256, NW = 8, CW = 32;
  constexpr int SZB = SZ_BF16 ? 2 : 4;
  // stage layout in 16-byte units: A [32 rows][32 chunks] (physical chunk
  // 8 s' + c of row r holds logical chunk c ^ swz(r) of slab s' ^ b(r),
  // b(r) = bit 3 of r: rows 512 bytes apart all start on bank 0, and the
  // slab flip puts rows r and r + 8 on different halves of the banks, so a
  // fragment read by 16 lanes touches 16 distinct 16-byte bank groups); weights
  // [256 columns][8 chunks] (logical chunk q = 2 s + half at q ^ swz(col));
  // scale / zero words [8 waves][2][64]
  constexpr int AO = 0, WO = BM * 32, ZO = WO + BN * 8, SSZ = ZO + NW * 2 * 64 / 4;
  constexpr int NS = 3;
  // loads per thread and super-slab: 2 A, 4 weights, scale, zero
  constexpr int PER = 2 + 4 + 2;
  static_assert(NS * SSZ == W4_DEEP_LDS, "the LDS layout");

  const int M_max = g.M_max, N = g.N, K = g.K, nh = g.nh, a_nrows = g.a_nrows;
  const int grp = g.group[0];
  int M = M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < M_max ? md : M_max);
  }
  if (gated && !gate_open(g, M)) return;   // the other launch's counts
  const int tiles_m_act = ((g.M_dev_z ? M_max : M) + BM - 1) / BM;
  const int tiles = tiles_n * tiles_m_act * batch;
  // parts for the whole chip whatever the launch's CU budget, so that the
  // sums do not depend on it
  const int P = w4_deep_parts(g, tiles, M, batch, N_CU);
  const int total = tiles * P;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int T = K / 256;                 // super-slabs
  const int gpr = K / grp;               // groups per weight row
  const int gps = 256 / grp;             // groups per super-slab (1 or 2)

  for (int unit = xcd * chunk + wg_in_xcd; unit < t_end; unit += per_xcd) {
    const int tile = unit % tiles, part = unit / tiles;
    const int nt = tile % tiles_n;
    const int mt = (tile / tiles_n) % tiles_m_act;
    const int z = tile / (tiles_n * tiles_m_act);
    // super-slabs [ta, tb) of the reduction
    const int ta = part * T / P, tb = (part + 1) * T / P, TT = tb - ta;
    const int m0 = mt * BM, n0 = nt * BN;
    if (g.M_dev_z) {                     // uniform
      const int mz = g.M_dev_z[z];
      M = mz < 0 ? 0 : (mz < M_max ? mz : M_max);
      if (m0 >= M) continue;
    }
    // A: load i of this wave covers stage chunks p = (8 i + wave) 64 + l:
    // row p / 32, slab (p % 32) / 8; rows past the count fetch nothing
    const void* a_buf = g.A + (int64_t)z * g.a_bstride;
    const int a_bytes = (int)(a_nrows * g.lda * 2);
    uint32_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = (8 * i + wave) * 64 + lane;
      const int r = p >> 5, c = p & 31;
      const int lc = (((c >> 3) ^ ((r >> 3) & 1)) << 3) | ((c & 7) ^ swz(r));
      const int t = m0 + r;
      int src = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
      if (src < 0 || src >= a_nrows) src = 0;          // row 0 stands in; dropped
      a_off[i] = t >= M ? BUF_OOB : (uint32_t)(((int64_t)src * g.lda + lc * 8) * 2);
    }
    // weights: this wave's 32 columns lie wholly in the K or the V half
    const int wc0 = n0 + CW * wave;
    const bool cols_ok = wc0 < N;
    const int which = wc0 >= nh ? 1 : 0;
    const int hc0 = wc0 - which * nh;
    const void* q_buf = (which ? g.q[1] : g.q[0]) + (int64_t)z * g.q_bstride;
    const int q_bytes = nh * (K / 2);
    const int64_t szs = which ? g.sz_bstride[1] : g.sz_bstride[0];
    const void* s_buf = (const char*)(which ? g.s[1] : g.s[0]) + z * szs * SZB;
    const void* z_buf = (const char*)(which ? g.zp[1] : g.zp[0]) + z * szs * SZB;
    const int sz_bytes = nh * gpr * SZB;
    // weight load m: wave columns 8 m + l / 8, 16-byte chunk (l % 8) ^ swz
    uint32_t wq_off[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int jc = 8 * m + (lane >> 3);
      const int cl = CW * wave + jc;
      wq_off[m] = cols_ok ? (uint32_t)((hc0 + jc) * (K / 2) + ((lane & 7) ^ swz(cl)) * 16) : BUF_OOB;
    }
    // scale / zero: lane l < 32 loads the word of column l holding the
    // super-slab's groups (the aligned word holding its group when a word
    // holds two and the super-slab one)
    const uint32_t sz_off = (cols_ok && lane < 32) ? (uint32_t)((hc0 + lane) * gpr * SZB) : BUF_OOB;

    auto issue = [&](int st, int t) {
      u32x4* l = L + st * SSZ;
#pragma unroll
      for (int i = 0; i < 2; ++i) buf_lds<16>(a_buf, a_bytes, a_off[i], t * 512, l + AO + (8 * i + wave) * 64);
#pragma unroll
      for (int m = 0; m < 4; ++m) buf_lds<16>(q_buf, q_bytes, wq_off[m], t * 128, l + WO + (wave * 4 + m) * 64);
      const int g0 = t * gps;
      const int go = (SZ_BF16 && gps == 1 ? (g0 & ~1) : g0) * SZB;
      uint32_t* lz = (uint32_t*)(l + ZO) + wave * 128;
      buf_lds<4>(s_buf, sz_bytes, sz_off, go, lz);
      buf_lds<4>(z_buf, sz_bytes, sz_off, go, lz + 64);
    };

    if (unit != xcd * chunk + wg_in_xcd) {
      // every wave is done with the previous tile's stages and epilogue
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // cache slot of row m0 + l (lane l < 32), looked up after the first wait
    int er = 0, sl = -1;
    {
      const int row = m0 + (lane & 31);
      const int rc = row < M ? row : M - 1;
      er = g.e_rows ? g.e_rows[rc] : rc;
    }
    issue(0, ta);
    if (TT > 1) issue(1, ta + 1);
    if (TT > 1) wait_barrier<PER, true>();
    else wait_barrier<0, true>();
    {
      const bool ok = m0 + (lane & 31) < M && er >= 0 && er < g.e_nrows;
      sl = ok ? g.slot[er] : -1;
    }

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    const int ra = lane & 31, cl = CW * wave + (lane & 31), fa = (ra >> 3) & 1;
    for (int i = 0; i < TT; ++i) {
      const int st = i % NS, t = ta + i;
      if (i > 0) {
        // super-slab t landed (t + 1 may still be in flight), and every
        // wave is done with super-slab t - 1, whose stage t + 2 reuses
        if (i + 1 < TT) wait_barrier<PER, true>();
        else wait_barrier<0, true>();
      }
      if (i + 2 < TT) issue((i + 2) % NS, t + 2);
      const u32x4* l = L + st * SSZ;
      const uint32_t* lz = (const uint32_t*)(l + ZO) + wave * 128;
      const uint32_t sw = lz[lane & 31], zw = lz[64 + (lane & 31)];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // the group of slab s: word half (64 s / grp) for two groups per
        // word, the super-slab's parity otherwise
        const int half = SZ_BF16 ? (gps == 2 ? (s >> 1) : (t & 1)) : 0;
        const uint32_t sb = SZ_BF16 ? (sw >> (16 * half)) & 0xFFFFu : sw;
        const uint32_t zb = SZ_BF16 ? (zw >> (16 * half)) & 0xFFFFu : zw;
        const float sc = SZ_BF16 ? __uint_as_float(sb << 16) : __uint_as_float(sb);
        const float ze = SZ_BF16 ? __uint_as_float(zb << 16) : __uint_as_float(zb);
        const float cc = -ze * sc;
        const u32x4 wq = l[WO + cl * 8 + ((2 * s + h) ^ swz(cl))];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, l[AO + ra * 32 + 8 * (s ^ fa) + ((4 * h + u) ^ swz(ra))]);
          uint32_t o[4];
          dequant8(wq[u], sc, cc, o);
          u32x4 v;
          v[0] = o[0]; v[1] = o[1]; v[2] = o[2]; v[3] = o[3];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), a, acc, 0, 0, 0);
        }
      }
    }

    if (P > 1) {
      // fp32 partial sums [part][z][row][N] of the rows on the device:
      // lane l holds row l % 32 and columns 8 gq + 4 (l / 32) + 0..3
      const int row = m0 + (lane & 31);
      if (row < M && cols_ok) {
        float* dst = g.part + (((int64_t)part * batch + z) * M + row) * N + wc0 + 4 * h;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *(f32x4*)(dst + 8 * gq) = f32x4{acc[4 * gq], acc[4 * gq + 1], acc[4 * gq + 2], acc[4 * gq + 3]};
      }
      continue;                          // next unit
    }
    // epilogue: the wave's 32 x 32 block as bf16 through LDS (its own
    // region in a stage the last super-slab did not use: past the last
    // barrier the waves read only that one), then row by row, 4 lanes x 16
    // bytes per row
    {
      constexpr int EP = CW + 8;
      const int free_st = (TT - 1) % NS == 0 ? 1 : 0;
      uint16_t* ep = (uint16_t*)(L + free_st * SSZ) + wave * BM * EP;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int r = lane & 31, c = 8 * gq + 4 * h;
        *(uint2*)(ep + r * EP + c) = uint2{pack_bf16x2(acc[4 * gq], acc[4 * gq + 1]),
                                           pack_bf16x2(acc[4 * gq + 2], acc[4 * gq + 3])};
      }
      const int ch = lane & 3;
      const int col = wc0 + 8 * ch;                   // 8 columns, all in K or all in V
      const bool isv = col >= nh;
#pragma unroll
      for (int i = 0; i < BM / 16; ++i) {
        const int r = i * 16 + (lane >> 2);
        const u32x4 v = *(const u32x4*)(ep + r * EP + 8 * ch);
        const int sr = __shfl(sl, r, 64);
        if (sr < 0 || sr >= g.n_slots || !cols_ok) continue;
        uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc);
        *(u32x4*)(dst + (int64_t)z * g.cache_bstride + (int64_t)sr * nh + (isv ? col - nh : col)) = v;
      }
    }
  }
}

template <bool SZ_BF16>
__global__ __launch_bounds__(512, 1) void w4_deep_kernel(GemmArgs g, int tiles_n, int batch) {
  __shared__ u32x4 L[W4_DEEP_LDS];
  w4_deep_body<SZ_BF16>(g, tiles_n, batch, L, true);
}

// One launch for both ranges of counts: the deep pipeline when its tiles
// fit one round (g.gate_units, g.gate_cus), else the 128-row int4 kernel
// (tn_deep, tn_big: their column tiles), on one LDS array, so that the
// count the launch does not take costs no launch of its own.
template <bool SZ_BF16, bool SZT>
__global__ __launch_bounds__(512, 1) void w4_either_kernel(GemmArgs g, int tn_deep, int tn_big, int batch) {
  constexpr int BIG = w4_lds_units<128, 8, false, SZT>();
  __shared__ u32x4 L[W4_DEEP_LDS > BIG ? W4_DEEP_LDS : BIG];
  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  if ((int64_t)((M + 31) / 32) * g.gate_units <= g.gate_cus) w4_deep_body<SZ_BF16>(g, tn_deep, batch, L, false);
  else w4_gemm_body<128, EPI_CACHE, SZ_BF16, 8, false, SZT>(g, tn_big, batch, L, false);
}

// The deep pipeline's shape conditions (the caller has checked those of
// the MFMA fill: d % 256 == 0, nh % 64 == 0, equal groups and scale types
// for K and V, spans below 2^31 bytes).
inline bool w4_deep_ok(const GemmArgs& g) {
  const int grp = g.group[0];
  if (g.K % 256 || grp <= 0) return false;
  if (g.sz_bf16[0]) return grp == 128 || (grp == 256 && (g.K / grp) % 2 == 0);
  return grp == 256;
}

// The parts of a split reduction added in order, rounded to bf16 and
// written to each row's cache slot: one thread per 8 columns of a row of the
// rows on the device; nothing when the projection took one part. cus: the
// CUs its parts were chosen for.
__global__ __launch_bounds__(256) void w4_deep_finish_kernel(GemmArgs g, int batch, int tiles_n, int cus) {
  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  if (!gate_open(g, M)) return;
  const int P = w4_deep_parts(g, tiles_n * ((M + 31) / 32) * batch, M, batch, cus);
  if (P == 1) return;
  const int N = g.N, nh = g.nh, per = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int p = (int)(idx % per);
  const int t = (int)((idx / per) % g.M_max);
  const int z = (int)(idx / ((int64_t)per * g.M_max));
  if (z >= batch || t >= M) return;
  const int e = g.e_rows ? g.e_rows[t] : t;
  if (e < 0 || e >= g.e_nrows) return;
  const int sl = g.slot[e];
  if (sl < 0 || sl >= g.n_slots) return;
  const int col = 8 * p;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < P; ++k) {
    const float* src = g.part + (((int64_t)k * batch + z) * M + t) * N + col;
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
  const bool isv = col >= nh;
  uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc);
  *(u32x4*)(dst + (int64_t)z * g.cache_bstride + (int64_t)sl * nh + (isv ? col - nh : col)) = o;
}

// The projection over `batch` layers for every count, one launch (the
// 128-row kernel's side without a split, M_max > 64), and with g.part set
// the finish kernel of the deep side's split.
inline void w4_either_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 255) / 256;
  const int grid = persistent_grid(launch_cu_budget());
  const bool szt = w4_tile_scales_ok(g);
  if (g.sz_bf16[0]) {
    if (szt) w4_either_kernel<true, true><<<grid, 512, 0, s>>>(g, tn, tn, batch);
    else w4_either_kernel<true, false><<<grid, 512, 0, s>>>(g, tn, tn, batch);
  } else {
    if (szt) w4_either_kernel<false, true><<<grid, 512, 0, s>>>(g, tn, tn, batch);
    else w4_either_kernel<false, false><<<grid, 512, 0, s>>>(g, tn, tn, batch);
  }
  if (g.part) {
    const int64_t threads = (int64_t)batch * g.M_max * (g.N / 8);
    w4_deep_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(g, batch, tn, N_CU);
  }
}

// The projection over `batch` layers, and (with g.part set) the finish
// kernel of its split: one workgroup per CU of the budget at most.
inline void w4_deep_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 255) / 256;
  const int tm = (g.M_max + 31) / 32;
  const int64_t tiles = (int64_t)tn * tm * batch;
  // with a split the units can outnumber the tiles: one workgroup per CU
  const int grid = g.part ? persistent_grid(launch_cu_budget()) : persistent_grid(tiles);
  if (g.sz_bf16[0]) w4_deep_kernel<true><<<grid, 512, 0, s>>>(g, tn, batch);
  else w4_deep_kernel<false><<<grid, 512, 0, s>>>(g, tn, batch);
  if (g.part) {
    const int64_t threads = (int64_t)batch * g.M_max * (g.N / 8);
    w4_deep_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(g, batch, tn, N_CU);
  }
}

}  // namespace river
