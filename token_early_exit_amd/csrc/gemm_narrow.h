// bf16 GEMM for decode-sized row counts: C[z] = A[z] . B[z]^T (both operands
// K-contiguous), fp32 accumulation, bf16 output (EPI_BF16), or EPI_CACHE:
// columns [0, nh) to the K cache and [nh, 2 nh) to the V cache at the slot
// of each row. The map GEMM of a fill whose row bound is at most 256 (a
// decode step's exits at one checkpoint), and the projection of such rows
// through folded products F = deq([Wk; Wv]) . M (EPI_CACHE).
//
// There the time goes into streaming the maps (B), d x d per layer, from
// HBM: 21 maps of 4096 x 4096 are 705 MB for 13 rows. The 128-row tiles of
// gemm.h keep three 64-wide slabs in flight, 48 KB of map rows per CU; at
// about 2 µs of HBM latency under load that is some 24 GB/s per CU, and the
// launch ran at 5.1 TB/s. Here a tile is 32 rows x 128 columns, so a 64-wide
// slab is 4 KB of rows and 16 KB of map, and an 8-stage ring (160 KB of LDS)
// keeps seven slabs, 112 KB of map, in flight.
//
// 4 waves, wave w owns columns [32 w, 32 w + 32) of the tile: one 32x32
// accumulator on v_mfma_f32_32x32x16_bf16, B first (lane l holds output
// row l % 32 and, per group of four registers, four consecutive columns).
// Sub-step s of a slab takes logical 16-byte chunk 4 h + s of each row, as
// gemm.h does.
//
// Over several maps each tile starts its walk over K at its own slab,
// (37 tile) mod K/64, and wraps around. All CUs start together and advance
// at about the same pace, so with a common start every load in flight on
// the chip would sit at the same 128-byte offset of an 8 KB map row;
// measured on a pure read of this pattern (21 maps of 4096^2) that reaches
// 4.1-4.8 TB/s, with staggered starts 5.7-6.1 (the GEMM: 129-135 -> 121-126
// us). The sums then run in another order than gemm_nt_kernel's: the
// results agree to rounding. Over one map (read from L2 by every row tile)
// there is no rotation, and the results are bit-identical to
// gemm_nt_kernel<128>'s.
//
// Loads: every wave load covers 8 rows x 128 contiguous bytes (8 lanes per
// row); chunk p of an operand block holds logical chunk (p % 8) ^ swz(row)
// of row p / 8, so the fragment reads are conflict-free. Rows past the
// count read zeros without a fetch; map rows past N read zeros.
#pragma once

#include "gemm.h"

namespace river {

constexpr int NARROW_BM = 32, NARROW_BN = 128, NARROW_NS = 8;

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_narrow_kernel(GemmArgs g, int tiles_n, int batch) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_CACHE, "bf16 output");
  constexpr int BM = NARROW_BM, BN = NARROW_BN;
  constexpr int SSZ = (BM + BN) * 8;     // one stage in 16-byte chunks (20 KB)
  constexpr int BD = BN * 8 / 256;       // B loads per thread per slab (A: one)
  constexpr int PER = 1 + BD;
  __shared__ u32x4 L[NARROW_NS * SSZ];

  const int M_max = g.M_max, N = g.N, K = g.K, a_nrows = g.a_nrows;
  int M = M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < M_max ? md : M_max);
  }
  constexpr int GM = 8;                  // row tiles per group of the tile walk
  const int tiles_m_act = (M + BM - 1) / BM;
  const int total = tiles_n * tiles_m_act * batch;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int KT = K / 64;                 // slabs, a multiple of 8

  for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
    const int z = tile / (tiles_n * tiles_m_act);
    const int tz = tile - z * tiles_n * tiles_m_act;
    const int g0 = tz / (GM * tiles_n) * GM;
    const int gsz = tiles_m_act - g0 < GM ? tiles_m_act - g0 : GM;
    const int tg = tz - g0 * tiles_n;
    const int m0 = (g0 + tg % gsz) * BM, n0 = (tg / gsz) * BN;

    // A load: chunk tid of the 32-row block (row tid / 8); a wave whose 8
    // rows all lie past the count loads nothing (uniform: its rows' results
    // are never stored, whatever LDS holds for them)
    const bool a_on = m0 + 8 * wave < M;
    const void* a_buf = g.A + (int64_t)z * g.a_bstride;
    const int a_bytes = (int)(a_nrows * g.lda * 2);
    uint32_t a_off;
    {
      const int r = tid >> 3, c = (tid & 7) ^ swz(r);
      const int t = m0 + r;
      int src = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
      if (src < 0 || src >= a_nrows) src = 0;   // row 0 stands in; dropped
      a_off = t >= M ? BUF_OOB : (uint32_t)(((int64_t)src * g.lda + c * 8) * 2);
    }
    // B load i: chunk (i * 4 + wave) * 64 + lane of the 128-row block
    const void* b_buf = g.B + (int64_t)z * g.b_bstride;
    const int b_bytes = (int)(N * g.ldb * 2);
    uint32_t b_off[BD];
#pragma unroll
    for (int i = 0; i < BD; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;
      const int r = p >> 3, c = (p & 7) ^ swz(r);
      b_off[i] = (uint32_t)(((int64_t)(n0 + r) * g.ldb + c * 8) * 2);
    }
    // the tile's k-th slab is slab (k + j0) mod KT of the operands (one
    // matrix, re-read from L2 by every row tile: no rotation)
    const int j0 = batch > 1 ? (tile * 37) % KT : 0;
    auto issue = [&](int st, int k) {
      u32x4* l = L + st * SSZ;
      const int j = k + j0 < KT ? k + j0 : k + j0 - KT;
      if (a_on) buf_lds<16>(a_buf, a_bytes, a_off, j * 128, l + wave * 64);
#pragma unroll
      for (int i = 0; i < BD; ++i) buf_lds<16>(b_buf, b_bytes, b_off[i], j * 128, l + BM * 8 + (i * 4 + wave) * 64);
    };
    const int ra = lane & 31, rb = wave * 32 + (lane & 31);
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    // slab j from stage st: all eight fragment reads, then the four MFMAs
    auto compute = [&](int st) {
      const u32x4* l = L + st * SSZ;
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = 4 * h + s;
        fa[s] = __builtin_bit_cast(bf16x8, l[ra * 8 + (ch ^ swz(ra))]);
        fb[s] = __builtin_bit_cast(bf16x8, l[BM * 8 + rb * 8 + (ch ^ swz(rb))]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s], fa[s], acc, 0, 0, 0);
    };

    if (tile != xcd * chunk + wg_in_xcd) {
      // every wave is done reading the previous tile's stages
      constexpr int imm = 15 | (3 << 14) | (7 << 4) | (0 << 8);   // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(imm);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int j = 0; j < NARROW_NS - 1; ++j) issue(j, j);

    // slab kt in stage kt % 8: the wait for it (and the barrier after which
    // the stage of slab kt - 1 is free), the loads of slab kt + 7 into that
    // stage, the MFMAs of slab kt
    auto iter = [&](auto st, int kt, auto w, auto iss) {
      constexpr int ST = decltype(st)::value;
      // the loads of this wave per slab: PER, or PER - 1 without its A rows
      if (a_on) wait_barrier<decltype(w)::value * PER, true>();
      else wait_barrier<decltype(w)::value * (PER - 1), true>();
      if constexpr (decltype(iss)::value) issue((ST + NARROW_NS - 1) % NARROW_NS, kt + NARROW_NS - 1);
      compute(ST);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using W6 = std::integral_constant<int, 6>;
    int kt = 0;
    for (; kt + 2 * NARROW_NS <= KT; kt += NARROW_NS) {
      iter(std::integral_constant<int, 0>{}, kt, W6{}, T_{});
      iter(std::integral_constant<int, 1>{}, kt + 1, W6{}, T_{});
      iter(std::integral_constant<int, 2>{}, kt + 2, W6{}, T_{});
      iter(std::integral_constant<int, 3>{}, kt + 3, W6{}, T_{});
      iter(std::integral_constant<int, 4>{}, kt + 4, W6{}, T_{});
      iter(std::integral_constant<int, 5>{}, kt + 5, W6{}, T_{});
      iter(std::integral_constant<int, 6>{}, kt + 6, W6{}, T_{});
      iter(std::integral_constant<int, 7>{}, kt + 7, W6{}, T_{});
    }
    // the last eight slabs: slab KT - 1 is the last load; then the waits
    // shrink to what is still in flight
    iter(std::integral_constant<int, 0>{}, kt, W6{}, T_{});
    iter(std::integral_constant<int, 1>{}, kt + 1, W6{}, F_{});
    iter(std::integral_constant<int, 2>{}, kt + 2, std::integral_constant<int, 5>{}, F_{});
    iter(std::integral_constant<int, 3>{}, kt + 3, std::integral_constant<int, 4>{}, F_{});
    iter(std::integral_constant<int, 4>{}, kt + 4, std::integral_constant<int, 3>{}, F_{});
    iter(std::integral_constant<int, 5>{}, kt + 5, std::integral_constant<int, 2>{}, F_{});
    iter(std::integral_constant<int, 6>{}, kt + 6, std::integral_constant<int, 1>{}, F_{});
    iter(std::integral_constant<int, 7>{}, kt + 7, std::integral_constant<int, 0>{}, F_{});

    // epilogue straight from the accumulator: row m0 + l % 32, columns
    // n0 + 32 wave + 8 gq + 4 h + 0..3 (EPI_CACHE: nh % 4 == 0, so the four
    // lie in one half; a row whose id or slot is out of range is dropped)
    const int row = m0 + (lane & 31);
    if constexpr (EPI == EPI_CACHE) {
      const int er = row < M ? (g.e_rows ? g.e_rows[row] : row) : -1;
      const int slot = er >= 0 && er < g.e_nrows ? g.slot[er] : -1;
      if (slot >= 0 && slot < g.n_slots) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = n0 + wave * 32 + 8 * gq + 4 * h;
          if (col >= N) continue;
          const bool isv = col >= g.nh;
          *(uint2*)((uint16_t*)(isv ? g.vc : g.kc) + (int64_t)z * g.cache_bstride + (int64_t)slot * g.nh +
                    (isv ? col - g.nh : col)) =
              uint2{pack_bf16x2(acc[4 * gq], acc[4 * gq + 1]), pack_bf16x2(acc[4 * gq + 2], acc[4 * gq + 3])};
        }
      }
    } else if (row < M) {
      uint16_t* C = (uint16_t*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = n0 + wave * 32 + 8 * gq + 4 * h;
        if (col >= N) continue;
        *(uint2*)(C + col) = uint2{pack_bf16x2(acc[4 * gq], acc[4 * gq + 1]),
                                   pack_bf16x2(acc[4 * gq + 2], acc[4 * gq + 3])};
      }
    }
  }
}

// K % 512 == 0 (slabs a multiple of 8), N % 4 == 0, and the requirements of
// gemm_launch; at most one workgroup per CU (160 KB of LDS).
inline bool gemm_narrow_ok(const GemmArgs& g) { return g.K % 512 == 0 && g.N % 4 == 0; }

template <int EPI = EPI_BF16>
inline void gemm_narrow_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + NARROW_BN - 1) / NARROW_BN;
  const int tm = (g.M_max + NARROW_BM - 1) / NARROW_BM;
  const int64_t tiles = (int64_t)tn * tm * batch;
  const int grid = persistent_grid(tiles);
  gemm_narrow_kernel<EPI><<<dim3(grid, 1), 256, 0, s>>>(g, tn, batch);
}

}  // namespace river
