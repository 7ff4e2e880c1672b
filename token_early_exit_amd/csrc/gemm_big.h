// bf16 GEMM for large row counts: C[z] = A[z] . B[z]^T (both operands
// K-contiguous, "NT"), fp32 accumulation, K a multiple of 128, bf16 output
// (EPI_BF16, or EPI_BF16N with the per-column gamma and the per-row partial
// sums of squares; see gemm.h), or EPI_CACHE: columns [0, nh) to the K
// cache and [nh, 2 nh) to the V cache at the slot of each row (the K/V
// projection on weights dequantised to bf16 beforehand).
//
// Workgroup tile 256 x 256, 512 threads = 8 waves in a 2 x 4 grid; each
// wave owns a 128 x 64 block: 4 x 2 accumulators of 32x32 fed by
// v_mfma_f32_32x32x16_bf16, so each 16-byte fragment read from LDS feeds
// 1.33 MFMAs (0.75 KB of LDS reads per MFMA, against 1 KB for 64 x 64 wave
// blocks). The K-slab is 32 wide: a stage holds 256 + 256 rows of 64 bytes
// (32 KB), and a 4-stage ring (128 KB) keeps three slabs in flight, as in
// gemm.h. The larger tile also halves the operand bytes each tile brings in
// from beyond L2 per flop, which bounds the 128 x 128 kernel once the
// operands no longer fit in the last-level cache.
//
// Rows of 4 chunks of 16 bytes; chunk c of row r is stored at
// r * 4 + (c ^ ((r >> 2) & 3)): a 16-lane group reading one logical chunk of
// 16 consecutive rows touches 16 distinct 16-byte bank groups.
//
// Inside a slab, sub-step s and lane half h contract chunk 2 h + s, for A
// and B alike, so the sum over the slab is unchanged.
//
// The epilogue stores straight from the accumulators (8 bytes per lane and
// fragment group; the output is a small part of the traffic at these sizes).
#pragma once

#include "gemm.h"

namespace river {

__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

template <int EPI>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs g, int tiles_n, int batch) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_BF16N || EPI == EPI_CACHE, "bf16 output");
  constexpr int BM = 256, BN = 256;
  constexpr int MI = 4, NI = 2;          // 32x32 fragments per wave
  constexpr int AD = BM * 4 / 512;       // A loads per thread per slab (2)
  constexpr int BD = BN * 4 / 512;       // B loads per thread per slab (2)
  constexpr int PER_SLAB = AD + BD;
  constexpr int SSZ = (BM + BN) * 4;     // one stage in 16-byte chunks: A rows, then B rows
  __shared__ u32x4 S0[SSZ], S1[SSZ], S2[SSZ], S3[SSZ];

  const int M_max = g.M_max, N = g.N, K = g.K, a_nrows = g.a_nrows;
  int M = M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < M_max ? md : M_max);
  }
  // persistent, XCD-aware tile walk with groups of GM row tiles (gemm.h)
  constexpr int GM = 4;
  const int tiles_m_act = (M + BM - 1) / BM;
  const int total = tiles_n * tiles_m_act * batch;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5;
  const int KT = K / 32;                 // a multiple of 4

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto stage = [&](auto st) -> u32x4* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return S0; else if constexpr (S == 1) return S1;
    else if constexpr (S == 2) return S2; else return S3;
  };

  for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
    const int z = tile / (tiles_n * tiles_m_act);
    const int tz = tile - z * tiles_n * tiles_m_act;
    const int g0 = tz / (GM * tiles_n) * GM;
    const int gsz = tiles_m_act - g0 < GM ? tiles_m_act - g0 : GM;
    const int tg = tz - g0 * tiles_n;
    const int mt = g0 + tg % gsz;
    const int nt = tg / gsz;
    const int m0 = mt * BM, n0 = nt * BN;

    // EPI_CACHE: the row ids of this lane's four output rows go out now, the
    // slots once the first slab has landed (its wait covers these loads)
    [[maybe_unused]] int er[MI], sl[MI];
    if constexpr (EPI == EPI_CACHE) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = m0 + wm * 128 + mi * 32 + (lane & 31);
        const int rc = row < M ? row : M - 1;
        er[mi] = g.e_rows ? g.e_rows[rc] : rc;
      }
    }

    // load i of this thread fills LDS chunk p = (i * 8 + wave) * 64 + lane
    // of the A (or B) rows: row p / 4, physical chunk p % 4, which holds
    // logical chunk (p % 4) ^ swz4(row)
    int a_src_row[AD];
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int t = m0 + (((i * 8 + wave) * 64 + lane) >> 2);
      a_src_row[i] = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
    }
    const void* a_buf = g.A + (int64_t)z * g.a_bstride;
    const int a_bytes = (int)(a_nrows * g.lda * 2);
    uint32_t a_off[AD];
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int p = (i * 8 + wave) * 64 + lane;
      const int r = p >> 2, c = (p & 3) ^ swz4(r);
      int src = a_src_row[i];
      if (src < 0 || src >= a_nrows) src = 0;   // row 0 stands in; dropped
      // rows past the count read zeros without a fetch (not stored either)
      a_off[i] = m0 + r >= M ? BUF_OOB : (uint32_t)(((int64_t)src * g.lda + c * 8) * 2);
    }
    const void* b_buf = g.B + (int64_t)z * g.b_bstride;
    const int b_bytes = (int)(N * g.ldb * 2);                   // rows past N read zeros
    uint32_t b_off[BD];
#pragma unroll
    for (int i = 0; i < BD; ++i) {
      const int p = (i * 8 + wave) * 64 + lane;
      const int r = p >> 2, c = (p & 3) ^ swz4(r);
      b_off[i] = (uint32_t)(((int64_t)(n0 + r) * g.ldb + c * 8) * 2);
    }
    auto issue = [&](auto st, int j) {
      u32x4* l = stage(st);
#pragma unroll
      for (int i = 0; i < AD; ++i) buf_lds<16>(a_buf, a_bytes, a_off[i], j * 64, l + (i * 8 + wave) * 64);
#pragma unroll
      for (int i = 0; i < BD; ++i) buf_lds<16>(b_buf, b_bytes, b_off[i], j * 64, l + BM * 4 + (i * 8 + wave) * 64);
    };

    struct Frag { bf16x8 a[MI], b[NI]; };
    auto frag = [&](const u32x4* l, int s, Frag& f) {
      const int ch = 2 * h + s;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * 128 + mi * 32 + (lane & 31);
        f.a[mi] = __builtin_bit_cast(bf16x8, l[r * 4 + (ch ^ swz4(r))]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        f.b[ni] = __builtin_bit_cast(bf16x8, l[BM * 4 + r * 4 + (ch ^ swz4(r))]);
      }
    };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    // B first: lane l holds output row l % 32 and, per group of four
    // registers, four consecutive columns
    auto mfma = [&](const Frag& f) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
    };

    if (tile != xcd * chunk + wg_in_xcd) {
      // every wave is done with the previous tile's stages
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    issue(I0{}, 0);
    issue(I1{}, 1);
    issue(I2{}, 2);
    wait_barrier<2 * PER_SLAB, true>();   // slab 0 landed
    if constexpr (EPI == EPI_CACHE) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = m0 + wm * 128 + mi * 32 + (lane & 31);
        const bool ok = row < M && er[mi] >= 0 && er[mi] < g.e_nrows;
        sl[mi] = ok ? g.slot[er[mi]] : -1;          // range-checked where it is used
      }
    }
    Frag f0, f1;
    frag(S0, 0, f0);

    // slab kt in stage kt % 4: issue slab kt + 3 into the stage of slab
    // kt - 1 (free since the previous barrier), sub-step 0, barrier for slab
    // kt + 1, then sub-step 1 over the first fragments of slab kt + 1
    auto iter = [&](auto st, int kt, auto w, auto issue_next) {
      constexpr int ST = decltype(st)::value;
      using NX = std::integral_constant<int, (ST + 1) & 3>;
      using PV = std::integral_constant<int, (ST + 3) & 3>;
      constexpr bool ISS = decltype(issue_next)::value;
      if constexpr (ISS) issue(PV{}, kt + 3);
      frag(stage(st), 1, f1);
      mfma(f0);
      interleave<1, MI * NI, MI + NI, ISS ? PER_SLAB : 0, 0>();
      wait_barrier<decltype(w)::value, true>();   // slab kt + 1 landed
      frag(stage(NX{}), 0, f0);                   // (a spare read after the last slab)
      mfma(f1);
      interleave<1, MI * NI, MI + NI, 0, 0>();
    };
    using W2 = std::integral_constant<int, 2 * PER_SLAB>;
    using W1 = std::integral_constant<int, PER_SLAB>;
    using W0 = std::integral_constant<int, 0>;
    using T_ = std::true_type;
    using F_ = std::false_type;
    int kt = 0;
    for (; kt + 4 < KT; kt += 4) {
      iter(I0{}, kt, W2{}, T_{});
      iter(I1{}, kt + 1, W2{}, T_{});
      iter(I2{}, kt + 2, W2{}, T_{});
      iter(I3{}, kt + 3, W2{}, T_{});
    }
    iter(I0{}, kt, W2{}, T_{});
    iter(I1{}, kt + 1, W1{}, F_{});
    iter(I2{}, kt + 2, W0{}, F_{});
    iter(I3{}, kt + 3, W0{}, F_{});

    // ---- epilogue, straight from the accumulators: lane l holds row
    // mi * 32 + l % 32 of the wave block and, per group gq, the four
    // consecutive columns ni * 32 + 8 gq + 4 (l / 32) + 0..3
    {
      const int rb = m0 + wm * 128, cb = n0 + wn * 64;
      [[maybe_unused]] uint2 gam[NI][4];
      if constexpr (EPI == EPI_BF16N) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = cb + ni * 32 + 8 * gq + 4 * h;
            gam[ni][gq] = col < N ? *(const uint2*)(g.gamma + (int64_t)z * g.gamma_bstride + col)
                                  : uint2{0u, 0u};
          }
        // partial sums of squares of this wave's 64 columns, per row
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          float ss = 0.f;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) ss = fmaf(acc[mi][ni][e], acc[mi][ni][e], ss);
          ss += __shfl_xor(ss, 32, 64);          // the row's other 32 columns
          const int row = rb + mi * 32 + (lane & 31);
          if (h == 0 && row < M && cb < N)
            g.ss[(int64_t)z * g.ss_bstride + (int64_t)row * (N >> 6) + (cb >> 6)] = ss;
        }
      }
      if constexpr (EPI == EPI_CACHE) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int row = rb + mi * 32 + (lane & 31);
          const int slot = sl[mi];
          if (row >= M || slot < 0 || slot >= g.n_slots) continue;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int col = cb + ni * 32 + 8 * gq + 4 * h;   // four columns, all in K or all in V
              if (col >= N) continue;
              const bool isv = col >= g.nh;
              uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc) + (int64_t)z * g.cache_bstride +
                              (int64_t)slot * g.nh + (isv ? col - g.nh : col);
              *(uint2*)dst = uint2{pack_bf16x2(acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1]),
                                   pack_bf16x2(acc[mi][ni][4 * gq + 2], acc[mi][ni][4 * gq + 3])};
            }
        }
        continue;                                  // next tile
      }
      uint16_t* C = (uint16_t*)g.C + (int64_t)z * g.c_bstride;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = rb + mi * 32 + (lane & 31);
        if (row >= M) continue;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = cb + ni * 32 + 8 * gq + 4 * h;
            if (col >= N) continue;
            f32x4 v = {acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1], acc[mi][ni][4 * gq + 2],
                       acc[mi][ni][4 * gq + 3]};
            if constexpr (EPI == EPI_BF16N) {
              v[0] *= bf16_lo(gam[ni][gq].x);
              v[1] *= bf16_hi(gam[ni][gq].x);
              v[2] *= bf16_lo(gam[ni][gq].y);
              v[3] *= bf16_hi(gam[ni][gq].y);
            }
            *(uint2*)(C + (int64_t)row * g.ldc + col) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      }
    }
  }  // tiles
}

// Launch: one workgroup of 8 waves per CU (128 KB of LDS), capped by the
// tile count and rounded up to whole XCDs. Requirements as gemm_launch's,
// K % 128 == 0, N % 4 == 0.
template <int EPI>
inline void gemm_big_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 255) / 256;
  const int tm = (g.M_max + 255) / 256;
  const int64_t tiles = (int64_t)tn * tm * batch;
  const int grid = persistent_grid(tiles);
  gemm_big_kernel<EPI><<<dim3(grid, 1), 512, 0, s>>>(g, tn, batch);
}

}  // namespace river
