// Tiled bf16 GEMM on gfx950 MFMA: C[z] = A[z] . B[z]^T with A [M][K] and
// B [N][K] both K-contiguous ("NT"), fp32 accumulation.
//
// Workgroup tile BM x 128 x 64 (K), 256 threads = 4 waves in a 2x2 grid;
// each wave owns a (BM/2) x 64 block of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16. Operand tiles reach LDS through direct
// global->LDS loads (no staging registers) in a 4-stage ring, three K-slabs
// ahead of the MFMAs; 16-byte chunks are XOR-swizzled by row (swz below)
// so that fragment reads are bank-conflict free.
//
// The kernel is persistent: one workgroup per CU walks the tiles. A may be
// gathered through a row index (the exited tokens) and its row count may
// live in device memory (the compaction's count); only the tiles of rows
// that exist are visited, so nothing waits on the host.
//
// B is either bf16 or group-quantized int4 ([Wk; Wv] stacked along N). The
// int4 weights are dequantized once per workgroup into an LDS bf16 tile:
//   w = (q - zero) * scale = fma(q, scale, -zero * scale)
// rounded to bf16 for the MFMA.
//
// Epilogues: bf16 store, fp32 store (+ a constant on the diagonal), or the
// K/V cache scatter: row t goes to slot[e_rows[t]] of layer z, columns
// [0, nh) to the K cache and [nh, 2 nh) to the V cache.
#pragma once

#include <type_traits>

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
  const uint32_t lo = opaque_and(w, 0x0F0F0F0Fu);          // elements 0, 2, 4, 6
  const uint32_t hi = opaque_and(w >> 4, 0x0F0F0F0Fu);     // elements 1, 3, 5, 7
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e0 = (float)((lo >> (8 * j)) & 0xFFu);
    const float e1 = (float)((hi >> (8 * j)) & 0xFFu);
    out[j] = pack_bf16x2(fmaf(e0, s, c), fmaf(e1, s, c));
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane l of the
// wave writes lds_base + 16 * l (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 16, 0, 0);
}

// 4 bytes per lane from global memory into LDS (lane l writes lds_base + 4 l)
__device__ __forceinline__ void dma4(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 4, 0, 0);
}

// Four-stage pipeline. Everything a K-slab needs goes to LDS stage
// slab % 4 through direct global->LDS loads (no staging registers), issued
// three slabs ahead. Each stage is a separate LDS array so the compiler
// can tell which load a read depends on.
// bf16 B: B tiles are staged like A.
// int4 B: wave w loads the packed weights (32 rows x 32 bytes) and the
// scale/zero of rows 32w..32w+31, exactly what its own threads dequantize,
// so the dequantization of slab k+1 (into one of two bf16 B buffers, during
// iteration k) needs only a wait on the wave's own loads, no barrier.
template <int BM, bool BQ4, int EPI, bool SZ_BF16 = true>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs g, int tiles_n, int tiles_m, int batch) {
  constexpr int BN = 128;
  constexpr int MI = BM / 64;            // 32-row fragments per wave
  constexpr int NI = BN / 64;            // 32-col fragments per wave
  constexpr int AD = BM * 8 / 256;       // A DMA instructions per thread per slab
  constexpr int BD = BQ4 ? 2 : 4;        // B DMA instructions per thread per slab
  constexpr int PER_SLAB = AD + BD;      // vector-memory ops per slab (all DMA)
  constexpr int SZB = SZ_BF16 ? 2 : 4;   // bytes per scale / zero
  // one LDS array per pipeline stage: A tile, then the B tile (bf16 B) or
  // the packed int4 rows and their scale/zero words (int4 B); the int4 path
  // has two more arrays for the dequantized bf16 B tile
  constexpr int SB = BQ4 ? 256 + 64 : BN * 8;           // 16-byte units after A
  __shared__ u32x4 S0[BM * 8 + SB], S1[BM * 8 + SB], S2[BM * 8 + SB], S3[BM * 8 + SB];
  __shared__ u32x4 D0[BQ4 ? BN * 8 : 1], D1[BQ4 ? BN * 8 : 1];

  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  // Persistent tiles: only the tiles of the M rows that exist are visited.
  // Tile t = (z * tiles_m_active + mt) * tiles_n + nt. Workgroups are
  // dispatched round-robin over the 8 XCDs; XCD x walks the contiguous range
  // [x * chunk, (x + 1) * chunk) so that neighbouring tiles (same A rows,
  // same layer's weights) share that XCD's L2.
  const int tiles_m_act = (M + BM - 1) / BM;
  const int total = tiles_n * tiles_m_act * batch;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;     // workgroups on this XCD
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;
  for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
  if (tile != xcd * chunk + wg_in_xcd) __syncthreads();   // LDS of the previous tile is free
  const int nt = tile % tiles_n;
  const int mt = (tile / tiles_n) % tiles_m_act;
  const int z = tile / (tiles_n * tiles_m_act);
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  (void)tiles_m;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int wm = wave >> 1, wn = wave & 1;

  // DMA block b = i * 4 + wave covers LDS chunks [64 b, 64 b + 64); lane l
  // fills chunk p = 64 b + l = (row p / 8, physical chunk p % 8), which
  // holds logical chunk (p % 8) ^ swz(row) of that row.
  // gathered row indices: all loads first (clamped, branch-free), then use
  int a_src_row[AD];
#pragma unroll
  for (int i = 0; i < AD; ++i) {
    const int t = m0 + (((i * 4 + wave) * 64 + lane) >> 3);
    a_src_row[i] = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
  }
  const uint16_t* a_src[AD];
#pragma unroll
  for (int i = 0; i < AD; ++i) {
    const int p = (i * 4 + wave) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ swz(r);
    int src = a_src_row[i];
    // rows past M or with an index outside A: row 0 stands in, output dropped
    if (m0 + r >= M || src < 0 || src >= g.a_nrows) src = 0;
    a_src[i] = g.A + (int64_t)z * g.a_bstride + (int64_t)src * g.lda + c * 8;
  }
  const uint16_t* b_src[BQ4 ? 1 : BD];
  if constexpr (!BQ4) {
#pragma unroll
    for (int i = 0; i < BD; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;
      const int r = p >> 3, c = (p & 7) ^ swz(r);
      const int nn = n0 + r < g.N ? n0 + r : 0;
      b_src[i] = g.B + (int64_t)z * g.b_bstride + (int64_t)nn * g.ldb + c * 8;
    }
  }
  // int4: thread tid = (row tid / 2, half tid % 2) owns 32 weights of one
  // row per slab; its wave's lane loads exactly those 16 bytes. For the
  // scale/zero load lane l < 32 fetches the scale and lane l >= 32 the zero
  // of row 32 * wave + l % 32, as the aligned 4-byte word that holds it (a
  // bf16 value sits in the low or high half by the parity of its group;
  // rows hold an even number of groups, so the word stays inside the row).
  const int q_row = tid >> 1, q_half = tid & 1;
  const uint8_t* q_src = nullptr;
  const char* sz_src = nullptr;
  int q_grp = 64;
  if constexpr (BQ4) {
    auto split = [&](int nn, int& which, int& rr) {
      if (nn >= 2 * g.nh) nn = 0;        // past the last tile's edge: any valid row
      which = nn >= g.nh ? 1 : 0;
      rr = nn - which * g.nh;
    };
    int which, rr;
    split(n0 + q_row, which, rr);
    q_grp = g.group[which];
    q_src = g.q[which] + (int64_t)z * g.q_bstride + (int64_t)rr * (g.K / 2) + q_half * 16;
    int w2, r2;
    split(n0 + 32 * wave + (lane & 31), w2, r2);
    const char* base = (const char*)(lane < 32 ? g.s[w2] : g.zp[w2]);
    sz_src = base + ((int64_t)z * g.sz_bstride[w2] + (int64_t)r2 * (g.K / g.group[w2])) * SZB;
    q_grp = g.group[which];
  }

  auto stageS = [&](auto st) -> u32x4* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return S0; else if constexpr (S == 1) return S1;
    else if constexpr (S == 2) return S2; else return S3;
  };
  auto stageA = [&](auto st) -> u32x4* { return stageS(st); };
  // bf16 B tile of stage ST; for int4 B, dequantized buffer ST (0 or 1)
  auto stageB = [&](auto st) -> u32x4* {
    if constexpr (BQ4) {
      constexpr int S = decltype(st)::value;
      if constexpr (S == 0) return D0; else return D1;
    } else {
      return stageS(st) + BM * 8;
    }
  };
  auto stageQ = [&](auto st) -> u32x4* { return stageS(st) + BM * 8; };
  auto stageZ = [&](auto st) -> uint32_t* { return (uint32_t*)(stageS(st) + BM * 8 + 256); };

  // issue every load of K-slab j into stage ST
  auto issue = [&](auto st, int j) {
    const int k0 = j * 64;
    u32x4* la = stageA(st);
#pragma unroll
    for (int i = 0; i < AD; ++i) dma16(a_src[i] + k0, la + (i * 4 + wave) * 64);
    if constexpr (!BQ4) {
      u32x4* lb = stageB(st);
#pragma unroll
      for (int i = 0; i < BD; ++i) dma16(b_src[i] + k0, lb + (i * 4 + wave) * 64);
    } else {
      dma16(q_src + k0 / 2, stageQ(st) + wave * 64);
      // group of this slab (groups are multiples of 64 wide)
      const int gi = k0 / q_grp;
      dma4(sz_src + (int64_t)(SZ_BF16 ? (gi & ~1) : gi) * SZB, stageZ(st) + wave * 64);
    }
  };
  // int4 slab j, held in stage ST: this thread's 32 weights and their
  // scale / zero (the wave loaded exactly these itself)
  struct DQ { u32x4 w; float sc, cc; };
  auto dq_load = [&](auto st, int j) -> DQ {
    DQ q;
    q.w = stageQ(st)[tid];
    const uint32_t* zb = stageZ(st) + wave * 64;
    const int rl = q_row & 31;
    float ze;
    if constexpr (SZ_BF16) {
      const int sh = ((j * 64 / q_grp) & 1) * 16;
      q.sc = __uint_as_float((zb[rl] >> sh) << 16);
      ze = __uint_as_float((zb[32 + rl] >> sh) << 16);
    } else {
      q.sc = __uint_as_float(zb[rl]);
      ze = __uint_as_float(zb[32 + rl]);
    }
    q.cc = -ze * q.sc;
    return q;
  };
  // dequantize the part-th 8 weights into bf16 buffer DB
  auto dq_part = [&](const DQ& q, auto db, int part) {
    uint32_t o[4];
    dequant8(q.w[part], q.sc, q.cc, o);
    u32x4 v;
    v[0] = o[0]; v[1] = o[1]; v[2] = o[2]; v[3] = o[3];
    const int ch = q_half * 4 + part;
    stageB(db)[q_row * 8 + (ch ^ swz(q_row))] = v;
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

  // the four 16-wide K sub-steps of one slab; the fragments of sub-step
  // s + 1 are read from LDS while the MFMAs of sub-step s run, and hook(s)
  // (VALU work) is issued behind them. The B fragment is the MFMA's first
  // operand, so the accumulator comes out transposed: lane l holds output
  // row l % 32 and, per group of four registers, four consecutive columns.
  auto compute = [&](u32x4* la, u32x4* lb, auto hook) {
    bf16x8 af[2][MI], bfr[2][NI];
    auto frags = [&](int s, bf16x8* a, bf16x8* b) {
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * (BM / 2) + mi * 32 + (lane & 31);
        a[mi] = __builtin_bit_cast(bf16x8, la[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * (BN / 2) + ni * 32 + (lane & 31);
        b[ni] = __builtin_bit_cast(bf16x8, lb[r * 8 + (ch ^ swz(r))]);
      }
    };
    frags(0, af[0], bfr[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // keep the program order: next fragments requested, then this
      // sub-step's MFMAs (which wait only for the older reads)
      if (s < 3) frags(s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][ni], af[s & 1][mi],
                                                               acc[mi][ni], 0, 0, 0);
      hook(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_hook = [](int) {};

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  const int KT = g.K / 64;

  // prologue: slabs 0, 1, 2 in flight (issued unconditionally, so the loop
  // is entered with a fixed number of loads outstanding: below three slabs
  // the last one is fetched again into a stage that is never read); int4
  // slab 0 dequantized once this wave's share of it has landed
  issue(I0{}, 0);
  issue(I1{}, KT > 1 ? 1 : KT - 1);
  issue(I2{}, KT > 2 ? 2 : KT - 1);
  if constexpr (BQ4) {
    wait_vm<2 * PER_SLAB>();
    const DQ q0 = dq_load(I0{}, 0);
#pragma unroll
    for (int part = 0; part < 4; ++part) dq_part(q0, I0{}, part);
  }

  // One iteration: slab kt lives in stage ST; slab kt+3 goes to stage
  // ST+3. Past the last slab the loads are still issued (slab KT-1 again,
  // into a stage that is never read), so every iteration waits for exactly
  // two slabs' worth of loads and the loop body has no data-dependent
  // branches.
  auto iter = [&](auto st, int kt) {
    constexpr int ST = decltype(st)::value;
    using NX = std::integral_constant<int, (ST + 3) & 3>;   // stage of slab kt + 3
    using N1 = std::integral_constant<int, (ST + 1) & 3>;   // stage of slab kt + 1
    using DB = std::integral_constant<int, ST & 1>;         // int4 bf16 buffer of slab kt
    using DN = std::integral_constant<int, (ST + 1) & 1>;   // ... and of slab kt + 1
    wait_barrier<2 * PER_SLAB, BQ4>();
    issue(NX{}, kt + 3 < KT ? kt + 3 : KT - 1);
    if constexpr (BQ4) {
      // slab kt+1 is dequantized behind the MFMAs of slab kt; this wave's
      // loads of it are done once the loads of the two slabs after it are
      // the only ones outstanding (after the last slab this converts a
      // spare copy into a buffer that is never read)
      wait_vm<2 * PER_SLAB>();
      const DQ q = dq_load(N1{}, kt + 1);
      compute(stageA(st), stageB(DB{}), [&](int part) { dq_part(q, DN{}, part); });
    } else {
      compute(stageA(st), stageB(st), no_hook);
    }
  };
  int kt = 0;
  for (; kt + 4 <= KT; kt += 4) {   // whole groups of four slabs, no exits inside
    iter(I0{}, kt);
    iter(I1{}, kt + 1);
    iter(I2{}, kt + 2);
    iter(I3{}, kt + 3);
  }
  const int rem = KT - kt;          // 0..3 slabs left, in stages 0.. (kt % 4 == 0)
  if (rem > 0) iter(I0{}, kt);
  if (rem > 1) iter(I1{}, kt + 1);
  if (rem > 2) iter(I2{}, kt + 2);
  wait_vm<0>();   // the spare loads land before the stages are reused or freed

  // ---- epilogue. Transposed 32x32 accumulator: lane l holds output row
  // l % 32 of its fragment and, for g = 0..3, the four consecutive columns
  // 8 g + 4 (l / 32) + 0..3 in registers 4 g .. 4 g + 3. N is a multiple of 4.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = m0 + wm * (BM / 2) + mi * 32 + (lane & 31);
    if (row >= M) continue;
    int sl = 0;
    if constexpr (EPI == EPI_CACHE) {
      const int er = g.e_rows ? g.e_rows[row] : row;
      if (er < 0 || er >= g.e_nrows) continue;
      sl = g.slot[er];
      if (sl < 0 || sl >= g.n_slots) continue;
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = n0 + wn * (BN / 2) + ni * 32 + 8 * gq + 4 * (lane >> 5);
        if (col >= g.N) continue;
        const float v0 = acc[mi][ni][4 * gq], v1 = acc[mi][ni][4 * gq + 1];
        const float v2 = acc[mi][ni][4 * gq + 2], v3 = acc[mi][ni][4 * gq + 3];
        if constexpr (EPI == EPI_F32) {
          f32x4 o = {v0, v1, v2, v3};
          if (row >= col && row < col + 4) o[row - col] += g.diag;
          *(f32x4*)((float*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col) = o;
        } else {
          const uint2 o = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          if constexpr (EPI == EPI_BF16) {
            *(uint2*)((uint16_t*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col) = o;
          } else {
            const bool isv = col >= g.nh;
            uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc);
            *(uint2*)(dst + (int64_t)z * g.cache_bstride + (int64_t)sl * g.nh + (isv ? col - g.nh : col)) = o;
          }
        }
      }
    }
  }
  }  // tiles
}

// Host-side launch of one tile configuration over a batch of `batch`
// problems (grid flattened for the XCD-aware tile order).
// One workgroup per CU (each needs 86-128 KB of LDS), capped by the tile
// count for the row bound and rounded up to whole XCDs; every workgroup
// walks its share of the tiles.
constexpr int N_CU = 256;
template <int BM, bool BQ4, int EPI>
inline void gemm_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 127) / 128;
  const int tm = (g.M_max + BM - 1) / BM;
  int64_t tiles = (int64_t)tn * tm * batch;
  int grid = (int)(tiles < N_CU ? tiles : N_CU);
  grid = (grid + 7) / 8 * 8;
  if (BQ4 && !g.sz_bf16[0])
    gemm_nt_kernel<BM, BQ4, EPI, false><<<dim3(grid, 1), 256, 0, s>>>(g, tn, tm, batch);
  else
    gemm_nt_kernel<BM, BQ4, EPI, true><<<dim3(grid, 1), 256, 0, s>>>(g, tn, tm, batch);
}

// Tile choice from the row bound: 64-row tiles for decode-sized batches,
// 128 otherwise.
template <bool BQ4, int EPI>
inline void gemm_auto(const GemmArgs& g, int batch, hipStream_t s) {
  if (g.M_max <= 64) gemm_launch<64, BQ4, EPI>(g, batch, s);
  else gemm_launch<128, BQ4, EPI>(g, batch, s);
}

}  // namespace river
