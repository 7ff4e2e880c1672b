// Tiled bf16 GEMM on gfx950 MFMA: C[z] = A[z] . B[z]^T with A [M][K] and
// B [N][K] both K-contiguous ("NT"), fp32 accumulation, K a multiple of 256.
//
// Workgroup tile BM x 128, 256 threads = 4 waves in a 2x2 grid; each wave
// owns a (BM/2) x 64 block of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16. Both operand tiles reach LDS through buffer
// loads straight into LDS (a uniform resource per operand, a fixed 32-bit
// offset per lane and a uniform offset per 64-wide K-slab, so the loop does
// no address arithmetic on the vector unit and rows past the end read as
// zeros), in a 4-stage ring, three slabs ahead of the MFMAs. 16-byte chunks
// are XOR-swizzled by row (swz) so fragment reads are bank-conflict free.
//
// Inside a slab the reduction index is permuted (sub-step s, lane half h
// contracts chunk 4 h + s) identically for A and B, which leaves the sum
// unchanged. The barrier for slab k + 1 sits before the last sub-step of
// slab k, so the first fragments of slab k + 1 are read while the last MFMAs
// of slab k run.
//
// The kernel is persistent: one workgroup per CU walks the tiles. A may be
// gathered through a row index (the exited tokens) and its row count may
// live in device memory (the compaction's count), so nothing waits on the
// host. Epilogues: bf16 store, or fp32 store plus a constant on the
// diagonal; each wave stages its block in LDS and writes whole rows of 64
// columns with 16-byte stores.
#pragma once

#include <type_traits>

#include "common.h"

namespace river {

// EPI_BF16N: bf16 output scaled by gamma[col], plus per-row partial sums
// of squares of the unscaled result (one per 64-column block): the input
// of a skipped layer's RMSNorm, applied in the K/V projection's epilogue.
// EPI_PART: fp32 partial sums of a split reduction, [ksplit][batch][M_max][N]
// (the map GEMM and the W4 projection at small row counts; a finishing
// kernel adds them in a fixed order).
enum { EPI_BF16 = 0, EPI_F32 = 1, EPI_CACHE = 2, EPI_BF16N = 3, EPI_PART = 4 };

struct GemmArgs {
  int M_max;
  const int32_t* M_dev;      // rows = clamp(*M_dev, 0, M_max) when set
  const int32_t* M_dev_z;    // W4 kernel: rows of batch entry z = clamp(M_dev_z[z], 0, M_max) when set
  int N, K;
  // A operand, bf16
  const uint16_t* A; int64_t lda; int64_t a_bstride;
  const int32_t* a_rows; int a_nrows;   // A row of output row t (NULL: t)
  // B operand, bf16
  const uint16_t* B; int64_t ldb; int64_t b_bstride;
  // B operand, int4 (w4gemm.h): rows [0, nh) from descriptor 0, [nh, 2 nh) from 1
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
  // EPI_BF16N: gamma [z][N] (bf16), partial sums ss[z][M_max][N / 64]
  const uint16_t* gamma; int64_t gamma_bstride;
  float* ss; int64_t ss_bstride;
  // K/V projection with the rest of the layer's K/V path (w4gemm.h):
  // row scale 1 / sqrt(sum_p ss_in[z][t][p] / K + eps) when ss_in is set
  // (ss_parts a multiple of 4, at most 128),
  // bias[which][z][col] (bf16) when set, rotary embedding of the K half
  // when pos is set (tables [n_pos][head_dim / 2] fp32, pos per e_row)
  const float* ss_in; int64_t ss_in_bstride; int ss_parts; float norm_eps;
  const uint16_t* bias[2]; int64_t bias_bstride;
  const int32_t* pos; const float* rcos; const float* rsin; int64_t n_pos; int head_dim;
  // split reduction (EPI_PART): K is cut into ksplit parts of K / ksplit
  int ksplit; float* part;
  // w4deep.h: bytes at part for partial sums whose parts the kernel
  // chooses from the row count on the device (0: no split)
  int64_t part_cap;
  // two launches of the int4 projection that split the row counts on the
  // device between them (w4deep.h): with gate = +1 a kernel runs only when
  // ceil(rows / 32) * gate_units <= gate_cus (the deep pipeline's tiles fit
  // one round), with gate = -1 only when not; gate = 0: always
  int gate, gate_units, gate_cus;
};

// whether the kernel of a gated projection launch runs for `rows` rows
__device__ __forceinline__ bool gate_open(const GemmArgs& g, int rows) {
  if (!g.gate) return true;
  const bool deep = (int64_t)((rows + 31) / 32) * g.gate_units <= g.gate_cus;
  return g.gate > 0 ? deep : !deep;
}

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

// Scheduling hint for the preceding code of a basic block, per sub-step:
// the LDS reads of the next fragments first (so their latency is covered),
// then one MFMA at a time with up to VALU vector instructions behind it and,
// every other MFMA, one of N_VMEM global loads, so the matrix unit is fed
// and no burst of loads stalls the wave.
template <int N_SUB, int MFMA_PER_SUB, int READS, int N_VMEM, int VALU = 6>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int sub = 0; sub < N_SUB; ++sub) {
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);                 // LDS reads first
#pragma unroll
    for (int i = 0; i < MFMA_PER_SUB; ++i) {
      const int k = sub * MFMA_PER_SUB + i;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
      if (VALU) __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);     // VALU
      if (k % 2 == 1 && k / 2 < N_VMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // load
    }
  }
}

// Scheduling hint that spreads a sub-step's memory instructions over its
// MFMAs: after MFMA k an LDS read while k % RSTEP == 0 and reads remain,
// otherwise one of N_VMEM global loads, so neither a burst of reads nor of
// loads stalls the in-order issue of the next MFMA.
template <int N_MFMA, int N_READ, int N_VMEM, int RSTEP>
__device__ __forceinline__ void interleave_spread() {
  int r = 0, v = 0;
#pragma unroll
  for (int k = 0; k < N_MFMA; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
    if (k % RSTEP == 0 && r < N_READ) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                  // LDS read
      ++r;
    } else if (v < N_VMEM) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                  // global load
      ++v;
    }
  }
}

constexpr int N_CU = 256;

// CUs that one persistent launch may occupy: all of them, unless a caller
// that runs two launch sequences side by side on two streams narrows it for
// one of them (CuBudget, host side), so that neither waits for the other's
// workgroups to leave a CU. A multiple of 8 (whole XCDs).
inline int& launch_cu_budget() {
  static thread_local int n = N_CU;
  return n;
}
struct CuBudget {
  int prev;
  explicit CuBudget(int n) : prev(launch_cu_budget()) { launch_cu_budget() = n; }
  ~CuBudget() { launch_cu_budget() = prev; }
};
// workgroups of a persistent launch over `tiles` tiles: one per CU of the
// budget at most, rounded up to whole XCDs
inline int persistent_grid(int64_t tiles) {
  const int cus = launch_cu_budget();
  const int grid = (int)(tiles < cus ? tiles : cus);
  return (grid + 7) / 8 * 8;
}

template <int BM, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs g, int tiles_n, int batch) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_F32 || EPI == EPI_BF16N || EPI == EPI_PART,
                "bf16 or fp32 output, or fp32 partial sums");
  constexpr int BN = 128;
  constexpr int MI = BM / 64;            // 32-row fragments per wave
  constexpr int NI = 2;                  // 32-column fragments per wave
  constexpr int AD = BM * 8 / 256;       // A loads per thread per slab
  constexpr int BD = BN * 8 / 256;       // B loads per thread per slab
  constexpr int PER_SLAB = AD + BD;
  constexpr int SSZ = (BM + BN) * 8;     // one stage: A tile, then B tile (16-byte chunks)
  __shared__ u32x4 S0[SSZ], S1[SSZ], S2[SSZ], S3[SSZ];

  const int M_max = g.M_max, N = g.N, K = g.K, a_nrows = g.a_nrows;
  int M = M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < M_max ? md : M_max);
  }
  // Persistent tiles: only the tiles of the M rows that exist are visited,
  // tiles_n * tiles_m_active of them per batch entry z. Workgroups are
  // dispatched round-robin over the 8 XCDs; XCD x walks the contiguous range
  // [x * chunk, (x + 1) * chunk) so that neighbouring tiles (one batch
  // entry, a few row and column tiles) share that XCD's L2.
  const int tiles_m_act = (M + BM - 1) / BM;
  const int ksplit = EPI == EPI_PART ? g.ksplit : 1;
  const int total = tiles_n * tiles_m_act * batch * ksplit;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int KT = K / 64 / ksplit;        // slabs per tile, a multiple of 4

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
    // Inside a batch entry the tiles go in groups of GM row tiles, column
    // tile by column tile, so the 32 tiles an XCD runs at once cover about
    // 4 row tiles x 8 column tiles: 12 operand tiles to bring into its L2
    // instead of 33 for one row tile across 32 column tiles.
    constexpr int GM = 4;
    const int ks = tile / (tiles_n * tiles_m_act * batch);   // part of the reduction
    const int tb = tile - ks * tiles_n * tiles_m_act * batch;
    const uint32_t k_off = (uint32_t)ks * KT * 128;           // its first slab, in bytes
    const int z = tb / (tiles_n * tiles_m_act);
    const int tz = tb - z * tiles_n * tiles_m_act;
    const int g0 = tz / (GM * tiles_n) * GM;                 // first row tile of the group
    const int gsz = tiles_m_act - g0 < GM ? tiles_m_act - g0 : GM;
    const int tg = tz - g0 * tiles_n;
    const int mt = g0 + tg % gsz;
    const int nt = tg / gsz;
    const int m0 = mt * BM, n0 = nt * BN;

    // load i of this thread fills LDS chunk p = (i * 4 + wave) * 64 + lane of
    // a tile, i.e. row p / 8, physical chunk p % 8, which holds logical
    // chunk (p % 8) ^ swz(row) of that row
    int a_src_row[AD];
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int t = m0 + (((i * 4 + wave) * 64 + lane) >> 3);
      a_src_row[i] = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
    }
    const void* a_buf = g.A + (int64_t)z * g.a_bstride;
    const int a_bytes = (int)(a_nrows * g.lda * 2);
    uint32_t a_off[AD];
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;
      const int r = p >> 3, c = (p & 7) ^ swz(r);
      int src = a_src_row[i];
      if (src < 0 || src >= a_nrows) src = 0;   // row 0 stands in; dropped
      // rows past the count read zeros without a fetch (not stored either)
      a_off[i] = m0 + r >= M ? BUF_OOB : (uint32_t)(((int64_t)src * g.lda + c * 8) * 2) + k_off;
    }
    const void* b_buf = g.B + (int64_t)z * g.b_bstride;
    const int b_bytes = (int)(N * g.ldb * 2);                   // rows past N read zeros
    uint32_t b_off[BD];
#pragma unroll
    for (int i = 0; i < BD; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;
      const int r = p >> 3, c = (p & 7) ^ swz(r);
      b_off[i] = (uint32_t)(((int64_t)(n0 + r) * g.ldb + c * 8) * 2) + k_off;
    }
    auto issue = [&](auto st, int j) {
      u32x4* l = stage(st);
#pragma unroll
      for (int i = 0; i < AD; ++i) buf_lds<16>(a_buf, a_bytes, a_off[i], j * 128, l + (i * 4 + wave) * 64);
#pragma unroll
      for (int i = 0; i < BD; ++i) buf_lds<16>(b_buf, b_bytes, b_off[i], j * 128, l + BM * 8 + (i * 4 + wave) * 64);
    };

    struct Frag { bf16x8 a[MI], b[NI]; };
    auto frag = [&](const u32x4* l, int s, Frag& f) {
      const int ch = 4 * h + s;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * (BM / 2) + mi * 32 + (lane & 31);
        f.a[mi] = __builtin_bit_cast(bf16x8, l[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        f.b[ni] = __builtin_bit_cast(bf16x8, l[BM * 8 + r * 8 + (ch ^ swz(r))]);
      }
    };
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    // B first: the accumulator comes out transposed (lane l holds output
    // row l % 32 and, per group of four registers, four consecutive columns)
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
    Frag f0, f1;
    frag(S0, 0, f0);

    // slab kt in stage kt % 4: issue slab kt + 3 into the stage of slab
    // kt - 1, sub-steps 0..2, barrier for slab kt + 1, then sub-step 3 over
    // the first fragments of slab kt + 1
    auto iter = [&](auto st, int kt, auto w, auto issue_next) {
      constexpr int ST = decltype(st)::value;
      using NX = std::integral_constant<int, (ST + 1) & 3>;
      using PV = std::integral_constant<int, (ST + 3) & 3>;
      constexpr bool ISS = decltype(issue_next)::value;
      if constexpr (ISS) issue(PV{}, kt + 3);
      frag(stage(st), 1, f1);
      mfma(f0);
      frag(stage(st), 2, f0);
      mfma(f1);
      frag(stage(st), 3, f1);
      mfma(f0);
      interleave<3, MI * NI, MI + NI, ISS ? PER_SLAB : 0, 0>();
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

    // ---- epilogue: each wave stages its (BM/2) x 64 block in its own
    // stage array (the other waves only make spare reads of stage 0 from
    // here on, whose values are never used), then writes whole rows of its
    // 64 columns with 16-byte stores.
    {
      constexpr bool F32OUT = EPI == EPI_F32 || EPI == EPI_PART;
      constexpr int ES = F32OUT ? 4 : 2;              // output element size
      constexpr int EP = (64 * ES + 16) / 4;          // row pitch in dwords (padded)
      constexpr int LPR = 64 * ES / 16;               // lanes per row: 8 (bf16) or 16 (f32)
      uint32_t* ep = (uint32_t*)(wave == 0 ? S0 : wave == 1 ? S1 : wave == 2 ? S2 : S3);
      [[maybe_unused]] uint2 gam[NI][4];
      if constexpr (EPI == EPI_BF16N) {
        // gamma of this lane's columns (four consecutive per group)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = n0 + wn * 64 + ni * 32 + 8 * gq + 4 * h;
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
          const int row = m0 + wm * (BM / 2) + mi * 32 + (lane & 31);
          if (h == 0 && row < M)
            g.ss[(int64_t)z * g.ss_bstride + (int64_t)row * (N >> 6) + (n0 >> 6) + wn] = ss;
        }
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int r = mi * 32 + (lane & 31), c = ni * 32 + 8 * gq + 4 * h;
            f32x4 v = {acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1], acc[mi][ni][4 * gq + 2],
                       acc[mi][ni][4 * gq + 3]};
            if constexpr (EPI == EPI_BF16N) {
              v[0] *= bf16_lo(gam[ni][gq].x);
              v[1] *= bf16_hi(gam[ni][gq].x);
              v[2] *= bf16_lo(gam[ni][gq].y);
              v[3] *= bf16_hi(gam[ni][gq].y);
            }
            if constexpr (F32OUT) {
              *(f32x4*)(ep + r * EP + c) = v;
            } else {
              *(uint2*)(ep + r * EP + c / 2) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
          }
      const int ch = lane % LPR;
      const int col = n0 + wn * 64 + ch * (16 / ES);
#pragma unroll
      for (int i = 0; i < (BM / 2) / (64 / LPR); ++i) {
        const int r = i * (64 / LPR) + lane / LPR;
        const u32x4 v = *(const u32x4*)(ep + r * EP + ch * 4);
        const int row = m0 + wm * (BM / 2) + r;
        if (row >= M || col >= N) continue;
        if constexpr (EPI == EPI_F32) {
          f32x4 o = __builtin_bit_cast(f32x4, v);
          if (row >= col && row < col + 4) o[row - col] += g.diag;
          *(f32x4*)((float*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col) = o;
        } else if constexpr (EPI == EPI_PART) {
          *(u32x4*)(g.part + (((int64_t)ks * batch + z) * M_max + row) * N + col) = v;
        } else {
          *(u32x4*)((uint16_t*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col) = v;
        }
      }
    }
  }  // tiles
}

// Host-side launch over a batch of `batch` problems (grid flattened for the
// XCD-aware tile order): one workgroup per CU (128 KB of LDS for BM = 128),
// capped by the tile count for the row bound and rounded up to whole XCDs.
// Requirements (checked by the callers): K % 256 == 0, N % 8 == 0 (bf16
// output) or N % 4 == 0 (fp32), 16-byte aligned rows, every operand's byte
// span below 2^31.
template <int BM, int EPI>
inline void gemm_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 127) / 128;
  const int tm = (g.M_max + BM - 1) / BM;
  const int64_t tiles = (int64_t)tn * tm * batch * (EPI == EPI_PART ? g.ksplit : 1);
  const int grid = persistent_grid(tiles);
  gemm_nt_kernel<BM, EPI><<<dim3(grid, 1), 256, 0, s>>>(g, tn, batch);
}

// Tile choice from the row bound: 64-row tiles for decode-sized batches,
// 128 otherwise.
template <int EPI>
inline void gemm_auto(const GemmArgs& g, int batch, hipStream_t s) {
  if (g.M_max <= 64) gemm_launch<64, EPI>(g, batch, s);
  else gemm_launch<128, EPI>(g, batch, s);
}

}  // namespace river
