// bf16 GEMM for large row counts with the reduction a multiple of 128:
// C[z] = A[z] . B[z]^T (both operands K-contiguous), fp32 accumulation,
// bf16 output (EPI_BF16), or EPI_CACHE (columns [0, nh) to the K cache and
// [nh, 2 nh) to the V cache at the slot of each row).
//
// Workgroup tile 256 x 256 as in gemm_big.h, but 4 waves, one per SIMD,
// each owning a 128 x 128 quadrant: 4 x 4 accumulators of 32x32 (256
// accumulator registers, held in the AGPRs), fed by
// v_mfma_f32_32x32x16_bf16, so each 16-byte fragment read from LDS feeds 4
// MFMAs.
//
// A stage is 64 wide in K: every global load of a wave covers 8 rows x 128
// contiguous bytes, whole 128-byte lines. With 64-byte row pieces (32-wide
// stages, the first version of this kernel) each line was requested from L2
// twice, once per half: measured on a 30704 x 5120 x 5120 product, 2.0e8
// L2 read requests against 1.0e8 now, and the texture address FIFO full 10x
// as often, which stalls the wave that issues the load and with it the
// MFMAs behind it in the in-order stream.
//
// Two pipelines over the 160 KB of LDS:
//  - K % 320 == 0: units of 32 KB, each the A rows or the B rows of one
//    stage, in a ring of 5: X(2t) = A(t), X(2t + 1) = B(t) in unit i % 5.
//    At the barrier of stage t - 1 the units of A(t - 1) and B(t - 1) free
//    up and take B(t + 1) and A(t + 2), so the A loads have two stages of
//    lead and the B loads one (measured 5% faster than two whole stages on
//    the 63472 x 5120 x 5120 x 48 map GEMM: 1275 against 1207 TFLOP/s).
//  - otherwise two stages of 64 KB: [A 0][A 1][B 0][B 1].
// The loads of a stage go out spread over the MFMAs of the stage before
// (one load per two MFMAs at most), as the address unit takes about 28
// cycles per 1 KB wave load.
//
// Every instruction of the main loop is placed by hand: a sub-step (slab j
// of the stage, K-half s) is 16 slots of one MFMA, then at most one LDS
// read (the next sub-step's fragments, in the order they are first used)
// and one global load, and a scheduling barrier. One workgroup barrier per
// stage, in the middle of its last sub-step: the next stage has landed and
// all reads of this one are done, so the rest of the sub-step reads the next
// stage's first fragments and starts loads into the freed space.
//
// A tile starts with the B rows of its first stage: their offsets need no
// row ids, so they go out while the row ids of the A rows (a gather) land.
// It ends through LDS: each wave writes its 128 x 128 block as bf16 into
// 32 KB of LDS and reads it back a row piece at a time, so that every store
// covers 4 rows x 256 contiguous bytes (where storing straight from the
// accumulators wrote 16-byte pieces of 32 rows per store). Measured on the
// same box, bit-identical: 30704 x 5120 x 5120 x 8 at 1288-1335 TFLOP/s
// against 1224-1290; on 63472 x 5120 x K x 8 the cost of a tile beyond its
// stages fell from about 13 to 10 µs (K from 320 to 5120).
//
// The MFMAs run in the same order on the same fragments as gemm_big.h
// (slab by slab, sub-step 0 then 1, K-chunk 2 h + s of the slab), so the
// results are bit-identical to it.
#pragma once

#include "gemm_big.h"

namespace river {

// waits for this wave's LDS reads, then the workgroup barrier (no wait on
// the global loads)
__device__ __forceinline__ void quad_lds_barrier() {
  constexpr int imm = 15 | (3 << 14) | (7 << 4) | (0 << 8);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-tile state of the 4-wave kernels: the tile walk, the load offsets,
// the fragment reads and the epilogue, shared by both pipelines.
template <int EPI>
struct QuadTile {
  static constexpr int BM = 256, BN = 256, MI = 4, NI = 4, AD = 8;
  struct Frag { bf16x8 a[MI], b[NI]; };

  const GemmArgs& g;
  int M, N, lane, wave, wm, wn, h;
  int z, m0, n0;
  const void* a_buf;
  const void* b_buf;
  int a_bytes, b_bytes, b_rowstep;
  uint32_t a_off[AD], b_off[2];
  int src[AD];                           // source rows of the A loads (row ids, then offsets())
  int pa[2][2], pb[2][2];                // read byte offsets within an operand block
  int er[MI], sl[MI];                    // EPI_CACHE: row ids, then slots

  __device__ __forceinline__ QuadTile(const GemmArgs& g_, int M_, int tile, int tiles_n, int tiles_m_act, int GM)
      : g(g_), M(M_), N(g_.N) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wm = wave >> 1;
    wn = wave & 1;
    h = lane >> 5;
    // persistent, XCD-aware tile walk with groups of GM row tiles (gemm.h)
    z = tile / (tiles_n * tiles_m_act);
    const int tz = tile - z * tiles_n * tiles_m_act;
    const int g0 = tz / (GM * tiles_n) * GM;
    const int gsz = tiles_m_act - g0 < GM ? tiles_m_act - g0 : GM;
    const int tg = tz - g0 * tiles_n;
    m0 = (g0 + tg % gsz) * BM;
    n0 = (tg / gsz) * BN;

    // EPI_CACHE: the row ids of this lane's four output rows go out now, the
    // slots once the first stage has landed (its wait covers these loads)
    if constexpr (EPI == EPI_CACHE) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = m0 + wm * 128 + mi * 32 + (lane & 31);
        const int rc = row < M ? row : M - 1;
        er[mi] = g.e_rows ? g.e_rows[rc] : rc;
      }
    }
    // load i of this thread fills chunk p = (i * 4 + wave) * 64 + lane of
    // an operand block: row p / 8 = 32 i + 8 wave + lane / 8, physical chunk
    // lane % 8 holding logical chunk (lane % 8) ^ swz(row); swz(row) depends
    // on i only through i % 2, so the B loads i and i + 2 differ by 64 rows
    // the row ids go out now; offsets() turns them into the A offsets
    a_buf = g.A + (int64_t)z * g.a_bstride;
    a_bytes = (int)(g.a_nrows * g.lda * 2);
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int t = m0 + i * 32 + wave * 8 + (lane >> 3);
      src[i] = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
    }
    b_buf = g.B + (int64_t)z * g.b_bstride;
    b_bytes = (int)(N * g.ldb * 2);
    b_rowstep = 64 * g.ldb * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = i * 32 + wave * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      // rows past N read zeros without a fetch; below N the offset lies
      // under b_bytes < 2^31 (32-bit arithmetic: a 64-bit form here made
      // the compiler wait for the row ids before the B loads)
      b_off[i] = n0 + r >= N ? BUF_OOB : (uint32_t)(n0 + r) * (uint32_t)(g.ldb * 2) + (uint32_t)(c * 16);
    }
    // read offsets: rows 32 apart differ in swz by 4, so row r + 32 m of
    // logical chunk ch sits at (r + 32 m) * 8 + (ch ^ swz(r) ^ 4 (m & 1));
    // with ch = 4 j + 2 h + s the chunk part is that of pa[s][j ^ (m & 1)]
    const int rowa = wm * 128 + (lane & 31), rowb = wn * 128 + (lane & 31);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jx = 0; jx < 2; ++jx) {
        pa[s][jx] = (rowa * 8 + ((4 * jx + 2 * h + s) ^ swz(rowa))) * 16;
        pb[s][jx] = (rowb * 8 + ((4 * jx + 2 * h + s) ^ swz(rowb))) * 16;
      }
  }

  // the A offsets from the row ids (waits for them)
  __device__ __forceinline__ void offsets() {
#pragma unroll
    for (int i = 0; i < AD; ++i) {
      const int r = i * 32 + wave * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const int t = m0 + r;
      int s = src[i];
      if (s < 0 || s >= g.a_nrows) s = 0;   // row 0 stands in; dropped
      // rows past the count read zeros without a fetch (not stored either);
      // s < a_nrows and a_nrows * lda * 2 < 2^31: exact in 32 bits
      a_off[i] = t >= M ? BUF_OOB : (uint32_t)s * (uint32_t)(g.lda * 2) + (uint32_t)(c * 16);
    }
  }

  // load x (0-7) of stage j's A rows, or of its B rows, into the 32 KB
  // block blk
  __device__ __forceinline__ void load_a(u32x4* blk, int j, int x) const {
    buf_lds<16>(a_buf, a_bytes, a_off[x], j * 128, blk + (x * 4 + wave) * 64);
  }
  __device__ __forceinline__ void load_b(u32x4* blk, int j, int x) const {
    buf_lds<16>(b_buf, b_bytes, b_off[x & 1], j * 128 + (x >> 1) * b_rowstep, blk + (x * 4 + wave) * 64);
  }

  // after the first stage has landed
  __device__ __forceinline__ void slots() {
    if constexpr (EPI == EPI_CACHE) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = m0 + wm * 128 + mi * 32 + (lane & 31);
        const bool ok = row < M && er[mi] >= 0 && er[mi] < g.e_nrows;
        sl[mi] = ok ? g.slot[er[mi]] : -1;
      }
    }
  }

  // read q of sub-step (j, s) from the operand blocks whose byte addresses
  // (offsets pa / pb plus the block base) are ab[s][.] and bb[s][.], in the
  // order of first use: a0, b0, b1, b2, b3, a1, a2, a3
  __device__ __forceinline__ static void read(const int (&ab)[2][2], const int (&bb)[2][2], int j, int s, int q,
                                              const u32x4* lds, Frag& f) {
    const int e = q == 0 ? 0 : (q <= 4 ? q + 3 : q - 4);
    const char* base = (const char*)lds;
    if (e < MI) f.a[e] = *(const bf16x8*)(base + ab[s][j ^ (e & 1)] + e * 4096);
    else f.b[e - MI] = *(const bf16x8*)(base + bb[s][j ^ (e & 1)] + (e - MI) * 4096);
  }

  // ---- epilogue through LDS. Lane l holds row mi * 32 + l % 32 of the
  // wave block and, per group gq, the four consecutive columns
  // ni * 32 + 8 gq + 4 (l / 32) + 0..3. The block goes as bf16 into the
  // wave's 32 KB of LDS (units 0-3; row r, 16-byte chunk c at
  // r * 16 + (c ^ (r & 15)): conflict-free both ways) and comes back as 4
  // rows x 16 chunks per read, each lane storing 16 bytes. EPI_CACHE: the
  // slots of the block's rows go to LDS as well (after the units, 512 bytes
  // per wave), since a lane stores other rows than it holds. Every wave
  // reads back only its own block, so one barrier (the last stage's reads
  // done) suffices; the next tile's first loads wait at its own barrier.
  __device__ __forceinline__ void store(const f32x16 (&acc)[MI][NI], u32x4* L) const {
    quad_lds_barrier();
    // the lane's byte offset in its row through a move the compiler cannot
    // hoist: otherwise it keeps the 16 chunk offsets of every lane live
    // across the tiles (and spills them)
    int lo;
    asm volatile("v_lshlrev_b32 %0, 3, %1" : "=v"(lo) : "v"(lane >> 5));
    const int x = lane & 15, r0 = lane & 31;
    char* W = (char*)(L + wave * 2048);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = mi * 32 + r0;                 // r & 15 == x
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int c = ni * 4 + gq;
          *(uint2*)(W + r * 256 + ((c ^ x) << 4) + lo) =
              uint2{pack_bf16x2(acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1]),
                    pack_bf16x2(acc[mi][ni][4 * gq + 2], acc[mi][ni][4 * gq + 3])};
        }
    }
    int* S = (int*)(L + 4 * 2048) + wave * 128;
    if constexpr (EPI == EPI_CACHE) {
      if (lane < 32) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) S[mi * 32 + lane] = sl[mi];
      }
    }
    const u32x4* R = L + wave * 2048;
    const int rb = m0 + wm * 128, cb = n0 + wn * 128;
    uint16_t* C = (uint16_t*)g.C + (int64_t)z * g.c_bstride;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) {
      const int r = i * 4 + (lane >> 4), c = lane & 15;
      const u32x4 v = R[r * 16 + (c ^ (r & 15))];
      const int row = rb + r, col = cb + c * 8;
      if (row >= M || col >= N) continue;
      if constexpr (EPI == EPI_CACHE) {
        const int slot = S[r];
        if (slot < 0 || slot >= g.n_slots) continue;
        const bool isv = col >= g.nh;
        // non-temporal: the cache rows are not read again here, so they
        // should not push the operand rows out of L2
        __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)(isv ? g.vc : g.kc) + (int64_t)z * g.cache_bstride +
                                                (int64_t)slot * g.nh + (isv ? col - g.nh : col)));
      } else {
        *(u32x4*)(C + (int64_t)row * g.ldc + col) = v;
      }
    }
  }
};

// slot k of a sub-step: MFMA of row block k / 4, column block k % 4; B
// first: lane l holds output row l % 32 and, per group of four registers,
// four consecutive columns
template <class Frag>
__device__ __forceinline__ void quad_mfma(f32x16 (&acc)[4][4], const Frag& f, int k) {
  acc[k >> 2][k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[k & 3], f.a[k >> 2], acc[k >> 2][k & 3], 0, 0, 0);
}

// byte offsets plus a block base, through a register move the compiler
// cannot hoist (otherwise it keeps one set per block live across the loop)
__device__ __forceinline__ void quad_addr(const int (&p)[2][2], int base, int (&o)[2][2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int jx = 0; jx < 2; ++jx) asm volatile("v_add_u32 %0, %1, %2" : "=v"(o[s][jx]) : "v"(p[s][jx]), "s"(base));
}

// groups of 8 row tiles: the 32 tiles an XCD runs together are 8 rows x 4
// columns of tiles (measured 5% faster than 4 x 8 on 30704 x 5120 x 5120)
constexpr int QUAD_GM = 8;

// ------------------------------------------------ K % 320: ring of 5 units
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_quad_kernel(GemmArgs g, int tiles_n, int batch) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_CACHE, "bf16 output");
  using T = QuadTile<EPI>;
  using Frag = typename T::Frag;
  __shared__ u32x4 L[5 * 2048];          // 5 units of 256 rows x 128 bytes

  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  const int tiles_m_act = (M + T::BM - 1) / T::BM;
  const int total = tiles_n * tiles_m_act * batch;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;
  const int KT = g.K / 64;               // stages, a multiple of 5

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
    if (tile != xcd * chunk + wg_in_xcd) quad_lds_barrier();   // the previous tile's reads done
    T q(g, M, tile, tiles_n, tiles_m_act, QUAD_GM);
    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

    // prologue: B(0) in unit 1 (while the row ids land), A(0) in 0, A(1)
    // in 2, B(1) loads 0-3 in 3; A(0) and B(0) landed
#pragma unroll
    for (int x = 0; x < 8; ++x) q.load_b(L + 2048, 0, x);
    __builtin_amdgcn_sched_barrier(0);
    q.offsets();
#pragma unroll
    for (int x = 0; x < 8; ++x) q.load_a(L, 0, x);
#pragma unroll
    for (int x = 0; x < 8; ++x) q.load_a(L + 2 * 2048, 1, x);
#pragma unroll
    for (int x = 0; x < 4; ++x) q.load_b(L + 3 * 2048, 1, x);
    wait_barrier<12, true>();
    q.slots();
    Frag f0, f1;
    {
      int ab[2][2], bb[2][2];
      quad_addr(q.pa, 0, ab);
      quad_addr(q.pb, 32768, bb);
#pragma unroll
      for (int r = 0; r < 8; ++r) T::read(ab, bb, 0, 0, r, L, f0);
    }

    // stage t (I = t % 5): A(t) in unit 2I % 5, B(t) in (2I + 1) % 5. B(t + 1)
    // loads 4-7 in sub-step 0 (0-3 went out after the previous barrier),
    // A(t + 2) in sub-steps 1 and 2; the barrier in the middle of sub-step 3
    // waits for all but A(t + 2); then the first reads of stage t + 1 and
    // B(t + 2) loads 0-3 into A(t)'s unit
    auto iter = [&](auto iv, int t, auto nb1, auto na2) {
      constexpr int I = decltype(iv)::value;
      constexpr int UA = (2 * I) % 5, UB = (2 * I + 1) % 5;
      constexpr int UA1 = (2 * I + 2) % 5, UB1 = (2 * I + 3) % 5, UA2 = (2 * I + 4) % 5;
      constexpr bool NB1 = decltype(nb1)::value;   // stage t + 1 exists
      constexpr bool NA2 = decltype(na2)::value;   // stage t + 2 exists
      int ab[2][2], bb[2][2];
      quad_addr(q.pa, UA * 32768, ab);
      quad_addr(q.pb, UB * 32768, bb);
#pragma unroll
      for (int k = 0; k < 16; ++k) {              // (0, 0) from f0; reads (0, 1)
        quad_mfma(acc, f0, k);
        if (k % 2 == 0) T::read(ab, bb, 0, 1, k / 2, L, f1);
        else if (NB1 && k / 2 < 4) q.load_b(L + UB1 * 2048, t + 1, 4 + k / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {              // (0, 1) from f1; reads (1, 0)
        quad_mfma(acc, f1, k);
        if (k % 2 == 0) T::read(ab, bb, 1, 0, k / 2, L, f0);
        else if (NA2 && k / 2 < 4) q.load_a(L + UA2 * 2048, t + 2, k / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {              // (1, 0) from f0; reads (1, 1)
        quad_mfma(acc, f0, k);
        if (k % 2 == 0) T::read(ab, bb, 1, 1, k / 2, L, f1);
        else if (NA2 && k / 2 < 4) q.load_a(L + UA2 * 2048, t + 2, 4 + k / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {               // (1, 1) from f1, first half
        quad_mfma(acc, f1, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NB1) {
        if constexpr (NA2) wait_barrier<8, true>();   // all but A(t + 2) landed
        else wait_barrier<0, true>();
        quad_addr(q.pa, UA1 * 32768, ab);
        quad_addr(q.pb, UB1 * 32768, bb);
      }
#pragma unroll
      for (int k = 8; k < 16; ++k) {              // second half; stage t + 1 reads
        quad_mfma(acc, f1, k);
        if (NB1) T::read(ab, bb, 0, 0, k - 8, L, f0);
        if (NA2 && k - 8 < 4) q.load_b(L + UA * 2048, t + 2, k - 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int t = 0;
    for (; t + 5 < KT; t += 5) {
      iter(I0{}, t, T_{}, T_{});
      iter(I1{}, t + 1, T_{}, T_{});
      iter(I2{}, t + 2, T_{}, T_{});
      iter(I3{}, t + 3, T_{}, T_{});
      iter(I4{}, t + 4, T_{}, T_{});
    }
    iter(I0{}, t, T_{}, T_{});
    iter(I1{}, t + 1, T_{}, T_{});
    iter(I2{}, t + 2, T_{}, T_{});
    iter(I3{}, t + 3, T_{}, F_{});
    iter(I4{}, t + 4, F_{}, F_{});
    q.store(acc, L);
  }
}

// ------------------------------------ K % 128: two stages of 64 KB
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_quad2_kernel(GemmArgs g, int tiles_n, int batch) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_CACHE, "bf16 output");
  using T = QuadTile<EPI>;
  using Frag = typename T::Frag;
  __shared__ u32x4 L[4 * 2048 + 128];    // [A 0][A 1][B 0][B 1], then the epilogue's slots

  int M = g.M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  const int tiles_m_act = (M + T::BM - 1) / T::BM;
  const int total = tiles_n * tiles_m_act * batch;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;
  const int KT = g.K / 64;               // stages, even

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
    if (tile != xcd * chunk + wg_in_xcd) quad_lds_barrier();
    T q(g, M, tile, tiles_n, tiles_m_act, QUAD_GM);
    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    // load x (0-15) of stage j into buffer S: 0-7 the A rows, 8-15 the B rows
    auto load = [&](int S, int j, int x) {
      if (x < 8) q.load_a(L + S * 2048, j, x);
      else q.load_b(L + 4096 + S * 2048, j, x - 8);
    };

    // B(0) first (while the row ids land), then A(0) and stage 1's loads 0-5
#pragma unroll
    for (int x = 8; x < 16; ++x) load(0, 0, x);
    __builtin_amdgcn_sched_barrier(0);
    q.offsets();
#pragma unroll
    for (int x = 0; x < 8; ++x) load(0, 0, x);
#pragma unroll
    for (int x = 0; x < 6; ++x) load(1, 1, x);
    wait_barrier<6, true>();               // stage 0 landed
    q.slots();
    Frag f0, f1;
    {
      int ab[2][2], bb[2][2];
      quad_addr(q.pa, 0, ab);
      quad_addr(q.pb, 65536, bb);
#pragma unroll
      for (int r = 0; r < 8; ++r) T::read(ab, bb, 0, 0, r, L, f0);
    }

    // stage t in buffer S: loads of stage t + 1 (other buffer) 0-5 after
    // the previous barrier, 6-11 in sub-step 0, 12-15 in sub-step 1; the
    // barrier in the middle of sub-step 3; then stage t + 1's first reads
    // and loads 0-5 of stage t + 2 into buffer S
    auto iter = [&](auto st, int t, auto nx, auto nx2) {
      constexpr int S = decltype(st)::value, O = 1 - S;
      constexpr bool NX = decltype(nx)::value;    // stage t + 1 exists
      constexpr bool NX2 = decltype(nx2)::value;  // stage t + 2 exists
      int ab[2][2], bb[2][2];
      quad_addr(q.pa, S * 32768, ab);
      quad_addr(q.pb, 65536 + S * 32768, bb);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        quad_mfma(acc, f0, k);
        if (k % 2 == 0) T::read(ab, bb, 0, 1, k / 2, L, f1);
        else if (NX && k / 2 < 6) load(O, t + 1, 6 + k / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        quad_mfma(acc, f1, k);
        if (k % 2 == 0) T::read(ab, bb, 1, 0, k / 2, L, f0);
        else if (NX && k / 2 < 4) load(O, t + 1, 12 + k / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        quad_mfma(acc, f0, k);
        if (k % 2 == 0) T::read(ab, bb, 1, 1, k / 2, L, f1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        quad_mfma(acc, f1, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NX) {
        wait_barrier<0, true>();              // stage t + 1 landed
        quad_addr(q.pa, O * 32768, ab);
        quad_addr(q.pb, 65536 + O * 32768, bb);
      }
#pragma unroll
      for (int k = 8; k < 16; ++k) {
        quad_mfma(acc, f1, k);
        if (NX) T::read(ab, bb, 0, 0, k - 8, L, f0);
        if (NX2 && k - 8 < 6) load(S, t + 2, k - 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int t = 0;
    for (; t + 3 < KT; t += 2) {
      iter(I0{}, t, T_{}, T_{});
      iter(I1{}, t + 1, T_{}, T_{});
    }
    iter(I0{}, t, T_{}, F_{});
    iter(I1{}, t + 1, F_{}, F_{});
    q.store(acc, L);
  }
}

// Launch: one workgroup of 4 waves per CU, capped by the tile count and
// rounded up to whole XCDs. quad_ok (the ring at K % 320 == 0), the other
// requirements as gemm_launch's.
template <int EPI>
inline void gemm_quad_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 255) / 256;
  const int tm = (g.M_max + 255) / 256;
  const int64_t tiles = (int64_t)tn * tm * batch;
  const int grid = persistent_grid(tiles);
  if (g.K % 320 == 0) gemm_quad_kernel<EPI><<<dim3(grid, 1), 256, 0, s>>>(g, tn, batch);
  else gemm_quad2_kernel<EPI><<<dim3(grid, 1), 256, 0, s>>>(g, tn, batch);
}

// The 4-wave kernels' conditions besides the launch's: K % 128 == 0, and
// the epilogue's 16-byte stores of 8 columns: N and the output row pitch (ldc,
// or nh for the cache) multiples of 8, the output 16-byte aligned.
template <int EPI>
inline bool quad_ok(const GemmArgs& g) {
  if (g.K % 128 || g.N % 8) return false;
  if constexpr (EPI == EPI_CACHE)
    return g.nh % 8 == 0 && g.cache_bstride % 8 == 0 && ((uintptr_t)g.kc | (uintptr_t)g.vc) % 16 == 0;
  else
    return g.ldc % 8 == 0 && g.c_bstride % 8 == 0 && (uintptr_t)g.C % 16 == 0;
}

// bf16-output GEMM: 256 x 256 tiles from 1024 rows on when they give at
// least one tile per CU (measured: 7782 rows of one 4096-wide layer, 496
// tiles, run 15% faster than on 128 x 128 tiles), the 128-row kernel
// otherwise. With the row count on the device the bound may be far above
// it (546 of 4096 rows in the GPT-2-shape step: 72 busy 256 x 256 tiles
// against 240 of 128 x 128; the whole fill measured 43 µs instead of 30),
// so there the big tiles need two per CU at the bound.
// The 256 x 256 tiles run on the 4-wave kernels of this file when K is a
// multiple of 128 and the output allows 16-byte stores (quad_ok; and the
// output has no norm epilogue), on gemm_big.h's 8-wave kernel otherwise (and
// always under gemm path 3).
template <int EPI>
inline void gemm_bf16_auto(const GemmArgs& g, int batch, hipStream_t s) {
  const int64_t big = (int64_t)((g.N + 255) / 256) * ((g.M_max + 255) / 256) * batch;
  const int path = river_host::gemm_path_override();
  const bool auto_big = g.M_dev ? big >= 2 * N_CU : (g.M_max >= 1024 && big >= N_CU);
  if (path == 2 || path == 3 || (path == 0 && auto_big)) {
    if constexpr (EPI == EPI_BF16) {
      if (path != 3 && quad_ok<EPI>(g)) {
        gemm_quad_launch<EPI>(g, batch, s);
        return;
      }
    }
    gemm_big_launch<EPI>(g, batch, s);
  } else {
    gemm_auto<EPI>(g, batch, s);
  }
}

// The projection on dequantised weights (EPI_CACHE), on the same choice of
// kernel by K and gemm path 3.
inline void gemm_cache_launch(const GemmArgs& g, int batch, hipStream_t s) {
  if (river_host::gemm_path_override() != 3 && quad_ok<EPI_CACHE>(g)) gemm_quad_launch<EPI_CACHE>(g, batch, s);
  else gemm_big_launch<EPI_CACHE>(g, batch, s);
}

}  // namespace river
