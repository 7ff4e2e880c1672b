// W4A16 GEMM on gfx950 MFMA with the K/V cache scatter as its epilogue:
//   C[z] = A[z] . deq(W[z])^T,   A bf16 [M][K], W int4 [N][K] (K-contiguous)
// where rows [0, nh) of W come from descriptor 0 (K projection) and
// [nh, 2 nh) from descriptor 1 (V projection), and
//   deq(q) = (q - zero) * scale = fma(q, scale, -zero * scale)
// per group of `group` input channels (a multiple of 64 here).
//
// Workgroup tile BM x 256, NW waves (8 by default: two per SIMD, which hide
// each other's latencies). Wave w owns the CW = 256 / NW output columns
// [CW w, CW w + CW) for all BM rows: BM/32 x CW/32 accumulators of 32x32 fed
// by v_mfma_f32_32x32x16_bf16. Only A goes through LDS as a tile (buffer
// loads straight into LDS, a 4-stage ring, three K-slabs ahead); every wave
// reads the same A fragments. The int4 weights of four slabs at a time
// (128 contiguous bytes of each column, so every wave load covers 8 columns
// x 128 bytes, whole lines) go into one of two LDS buffers, three slabs
// ahead of their first use; each lane takes from there the 16 bytes it needs
// per slab and dequantizes them in registers into the MFMA's B operand: no
// dequantized tile goes through LDS, and each weight is dequantized once per
// workgroup. (Loading each slab's 32 bytes per column separately touched 32
// lines per wave load; the L1 then stalled the address unit on 35 of its 52
// cycles per load.)
//
// The reduction index inside a 64-wide slab is permuted so that one 16-byte
// load per lane and column fragment covers the whole slab: in sub-step s
// (16 channels), lane half h = lane / 32 contracts channels
// 32 h + 8 s .. 32 h + 8 s + 7 (A chunk 4 h + s of its row, dword s of the
// lane's 16 weight bytes). The sum over the slab is the same sum.
//
// Per 64-slab and workgroup (BM = 128): 128 MFMAs of 32 cycles per SIMD
// (1024 cycles), 16 dequant8 per SIMD (about 23 vector instructions each,
// the binding cost: about 5 vector instructions hide behind one MFMA), 16 KB
// of A and 12 KB of weight staging written to LDS and 8 x 16 KB of A
// fragments read from it, 28 KB from L2.
//
// LAYER adds the rest of a layer's K/V path to the cache epilogue, on the
// fp32 accumulators: the input RMSNorm's row scale (from per-row partial
// sums of squares of the layer input), the K/V bias, and the rotary
// embedding of K. For the rotation each wave computes, instead of 32
// consecutive output channels, the 16 channels o0 .. o0 + 15 of one head and
// their partners o0 + hd/2 .. o0 + hd/2 + 15, so that both elements of every
// rotated pair sit in the same lane (accumulator groups gq and gq + 2).
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace river {

// The rest of a layer's K/V path on the fp32 accumulators of one wave
// (32 columns, MI fragments of 32 rows): lane l holds row mi * 32 + l % 32
// and, per group gq, the four consecutive wave columns 8 gq + 4 (l / 32) + i.
//   v = acc * r_row + bias[chan]                 (r_row = 1 without a norm)
//   K only, with rotation: for gq < 2 the pair (v[gq][i], v[gq + 2][i]) of
//   channels (o0 + j, hd/2 + o0 + j), j = 8 gq + 4 (l / 32) + i, turns by the
//   table angle of frequency o0 + j at the row's position.
// The row sums of squares are reduced by the whole workgroup into rsum (RG
// partial sums per row, added in a fixed order), so every wave of the
// workgroup calls this. A row whose position is outside the table gets
// slot -1 (not written).
template <int MI, int BM, int RG, int RCH, int RJ, typename Chan>
__device__ __forceinline__ void layer_epilogue(const GemmArgs& g, f32x16 (&acc)[MI][1], int z, int m0,
                                               int M_max, int K, int which, bool cols_ok, int tid,
                                               int lane, int h, bool rope, int o0, int half,
                                               float* rsum, Chan chan, const int (&ps)[RJ],
                                               int (&sl)[RJ]) {
  const bool rot = rope && which == 0 && cols_ok;
  // the rotary tables of this lane's rows and the bias of its 16 channels
  // go out first; the row sums' loads follow, and their first wait covers
  // every load, so they share one latency
  f32x4 c[MI][2], s[MI][2];
  if (rot) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rr = mi * 32;                    // rows mi * 32 + l % 32 sit in register rr / 64
      const int p = __shfl(ps[rr / 64], rr % 64 + (lane & 31), 64);
      const bool pok = p >= 0 && p < g.n_pos;
      const int64_t base = (int64_t)(pok ? p : 0) * half + o0 + 4 * h;
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        c[mi][gq] = *(const f32x4*)(g.rcos + base + 8 * gq);
        s[mi][gq] = *(const f32x4*)(g.rsin + base + 8 * gq);
      }
    }
  }
  uint2 bw[4];
  const uint16_t* bp = g.bias[which];
#pragma unroll
  for (int gq = 0; gq < 4; ++gq)
    bw[gq] = (bp && cols_ok) ? *(const uint2*)(bp + (int64_t)z * g.bias_bstride + chan(8 * gq + 4 * h))
                             : uint2{0u, 0u};
  // partial sums of the tile's rows: RG threads per row, RCH 16-byte chunks
  // per thread and round (one round for d <= 64 * 4 * RG * RCH)
  float a = 0.f;
  if (g.ss_in) {
    const int rr = tid % BM, rg = tid / BM;
    int t = m0 + rr;
    if (t >= M_max) t = 0;                       // rows past the count are never stored
    const f32x4* src = (const f32x4*)(g.ss_in + (int64_t)z * g.ss_in_bstride + (int64_t)t * g.ss_parts);
    const int nchk = g.ss_parts >> 2;
    for (int c0 = 0; c0 < nchk; c0 += RG * RCH) {
      f32x4 pv[RCH];
#pragma unroll
      for (int i = 0; i < RCH; ++i) {
        const int ci = c0 + rg + i * RG;
        pv[i] = ci < nchk ? src[ci] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < RCH; ++i) a += (pv[i][0] + pv[i][1]) + (pv[i][2] + pv[i][3]);
    }
  }
  float rs[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) rs[mi] = 1.0f;
  if (g.ss_in) {
    rsum[(tid / BM) * BM + tid % BM] = a;
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = mi * 32 + (lane & 31);
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < RG; ++q) t += rsum[q * BM + r];
      rs[mi] = rsqrtf(t / (float)K + g.norm_eps);
    }
  }
  float b[4][4];
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    b[gq][0] = bf16_lo(bw[gq].x); b[gq][1] = bf16_hi(bw[gq].x);
    b[gq][2] = bf16_lo(bw[gq].y); b[gq][3] = bf16_hi(bw[gq].y);
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    float v[4][4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[gq][i] = fmaf(acc[mi][0][4 * gq + i], rs[mi], b[gq][i]);
    if (rot) {
#pragma unroll
      for (int gq = 0; gq < 2; ++gq)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = v[gq][i], hi = v[gq + 2][i];
          v[gq][i] = lo * c[mi][gq][i] - hi * s[mi][gq][i];
          v[gq + 2][i] = lo * s[mi][gq][i] + hi * c[mi][gq][i];
        }
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mi][0][4 * gq + i] = v[gq][i];
  }
  // rows whose position is outside the tables are not written
  if (rope) {
#pragma unroll
    for (int j = 0; j < RJ; ++j)
      if (ps[j] < 0 || ps[j] >= g.n_pos) sl[j] = -1;
  }
}

// LDS of the int4 projection, in 16-byte units (the layout is described in
// w4_gemm_body)
template <int BM, int NW, bool LAYER, bool SZT>
constexpr int w4_lds_units() {
  return 4 * (BM * 8 + (SZT ? 0 : NW * 32)) + 2 * 256 * 8 + (SZT ? NW * 256 : 0) + (LAYER ? (64 * NW / BM) * BM / 4 : 0);
}

// The projection's work on LDS (w4_lds_units of it) given by the caller.
// gated: honour the gate of a split launch (w4deep.h).
template <int BM, int EPI, bool SZ_BF16, int NW, bool LAYER, bool SZT>
__device__ __forceinline__ void w4_gemm_body(const GemmArgs& g, int tiles_n, int batch, u32x4* LDS, bool gated) {
  static_assert(!LAYER || (NW == 8 && EPI == EPI_CACHE), "the layer epilogue takes 32-column waves");
  static_assert(!SZT || (NW == 8 && !LAYER), "tile-wide scales: 32-column waves, plain channels");
  static_assert(EPI == EPI_CACHE || EPI == EPI_PART, "cache or partial-sum output");
  constexpr int BN = 256;
  constexpr int MI = BM / 32;            // 32-row fragments (all rows of the tile)
  constexpr int NI = 8 / NW;             // 32-column fragments per wave (NW = 4 or 8 waves)
  constexpr int CW = 32 * NI;            // columns per wave
  constexpr int AD = BM * 8 / (64 * NW); // A DMA instructions per thread per slab
  constexpr int SZB = SZ_BF16 ? 2 : 4;
  // vector-memory instructions per thread per slab: A DMAs and (unless
  // SZT) one scale and one zero load; per four slabs WQD weight loads (8
  // columns x 128 bytes)
  constexpr int PER_SLAB = AD + (SZT ? 0 : 2);
  constexpr int WQD = CW / 8;
  // LDS, in 16-byte units:
  // - four pipeline stages: the A tile (BM x 64 bf16, swizzled) and, unless
  //   SZT, per wave the scale and zero words of 64 columns from its first
  //   one (2 x 64 x 4 B);
  // - the weights of four slabs: column c (0..255 of the tile) holds its
  //   128 bytes at chunks 8 c + (q ^ swz(c)), q = 2 (slab % 4) + half; two
  //   buffers;
  // - SZT: the scales and zeros of the whole tile, per wave 32 columns x
  //   up to 64 bytes each (the rows of its columns, as stored);
  // - LAYER: per-row sums of squares of the tile's input rows, reduced by
  //   the whole workgroup in the epilogue (RG threads per row, RCH 16-byte
  //   chunks of partial sums per thread and round).
  // The epilogue reuses the first NW x BM x (CW + 8) x 2 bytes.
  constexpr int ZOFF = BM * 8;
  constexpr int SSZ = ZOFF + (SZT ? 0 : NW * 32);
  constexpr int WQO = 4 * SSZ;
  constexpr int SZO = WQO + 2 * BN * 8;
  constexpr int SZW = 256;                        // per wave: scales [0, 128), zeros [128, 256)
  constexpr int RG = 64 * NW / BM;
  constexpr int RCH = 4;
  constexpr int RSO = SZO + (SZT ? NW * SZW : 0);
  static_assert(RSO + (LAYER ? RG * BM / 4 : 0) == w4_lds_units<BM, NW, LAYER, SZT>(), "the LDS layout");
  u32x4* const WQ = LDS + WQO;
  [[maybe_unused]] float* const RSUM = (float*)(LDS + RSO);

  // kernel arguments used below, read up front
  const int M_max = g.M_max, N = g.N, K = g.K, nh = g.nh, a_nrows = g.a_nrows;
  const int grp = g.group[0];            // equal for both descriptors here
  int M = M_max;
  if (g.M_dev) {
    const int md = *g.M_dev;
    M = md < 0 ? 0 : (md < M_max ? md : M_max);
  }
  if (gated && !gate_open(g, M)) return;   // the other launch's counts
  // with per-entry row counts every entry walks the row tiles of M_max and
  // skips those past its own count
  const int tiles_m_act = ((g.M_dev_z ? M_max : M) + BM - 1) / BM;
  const int ksplit = EPI == EPI_PART ? g.ksplit : 1;
  const int total = tiles_n * tiles_m_act * batch * ksplit;
  // persistent tiles, contiguous per XCD (see gemm_nt_kernel)
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;
  const int per_xcd = (gridDim.x + 7 - xcd) >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = (xcd + 1) * chunk < total ? (xcd + 1) * chunk : total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int KT = K / 64 / ksplit;        // slabs per tile, a multiple of 4 on this path
  const int slabs_per_group = grp >> 6;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto stage = [&](auto st) -> u32x4* { return LDS + decltype(st)::value * SSZ; };

  // MA: the row fragments the loop computes. A launch whose row count (on
  // the device) is at most 32 runs every tile on its first row fragment
  // only: a quarter of the MFMAs and A reads at BM = 128, the same
  // dequantisation; the other fragments stay zero, their rows are past the
  // count and not stored.
  auto run = [&](auto ma) {
    constexpr int MA = decltype(ma)::value;
    for (int tile = xcd * chunk + wg_in_xcd; tile < t_end; tile += per_xcd) {
      const int nt = tile % tiles_n;
      const int mt = (tile / tiles_n) % tiles_m_act;
      const int z = (tile / (tiles_n * tiles_m_act)) % batch;
      const int ks = tile / (tiles_n * tiles_m_act * batch);   // part of the reduction
      const int j0 = ks * KT;                                  // its first slab
      const int m0 = mt * BM, n0 = nt * BN;
      if (g.M_dev_z) {                                         // uniform
        const int mz = g.M_dev_z[z];
        M = mz < 0 ? 0 : (mz < M_max ? mz : M_max);
        if (m0 >= M) continue;
      }

      // A: DMA block b = i * 4 + wave covers LDS chunks [64 b, 64 b + 64);
      // lane l fills chunk p = 64 b + l = (row p / 8, physical chunk p % 8),
      // which holds logical chunk (p % 8) ^ swz(row) of that row.
      int a_src_row[AD];
#pragma unroll
      for (int i = 0; i < AD; ++i) {
        const int t = m0 + (((i * NW + wave) * 64 + lane) >> 3);
        a_src_row[i] = g.a_rows ? g.a_rows[t < M ? t : M - 1] : t;
      }
      // Operands come in through buffer loads straight into LDS: a uniform
      // resource (base and byte size of the buffer), a fixed 32-bit offset per
      // lane and a uniform offset per slab, so no per-slab address arithmetic
      // runs on the vector unit; a read past the stated size returns zeros.
      // A: row src of this tile's layer, 16-byte chunk c of the slab.
      const void* a_buf = g.A + (int64_t)z * g.a_bstride;
      const int a_bytes = (int)(a_nrows * g.lda * 2);
      uint32_t a_off[AD];
#pragma unroll
      for (int i = 0; i < AD; ++i) {
        const int p = (i * NW + wave) * 64 + lane;
        const int r = p >> 3, c = (p & 7) ^ swz(r);
        int src = a_src_row[i];
        if (src < 0 || src >= a_nrows) src = 0;   // row 0 stands in; dropped
        // rows past the count read zeros without a fetch (not stored either)
        a_off[i] = m0 + r >= M ? BUF_OOB : (uint32_t)(((int64_t)src * g.lda + c * 8) * 2);
      }
      // B: this wave's CW columns n0 + CW wave .. lie wholly in the K or the V
      // half (nh % 64 == 0): one resource per operand for the layer's
      // half. Column fragment ni, lane (l % 32, h): weight bytes [16 h, 16 h +
      // 16) of the 32-byte run of column 32 ni + l % 32 in each slab; scale and
      // zero: lane l loads the word of column l.
      const int wc0 = n0 + CW * wave;                         // uniform
      const int which = wc0 >= nh ? 1 : 0;
      const int hc0 = wc0 - which * nh;                       // first column inside the half
      const int64_t szs = which ? g.sz_bstride[1] : g.sz_bstride[0];
      const int gpr = K / grp;                                // groups per row
      const void* q_buf = (which ? g.q[1] : g.q[0]) + (int64_t)z * g.q_bstride;
      const int q_bytes = nh * (K / 2);
      const void* s_buf = (const char*)(which ? g.s[1] : g.s[0]) + z * szs * SZB;
      const void* z_buf = (const char*)(which ? g.zp[1] : g.zp[0]) + z * szs * SZB;
      const int sz_bytes = nh * gpr * SZB;
      // weight load m of this wave (per four slabs): wave columns 8 m + l / 8,
      // 16-byte chunk (l % 8) ^ swz(column) of their 128-byte run
      uint32_t wq_off[WQD];
      [[maybe_unused]] const uint32_t sz_off_plain = (uint32_t)((hc0 + lane) * gpr * SZB);
      // LAYER with rotary embedding: output channel of wave column j (0..31)
      // is hb + o0 + j for j < 16 and hb + hd/2 + o0 + j - 16 otherwise
      [[maybe_unused]] const bool rope = LAYER && g.pos != nullptr;
      [[maybe_unused]] int hb = 0, o0 = 0, half = 0;
      if constexpr (LAYER) {
        if (rope) {
          const int hd = g.head_dim;
          half = hd >> 1;
          hb = hc0 / hd * hd;
          o0 = ((hc0 - hb) >> 5) << 4;
        }
      }
      auto chan = [&](int j) -> int {    // channel (inside the K or V half) of wave column j
        if constexpr (LAYER) {
          if (rope) return hb + o0 + (j < 16 ? j : half + j - 16);
        }
        return hc0 + j;
      };
#pragma unroll
      for (int m = 0; m < WQD; ++m) {
        const int jc = 8 * m + (lane >> 3);                   // wave column
        const int cl = CW * wave + jc;                        // tile column
        wq_off[m] = (uint32_t)(chan(jc) * (K / 2) + ((lane & 7) ^ swz(cl)) * 16);
      }
      const uint32_t sz_off = LAYER ? (uint32_t)(chan(lane & 31) * gpr * SZB) : sz_off_plain;

      // the weights of slabs j .. j + 3 (j - j0 a multiple of 4) into buffer
      // ((j - j0) / 4) % 2
      auto issue_w = [&](int j) {
        u32x4* lw = WQ + (((j - j0) >> 2) & 1) * (BN * 8);
#pragma unroll
        for (int m = 0; m < WQD; ++m) buf_lds<16>(q_buf, q_bytes, wq_off[m], j * 32, lw + (wave * WQD + m) * 64);
      };
      // every load of K-slab j into LDS stage ST (and, for the first slab of
      // four, their weights after them)
      auto issue = [&](auto st, int j) {
        u32x4* la = stage(st);
#pragma unroll
        for (int i = 0; i < AD; ++i) buf_lds<16>(a_buf, a_bytes, a_off[i], j * 128, la + (i * NW + wave) * 64);
        if constexpr (!SZT) {
          const int gi = j / slabs_per_group;   // uniform
          // bf16 scale / zero: the aligned word holding group gi (rows hold an
          // even number of groups, so the word stays inside the row)
          const int go = (SZ_BF16 ? (gi & ~1) : gi) * SZB;
          uint32_t* lz = (uint32_t*)(la + ZOFF) + wave * 128;
          buf_lds<4>(s_buf, sz_bytes, sz_off, go, lz);
          buf_lds<4>(z_buf, sz_bytes, sz_off, go, lz + 64);
        }
        if (((j - j0) & 3) == 0) issue_w(j);   // uniform
      };
      // SZT: the scale and zero rows of the wave's 32 columns (contiguous,
      // 32 gpr SZB bytes each, at most 2 KB), two 1 KB loads per array whose
      // lanes past the end fetch nothing
      [[maybe_unused]] auto issue_sz = [&]() {
        u32x4* lw = LDS + SZO + wave * SZW;
        const int nchk = 32 * gpr * SZB / 16;
        const uint32_t base = (uint32_t)(hc0 * gpr * SZB);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int c = r * 64 + lane;
          const uint32_t off = c < nchk ? base + c * 16 : BUF_OOB;
          buf_lds<16>(s_buf, sz_bytes, off, 0, lw + r * 64);
          buf_lds<16>(z_buf, sz_bytes, off, 0, lw + 128 + r * 64);
        }
      };
      // this lane's weights of slab j (held in stage la) from LDS
      struct BRegs { u32x4 q[NI]; uint32_t s[NI], zz[NI]; };
      auto fetch = [&](const u32x4* la, int j, BRegs& b) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int cl = CW * wave + 32 * ni + (lane & 31);
          const int q = 2 * ((j - j0) & 3) + h;
          b.q[ni] = WQ[(((j - j0) >> 2) & 1) * (BN * 8) + cl * 8 + (q ^ swz(cl))];
          if constexpr (SZT) {
            // group j / slabs_per_group of column l % 32 in the wave's rows
            const int e = (lane & 31) * gpr + j / slabs_per_group;
            const char* lw = (const char*)(LDS + SZO + wave * SZW);
            if constexpr (SZ_BF16) {
              b.s[ni] = ((const uint16_t*)lw)[e];
              b.zz[ni] = ((const uint16_t*)(lw + 2048))[e];
            } else {
              b.s[ni] = ((const uint32_t*)lw)[e];
              b.zz[ni] = ((const uint32_t*)(lw + 2048))[e];
            }
          } else {
            const uint32_t* lz = (const uint32_t*)(la + ZOFF) + wave * 128;
            const int sh = SZ_BF16 ? ((j / slabs_per_group) & 1) * 16 : 0;
            const uint32_t sw = lz[ni * 32 + (lane & 31)];
            const uint32_t zw = lz[64 + ni * 32 + (lane & 31)];
            b.s[ni] = SZ_BF16 ? (sw >> sh) & 0xFFFFu : sw;
            b.zz[ni] = SZ_BF16 ? (zw >> sh) & 0xFFFFu : zw;
          }
        }
      };
      struct SC { float s[NI], c[NI]; };
      auto scales = [&](const BRegs& b) {
        SC r;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          r.s[ni] = SZ_BF16 ? __uint_as_float(b.s[ni] << 16) : __uint_as_float(b.s[ni]);
          const float ze = SZ_BF16 ? __uint_as_float(b.zz[ni] << 16) : __uint_as_float(b.zz[ni]);
          r.c[ni] = -ze * r.s[ni];
        }
        return r;
      };
      // the A fragments (from LDS) and dequantized B fragments of sub-step s
      struct Frag { bf16x8 a[MI], b[NI]; };
      auto frag = [&](const u32x4* la, const BRegs& b, const SC& sc, int s, Frag& f) {
        const int ch = 4 * h + s;
#pragma unroll
        for (int mi = 0; mi < MA; ++mi) {
          const int r = mi * 32 + (lane & 31);
          f.a[mi] = __builtin_bit_cast(bf16x8, la[r * 8 + (ch ^ swz(r))]);
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          uint32_t o[4];
          dequant8(b.q[ni][s], sc.s[ni], sc.c[ni], o);
          u32x4 v;
          v[0] = o[0]; v[1] = o[1]; v[2] = o[2]; v[3] = o[3];
          f.b[ni] = __builtin_bit_cast(bf16x8, v);
        }
      };

      f32x16 acc[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
      auto mfma = [&](const Frag& f) {
#pragma unroll
        for (int mi = 0; mi < MA; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
      };

      // Pipeline. Slab kt lives in LDS stage kt % 4 and register set kt % 4.
      // The barrier for slab kt + 1 sits before the last sub-step of slab kt,
      // so the first fragments of slab kt + 1 are read and dequantized while
      // the last MFMAs of slab kt run; after it, the stage of slab kt is free
      // and slab kt + 4 is issued into it. The last four slabs issue nothing
      // and wait for exactly what is still outstanding.
      if (tile != xcd * chunk + wg_in_xcd) {
        // every wave is done with the previous tile's stages
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      // cache slots of the tile's rows for the epilogue: lane l looks up rows
      // m0 + 64 j + l. The e_rows loads go out before the first slab's (so the
      // first wait covers them), the slot loads right after it.
      constexpr int RJ = BM / 64;
      [[maybe_unused]] int er[RJ], sl[RJ], ps[RJ];
      if constexpr (EPI == EPI_CACHE) {
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
          const int row = m0 + 64 * j + lane;
          const int rc = row < M ? row : M - 1;
          er[j] = g.e_rows ? g.e_rows[rc] : rc;
        }
      }
      if constexpr (SZT) issue_sz();         // before slab 0's loads: its wait covers them
      issue(I0{}, j0);
      issue(I1{}, j0 + 1);
      issue(I2{}, j0 + 2);
      wait_barrier<2 * PER_SLAB, true>();   // slab 0 landed
      if constexpr (EPI == EPI_CACHE) {
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
          const bool ok = m0 + 64 * j + lane < M && er[j] >= 0 && er[j] < g.e_nrows;
          sl[j] = ok ? g.slot[er[j]] : -1;          // range-checked where it is used
          if constexpr (LAYER) ps[j] = (ok && rope) ? g.pos[er[j]] : 0;
        }
      }
      Frag f0, f1;
      BRegs bA, bB;
      fetch(stage(I0{}), j0, bA);
      SC sc = scales(bA);
      frag(stage(I0{}), bA, sc, 0, f0);

      // Pipeline. Slab kt lives in LDS stage kt % 4. Iteration kt issues slab
      // kt + 3 into the stage of slab kt - 1 (free since the previous barrier),
      // spread between the MFMAs of sub-steps 0..2, so that no wave stalls on
      // a burst of loads; the barrier for slab kt + 1 sits before the last
      // sub-step, whose MFMAs then cover the fetch and dequantization of the
      // first fragments of slab kt + 1. W = loads allowed outstanding at the
      // barrier (those of the slabs after kt + 1); ISSUE = slab kt + 3 exists.
      auto iter = [&](auto st, BRegs& cur, BRegs& nxt, int kt, auto w, auto issue_next) {
        constexpr int ST = decltype(st)::value;
        using NX = std::integral_constant<int, (ST + 1) & 3>;
        using PV = std::integral_constant<int, (ST + 3) & 3>;
        constexpr bool ISS = decltype(issue_next)::value;
        if constexpr (ISS) issue(PV{}, j0 + kt + 3);
        frag(stage(st), cur, sc, 1, f1);
        mfma(f0);
        frag(stage(st), cur, sc, 2, f0);
        mfma(f1);
        frag(stage(st), cur, sc, 3, f1);
        mfma(f0);
        interleave<3, MA * NI, MA, ISS ? PER_SLAB : 0>();
        wait_barrier<decltype(w)::value, true>();   // slab kt + 1 landed
        fetch(stage(NX{}), j0 + kt + 1, nxt);      // (spare reads after the last slab)
        sc = scales(nxt);
        frag(stage(NX{}), nxt, sc, 0, f0);
        mfma(f1);
        interleave<1, MA * NI, MA + 3 * NI, 0>();
      };
      // at the barrier of slab kt + 1 the loads of slabs kt + 2 and kt + 3
      // may be outstanding, with the weights issued after slab kt + 4 m's
      using W2 = std::integral_constant<int, 2 * PER_SLAB>;
      using W2Q = std::integral_constant<int, 2 * PER_SLAB + WQD>;
      using W1 = std::integral_constant<int, PER_SLAB>;
      using W0 = std::integral_constant<int, 0>;
      using T_ = std::true_type;
      using F_ = std::false_type;
      int kt = 0;
      for (; kt + 4 < KT; kt += 4) {       // every slab here issues slab kt + 3
        iter(I0{}, bA, bB, kt, W2{}, T_{});
        iter(I1{}, bB, bA, kt + 1, W2Q{}, T_{});
        iter(I2{}, bA, bB, kt + 2, W2Q{}, T_{});
        iter(I3{}, bB, bA, kt + 3, W2{}, T_{});
      }
      // last four slabs: only the first still has a slab to issue
      iter(I0{}, bA, bB, kt, W2{}, T_{});
      iter(I1{}, bB, bA, kt + 1, W1{}, F_{});
      iter(I2{}, bA, bB, kt + 2, W0{}, F_{});
      iter(I3{}, bB, bA, kt + 3, W0{}, F_{});

      if constexpr (EPI == EPI_PART) {
        // fp32 partial sums straight from the accumulators: lane l holds row
        // mi * 32 + l % 32 and the four columns 8 gq + 4 (l / 32) + 0..3
        float* P = g.part + ((int64_t)ks * batch + z) * M_max * N;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int r = m0 + mi * 32 + (lane & 31);
              const int c = n0 + CW * wave + ni * 32 + 8 * gq + 4 * h;
              if (r < M && c < N)
                *(f32x4*)(P + (int64_t)r * N + c) = f32x4{acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1],
                                                          acc[mi][ni][4 * gq + 2], acc[mi][ni][4 * gq + 3]};
            }
        continue;                                  // next tile
      }

      // ---- epilogue. The transposed 32x32 accumulator gives lane l output
      // row l % 32 of fragment mi and, for gq = 0..3, the four consecutive
      // columns 8 gq + 4 (l / 32) + 0..3 of fragment ni. Each wave first writes
      // its BM x CW block as bf16 into LDS (its own region at the start of the
      // array, free now: past the last slab's barrier the other waves only
      // make spare reads of stage 0, the weights and the scales, whose values
      // are never used), then stores it row by row: LPR lanes x 16 bytes cover
      // one row's CW columns, 64 / LPR rows per store.
      {
        constexpr int EP = CW + 8;                  // row pitch in bf16 (padded)
        constexpr int LPR = CW / 8;                 // lanes per row
        constexpr int RPI = 64 / LPR;               // rows per store instruction
        static_assert(NW * BM * EP * 2 <= RSO * 16, "the epilogue's blocks fit before the row sums");
        uint16_t* ep = (uint16_t*)LDS + wave * BM * EP;
        // (a wave whose columns lie past N reads no bias; its stores are dropped)
        if constexpr (LAYER)
          layer_epilogue<MI, BM, RG, RCH>(g, acc, z, m0, M_max, K, which, wc0 < N, tid, lane, h, rope, o0,
                                          half, RSUM, chan, ps, sl);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int r = mi * 32 + (lane & 31), c = ni * 32 + 8 * gq + 4 * h;
              *(uint2*)(ep + r * EP + c) = uint2{pack_bf16x2(acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1]),
                                                 pack_bf16x2(acc[mi][ni][4 * gq + 2], acc[mi][ni][4 * gq + 3])};
            }
        const int ch = lane % LPR;
        int col = n0 + CW * wave + 8 * ch;         // 8 columns, all in K or all in V
        const bool col_ok = col < N;
        const bool isv = col >= nh;
        if constexpr (LAYER) col = (isv ? nh : 0) + chan(8 * ch);
#pragma unroll
        for (int i = 0; i < BM / RPI; ++i) {
          const int r = i * RPI + lane / LPR;
          const u32x4 v = *(const u32x4*)(ep + r * EP + 8 * ch);
          if constexpr (EPI == EPI_CACHE) {
            // slot of row r: looked up by lane r % 64 in its register r / 64
            const int sr = __shfl(sl[(i * RPI) / 64], (i * RPI) % 64 + lane / LPR, 64);
            if (sr < 0 || sr >= g.n_slots || !col_ok) continue;
            uint16_t* dst = (uint16_t*)(isv ? g.vc : g.kc);
            *(u32x4*)(dst + (int64_t)z * g.cache_bstride + (int64_t)sr * nh + (isv ? col - nh : col)) = v;
          } else {
            const int row = m0 + r;
            if (row >= M || !col_ok) continue;
            *(u32x4*)((uint16_t*)g.C + (int64_t)z * g.c_bstride + (int64_t)row * g.ldc + col) = v;
          }
        }
      }
    }  // tiles
  };
  if constexpr (MI > 1 && !LAYER) {   // (the layer epilogue's registers leave no room for two loops)
    if (!g.M_dev_z && M <= 32) run(std::integral_constant<int, 1>{});   // uniform
    else run(std::integral_constant<int, MI>{});
  } else {
    run(std::integral_constant<int, MI>{});
  }
}

template <int BM, int EPI, bool SZ_BF16, int NW, bool LAYER, bool SZT>
__global__ __launch_bounds__(64 * NW) void w4_gemm_kernel(GemmArgs g, int tiles_n, int batch) {
  __shared__ u32x4 LDS[w4_lds_units<BM, NW, LAYER, SZT>()];
  w4_gemm_body<BM, EPI, SZ_BF16, NW, LAYER, SZT>(g, tiles_n, batch, LDS, true);
}

// Launch over a batch of `batch` layers: one workgroup per CU (144 KB of
// LDS for BM = 128), capped by the tile count and rounded to whole XCDs.
// W4_WAVES: 4 waves (64 columns each, one per SIMD) or 8 (32 columns each,
// two per SIMD, which hide each other's latencies).
constexpr int W4_WAVES = 8;
// The parts of a split reduction added in order, rounded to bf16 and
// written to each row's cache slot (the EPI_CACHE epilogue's addressing):
// one thread per 8 columns of a row.
__global__ __launch_bounds__(256) void w4_part_finish_kernel(GemmArgs g, int batch) {
  const int N = g.N, nh = g.nh;
  const int per = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int p = (int)(idx % per);
  const int t = (int)((idx / per) % g.M_max);
  const int z = (int)(idx / ((int64_t)per * g.M_max));
  if (z >= batch) return;
  int M = g.M_max;
  const int32_t* md_p = g.M_dev_z ? g.M_dev_z + z : g.M_dev;
  if (md_p) {
    const int md = *md_p;
    M = md < 0 ? 0 : (md < g.M_max ? md : g.M_max);
  }
  if (!g.M_dev_z && !gate_open(g, M)) return;
  if (t >= M) return;
  const int e = g.e_rows ? g.e_rows[t] : t;
  if (e < 0 || e >= g.e_nrows) return;
  const int sl = g.slot[e];
  if (sl < 0 || sl >= g.n_slots) return;
  const int col = 8 * p;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < g.ksplit; ++ks) {
    const float* src = g.part + (((int64_t)ks * batch + z) * g.M_max + t) * N + col;
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

// The scales and zeros of a whole tile fit its LDS (each wave's 32 columns
// hold at most 64 bytes of them per array) and sit at 16-byte boundaries:
// then they are loaded once per tile, in whole lines, instead of a 4-byte
// word per column and slab, each load touching 32 lines (two vector-memory
// instructions fewer per thread and slab; at the 8B decode shape, 13 rows x
// 21 blocks, 50.0-50.7 us against 51.6, bit-identical).
inline bool w4_tile_scales_ok(const GemmArgs& g) {
  const int szb = g.sz_bf16[0] ? 2 : 4;
  const int gpr = g.K / g.group[0];
  bool ok = W4_WAVES == 8 && gpr * szb <= 64;
  for (int i = 0; i < 2; ++i)
    ok = ok && ((uintptr_t)g.s[i] % 16) == 0 && ((uintptr_t)g.zp[i] % 16) == 0 && (g.sz_bstride[i] * szb) % 16 == 0;
  return ok;
}

template <int BM, int EPI, bool LAYER>
inline void w4_gemm_launch(const GemmArgs& g, int batch, hipStream_t s) {
  const int tn = (g.N + 255) / 256;
  const int tm = (g.M_max + BM - 1) / BM;
  const int64_t tiles = (int64_t)tn * tm * batch * (EPI == EPI_PART ? g.ksplit : 1);
  const int grid = persistent_grid(tiles);
  // (not for the parts of a split: a part uses only its share of the rows)
  if constexpr (!LAYER && EPI != EPI_PART) {
    if (w4_tile_scales_ok(g)) {
      if (g.sz_bf16[0]) w4_gemm_kernel<BM, EPI, true, W4_WAVES, false, true><<<grid, 64 * W4_WAVES, 0, s>>>(g, tn, batch);
      else w4_gemm_kernel<BM, EPI, false, W4_WAVES, false, true><<<grid, 64 * W4_WAVES, 0, s>>>(g, tn, batch);
      return;
    }
  }
  if (g.sz_bf16[0]) w4_gemm_kernel<BM, EPI, true, W4_WAVES, LAYER, false><<<grid, 64 * W4_WAVES, 0, s>>>(g, tn, batch);
  else w4_gemm_kernel<BM, EPI, false, W4_WAVES, LAYER, false><<<grid, 64 * W4_WAVES, 0, s>>>(g, tn, batch);
}

template <int EPI, bool LAYER = false>
inline void w4_gemm_auto(const GemmArgs& g, int batch, hipStream_t s) {
  if (g.M_max <= 64) w4_gemm_launch<64, EPI, LAYER>(g, batch, s);
  else w4_gemm_launch<128, EPI, LAYER>(g, batch, s);
}

}  // namespace river
