// compact: stable split of a batch by its exit mask, row gather of the
// continuing tokens and scatter of the exited ones.
//
// TIDE, 模块4 (融合 CUDA 内核): "Batch Compact" separates continuing from
// exiting tokens, with a ballot for small batches and a prefix-sum scatter
// for large ones; "Exit Scatter" copies exited hidden states back to their
// original rows of an output buffer.
//
// Default for n <= 65536: one fused launch (indices and rows, see below).
// Otherwise, or when forced for testing, index kernels (one launch, or two
// for very large batches) then a row kernel:
//   n <= 64      one wave: ballot + lane-rank (mbcnt)
//   n <= 16384   one workgroup of 1024 threads: per-thread counts, wave
//                prefix scans, scan of the 16 wave totals in LDS
//   larger       per-chunk counts, then every chunk sums the counts of the
//                chunks before it (deterministic, no atomics)
// Row kernel: one pass over the destination rows; reads the counts from
// device memory, so nothing waits on the host.
#include "common.h"

namespace river {

constexpr int CB_THREADS = 1024;
constexpr int GRID_ITEMS = 16;                  // items per thread, grid path
constexpr int GRID_CHUNK = 256 * GRID_ITEMS;    // items per workgroup, grid path

struct CompactIdx {
  int n;
  const uint8_t* mask;
  const int32_t* row_ids;
  int32_t* cont_idx;
  int32_t* exit_idx;
  int32_t* counts;
  int32_t* row_ids_cont;
};

__device__ __forceinline__ void emit(const CompactIdx& a, int i, bool ex, int exit_rank) {
  if (ex) {
    a.exit_idx[exit_rank] = i;
  } else {
    const int cr = i - exit_rank;
    a.cont_idx[cr] = i;
    if (a.row_ids_cont) a.row_ids_cont[cr] = a.row_ids ? a.row_ids[i] : i;
  }
}

__global__ __launch_bounds__(64) void compact_wave_kernel(CompactIdx a) {
  const int l = threadIdx.x;
  const bool ex = l < a.n && a.mask[l] != 0;
  const uint64_t bits = __ballot(ex);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
  if (l < a.n) emit(a, l, ex, rank);
  if (l == 0) {
    const int ne = __popcll(bits);
    a.counts[0] = a.n - ne;
    a.counts[1] = ne;
  }
}

// exclusive prefix over the threads of a workgroup (blockDim <= 1024);
// returns the exclusive prefix of v and the workgroup total
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = s_wave[w];
      s_wave[w] = run;
      run += t;
    }
    s_wave[nw] = run;
  }
  __syncthreads();
  *total = s_wave[nw];
  return s_wave[wave] + inc - v;
}

// One workgroup; thread t owns items [t*items, (t+1)*items).
__global__ __launch_bounds__(CB_THREADS) void compact_block_kernel(CompactIdx a, int items) {
  __shared__ int s_wave[CB_THREADS / 64 + 1];
  const int i0 = threadIdx.x * items;
  const int i1 = min(a.n, i0 + items);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += a.mask[i] != 0;
  int total;
  int er = block_exclusive_scan(cnt, s_wave, &total);
  for (int i = i0; i < i1; ++i) {
    const bool ex = a.mask[i] != 0;
    emit(a, i, ex, er);
    er += ex;
  }
  if (threadIdx.x == 0) {
    a.counts[0] = a.n - total;
    a.counts[1] = total;
  }
}

// grid path, pass 1: exits per chunk of GRID_CHUNK items
__global__ __launch_bounds__(256) void compact_grid_count_kernel(CompactIdx a, int32_t* chunk_cnt) {
  __shared__ int s_wave[5];
  const int c0 = blockIdx.x * GRID_CHUNK;
  const int i0 = c0 + threadIdx.x * GRID_ITEMS;
  const int i1 = min(a.n, i0 + GRID_ITEMS);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += a.mask[i] != 0;
  int total;
  block_exclusive_scan(cnt, s_wave, &total);
  if (threadIdx.x == 0) chunk_cnt[blockIdx.x] = total;
}

// grid path, pass 2: offset = exits in the chunks before this one
__global__ __launch_bounds__(256) void compact_grid_write_kernel(CompactIdx a, const int32_t* chunk_cnt,
                                                                 int n_chunks) {
  __shared__ int s_wave[5];
  __shared__ int s_base;
  if (threadIdx.x == 0) {
    int base = 0;
    for (int c = 0; c < (int)blockIdx.x; ++c) base += chunk_cnt[c];
    s_base = base;
  }
  const int c0 = blockIdx.x * GRID_CHUNK;
  const int i0 = c0 + threadIdx.x * GRID_ITEMS;
  const int i1 = min(a.n, i0 + GRID_ITEMS);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += a.mask[i] != 0;
  int total;
  int er = block_exclusive_scan(cnt, s_wave, &total);   // contains a barrier: s_base visible
  er += s_base;
  for (int i = i0; i < i1; ++i) {
    const bool ex = a.mask[i] != 0;
    emit(a, i, ex, er);
    er += ex;
  }
  if (threadIdx.x == 0 && (int)blockIdx.x == n_chunks - 1) {
    const int ne = s_base + total;
    a.counts[0] = a.n - ne;
    a.counts[1] = ne;
  }
}

// nonzero bytes of a dword (the high bit of each byte of the result is set
// iff that byte is nonzero)
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return __popc((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u);
}

// ---------------------------------------------------------- fused path
// One launch for indices and rows, n <= FUSED_MAX: workgroup c owns the
// FCH tokens [FCH c, FCH c + FCH). Every wave reads the chunk's mask bytes
// and ballots them. The rows to copy (exits when `out` is set, continuing
// rows when `h_cont` is) are dealt round-robin to the four waves, and each
// wave issues the loads of all its rows before the count of the exits
// before the chunk (16-byte reads of the mask prefix, issued first) is
// reduced: a row costs one memory latency for its loads and one for its
// stores, whatever the number of rows per wave. The workgroup then writes
// both index lists and stores the rows: an exited row to out[row_ids[i]],
// a continuing one to h_cont[i - (exits before i)]. Rows longer than
// 64 KP 16-byte pieces per lane go in several passes.
constexpr int FUSED_MAX = 65536;

template <int FCH>
__global__ __launch_bounds__(256) void compact_fused_kernel(CompactIdx a, const char* h, int64_t ld_h,
                                                            int row_bytes, char* h_cont, int64_t ld_cont,
                                                            char* out, int64_t ld_out, int64_t n_out_rows) {
  constexpr int RW = FCH / 4;                     // row slots per wave
  constexpr int KP = FCH <= 16 ? 2 : 1;           // 16-byte pieces per lane, row and pass
  __shared__ int s_part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * FCH;
  const int n = a.n;
  const int chunks = row_bytes >> 4;
  // this chunk's tokens: lane l < FCH of every wave holds token c0 + l; the
  // mask byte and the row id load together (the id is used only for exits)
  const int i_own = c0 + lane;
  const bool in = lane < FCH && i_own < n;
  const bool ex_own = in && a.mask[i_own] != 0;
  const int rid_own = (out && in) ? (a.row_ids ? a.row_ids[i_own] : i_own) : -1;
  const uint64_t bits = __ballot(ex_own);         // exits of the chunk
  const uint64_t valid = __ballot(in);            // tokens of the chunk
  const uint64_t need = (h && out ? bits : 0ull) | (h && h_cont ? valid & ~bits : 0ull);
  // slot j of this wave: the row of rank 4 j + wave among the rows to copy
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(need >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)need, 0u));
  const bool mine = lane < FCH && ((need >> lane) & 1);
  int row[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    const uint64_t b = __ballot(mine && rank == 4 * j + wave);
    row[j] = b ? __builtin_ctzll(b) : -1;
  }
  const bool any = row[0] >= 0;                   // uniform
  // every load below is unconditional: a free slot's buffer has no bytes,
  // and a piece past the end of a buffer reads zeros without a memory access
  const char* src[RW];
  int sbytes[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    src[j] = h + (int64_t)(c0 + (row[j] >= 0 ? row[j] : 0)) * ld_h;
    sbytes[j] = row[j] >= 0 ? row_bytes : 0;
  }
  u32x4 v[RW][KP];
#pragma unroll
  for (int j = 0; j < RW; ++j)
#pragma unroll
    for (int k = 0; k < KP; ++k) v[j][k] = buf_load16(src[j], sbytes[j], (uint32_t)(lane + 64 * k) * 16);
  // exits in [0, c0): its first 16-byte pieces load with the rows, the rest
  // (prefixes over 16 KB) in a loop
  constexpr int PF = 4;
  u32x4 pm[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) pm[k] = buf_load16(a.mask, c0, (uint32_t)(tid + 256 * k) * 16);
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < PF; ++k)
    cnt += nonzero_bytes(pm[k][0]) + nonzero_bytes(pm[k][1]) + nonzero_bytes(pm[k][2]) + nonzero_bytes(pm[k][3]);
  const u32x4* m16 = (const u32x4*)a.mask;
  for (int q = tid + 256 * PF; q < (c0 >> 4); q += 256) {
    const u32x4 w = m16[q];
    cnt += nonzero_bytes(w[0]) + nonzero_bytes(w[1]) + nonzero_bytes(w[2]) + nonzero_bytes(w[3]);
  }
  cnt = (int)row_sum<16>((float)cnt);       // exact: counts stay far below 2^24
  cnt += __shfl_xor(cnt, 16, WAVE);
  cnt += __shfl_xor(cnt, 32, WAVE);
  if (lane == 0) s_part[wave] = cnt;
  __syncthreads();
  const int base = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  if (wave == 0) {
    const int rk = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
    if (in) emit(a, i_own, ex_own, rk);
    if (c0 + FCH >= n && lane == 0) {          // the last chunk knows the total
      const int ne = base + __popcll(bits);
      a.counts[0] = n - ne;
      a.counts[1] = ne;
    }
  }
  if (!any) return;
  // destination of each slot's row (null: nothing to store)
  u32x4* dst[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    dst[j] = nullptr;
    const int t = row[j];
    if (t < 0) continue;
    if ((bits >> t) & 1) {
      const int rid = __builtin_amdgcn_readlane(rid_own, t);
      if (rid >= 0 && rid < n_out_rows) dst[j] = (u32x4*)(out + (int64_t)rid * ld_out);
    } else {
      const int er = base + __popcll(bits & ((1ull << t) - 1));
      dst[j] = (u32x4*)(h_cont + (int64_t)(c0 + t - er) * ld_cont);
    }
  }
  for (int p0 = 0;;) {
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int c = p0 + lane + 64 * k;
        if (dst[j] && c < chunks) dst[j][c] = v[j][k];
      }
    p0 += 64 * KP;
    if (p0 >= chunks) break;
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
      for (int k = 0; k < KP; ++k) v[j][k] = buf_load16(src[j], sbytes[j], (uint32_t)(p0 + lane + 64 * k) * 16);
  }
}

__global__ void compact_zero_counts_kernel(int32_t* counts) {
  if (threadIdx.x == 0) { counts[0] = 0; counts[1] = 0; }
}

// ---------------------------------------------------------------- rows
// Destination row j < n_cont: h_cont[j] = h[cont_idx[j]].
// Destination row j >= n_cont: out[row_ids[e]] = h[e], e = exit_idx[j - n_cont].
struct CompactRows {
  int n, row_bytes;                 // row_bytes multiple of 16
  const char* h; int64_t ld_h;      // strides in bytes
  const int32_t* row_ids;
  const int32_t* cont_idx; const int32_t* exit_idx; const int32_t* counts;
  char* h_cont; int64_t ld_cont;
  char* out; int64_t ld_out; int64_t n_out_rows;
};

constexpr int ROWS_PER_WG = 4;

__global__ __launch_bounds__(256) void compact_rows_kernel(CompactRows a) {
  const int n_cont = a.counts[0];
  const int chunks = a.row_bytes >> 4;
#pragma unroll 1
  for (int r = 0; r < ROWS_PER_WG; ++r) {
    const int j = blockIdx.x * ROWS_PER_WG + r;
    if (j >= a.n) return;
    const char* src;
    char* dst;
    if (j < n_cont) {
      if (!a.h_cont) continue;
      src = a.h + (int64_t)a.cont_idx[j] * a.ld_h;
      dst = a.h_cont + (int64_t)j * a.ld_cont;
    } else {
      if (!a.out) continue;
      const int e = a.exit_idx[j - n_cont];
      const int64_t rid = a.row_ids ? a.row_ids[e] : e;
      if (rid < 0 || rid >= a.n_out_rows) continue;
      src = a.h + (int64_t)e * a.ld_h;
      dst = a.out + rid * a.ld_out;
    }
    for (int c = threadIdx.x; c < chunks; c += blockDim.x)
      ((u32x4*)dst)[c] = ((const u32x4*)src)[c];
  }
}

}  // namespace river

namespace river_host {
using namespace river;

size_t compact_workspace(int n) {
  const size_t chunks = (size_t)(n + GRID_CHUNK - 1) / GRID_CHUNK;
  return align_up(chunks * sizeof(int32_t), 256);
}

river_status launch_compact(int n, int d, river_dtype dt, const uint8_t* mask, const void* h,
                            int64_t ld_h, const int32_t* row_ids, int32_t* cont_idx,
                            int32_t* exit_idx, int32_t* counts, void* h_cont, int64_t ld_cont,
                            int32_t* row_ids_cont, void* out, int64_t ld_out, int64_t n_out_rows,
                            void* workspace, size_t ws_bytes, hipStream_t s) {
  (void)ws_bytes;
  if (n == 0) {
    compact_zero_counts_kernel<<<1, 64, 0, s>>>(counts);
    return check_launch("compact (empty)");
  }
  CompactIdx a{n, mask, row_ids, cont_idx, exit_idx, counts, row_ids_cont};
  int path = compact_path_override();
  if (path == 0) path = n <= FUSED_MAX ? 4 : 3;
  const int64_t es = (int64_t)esize(dt);
  if (path == 4) {
    // 8 tokens per workgroup up to 8192 tokens (measured at 4096 tokens of
    // d = 768: 4.14 µs against 4.57 with 16 and 4.22 with 4), 16 while the
    // mask prefixes the workgroups read stay small (n^2 / 32 bytes in all),
    // 64 beyond
    const char* hh = (h_cont || out) ? (const char*)h : nullptr;
    if (n <= 8192)
      compact_fused_kernel<8><<<(n + 7) / 8, 256, 0, s>>>(a, hh, ld_h * es, (int)(d * es), (char*)h_cont,
                                                          ld_cont * es, (char*)out, ld_out * es, n_out_rows);
    else if (n <= 16384)
      compact_fused_kernel<16><<<(n + 15) / 16, 256, 0, s>>>(a, hh, ld_h * es, (int)(d * es), (char*)h_cont,
                                                             ld_cont * es, (char*)out, ld_out * es, n_out_rows);
    else
      compact_fused_kernel<64><<<(n + 63) / 64, 256, 0, s>>>(a, hh, ld_h * es, (int)(d * es), (char*)h_cont,
                                                             ld_cont * es, (char*)out, ld_out * es, n_out_rows);
    return check_launch("compact fused");
  }
  if (path == 1) {
    compact_wave_kernel<<<1, 64, 0, s>>>(a);
  } else if (path == 2) {
    const int items = (n + CB_THREADS - 1) / CB_THREADS;
    compact_block_kernel<<<1, CB_THREADS, 0, s>>>(a, items);
  } else {
    const int chunks = (n + GRID_CHUNK - 1) / GRID_CHUNK;
    int32_t* cc = (int32_t*)workspace;
    compact_grid_count_kernel<<<chunks, 256, 0, s>>>(a, cc);
    river_status st = check_launch("compact count");
    if (st != RIVER_OK) return st;
    compact_grid_write_kernel<<<chunks, 256, 0, s>>>(a, cc, chunks);
  }
  river_status st = check_launch("compact index");
  if (st != RIVER_OK || (!h_cont && !out)) return st;
  CompactRows r{n, (int)(d * es), (const char*)h, ld_h * es, row_ids, cont_idx, exit_idx, counts,
                (char*)h_cont, ld_cont * es, (char*)out, ld_out * es, n_out_rows};
  compact_rows_kernel<<<(n + ROWS_PER_WG - 1) / ROWS_PER_WG, 256, 0, s>>>(r);
  return check_launch("compact rows");
}

}  // namespace river_host
