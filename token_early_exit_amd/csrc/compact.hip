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
// One launch for indices and rows, n <= FUSED_MAX: workgroup c owns tokens
// [64 c, 64 c + 64). Every wave reads the chunk's 64 mask bytes and ballots
// them, so each wave knows which of the chunk's rows exit. Exited rows go to
// out[row_ids[i]], which does not depend on any rank, so they are copied
// while the exits before the chunk are still being counted (16-byte reads
// of the mask prefix, at most n bytes). With that count the workgroup writes
// both index lists and copies its continuing rows to h_cont.
constexpr int FCH = 64;
constexpr int FUSED_MAX = 65536;

// One row of `chunks` 16-byte pieces copied by one wave: up to 8 loads per
// lane in flight before their stores, so a long row costs one memory
// latency per 8 x 1 KB instead of one per kilobyte.
__device__ __forceinline__ void copy_row(u32x4* __restrict__ d, const u32x4* __restrict__ src, int chunks,
                                         int lane) {
  for (int c0 = 0; c0 < chunks; c0 += 8 * 64) {
    u32x4 v[8];
    // unconditional loads (a lane past the row reloads its last piece), so
    // that no branch makes the wave wait between them
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + lane + 64 * i;
      v[i] = src[c < chunks ? c : chunks - 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + lane + 64 * i;
      if (c < chunks) d[c] = v[i];
    }
  }
}

__global__ __launch_bounds__(256) void compact_fused_kernel(CompactIdx a, const char* h, int64_t ld_h,
                                                            int row_bytes, char* h_cont, int64_t ld_cont,
                                                            char* out, int64_t ld_out, int64_t n_out_rows) {
  __shared__ int s_part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * FCH;
  const int n = a.n;
  const int chunks = row_bytes >> 4;
  // this chunk's tokens, in every wave
  const int i_own = c0 + lane;
  // the mask byte and the row id load together (the id is used only for
  // exits)
  const bool in = i_own < n;
  const bool ex_own = in && a.mask[i_own] != 0;
  const int rid_all = (out && in) ? (a.row_ids ? a.row_ids[i_own] : i_own) : -1;
  const int rid_own = ex_own ? rid_all : -1;
  // exits in [0, c0) (loads issued now, summed below)
  int cnt = 0;
  const u32x4* m16 = (const u32x4*)a.mask;
  for (int v = tid; v < (c0 >> 4); v += 256) {
    const u32x4 w = m16[v];
    cnt += nonzero_bytes(w[0]) + nonzero_bytes(w[1]) + nonzero_bytes(w[2]) + nonzero_bytes(w[3]);
  }
  const uint64_t bits = __ballot(ex_own);
  // exit scatter: rows t = wave, wave + 4, ... of the chunk
  if (h && out) {
    for (int t = wave; t < FCH; t += 4) {
      if (!((bits >> t) & 1)) continue;                     // uniform
      const int rid = __builtin_amdgcn_readlane(rid_own, t);
      if (rid < 0 || rid >= n_out_rows) continue;
      copy_row((u32x4*)(out + (int64_t)rid * ld_out), (const u32x4*)(h + (int64_t)(c0 + t) * ld_h),
               chunks, lane);
    }
  }
  cnt = (int)row_sum<16>((float)cnt);       // exact: counts stay far below 2^24
  cnt += __shfl_xor(cnt, 16, WAVE);
  cnt += __shfl_xor(cnt, 32, WAVE);
  if (lane == 0) s_part[wave] = cnt;
  __syncthreads();
  const int base = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  if (wave == 0) {
    const int rank = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
    if (i_own < n) emit(a, i_own, ex_own, rank);
    if (c0 + FCH >= n && lane == 0) {          // the last chunk knows the total
      const int ne = base + __popcll(bits);
      a.counts[0] = n - ne;
      a.counts[1] = ne;
    }
  }
  // continuing rows: row t goes to h_cont[(c0 + t) - (exits before it)]
  if (h && h_cont) {
    for (int t = wave; t < FCH && c0 + t < n; t += 4) {
      if ((bits >> t) & 1) continue;                        // uniform
      const int er = base + __popcll(bits & ((1ull << t) - 1));
      copy_row((u32x4*)(h_cont + (int64_t)(c0 + t - er) * ld_cont),
               (const u32x4*)(h + (int64_t)(c0 + t) * ld_h), chunks, lane);
    }
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
    compact_fused_kernel<<<(n + FCH - 1) / FCH, 256, 0, s>>>(
        a, (h_cont || out) ? (const char*)h : nullptr, ld_h * es, (int)(d * es), (char*)h_cont,
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
