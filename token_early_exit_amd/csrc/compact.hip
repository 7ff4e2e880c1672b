// compact: stable split of a batch by its exit mask, row gather of the
// continuing tokens and scatter of the exited ones.
//
// TIDE, 模块4 (融合 CUDA 内核): "Batch Compact" separates continuing from
// exiting tokens, with a ballot for small batches and a prefix-sum scatter
// for large ones; "Exit Scatter" copies exited hidden states back to their
// original rows of an output buffer.
//
// Index kernels (one launch, or two for very large batches):
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
  if (path == 0) path = n <= 64 ? 1 : (n <= CB_THREADS * 16 ? 2 : 3);
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
  const int64_t es = (int64_t)esize(dt);
  CompactRows r{n, (int)(d * es), (const char*)h, ld_h * es, row_ids, cont_idx, exit_idx, counts,
                (char*)h_cont, ld_cont * es, (char*)out, ld_out * es, n_out_rows};
  compact_rows_kernel<<<(n + ROWS_PER_WG - 1) / ROWS_PER_WG, 256, 0, s>>>(r);
  return check_launch("compact rows");
}

}  // namespace river_host
