// Shared device helpers of the river library (gfx950 / CDNA4, wave64); the
// host-side plumbing is in host.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "river.h"

namespace river {

// ------------------------------------------------------------ vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ------------------------------------------------------------ bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// x & m, opaque to the compiler's known-bits analysis (so that a later
// (float)((x >> 8 j) & 0xff) becomes a single v_cvt_f32_ubyte<j>)
__device__ __forceinline__ uint32_t opaque_and(uint32_t x, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
  return r;
}

// load element i of a dt array as fp32
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

// ----------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// sum over aligned groups of G consecutive lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// Cross-lane moves inside a row of 16 lanes (DPP, no LDS round trip).
// CTRL: 0xB1 swaps neighbours (quad_perm 1,0,3,2), 0x4E swaps pairs
// (quad_perm 2,3,0,1), 0x141 mirrors each half row, 0x140 mirrors the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of 8 or 16 lanes, left in every lane of the group
template <int G>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  if constexpr (G == 16) v += dpp_mov<0x140>(v);
  return v;
}

// ------------------------------------------------- LDS tiles and waits
// LDS swizzle of 16-byte chunk c of tile row r (8 chunks per row): stored at
// r * 8 + (c ^ swz(r)). With 64 lanes reading one chunk of 32 consecutive
// rows, each 16-lane group touches 16 distinct bank groups (measured on
// gfx950: no bank-conflict cycles, where c ^ (r & 7) costs 4 per read).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding (and, with LGKM0, all LDS writes are done), then a
// workgroup barrier. The empty asm statements keep the compiler from
// moving memory operations across; unlike __syncthreads() there is no
// release fence, which would force vmcnt(0) and drain the load pipeline.
template <int N, bool LGKM0>
__device__ __forceinline__ void wait_barrier() {
  constexpr int vm = N > 63 ? 63 : N;
  constexpr int imm = (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding, no barrier (for data this wave loaded itself).
template <int N>
__device__ __forceinline__ void wait_vm() {
  constexpr int vm = N > 63 ? 63 : N;
  constexpr int imm = (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------- buffer loads
// a buffer offset past every resource here (they span under 2^31 bytes):
// the load returns zeros and fetches nothing
constexpr uint32_t BUF_OOB = 0x80000000u;

// dword 3 of a raw (untyped) buffer resource on gfx9-family GPUs: 32-bit
// data format, no swizzle, no index stride
constexpr int RSRC_WORD3 = 0x00020000;

// 16 bytes per lane from the buffer [base, base + bytes) at byte offset voff
// into registers; a lane whose 16 bytes lie past the end reads zeros and
// touches no memory (bytes and voff multiples of 16). No branch guards the
// load, so a wave keeps several in flight.
__device__ __forceinline__ u32x4 buf_load16(const void* base, int bytes, uint32_t voff) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, RSRC_WORD3);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// SIZE bytes per lane from the buffer [base, base + bytes) at byte offset
// voff + soff straight into LDS (lane l writes lds + SIZE * l); a lane whose
// bytes lie past the end reads zeros. base, bytes and soff are uniform, so
// the resource sits in scalar registers and is built once per loop.
template <int SIZE>   // 16 or 4
__device__ __forceinline__ void buf_lds(const void* base, int bytes, uint32_t voff, int soff, void* lds) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, RSRC_WORD3);
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)voff, soff, 0, 0);
}


}  // namespace river

#include "host.h"
