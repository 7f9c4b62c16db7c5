// LDS tile layout and HBM -> LDS copy helpers shared by the gfx950 bf16 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// Word 3 of a raw (unswizzled, stride 0) buffer descriptor on gfx9 parts:
// 32-bit data format, range-checked against num_records.
constexpr int kBufferFlags = 0x00020000;

// (The buffer builtins sit in plain device functions: called from a lambda in
// the kernel they stop the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int num_records) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, num_records, kBufferFlags);
}

// 16 bytes per lane from `rsrc` at byte offset `voffset` into LDS at
// lds_base + 16 * lane; lanes past num_records write zeros.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds_base,
                                                  unsigned voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)lds_base, 16, voffset, 0, 0, 0);
}

// Chunk swizzle of an LDS tile row: logical 16-byte chunk c of row r lives at
// physical chunk c ^ swz(r). For head_dim 128 (16 chunks per 256-byte row) the
// 16 rows read together by a K operand load get 16 distinct chunks, and the 4
// consecutive rows of a transposed V read (two 16-lane groups, 16 columns
// apart) land on 16 distinct chunks; head_dim 64 (8 chunks per 128-byte row,
// two rows per bank sweep) gets the same property from row bits 1..3.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row, logical 16-byte chunk) inside an LDS tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + 8 * (chunk ^ swz<D>(row));
}

// Wait until at most N vector-memory operations of this wavefront are in
// flight, then meet the other wavefronts. Copies complete in issue order, so N
// = the copies issued last stay in flight. (A plain __syncthreads() would wait
// for all of them.) The memory clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void wait_vmem_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_vmem() {
  // vmcnt(0), leaving the LDS/export counters unconstrained.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace fa
