// Device helpers shared by the HIP sources of libslora (gfx950): vector
// types, 16-byte loads and stores, wave-uniform values, the LDS-only barrier
// and the two swizzled LDS layouts the matrix-core tiles stage operands in.
#pragma once

#include <hip/hip_runtime.h>

#include "slora_internal.h"

namespace slora {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Values every lane of a wavefront holds alike (tile header fields, the wave
// index) are moved to scalar registers.  Control flow on them then branches
// instead of masking lanes, which matters for MFMA: a matrix instruction runs
// on the whole wavefront whatever the EXEC mask says, so it must never sit
// behind a lane mask to be skipped.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its global
// loads still in flight (prefetches included) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rows of kShrinkKc (64) fp16 k values, k-contiguous: 16-byte chunk c of row
// `row` at this dword offset; the chunks are XOR-swizzled by row so that the
// 16 rows one MFMA operand read touches spread over the banks.
__device__ __forceinline__ int chunk_dw(int row, int c) { return row * (kShrinkKc / 2) + 4 * (c ^ (row & 7)); }

// Rows of kMfmaPass (128) fp16 columns, column-contiguous (a staged slice of
// B or W rows).
constexpr int kSliceRowDw = kMfmaPass / 2;      // dwords per 128-column row
// Dword offset of column quad q (4 columns) of row r of a staged slice.  The
// quads are XOR-swizzled by row so that the 8 rows the two lane groups of a
// half-wave read together (8g + t, t = 0..3) land in distinct banks.
__device__ __forceinline__ int quad_dw(int r, int q) {
  return r * kSliceRowDw + 2 * (q ^ (4 * ((r & 3) + 4 * ((r >> 3) & 1))));
}


}  // namespace slora
