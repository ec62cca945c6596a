// Bandwidth probes (measurement only, include/slora_probe.h): a contiguous
// streaming read and a gather of whole rows, each one launch, so that the
// delta kernels' achieved bandwidth can be set beside what a plain read of the
// same size reaches on the same GPU.
#include <string>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "slora_internal.h"
#include "slora_probe.h"

namespace {

constexpr int kProbeThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferFormat = 0x00020000;   // descriptor word 3: raw 32-bit buffer
constexpr int kNontemporal = 2;             // cache-policy bits of a buffer load: streaming

// A buffer load returns zero, without touching memory, for any offset at or
// past the descriptor's byte count: the probes read ragged ends and skipped
// rows with no branch, so every load of a thread stays in flight together.
__device__ __forceinline__ u32x4 load16(const char* base, uint32_t bytes, uint32_t offset, bool nt) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)bytes,
                                                                      kBufferFormat);
  return nt ? __builtin_amdgcn_raw_buffer_load_b128(rs, offset, 0, kNontemporal)
            : __builtin_amdgcn_raw_buffer_load_b128(rs, offset, 0, 0);
}

// The loads feed an xor that decides whether one store runs; the store never
// runs for real data, but the compiler cannot drop the loads.
__device__ __forceinline__ void sink_if(u32x4 acc, u32x4* sink) {
  if (acc.x == 0x5A5A5A5Au && acc.y == 0xA5A5A5A5u && acc.z == 0x0F0F0F0Fu && acc.w == 0xF0F0F0F0u)
    sink[0] = acc;
}

// Workgroup b reads chunks [b * 256 * ITEMS, (b + 1) * 256 * ITEMS): at step k
// thread tid reads chunk k * 256 + tid of that span, so every load instruction
// of a wave covers 1 KB of contiguous memory.  All ITEMS loads are issued
// before any is used; the last workgroup's loads past the end return zero.
template <int ITEMS, bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const char* src, int64_t bytes, u32x4* sink) {
  constexpr int64_t kSpan = (int64_t)kProbeThreads * ITEMS * 16;
  const int64_t start = (int64_t)blockIdx.x * kSpan;
  const int64_t left = bytes - start;
  const uint32_t span = (uint32_t)(left < kSpan ? left : kSpan);
  u32x4 v[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) v[k] = load16(src + start, span, (k * kProbeThreads + threadIdx.x) * 16, NT);
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) acc ^= v[k];
  sink_if(acc, sink);
}

struct GatherArray {
  const char* base;
  int64_t stride;
  const int32_t* rows;
  uint32_t n;           // rows listed
  uint32_t row_bytes;
  uint32_t cpt;         // 256-thread passes per row: ceil(row_bytes / 4096)
  uint32_t pad;
};

struct GatherArgs {
  GatherArray a[2];
  uint32_t blocks0;     // workgroups of the first array
};

// Each row is cut into cpt passes of 256 16-byte chunks (the last one ragged);
// the passes of the listed rows, row after row, are dealt ITEMS to a
// workgroup: [0, blocks0) over the first array, the rest over the second.
// A pass lies in one row, so the row id of every load instruction is uniform
// (one scalar load) and the instruction covers 1 KB of that row; chunks past
// the row's end, and passes past the last listed row, read nothing.
template <int ITEMS>
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(GatherArgs G, u32x4* sink) {
  uint32_t b = blockIdx.x;
  const bool second = b >= G.blocks0;
  const GatherArray A = second ? G.a[1] : G.a[0];
  if (second) b -= G.blocks0;
  const uint32_t p0 = b * ITEMS;
  uint32_t row = p0 / A.cpt, pc = p0 - row * A.cpt;
  uint32_t id[ITEMS], bytes[ITEMS], off[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const bool listed = row < A.n;
    id[k] = (uint32_t)A.rows[listed ? row : A.n - 1];
    bytes[k] = listed ? A.row_bytes : 0u;
    off[k] = (pc * kProbeThreads + threadIdx.x) * 16;
    ++pc;
    const bool wrap = pc == A.cpt;
    row += wrap ? 1u : 0u;
    pc = wrap ? 0u : pc;
  }
  u32x4 v[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) v[k] = load16(A.base + (int64_t)id[k] * A.stride, bytes[k], off[k], true);
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) acc ^= v[k];
  sink_if(acc, sink);
}

slora_status probe_fail(slora_status s, const std::string& m) {
  slora::set_last_error(m.c_str());
  return s;
}

template <typename K>
hipError_t launch(K kernel, int64_t blocks, void** args, void* stream, void* ev0, void* ev1) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!ev0 && !ev1)
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks), dim3(kProbeThreads),
                           args, 0, st);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks), dim3(kProbeThreads),
                            args, 0, st, static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0);
}

template <int ITEMS>
const void* read_fn(bool nt) {
  return nt ? reinterpret_cast<const void*>(&probe_read_kernel<ITEMS, true>)
            : reinterpret_cast<const void*>(&probe_read_kernel<ITEMS, false>);
}

}  // namespace

extern "C" {

slora_status slora_probe_read(const void* src, int64_t bytes, int32_t items, int32_t nontemporal,
                              void* sink, void* stream, void* ev0, void* ev1) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) || ((reinterpret_cast<uintptr_t>(src) |
                                                       reinterpret_cast<uintptr_t>(sink)) & 15))
    return probe_fail(SLORA_E_INVAL, "slora_probe_read: NULL, unaligned or empty buffer");
  const void* k = nullptr;
  switch (items) {
    case 1: k = read_fn<1>(nontemporal); break;
    case 2: k = read_fn<2>(nontemporal); break;
    case 4: k = read_fn<4>(nontemporal); break;
    case 8: k = read_fn<8>(nontemporal); break;
    case 16: k = read_fn<16>(nontemporal); break;
    default: return probe_fail(SLORA_E_INVAL, "slora_probe_read: items must be 1, 2, 4, 8 or 16");
  }
  const int64_t per = (int64_t)kProbeThreads * items * 16;
  const int64_t blocks = (bytes + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return probe_fail(SLORA_E_INVAL, "slora_probe_read: too many bytes");
  const char* s = static_cast<const char*>(src);
  u32x4* o = static_cast<u32x4*>(sink);
  void* args[] = {&s, &bytes, &o};
  const hipError_t e = launch(k, blocks, args, stream, ev0, ev1);
  if (e != hipSuccess) return probe_fail(SLORA_E_HIP, std::string("slora_probe_read: ") + hipGetErrorString(e));
  return SLORA_OK;
}

slora_status slora_probe_gather(const void* base0, int64_t stride0, int64_t row_bytes0, const int32_t* rows0,
                                int64_t n0, const void* base1, int64_t stride1, int64_t row_bytes1,
                                const int32_t* rows1, int64_t n1, int32_t items, void* sink, void* stream,
                                void* ev0, void* ev1) {
  if (!base0 || !rows0 || n0 <= 0 || row_bytes0 <= 0 || (row_bytes0 & 15) || stride0 < row_bytes0 ||
      (stride0 & 15) || !sink || n1 < 0 || (n1 > 0 && (!base1 || !rows1 || row_bytes1 <= 0 || (row_bytes1 & 15) ||
                                                       stride1 < row_bytes1 || (stride1 & 15))))
    return probe_fail(SLORA_E_INVAL, "slora_probe_gather: bad row arrays");
  if (items != 1 && items != 2 && items != 4 && items != 8 && items != 16)
    return probe_fail(SLORA_E_INVAL, "slora_probe_gather: items must be 1, 2, 4, 8 or 16");
  if (n0 >= ((int64_t)1 << 31) || n1 >= ((int64_t)1 << 31) || row_bytes0 >= ((int64_t)1 << 30) ||
      (n1 > 0 && row_bytes1 >= ((int64_t)1 << 30)))
    return probe_fail(SLORA_E_INVAL, "slora_probe_gather: too many rows or row too long");
  GatherArgs G{};
  const void* bases[2] = {base0, base1};
  const int64_t strides[2] = {stride0, stride1}, rbytes[2] = {row_bytes0, row_bytes1}, ns[2] = {n0, n1};
  const int32_t* rows[2] = {rows0, rows1};
  int64_t blocks[2] = {0, 0};
  for (int a = 0; a < 2; ++a) {
    const int src = ns[a] > 0 ? a : 0;  // an empty second array repeats the first's fields
    GatherArray& A = G.a[a];
    A.base = static_cast<const char*>(bases[src]);
    A.stride = strides[src];
    A.rows = rows[src];
    A.n = (uint32_t)ns[a];
    A.row_bytes = (uint32_t)rbytes[src];
    A.cpt = (uint32_t)((rbytes[src] + 16 * kProbeThreads - 1) / (16 * kProbeThreads));
    blocks[a] = (ns[a] * A.cpt + items - 1) / items;
    if (ns[a] * A.cpt + items >= ((int64_t)1 << 32))
      return probe_fail(SLORA_E_INVAL, "slora_probe_gather: too many rows");
  }
  if (blocks[0] + blocks[1] > 0x7FFFFFFF) return probe_fail(SLORA_E_INVAL, "slora_probe_gather: too many rows");
  G.blocks0 = (uint32_t)blocks[0];
  u32x4* o = static_cast<u32x4*>(sink);
  void* args[] = {&G, &o};
  const int64_t nblocks = blocks[0] + blocks[1];
  hipError_t e;
  switch (items) {
    case 1: e = launch(&probe_gather_kernel<1>, nblocks, args, stream, ev0, ev1); break;
    case 2: e = launch(&probe_gather_kernel<2>, nblocks, args, stream, ev0, ev1); break;
    case 4: e = launch(&probe_gather_kernel<4>, nblocks, args, stream, ev0, ev1); break;
    case 8: e = launch(&probe_gather_kernel<8>, nblocks, args, stream, ev0, ev1); break;
    default: e = launch(&probe_gather_kernel<16>, nblocks, args, stream, ev0, ev1); break;
  }
  if (e != hipSuccess) return probe_fail(SLORA_E_HIP, std::string("slora_probe_gather: ") + hipGetErrorString(e));
  return SLORA_OK;
}

}  // extern "C"
