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

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// The loads feed an xor that decides whether one store runs; the store never
// runs for real data, but the compiler cannot drop the loads.
__device__ __forceinline__ void sink_if(u32x4 acc, u32x4* sink) {
  if (acc.x == 0x5A5A5A5Au && acc.y == 0xA5A5A5A5u && acc.z == 0x0F0F0F0Fu && acc.w == 0xF0F0F0F0u)
    sink[0] = acc;
}

// Workgroup b reads chunks [b * 256 * ITEMS, (b + 1) * 256 * ITEMS): at step k
// thread tid reads chunk base + k * 256 + tid, so every load instruction of a
// wave covers 1 KB of contiguous memory.  All ITEMS loads are issued before
// any is used.
template <int ITEMS, bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* src, int64_t n_chunks,
                                                                   u32x4* sink) {
  const int64_t base = (int64_t)blockIdx.x * kProbeThreads * ITEMS + threadIdx.x;
  u32x4 v[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int64_t c = base + (int64_t)k * kProbeThreads;
    v[k] = load16<NT>(src + (c < n_chunks ? c : n_chunks - 1));
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) acc ^= v[k];
  sink_if(acc, sink);
}

struct GatherArgs {
  const char* base[2];
  int64_t stride[2];
  const int32_t* rows[2];
  uint32_t cpr[2];       // 16-byte chunks per row
  uint32_t n_chunks0;    // chunks of the first array's rows
  uint32_t n_chunks;     // all chunks
};

// The listed rows' chunks, numbered first array first, row by row; workgroup
// b reads numbers [b * 256 * ITEMS, ...) as the read probe does, each through
// its row id.
template <int ITEMS>
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(GatherArgs G, u32x4* sink) {
  const uint32_t base = blockIdx.x * (uint32_t)(kProbeThreads * ITEMS) + threadIdx.x;
  u32x4 v[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    uint32_t i = base + (uint32_t)k * kProbeThreads;
    i = i < G.n_chunks ? i : G.n_chunks - 1;
    const int a = i < G.n_chunks0 ? 0 : 1;
    const uint32_t j = a ? i - G.n_chunks0 : i;
    const uint32_t row = j / G.cpr[a], c = j - row * G.cpr[a];
    const char* p = G.base[a] + (int64_t)(uint32_t)G.rows[a][row] * G.stride[a] + (int64_t)c * 16;
    v[k] = load16<true>(reinterpret_cast<const u32x4*>(p));
  }
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
  const int64_t n_chunks = bytes / 16;
  const void* k = nullptr;
  switch (items) {
    case 1: k = read_fn<1>(nontemporal); break;
    case 2: k = read_fn<2>(nontemporal); break;
    case 4: k = read_fn<4>(nontemporal); break;
    case 8: k = read_fn<8>(nontemporal); break;
    case 16: k = read_fn<16>(nontemporal); break;
    default: return probe_fail(SLORA_E_INVAL, "slora_probe_read: items must be 1, 2, 4, 8 or 16");
  }
  const int64_t per = (int64_t)kProbeThreads * items;
  const int64_t blocks = (n_chunks + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return probe_fail(SLORA_E_INVAL, "slora_probe_read: too many bytes");
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* o = static_cast<u32x4*>(sink);
  void* args[] = {&s, const_cast<int64_t*>(&n_chunks), &o};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = (!ev0 && !ev1)
      ? hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kProbeThreads), args, 0, st)
      : hipExtLaunchKernel(k, dim3((unsigned)blocks), dim3(kProbeThreads), args, 0, st,
                           static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0);
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
  GatherArgs G{};
  G.base[0] = static_cast<const char*>(base0);
  G.base[1] = n1 > 0 ? static_cast<const char*>(base1) : G.base[0];
  G.stride[0] = stride0;
  G.stride[1] = n1 > 0 ? stride1 : stride0;
  G.rows[0] = rows0;
  G.rows[1] = n1 > 0 ? rows1 : rows0;
  G.cpr[0] = (uint32_t)(row_bytes0 / 16);
  G.cpr[1] = n1 > 0 ? (uint32_t)(row_bytes1 / 16) : G.cpr[0];
  const int64_t c0 = n0 * (row_bytes0 / 16), c1 = n1 * (n1 > 0 ? row_bytes1 / 16 : 0);
  if (c0 + c1 >= ((int64_t)1 << 31)) return probe_fail(SLORA_E_INVAL, "slora_probe_gather: too many chunks");
  G.n_chunks0 = (uint32_t)c0;
  G.n_chunks = (uint32_t)(c0 + c1);
  u32x4* o = static_cast<u32x4*>(sink);
  void* args[] = {&G, &o};
  const int64_t per = (int64_t)kProbeThreads * items;
  const int64_t blocks = (c0 + c1 + per - 1) / per;
  hipError_t e;
  switch (items) {
    case 1: e = launch(&probe_gather_kernel<1>, blocks, args, stream, ev0, ev1); break;
    case 2: e = launch(&probe_gather_kernel<2>, blocks, args, stream, ev0, ev1); break;
    case 4: e = launch(&probe_gather_kernel<4>, blocks, args, stream, ev0, ev1); break;
    case 8: e = launch(&probe_gather_kernel<8>, blocks, args, stream, ev0, ev1); break;
    case 16: e = launch(&probe_gather_kernel<16>, blocks, args, stream, ev0, ev1); break;
    default: return probe_fail(SLORA_E_INVAL, "slora_probe_gather: items must be 1, 2, 4, 8 or 16");
  }
  if (e != hipSuccess) return probe_fail(SLORA_E_HIP, std::string("slora_probe_gather: ") + hipGetErrorString(e));
  return SLORA_OK;
}

}  // extern "C"
