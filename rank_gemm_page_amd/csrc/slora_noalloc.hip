// slora_lora_forward_noalloc: slora_lora_forward with its workspace (the fp32
// x A products of the batch and their K-split partials) in a device array of
// the library instead of caller memory, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops and harnesses
// that forbid it).
//
// The array is a file-scope __device__ array: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the array's name as an address (it is a host-side stand-in
// there): the first call on a device, with that device current, asks the
// runtime for that device's address with hipGetSymbolAddress, checks the
// result and keeps it per device; every kernel argument and copy uses that
// address.  The entry point itself allocates nothing.
#include <mutex>
#include <string>

#include <hip/hip_runtime.h>

#include "slora_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;   // 8 MiB: the 7B prefill batch needs 5.5 MB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

slora_status fail(slora_status st, const std::string& msg) {
  slora::set_last_error(msg.c_str());
  return st;
}

}  // namespace

extern "C" slora_status slora_lora_forward_noalloc(slora_pool* pool, const slora_segments* seg, int32_t proj,
                                                   const void* x, const void* w, void* y, void* stream) {
  const char* fn = "slora_lora_forward_noalloc";
  if (!pool || !seg) return fail(SLORA_E_INVAL, std::string(fn) + ": NULL pool or segments");
  const size_t need = slora::segments_workspace_bytes(seg);
  if (need > kScratchBytes)
    return fail(SLORA_E_NOMEM, std::string(fn) + ": the batch needs " + std::to_string(need) +
                                   " bytes of workspace, more than the library's " +
                                   std::to_string(kScratchBytes) + " (use slora_lora_forward with a workspace)");
  slora_status st = slora::pool_device_current(pool);
  if (st != SLORA_OK) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SLORA_E_HIP, std::string(fn) + ": hipGetDevice: " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SLORA_E_INVAL, std::string(fn) + ": device index out of range");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(SLORA_E_HIP, std::string(fn) + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return slora_lora_forward(pool, seg, proj, x, w, y, ptr, kScratchBytes, stream);
}
