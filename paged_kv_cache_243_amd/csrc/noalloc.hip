// noalloc.hip -- paged_attention_noalloc: paged attention for callers that
// cannot allocate device memory (graph capture, serving loops, harnesses that
// forbid hipMalloc).  Its workspace is `scratch`, a fixed array in the
// library's own device memory; the HIP runtime places one copy on each GPU the
// library runs on, held until the process ends.
//
// `scratch` names a host-side stand-in in host code, not a device address.  Its
// device address is taken once per device, at the first call on that device
// and with that device current, by hipGetSymbolAddress; host code then uses
// only that address (kernel arguments), never the array's name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "pagedkv.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of device `dev`'s copy of `scratch` (nullptr on a HIP error).
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_lock);
  if (g_scratch[dev] == nullptr) {
    int current = -1;
    if (hipGetDevice(&current) != hipSuccess) return nullptr;
    if (current != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (current != dev) (void)hipSetDevice(current);
    if (err != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int paged_attention_noalloc(const pkv_tensor* q, const pkv_tensor* key_pool,
                                       const pkv_tensor* value_pool, const pkv_tensor* block_table,
                                       const pkv_tensor* seq_lens, const pkv_tensor* query_start_loc,
                                       float scale, pkv_tensor* out, const pkv_attn_opts* opts,
                                       void* stream) {
  return pkv::attention_in_region(q, key_pool, value_pool, block_table, seq_lens, query_start_loc, scale, out,
                                  opts, PKV_NOALLOC_SCRATCH_BYTES, scratch_on, stream);
}
