// decode_scratch.hip -- the fixed device workspace behind the allocation-free
// decode entry point (kvq_decode_attention_noalloc).
//
// The decode's split partial records (one binary32 (max, sum, output row)
// record per sequence, kv head and context split) live here instead of in a
// caller-provided buffer, for callers that cannot allocate device memory.
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  On the
// host the array's name is only a stand-in for the symbol, so the device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels receive that address, never the name.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

static __device__ __align__(256) unsigned char scratch[KVQ_DECODE_SCRATCH_BYTES];

namespace kvq {
namespace {

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace kvq
