// Library-owned scratch memory for the entry point that allocates nothing
// (vmla_chunk_attention_noalloc): a file-scope device array, one copy per GPU,
// holding the query prologue's Qhat rows between the prologue and the
// attention kernel. Its size is VMLA_NOALLOC_SCRATCH_BYTES.
//
// In host code the array's name is only a stand-in, not a device address: the
// address comes from hipGetSymbolAddress, looked up once per device (with that
// device current) on the entry point's first call there, and kept per device.
// Every call on a GPU shares that GPU's array and leaves its contents behind;
// the prologue rewrites every Qhat row that the attention reads, so nothing
// needs to start at zero.
#include <atomic>
#include <mutex>

#include "kernels.h"
#include "vmla.h"

namespace vmla {

static __device__ __align__(256) unsigned char scratch[VMLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;
}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace vmla
