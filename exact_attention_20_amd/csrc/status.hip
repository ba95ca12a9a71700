// Device status word. The paged kernels tolerate bad device metadata: a
// page-table entry outside the pool reads as zeros (attention) or is not
// written (KV append), and an appended token past its page-table row is
// skipped. So that this does not pass unnoticed, the kernel that meets it also
// ORs a bit into this word, which fa_device_status reads back (and clears).
//
// Each GPU the library runs on holds its own copy of the word for the life of
// the process, and every call on that GPU shares it.
#include <mutex>

#include "fa_internal.h"

namespace fa {

static __device__ __align__(256) unsigned int g_status;

namespace {
constexpr int kMaxStatusDevices = 64;
std::mutex g_status_mu;
unsigned* g_status_addr[kMaxStatusDevices] = {};
}  // namespace

// In host code the word's name is only a host-side handle, so its address is
// asked of the runtime once per device, with that device current, and kept.
hipError_t device_status_ptr(unsigned** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxStatusDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_status_mu);
  if (!g_status_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_status));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_status_addr[dev] = static_cast<unsigned*>(p);
  }
  *ptr = g_status_addr[dev];
  return hipSuccess;
}

}  // namespace fa
