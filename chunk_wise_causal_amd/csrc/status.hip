// Per-device status word: kernels OR WF_STATUS_* bits into it when they meet
// device data the host could not check (a page-table entry outside the
// pool).  Each GPU holds its own copy of the variable; the host resolves its
// address once per device and passes that address to kernels.
#include <mutex>

#include "wf_internal.h"

__device__ int wf_status_word;

namespace wf {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int* g_ptr[kMaxDevices] = {};
}  // namespace

int* status_word_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(wf_status_word));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = static_cast<int*>(p);
  }
  *err = hipSuccess;
  return g_ptr[dev];
}

}  // namespace wf
