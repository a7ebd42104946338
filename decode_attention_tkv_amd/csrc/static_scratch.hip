// The library's static device scratch: device memory that the
// no-allocation entry point (tkv_reassign_static) uses in place of the
// buffers tkv_reassign grows with hipMalloc.  Each GPU the library runs on
// holds its own copy of the array until the process ends.
#include <mutex>

#include "handle.hpp"
#include "host_util.hpp"

namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

// In host code this name stands for the array; kernels get its device
// address, looked up once per device below, never the name itself.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // scratch's address on each device, once looked up

}  // namespace

// Address of the calling handle's GPU's copy of the scratch (looked up with
// that device current, once per device) and its size.
int static_scratch(tkv* t, void** base, size_t* cap) {
  const int dev = t->device;
  if (dev < 0 || dev >= kMaxDevices) return tkv_fail(t, TKV_EINVAL, "device %d out of range for the static scratch", dev);
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    HIP_TRY(t, hipGetDevice(&cur));
    if (cur != dev) HIP_TRY(t, hipSetDevice(dev));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return tkv_fail(t, TKV_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    }
    g_ptr[dev] = p;
  }
  *base = g_ptr[dev];
  *cap = kStaticScratchBytes;
  return TKV_OK;
}
