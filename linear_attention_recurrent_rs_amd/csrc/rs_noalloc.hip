// Workspace of the allocation-free verify entry point (rs_gdn_verify_noalloc).
//
// The verify's one scratch buffer is the key-group fold counter ([batch, hk] int32: the
// last workgroup of a key group to read the old ring prefix rewrites its rows).  For
// callers that cannot allocate, it lives here in a file-scope device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy until the process
// ends; host code never passes the array's name to a kernel (on the host it is only a
// stand-in), but the device address hipGetSymbolAddress returns for the current device,
// looked up once per device and kept.
#include <mutex>

#include "rs_device.h"
#include "rs_internal.h"

namespace rs {

static __device__ __align__(256) int32_t scratch[kNoAllocCounters];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
int32_t* g_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(kThreads) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t noalloc_counters(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

// Clears the first n counters on the stream with a fill kernel (no memset node, so that a
// captured graph replays it faithfully).
hipError_t launch_zero_counters(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     p, n);
  return hipGetLastError();
}

}  // namespace rs
