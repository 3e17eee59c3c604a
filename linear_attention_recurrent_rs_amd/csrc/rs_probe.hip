// The bandwidth reference for the verify kernels: a plain streaming read with the same
// load instructions (non-temporal 16-byte vector loads) and workgroup size (256 threads)
// as the verify's state-tile loads, and nothing else.  Its rate on a buffer of the verify's
// size is the read rate this GPU reaches for that access pattern and transfer size, the
// ceiling the verify's achieved rate is compared with (next to the HBM peak).
#include <cstdint>

#include "rs.h"
#include "rs_device.h"

namespace rs {

namespace {

constexpr int kLoadsPerThread = 4;           // 16 KiB per workgroup, contiguous

// Workgroup b reads 16-byte words [b * 1024, (b + 1) * 1024); thread t reads every 256th.
// The sum is written only when it equals a value a zero or random buffer does not give,
// so that the loads are not removed; sink holds 256 floats.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const f4* __restrict__ src,
                                                               uint64_t n16, float* sink) {
  const uint64_t base = (uint64_t)blockIdx.x * kThreads * kLoadsPerThread + threadIdx.x;
  f4 v[kLoadsPerThread];
#pragma unroll
  for (int k = 0; k < kLoadsPerThread; ++k) {
    const uint64_t i = base + (uint64_t)kThreads * k;
    v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : f4{0.f, 0.f, 0.f, 0.f};
  }
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kLoadsPerThread; ++k) acc += v[k];
  if (acc[0] == 1234.5f && acc[1] == -1234.5f) sink[threadIdx.x] = acc[2] + acc[3];
}

}  // namespace

}  // namespace rs

extern "C" rs_status rs_stream_read(const void* src, uint64_t bytes, float* sink,
                                    hipStream_t stream) {
  if (!src || !sink) return RS_E_NULLPTR;
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return RS_E_SHAPE;
  const uint64_t n16 = bytes / 16;
  const uint64_t per_block = (uint64_t)rs::kThreads * rs::kLoadsPerThread;
  const uint64_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return RS_E_SHAPE;
  hipLaunchKernelGGL(rs::stream_read_kernel, dim3((unsigned)blocks), dim3(rs::kThreads), 0,
                     stream, static_cast<const rs::f4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? RS_OK : RS_E_LAUNCH;
}
