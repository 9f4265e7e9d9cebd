// Streaming-read probe for the per-workload report: how fast one kernel can
// read a buffer from HBM on this device (16-byte loads, grid-stride, one store
// per thread).  It is the practical ceiling the HBM-bound stages are compared
// with; it is not part of the library's interface.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

__global__ void __launch_bounds__(256) read_kernel(const float4* __restrict__ a, size_t n4, float* __restrict__ out) {
  float s = 0.0f;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 v = a[i];
    s += v.x + v.y + v.z + v.w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;  // keeps the loads
}

}  // namespace

// Reads `bytes` (a multiple of 16, buf 16-byte aligned) `reps` times back to
// back on `stream` with `grid` work-groups of 256 threads; sink holds grid*256
// floats.  Writes the mean microseconds per launch.  Returns 0, 1 on invalid
// arguments, or the HIP error code.
extern "C" int read_rate_probe(const void* buf, size_t bytes, float* sink, int grid, int reps, float* us_per_call,
                               void* stream) {
  if (!buf || !sink || !us_per_call || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15) || grid < 1 || reps < 1)
    return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float4* a = reinterpret_cast<const float4*>(buf);
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, a, bytes / 16, sink);
  hipEvent_t e0, e1;
  hipError_t e = hipEventCreate(&e0);
  if (e != hipSuccess) return (int)e;
  e = hipEventCreate(&e1);
  if (e != hipSuccess) {
    hipEventDestroy(e0);
    return (int)e;
  }
  hipEventRecord(e0, s);
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, a, bytes / 16, sink);
  hipEventRecord(e1, s);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  *us_per_call = ms * 1e3f / reps;
  return 0;
}
