// topk_select_noalloc: topk_select without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops that must not call the allocator).  The split path's workspace is a
// fixed-size array in device memory owned by the library (each GPU holds its
// own copy until the process ends); every call on a GPU shares that GPU's
// copy, so such calls must not overlap on one GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/libcsa.h"
#include "common.h"

namespace {

constexpr size_t kScratchBytes = (size_t)CSA_TOPK_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte granules");

// The array's name is a host-side stand-in: host code uses only the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

__global__ void __launch_bounds__(256) clear_words(uint4* p, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Device address of this device's scratch, found once per device; the first
// call on a device also clears the array with a fill kernel on `s` (the array
// starts zeroed when the code object loads; the clear makes that explicit),
// after which every successful call leaves the part that must start at zero
// at zero.
hipError_t scratch_for_current_device(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    const size_t n16 = kScratchBytes / 16;
    hipLaunchKernelGGL(clear_words, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, static_cast<uint4*>(p), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace csa {
int abi_hip_status(hipError_t e);
}

extern "C" int topk_select_noalloc(const void* scores, int32_t score_dtype, int32_t batch, int32_t n_q,
                                   int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int32_t ratio,
                                   int32_t k, int32_t* idx_out, void* stream) {
  // the checks of topk_select, with the library's array as the workspace
  if (score_dtype != CSA_BF16 && score_dtype != CSA_F32) return CSA_ERR_DTYPE;
  if (batch < 0 || n_q < 0 || n_cap < 0 || k < 1 || ratio < 1) return CSA_ERR_SHAPE;
  if (batch > 65535 || n_q > 0x7fffffff) return CSA_ERR_SHAPE;
  if ((int64_t)batch * n_q == 0) return CSA_OK;
  if (!n_entries || !q_pos || !idx_out || (n_cap > 0 && !scores)) return CSA_ERR_NULL;
  const size_t need = csa::topk_ws_bytes(batch, n_q, n_cap, k, score_dtype);
  if (need > kScratchBytes) return CSA_ERR_WORKSPACE;  // beyond the fixed array: use topk_select
  const hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_for_current_device(s, &ws);
    if (e != hipSuccess) return csa::abi_hip_status(e);
  }
  return csa::abi_hip_status(
      csa::launch_topk(scores, score_dtype, batch, n_q, n_cap, n_entries, q_pos, ratio, k, idx_out, ws, s));
}
