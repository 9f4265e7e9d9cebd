// Stand-ins for the device side of libcsa, so that the library's host code
// (argument checks of the C-ABI, the snapshot files of prefix reuse) can be
// built with AddressSanitizer and UndefinedBehaviorSanitizer and run on a
// machine without a GPU.  Test infrastructure only: "device" pointers are host
// pointers, copies are memcpy, kernels are never launched (every launcher
// reports hipErrorNoDevice), and the workspace sizes are those of the float32
// path (no workspace).
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "common.h"

extern "C" {
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memmove(dst, src, n);
  return hipSuccess;
}
}

namespace csa {
constexpr hipError_t kNoLaunch = hipErrorNoDevice;
hipError_t launch_kv_pack(const void*, int, int64_t, int64_t, void*, int, int64_t, hipStream_t) { return kNoLaunch; }
hipError_t launch_kv_append(const void*, int, int, const int64_t*, void*, int, int64_t, int64_t, void*, int, int64_t,
                            int64_t, hipStream_t) {
  return kNoLaunch;
}
hipError_t launch_mxfp4_quantize(const float*, int64_t, int, uint8_t*, uint8_t*, hipStream_t) { return kNoLaunch; }
hipError_t launch_csa_compress(const void*, int, int, int64_t, int64_t, const float*, const float*, int64_t, int, void*,
                               int, int64_t, const float*, int, void*, uint8_t*, int, hipStream_t) {
  return kNoLaunch;
}
hipError_t launch_hca_compress(const void*, int, int, int64_t, int64_t, const float*, const float*, int64_t, int, void*,
                               int, int64_t, hipStream_t) {
  return kNoLaunch;
}
hipError_t launch_indexer_f32(const float*, const float*, const float*, int, int, int, int, int64_t, const int32_t*,
                              const int64_t*, int, float*, hipStream_t) {
  return kNoLaunch;
}
hipError_t launch_indexer_mxfp4(const void*, bool, const uint8_t*, const float*, const uint8_t*, const uint8_t*, int,
                                int, int, int, int64_t, const int32_t*, const int64_t*, int, uint16_t*, hipStream_t,
                                uint32_t*, int, hipEvent_t, hipEvent_t, EntryPages) {
  return kNoLaunch;
}
size_t topk_ws_bytes(int, int, int64_t, int, int) { return 0; }
hipError_t launch_topk(const void*, int, int, int, int64_t, const int32_t*, const int64_t*, int, int, int32_t*, void*,
                       hipStream_t, bool) {
  return kNoLaunch;
}
bool topk_uses_split(int64_t, int64_t, int) { return false; }
uint32_t* topk_split_totals(void* ws, int* row_words) {
  *row_words = 0;
  return static_cast<uint32_t*>(ws);
}
hipError_t launch_decode_append(const csa_decode_cache&, const void*, const void*, int, int64_t*, int32_t*, const float*,
                                uint8_t*, uint8_t*, hipStream_t, int, bool) {
  return kNoLaunch;
}
hipError_t launch_decode_prime(const csa_decode_cache&, const void*, const void*, int, int, hipStream_t) {
  return kNoLaunch;
}
hipError_t launch_decode_fork(const csa_decode_cache&, int, int, hipStream_t) { return kNoLaunch; }
size_t attn_ws_bytes(int, int, int, int64_t, int, int) { return 0; }
hipError_t launch_attention(const AttnArgs&, int64_t, hipStream_t) { return kNoLaunch; }
hipError_t launch_attention_pair(const AttnArgs&, int64_t, const AttnArgs&, int64_t, hipStream_t) { return kNoLaunch; }
}  // namespace csa
