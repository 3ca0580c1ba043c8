// Host-only stand-ins for the kernel launchers of libtattn.so, so that the
// C-ABI layer (tattn.cpp) can be built by the host compiler alone, with
// AddressSanitizer and UndefinedBehaviorSanitizer, and its validation paths
// exercised on a machine without a GPU. Nothing here computes anything: a
// launcher that is reached records the call and reports success.
#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace tattn {

int g_stub_launches = 0;

hipError_t launch_mha_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int, int, int,
                               int, bool, int, const uint8_t*, float, int, int, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

hipError_t launch_mha_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int, int, int,
                              bool, float, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

size_t mla_workspace_bytes(int B, int H, int n_split) {
  return (size_t)(n_split + B) * (size_t)H * 1028u + 4096u;
}

hipError_t launch_mla_decode(const void*, const void*, const void*, const void*, void*, float*, int, int,
                             const int32_t*, float, int, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

hipError_t mla_noalloc_scratch(void** ptr) {
  static char host_stand_in[64];
  *ptr = host_stand_in;
  return hipSuccess;
}

hipError_t launch_ssd_scan_bf16(const void*, const float*, const float*, const void*, const void*, void*,
                                const float*, float*, int, int, int, int, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

}  // namespace tattn
