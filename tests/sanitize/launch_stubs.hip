// Kernel launchers that refuse to launch: linked into the sanitizer build of the library's host
// code (tests/test_host_sanitizers.py), which exercises only the entry points that do no GPU
// work.  Any launch reached from them would be a bug; each stub reports it and fails.
#include <cstdio>

#include "../../audio_encoder_amd/csrc/ae_internal.h"

namespace ae {
namespace {
hipError_t refused(const char* what) {
  std::fprintf(stderr, "host-only run reached a kernel launch: %s\n", what);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_log_mel(const float*, const ClipSpan*, int32_t, int64_t, const MelTables&, float*, uint32_t*,
                          hipStream_t) { return refused("log_mel"); }
hipError_t launch_clear_u32(uint32_t*, int64_t, hipStream_t) { return refused("clear_u32"); }
hipError_t launch_batch_spans(ClipSpan*, int32_t, int64_t, hipStream_t) { return refused("batch_spans"); }
hipError_t launch_mel_normalize(const float*, const uint32_t*, int64_t, int32_t, float*, hipStream_t) {
  return refused("mel_normalize");
}
template <typename T>
hipError_t launch_conv1(const PassGeom&, const float*, const uint32_t*, const float*, const float*, const float*,
                        int32_t, T*, hipStream_t) { return refused("conv1"); }
template <typename T>
hipError_t launch_linear(const LinearArgs&, int, int, hipStream_t) { return refused("linear"); }
template <typename T>
hipError_t launch_conv_igemm(const PassGeom&, int, const T*, const T*, const float*, int32_t, T*, hipStream_t,
                             int32_t) {
  return refused("conv_igemm");
}
template <typename T>
hipError_t launch_layernorm(const float*, const float*, const float*, T*, int64_t, int32_t, float, hipStream_t) {
  return refused("layernorm");
}
template <typename T>
hipError_t launch_attention(const T*, const Win*, const int32_t*, int32_t, int32_t, int32_t, T*, hipStream_t) {
  return refused("attention");
}
template <typename T>
hipError_t launch_swiglu_split(const T*, int64_t, int32_t, T*, hipStream_t) { return refused("swiglu_split"); }
template <typename T>
hipError_t launch_to_f32(const T*, int64_t, float*, hipStream_t) { return refused("to_f32"); }
hipError_t launch_resample(const float*, int64_t, int32_t, int32_t, int32_t, int32_t, const float*, float*, int64_t,
                           hipStream_t) { return refused("resample"); }
template <typename T>
hipError_t launch_splice(const T*, int64_t, int32_t, const int64_t*, T*, int64_t, int32_t*, hipStream_t) {
  return refused("splice");
}

#define AE_STUB_TYPES(T)                                                                                   \
  template hipError_t launch_conv1<T>(const PassGeom&, const float*, const uint32_t*, const float*,        \
                                      const float*, const float*, int32_t, T*, hipStream_t);               \
  template hipError_t launch_linear<T>(const LinearArgs&, int, int, hipStream_t);                          \
  template hipError_t launch_conv_igemm<T>(const PassGeom&, int, const T*, const T*, const float*, int32_t, \
                                           T*, hipStream_t, int32_t);                                      \
  template hipError_t launch_layernorm<T>(const float*, const float*, const float*, T*, int64_t, int32_t,  \
                                          float, hipStream_t);                                             \
  template hipError_t launch_attention<T>(const T*, const Win*, const int32_t*, int32_t, int32_t, int32_t, \
                                          T*, hipStream_t);                                                \
  template hipError_t launch_swiglu_split<T>(const T*, int64_t, int32_t, T*, hipStream_t);                 \
  template hipError_t launch_to_f32<T>(const T*, int64_t, float*, hipStream_t);                            \
  template hipError_t launch_splice<T>(const T*, int64_t, int32_t, const int64_t*, T*, int64_t, int32_t*,  \
                                       hipStream_t);
AE_STUB_TYPES(bf16_t)
AE_STUB_TYPES(float)

}  // namespace ae
