// Audio injection: the rows of a prompt's token-embedding table that hold audio placeholders are
// replaced by the adapter's output frames, in order ("cstr/MOSS-Transcribe-preview-2B-GGUF"
// card, "Architecture", row "Audio injection").
//
// A pure row scatter: one workgroup per frame copies its row with 16-byte accesses.  Positions
// outside the table are skipped and counted, so a bad position never writes out of bounds.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void splice_kernel(const T* __restrict__ frames, int64_t n,
                                                     int32_t dim, const int64_t* __restrict__ pos,
                                                     T* __restrict__ table, int64_t rows,
                                                     int32_t* __restrict__ n_skipped) {
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t p = pos[i];
    if (p < 0 || p >= rows) {
      if (threadIdx.x == 0 && n_skipped) atomicAdd(n_skipped, 1);
      continue;
    }
    const uint4* src = reinterpret_cast<const uint4*>(frames + i * (int64_t)dim);
    uint4* dst = reinterpret_cast<uint4*>(table + p * (int64_t)dim);
    const int chunks = dim * (int)sizeof(T) / 16;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) dst[c] = src[c];
  }
}

}  // namespace

template <typename T>
hipError_t launch_splice(const T* frames, int64_t n, int32_t dim, const int64_t* pos, T* table,
                         int64_t rows, int32_t* n_skipped, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if ((dim * (int64_t)sizeof(T)) % 16 != 0) return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>(n, 65535);
  hipLaunchKernelGGL(splice_kernel<T>, dim3(blocks), dim3(256), 0, s, frames, n, dim, pos, table,
                     rows, n_skipped);
  return hipGetLastError();
}

template hipError_t launch_splice<bf16_t>(const bf16_t*, int64_t, int32_t, const int64_t*, bf16_t*,
                                          int64_t, int32_t*, hipStream_t);
template hipError_t launch_splice<float>(const float*, int64_t, int32_t, const int64_t*, float*,
                                         int64_t, int32_t*, hipStream_t);

}  // namespace ae
