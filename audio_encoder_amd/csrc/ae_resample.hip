// Input conditioning: any channel count and sample rate -> the 16 kHz mono signal the front end
// takes ("SILVERTHRONE/Ossicle-4B" card, model summary line "Audio input": mono or stereo, any
// sample rate; "cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Quick Start": the tower itself
// takes 16 kHz mono, which that card pre-converts).
//
// The pages name no filter.  Reading used here (documented with the oracle that defines it):
//   downmix   the mean of the channels;
//   16 kHz    passed through unchanged;
//   otherwise band-limited interpolation with a Hann-windowed sinc: with L/M = 16000/fs in
//             lowest terms, output sample j sits at input position t_j = j*M/L; the low-pass
//             cutoff is fc = 0.945 * min(1, L/M) / 2 cycles per input sample and the window spans
//             16 zero crossings of the sinc on each side (R = 16 / (2 fc) input samples);
//             the taps of each of the L phases are normalised to sum to 1 (unit DC gain);
//             samples outside the signal are zero.  n_out = ceil(n_in * L / M).
// The host builds the L x 2K tap table (fp64, stored fp32); one thread per output sample sums
// its 2K taps in fp32, downmixing the interleaved input on the fly.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

__global__ __launch_bounds__(256) void resample_kernel(const float* __restrict__ in, int64_t n_in,
                                                       int32_t channels, int32_t L, int32_t M,
                                                       int32_t K, const float* __restrict__ taps,
                                                       float* __restrict__ out, int64_t n_out) {
  const float inv_c = 1.0f / (float)channels;
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n_out;
       j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t num = j * (int64_t)M;
    const int64_t base = num / L;
    const int p = (int)(num - base * L);
    const float* h = taps + (int64_t)p * 2 * K;
    float acc = 0.0f;
    for (int k = 0; k < 2 * K; ++k) {
      const int64_t i = base - K + 1 + k;
      if (i < 0 || i >= n_in) continue;
      float x = 0.0f;
      for (int c = 0; c < channels; ++c) x += in[i * channels + c];
      acc = fmaf(h[k], x * inv_c, acc);
    }
    out[j] = acc;
  }
}

__global__ __launch_bounds__(256) void downmix_kernel(const float* __restrict__ in, int64_t n,
                                                      int32_t channels, float* __restrict__ out) {
  const float inv_c = 1.0f / (float)channels;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float x = 0.0f;
    for (int c = 0; c < channels; ++c) x += in[i * channels + c];
    out[i] = channels == 1 ? x : x * inv_c;
  }
}

inline int grid_for(int64_t n) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 16384));
}

}  // namespace

hipError_t launch_resample(const float* in, int64_t n_in, int32_t channels, int32_t L, int32_t M,
                           int32_t K, const float* taps, float* out, int64_t n_out, hipStream_t s) {
  if (n_out <= 0) return hipSuccess;
  if (L == 1 && M == 1) {
    hipLaunchKernelGGL(downmix_kernel, dim3(grid_for(n_out)), dim3(256), 0, s, in, n_out, channels, out);
  } else {
    hipLaunchKernelGGL(resample_kernel, dim3(grid_for(n_out)), dim3(256), 0, s, in, n_in, channels, L,
                       M, K, taps, out, n_out);
  }
  return hipGetLastError();
}

}  // namespace ae
