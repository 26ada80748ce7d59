// conv1: the first 3x3 stride-2 Conv2D (1 -> C channels) + bias + GELU of the conv front end
// ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture", row "Conv front-end").
//
// The image of one window is [128 mel bins (frequency), L0 frames (time)], zero outside.  The
// kernel reads the raw log10 mel and applies the Whisper normalisation (max(L, max - 8) + 4) / 4
// on load, so the normalised mel is never written to HBM.  Each thread produces 8 consecutive
// output channels of one (time, frequency) position and writes them as one 16-byte store into
// the channels-last activation [window][4W time][64 freq][C], which is the layout the implicit
// GEMM of conv2 reads.  With one input channel this layer has K = 9 and no MFMA shape fits;
// it is bound by its HBM writes.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

__device__ inline float key_to_float_c(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <typename T> struct Pack8;
template <> struct Pack8<bf16_t> {
  __device__ static inline void store(bf16_t* p, const float* v) {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = o;
  }
};
template <> struct Pack8<float> {
  __device__ static inline void store(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void conv1_kernel(const Win* __restrict__ wins, int32_t n_win,
                                                    int32_t W, const float* __restrict__ mel,
                                                    int64_t T_frames,
                                                    const uint32_t* __restrict__ max_key,
                                                    const float* __restrict__ wt,
                                                    const float* __restrict__ bias, int32_t C,
                                                    T* __restrict__ act1) {
  extern __shared__ float sw[];  // [C][10]: 9 taps + bias
  for (int i = threadIdx.x; i < C * 9; i += blockDim.x) sw[(i / 9) * 10 + (i % 9)] = wt[i];
  for (int i = threadIdx.x; i < C; i += blockDim.x) sw[i * 10 + 9] = bias[i];
  __syncthreads();

  const int CG = C / 8;
  const int64_t L1max = 4 * (int64_t)W;
  const int64_t total = (int64_t)n_win * L1max * 64 * CG;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int cg = (int)(i % CG);
    int64_t r = i / CG;
    const int f1 = (int)(r % 64);
    r /= 64;
    const int t1 = (int)(r % L1max);
    const int wi = (int)(r / L1max);
    const Win wn = wins[wi];
    if (t1 >= wn.L1) continue;
    const float lo = key_to_float_c(max_key[wn.clip]) - 8.0f;
    const float* mrow = mel + ((int64_t)wn.clip * T_frames + wn.start) * 128;
    float xv[9];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const int f = 2 * f1 + a - 1;  // frequency tap
        const int t = 2 * t1 + b - 1;  // time tap
        const bool ok = f >= 0 && f < 128 && t >= 0 && t < wn.L0;
        xv[a * 3 + b] = ok ? (fmaxf(mrow[(int64_t)t * 128 + f], lo) + 4.0f) * 0.25f : 0.0f;
      }
    }
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float* wc = sw + (cg * 8 + c) * 10;
      float acc = wc[9];
#pragma unroll
      for (int q = 0; q < 9; ++q) acc = fmaf(wc[q], xv[q], acc);
      o[c] = gelu_erf(acc);
    }
    Pack8<T>::store(act1 + (((int64_t)wi * L1max + t1) * 64 + f1) * C + cg * 8, o);
  }
}

}  // namespace

template <typename T>
hipError_t launch_conv1(const PassGeom& g, const float* mel, int64_t T_frames,
                        const uint32_t* max_key, const float* w, const float* b, int32_t C,
                        T* act1, hipStream_t s) {
  const int64_t total = (int64_t)g.n_win * 4 * g.W * 64 * (C / 8);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 1 << 16));
  hipLaunchKernelGGL(conv1_kernel<T>, dim3(blocks), dim3(256), C * 10 * sizeof(float), s, g.wins,
                     g.n_win, g.W, mel, T_frames, max_key, w, b, C, act1);
  return hipGetLastError();
}

template hipError_t launch_conv1<bf16_t>(const PassGeom&, const float*, int64_t, const uint32_t*,
                                         const float*, const float*, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_conv1<float>(const PassGeom&, const float*, int64_t, const uint32_t*,
                                        const float*, const float*, int32_t, float*, hipStream_t);

}  // namespace ae
