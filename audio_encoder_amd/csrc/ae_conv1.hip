// conv1: the first 3x3 stride-2 Conv2D (1 -> C channels) + bias + GELU of the conv front end
// ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture", row "Conv front-end").
//
// The image of one window is [128 mel bins (frequency), L0 frames (time)], zero outside.  The
// kernel reads the raw log10 mel and applies the Whisper normalisation (max(L, max - 8) + 4) / 4
// on load, so the normalised mel is never written to HBM.  The output is the channels-last
// activation [window][4W time][64 freq][C] that the implicit GEMM of conv2 reads.
//
// With one input channel the layer has K = 9: no MFMA shape fits and it is bound by its HBM
// writes (2*C bytes per output position).  A workgroup owns RT consecutive output time steps of
// one window.  It stages the 2*RT+1 normalised mel frames those steps touch in LDS (zero rows and
// columns for the padding).  Each thread keeps the 9 taps and the bias of its 8 output channels
// in registers and emits 16-byte stores; CG = C/8 consecutive threads write one contiguous
// C-channel position.  Window w's rows start at w * L1s (the pass's time stride).
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

constexpr int RT = 4;  // output time steps per workgroup

__device__ inline float key_to_float_c(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <typename T> struct Pack8;
template <> struct Pack8<bf16_t> {
  __device__ static inline void store(bf16_t* p, const float* v) {
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = o;
  }
};
template <> struct Pack8<float> {
  __device__ static inline void store(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// blockDim.x = CG * FQ; thread -> channel group cg = tid % CG, frequency phase fq = tid / CG
template <typename T>
__global__ __launch_bounds__(256) void conv1_kernel(const Win* __restrict__ wins, int32_t L1s,
                                                    const float* __restrict__ mel,
                                                    const uint32_t* __restrict__ max_key,
                                                    const float* __restrict__ max_f,
                                                    const float* __restrict__ wt,
                                                    const float* __restrict__ bias, int32_t C,
                                                    T* __restrict__ act1) {
  __shared__ float xs[2 * RT + 1][130];  // frames 2*t1_0-1 .. 2*(t1_0+RT-1)+1, freq -1..128
  const int CG = C >> 3;
  const int FQ = blockDim.x / CG;
  const int tid = threadIdx.x;
  const int cg = tid % CG, fq = tid / CG;
  const int nrb = (L1s + RT - 1) / RT;
  const int w = blockIdx.x / nrb;
  const int t1_0 = (blockIdx.x - w * nrb) * RT;
  const Win wn = wins[w];
  if (t1_0 >= wn.L1) return;

  // the clip's maximum: ordered-integer key from the log-mel kernel, or a float (kernel-level
  // entry); uniform over the workgroup
  const float lo = (max_f ? max_f[wn.clip] : key_to_float_c(max_key[wn.clip])) - 8.0f;
  const float* mrow = mel + (int64_t)wn.mel_row * 128;
  for (int i = tid; i < (2 * RT + 1) * 130; i += blockDim.x) {
    const int r = i / 130, c = i - r * 130;
    const int t = 2 * t1_0 - 1 + r, f = c - 1;
    float v = 0.0f;
    if (t >= 0 && t < wn.L0 && f >= 0 && f < 128) v = (fmaxf(mrow[t * 128 + f], lo) + 4.0f) * 0.25f;
    xs[r][c] = v;
  }
  float wr[8][9], br[8];
  if (fq < FQ) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      br[c] = bias[cg * 8 + c];
#pragma unroll
      for (int q = 0; q < 9; ++q) wr[c][q] = wt[(cg * 8 + c) * 9 + q];
    }
  }
  __syncthreads();
  if (fq >= FQ) return;

  const int rows = min(RT, wn.L1 - t1_0);
  for (int r = 0; r < rows; ++r) {
    T* orow = act1 + (((int64_t)w * L1s + t1_0 + r) * 64) * C + cg * 8;
    for (int f1 = fq; f1 < 64; f1 += FQ) {
      float xv[9];
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) xv[a * 3 + b] = xs[2 * r + b][2 * f1 + a];  // (freq a, time b)
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float acc = br[c];
#pragma unroll
        for (int q = 0; q < 9; ++q) acc = fmaf(wr[c][q], xv[q], acc);
        o[c] = gelu_erf(acc);
      }
      Pack8<T>::store(orow + (int64_t)f1 * C, o);
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_conv1(const PassGeom& g, const float* mel, const uint32_t* max_key, const float* max_f,
                        const float* w, const float* b, int32_t C, T* act1, hipStream_t s) {
  const int CG = C / 8;
  const int FQ = std::max(1, std::min(64, 256 / CG));
  const int threads = CG * FQ;
  if (threads > 256 || threads < 1) return hipErrorInvalidValue;
  if (g.L1s < 1 || g.L1s > 4 * g.W) return hipErrorInvalidValue;
  const int nrb = (g.L1s + RT - 1) / RT;
  const int64_t blocks = (int64_t)g.n_win * nrb;
  if (blocks == 0) return hipSuccess;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(conv1_kernel<T>, dim3((unsigned)blocks), dim3(threads), 0, s, g.wins, g.L1s,
                     mel, max_key, max_f, w, b, C, act1);
  return hipGetLastError();
}

template hipError_t launch_conv1<bf16_t>(const PassGeom&, const float*, const uint32_t*, const float*,
                                         const float*, const float*, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_conv1<float>(const PassGeom&, const float*, const uint32_t*, const float*,
                                        const float*, const float*, int32_t, float*, hipStream_t);

}  // namespace ae
