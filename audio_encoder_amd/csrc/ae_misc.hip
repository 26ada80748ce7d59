// Row-wise kernels: the pre-LN LayerNorms (card "cstr/MOSS-Transcribe-preview-2B-GGUF",
// "Architecture": pre-LN Transformer and ln_post), the standalone SwiGLU of the fp32 path and
// float32 conversion for stage dumps.  All are HBM-bound.
//
// LayerNorm: one wave per row; each lane keeps its D/64 values in registers (float4 loads,
// fully coalesced), so the row is read once; mean and biased variance come from two wave
// reductions in fp32 (DPP within rows of 16 lanes, then the four row sums), and the normalised
// row is written in the GEMM operand type.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the 64 lanes, returned in every lane, without LDS permutes: DPP swaps within each row
// of 16 lanes (neighbours, pairs of neighbours, then the two half-rows and the two row halves
// mirrored), then the four row sums read as scalars.
template <int CTRL>
__device__ inline float dpp_swap_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                    0xf, 0xf, false));
}
__device__ inline float wave_sum_dpp(float v) {
  v = dpp_swap_add<0xb1>(v);   // quad_perm [1,0,3,2]
  v = dpp_swap_add<0x4e>(v);   // quad_perm [2,3,0,1]
  v = dpp_swap_add<0x141>(v);  // row_half_mirror: lane i of 8 <- lane 7-i
  v = dpp_swap_add<0x140>(v);  // row_mirror: lane i of 16 <- lane 15-i
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <typename T> struct Store4;
template <> struct Store4<bf16_t> {
  __device__ static inline void put(bf16_t* p, float a, float b, float c, float d) {
    uint2 o;
    o.x = pack_bf16x2(a, b);
    o.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = o;
  }
};
template <> struct Store4<float> {
  __device__ static inline void put(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

// D = 256 * NJ
template <typename T, int NJ>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ g,
                                                        const float* __restrict__ b,
                                                        T* __restrict__ y, int64_t M, float eps) {
  constexpr int D = 256 * NJ;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * D);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  // gain and bias are loaded with the row, so their latency is not paid after the reductions
  float4 v[NJ], gg[NJ], bb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = xr[lane + 64 * j];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    gg[j] = g4[lane + 64 * j];
    bb[j] = b4[lane + 64 * j];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the gain/bias loads ahead of the reductions
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_sum_dpp(s) * (1.0f / D);
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float a0 = v[j].x - mean, a1 = v[j].y - mean, a2 = v[j].z - mean, a3 = v[j].w - mean;
    q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
  }
  const float rstd = rsqrtf(wave_sum_dpp(q) * (1.0f / D) + eps);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c4 = lane + 64 * j;
    Store4<T>::put(y + row * D + 4 * c4, (v[j].x - mean) * rstd * gg[j].x + bb[j].x,
                   (v[j].y - mean) * rstd * gg[j].y + bb[j].y, (v[j].z - mean) * rstd * gg[j].z + bb[j].z,
                   (v[j].w - mean) * rstd * gg[j].w + bb[j].w);
  }
}

// any D % 64 == 0: three passes over the (cached) row
template <typename T>
__global__ __launch_bounds__(256) void layernorm_generic_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ g,
                                                                const float* __restrict__ b,
                                                                T* __restrict__ y, int64_t M,
                                                                int32_t D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + row * D;
  float s = 0.0f;
  for (int c = lane; c < D; c += 64) s += xr[c];
  const float mean = wave_sum(s) / D;
  float q = 0.0f;
  for (int c = lane; c < D; c += 64) {
    const float a = xr[c] - mean;
    q += a * a;
  }
  const float rstd = rsqrtf(wave_sum(q) / D + eps);
  for (int c = lane; c < D; c += 64) StoreT<T>::put(y + row * D + c, (xr[c] - mean) * rstd * g[c] + b[c]);
}

// gu [M, N2] with 32-column interleaved gate/up groups -> out [M, N2/2]
template <typename T>
__global__ void swiglu_split_kernel(const T* __restrict__ gu, int64_t M, int32_t N2,
                                    T* __restrict__ out) {
  const int32_t Nh = N2 / 2;
  const int64_t total = M * Nh;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / Nh;
    const int j = (int)(i - r * Nh);
    const int64_t src = r * N2 + 64 * (j / 32) + (j % 32);
    float gv, uv;
    if constexpr (std::is_same<T, bf16_t>::value) {
      gv = bf16_to_f32(gu[src]);
      uv = bf16_to_f32(gu[src + 32]);
    } else {
      gv = gu[src];
      uv = gu[src + 32];
    }
    StoreT<T>::put(out + i, silu(gv) * uv);
  }
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ src, int64_t n, float* __restrict__ dst) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    if constexpr (std::is_same<T, bf16_t>::value) dst[i] = bf16_to_f32(src[i]);
    else dst[i] = src[i];
  }
}

inline int grid_for(int64_t n) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 16384));
}

}  // namespace

template <typename T>
hipError_t launch_layernorm(const float* x, const float* g, const float* b, T* y, int64_t M,
                            int32_t D, float eps, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((M + 3) / 4));
  switch (D) {
    case 256: hipLaunchKernelGGL((layernorm_kernel<T, 1>), grid, dim3(256), 0, s, x, g, b, y, M, eps); break;
    case 512: hipLaunchKernelGGL((layernorm_kernel<T, 2>), grid, dim3(256), 0, s, x, g, b, y, M, eps); break;
    case 1024: hipLaunchKernelGGL((layernorm_kernel<T, 4>), grid, dim3(256), 0, s, x, g, b, y, M, eps); break;
    case 1280: hipLaunchKernelGGL((layernorm_kernel<T, 5>), grid, dim3(256), 0, s, x, g, b, y, M, eps); break;
    case 2048: hipLaunchKernelGGL((layernorm_kernel<T, 8>), grid, dim3(256), 0, s, x, g, b, y, M, eps); break;
    default:
      if (D % 64 != 0) return hipErrorInvalidValue;
      hipLaunchKernelGGL((layernorm_generic_kernel<T>), grid, dim3(256), 0, s, x, g, b, y, M, D, eps);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_swiglu_split(const T* gu, int64_t M, int32_t N2, T* out, hipStream_t s) {
  hipLaunchKernelGGL((swiglu_split_kernel<T>), dim3(grid_for(M * (N2 / 2))), dim3(256), 0, s, gu,
                     M, N2, out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_to_f32(const T* src, int64_t n, float* dst, hipStream_t s) {
  hipLaunchKernelGGL((to_f32_kernel<T>), dim3(grid_for(n)), dim3(256), 0, s, src, n, dst);
  return hipGetLastError();
}

template hipError_t launch_layernorm<bf16_t>(const float*, const float*, const float*, bf16_t*,
                                             int64_t, int32_t, float, hipStream_t);
template hipError_t launch_layernorm<float>(const float*, const float*, const float*, float*,
                                            int64_t, int32_t, float, hipStream_t);
template hipError_t launch_swiglu_split<bf16_t>(const bf16_t*, int64_t, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_swiglu_split<float>(const float*, int64_t, int32_t, float*, hipStream_t);
template hipError_t launch_to_f32<bf16_t>(const bf16_t*, int64_t, float*, hipStream_t);
template hipError_t launch_to_f32<float>(const float*, int64_t, float*, hipStream_t);

}  // namespace ae
