// Windowed (block-diagonal) self-attention ("cstr/MOSS-Transcribe-preview-2B-GGUF" card,
// "Architecture", row "Audio encoder").  A token attends to the tokens of its own window
// only, so one workgroup owns one (window, head) pair and computes just that diagonal block;
// no score outside a window is ever formed.  Scores are scaled by 1/sqrt(64), keys past the
// window's valid length are masked, and the softmax runs in fp32.
//
// bf16 path (windows of up to 128 tokens): four waves, each owning 32 query rows.
//   S = Q K^T  : 4 key blocks x 4 K-steps of v_mfma_f32_32x32x16_bf16 (Q fragments straight
//                from HBM, K staged in LDS with XOR-swizzled 16-byte chunks)
//   softmax    : row max and row sum with cross-lane shuffles inside each 32-lane half (a
//                32x32 MFMA result row is spread over the 32 lanes of one half)
//   O = P V    : P goes through LDS to become an A operand; V is staged transposed so each
//                lane reads 8 consecutive keys of one feature as a B operand.
// fp32 path: one thread per query row with an online softmax over the window's keys.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

struct WinRef {
  const int32_t* p;
  int32_t stride, tok_off, len_off;
};

constexpr int QMAX = 128;   // maximum window length
constexpr int HD = 64;      // head dimension
constexpr int VTS = QMAX + 8;  // row stride (elements) of the transposed V and of P

__global__ __launch_bounds__(256) void attn_bf16_kernel(const bf16_t* __restrict__ qkv, WinRef wr,
                                                        int32_t n_heads, int32_t d,
                                                        bf16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[QMAX * HD];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[HD * VTS];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[4][32 * VTS];

  const int w = blockIdx.x / n_heads;
  const int h = blockIdx.x - w * n_heads;
  const int tok0 = wr.p[(int64_t)w * wr.stride + wr.tok_off];
  const int n = wr.p[(int64_t)w * wr.stride + wr.len_off];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t ld = 3 * (int64_t)d;
  const bf16_t* base = qkv + (int64_t)tok0 * ld + h * HD;

  // stage K (row-major, swizzled) and V (transposed)
  {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
      if (r < n) {
        kv = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + d + c * 8);
        vv = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + 2 * d + c * 8);
      }
      *reinterpret_cast<uint4*>(&Ks[r * HD + ((c ^ (r & 7)) * 8)]) = kv;
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(c * 8 + 2 * e) * VTS + r] = (bf16_t)(vw[e] & 0xffffu);
        Vt[(c * 8 + 2 * e + 1) * VTS + r] = (bf16_t)(vw[e] >> 16);
      }
    }
  }
  // Q fragments of this wave's 32 rows: lane -> row lane%32, 8 features per K-step
  const int q0 = wv * 32;
  const int qr = q0 + (lane & 31);
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (qr < n) v = *reinterpret_cast<const uint4*>(base + (int64_t)qr * ld + ks * 16 + (lane >> 5) * 8);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
  __syncthreads();

  f32x16_t S[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) S[jb][v] = 0.0f;
    const int key = jb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[key * HD + ((ch ^ (key & 7)) * 8)]);
      S[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, S[jb], 0, 0, 0);
    }
  }

  // softmax over keys; lane holds key column lane%32 of each block for 16 rows
  const float scale = 0.125f;  // 1/sqrt(64)
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float m = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int key = jb * 32 + (lane & 31);
      const float s = key < n ? S[jb][v] * scale : -INFINITY;
      S[jb][v] = s;
      m = fmaxf(m, s);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.0f;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const float e = __expf(S[jb][v] - m);
      S[jb][v] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o);
    const float inv = 1.0f / sum;
    const int prow = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      Ps[wv][prow * VTS + jb * 32 + (lane & 31)] = f32_to_bf16(S[jb][v] * inv);
  }
  __syncthreads();

  // O = P V
  f32x16_t O[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < QMAX / 16; ++ks) {
    const int kk = ks * 16 + (lane >> 5) * 8;
    const bf16x8_t pf = *reinterpret_cast<const bf16x8_t*>(&Ps[wv][(lane & 31) * VTS + kk]);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dim = db * 32 + (lane & 31);
      const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(&Vt[dim * VTS + kk]);
      O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, vf, O[db], 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = q0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (row >= n) continue;
    bf16_t* o = out + (int64_t)(tok0 + row) * d + h * HD;
#pragma unroll
    for (int db = 0; db < 2; ++db) o[db * 32 + (lane & 31)] = f32_to_bf16(O[db][v]);
  }
}

__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ qkv, WinRef wr,
                                                       int32_t n_heads, int32_t d,
                                                       float* __restrict__ out) {
  __shared__ float Kf[QMAX][HD + 1];
  __shared__ float Vf[QMAX][HD + 1];
  const int w = blockIdx.x / n_heads;
  const int h = blockIdx.x - w * n_heads;
  const int tok0 = wr.p[(int64_t)w * wr.stride + wr.tok_off];
  const int n = wr.p[(int64_t)w * wr.stride + wr.len_off];
  const int64_t ld = 3 * (int64_t)d;
  const float* base = qkv + (int64_t)tok0 * ld + h * HD;
  for (int i = threadIdx.x; i < n * HD; i += blockDim.x) {
    const int r = i / HD, c = i - r * HD;
    Kf[r][c] = base[(int64_t)r * ld + d + c];
    Vf[r][c] = base[(int64_t)r * ld + 2 * d + c];
  }
  __syncthreads();
  const int q = threadIdx.x;
  if (q >= n) return;
  float qv[HD], o[HD];
  for (int c = 0; c < HD; ++c) { qv[c] = base[(int64_t)q * ld + c] * 0.125f; o[c] = 0.0f; }
  float m = -INFINITY, l = 0.0f;
  for (int j = 0; j < n; ++j) {
    float s = 0.0f;
    for (int c = 0; c < HD; ++c) s = fmaf(qv[c], Kf[j][c], s);
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float p = expf(s - mn);
    l = l * corr + p;
    for (int c = 0; c < HD; ++c) o[c] = fmaf(p, Vf[j][c], o[c] * corr);
    m = mn;
  }
  const float inv = 1.0f / l;
  float* dst = out + (int64_t)(tok0 + q) * d + h * HD;
  for (int c = 0; c < HD; ++c) dst[c] = o[c] * inv;
}

}  // namespace

template <typename T>
hipError_t launch_attention(const T* qkv, const Win* wins, const int32_t* win2, int32_t n_win,
                            int32_t n_heads, int32_t d, T* out, hipStream_t s) {
  if (n_win <= 0) return hipSuccess;
  WinRef wr;
  if (wins) {
    wr.p = reinterpret_cast<const int32_t*>(wins);
    wr.stride = sizeof(Win) / sizeof(int32_t);
    wr.tok_off = offsetof(Win, tok) / sizeof(int32_t);
    wr.len_off = offsetof(Win, L3) / sizeof(int32_t);
  } else {
    wr.p = win2;
    wr.stride = 2;
    wr.tok_off = 0;
    wr.len_off = 1;
  }
  const dim3 grid((unsigned)(n_win * n_heads));
  if constexpr (std::is_same<T, bf16_t>::value) {
    hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(256), 0, s, qkv, wr, n_heads, d, out);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(128), 0, s, qkv, wr, n_heads, d, out);
  }
  return hipGetLastError();
}

template hipError_t launch_attention<bf16_t>(const bf16_t*, const Win*, const int32_t*, int32_t,
                                             int32_t, int32_t, bf16_t*, hipStream_t);
template hipError_t launch_attention<float>(const float*, const Win*, const int32_t*, int32_t,
                                            int32_t, int32_t, float*, hipStream_t);

}  // namespace ae
