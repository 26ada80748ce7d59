// Windowed (block-diagonal) self-attention ("cstr/MOSS-Transcribe-preview-2B-GGUF" card,
// "Architecture", row "Audio encoder").  A token attends to the tokens of its own window
// only, so one workgroup owns one (window, head) pair and computes just that diagonal block;
// no score outside a window is ever formed.  Scores are scaled by 1/sqrt(64), keys past the
// window's valid length are masked, and the softmax runs in fp32.
//
// bf16 path (windows of up to 128 tokens): four waves, each owning 32 queries.
//   S^T = K Q^T : 4 key blocks x 4 K-steps of v_mfma_f32_32x32x16_bf16.  K is staged in LDS
//                 (XOR-swizzled 16-byte chunks); Q fragments come straight from HBM.  In the
//                 transposed product each lane owns one query column, so the softmax max and
//                 sum run over its own registers plus a single exchange with lane ^ 32
//                 (v_permlane32_swap, no LDS).
//   O^T = V^T P^T: the unnormalised probabilities are packed to bf16 in registers and reordered
//                 into the B-operand layout with two v_permlane32_swap per K-step (no LDS round
//                 trip); V is staged transposed so each lane reads 8 consecutive keys of one
//                 feature.  The 1/sum scale is applied to O in fp32.
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

// Four workgroups per CU (the occupancy hint caps the kernel at 128 VGPRs; LDS 33 KB each):
// 1024 resident (window, head) pairs instead of the 768 the unconstrained allocation allows.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_bf16_kernel(const bf16_t* __restrict__ qkv, WinRef wr,
                                                        int32_t n_heads, int32_t d,
                                                        bf16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[QMAX * HD];   // [key][64], chunk-swizzled
  __shared__ __attribute__((aligned(16))) bf16_t Vt[HD * VTS];    // [feature][key]

  const int w = blockIdx.x / n_heads;
  const int h = blockIdx.x - w * n_heads;
  const int tok0 = wr.p[(int64_t)w * wr.stride + wr.tok_off];
  const int n = wr.p[(int64_t)w * wr.stride + wr.len_off];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t ld = 3 * (int64_t)d;
  const bf16_t* base = qkv + (int64_t)tok0 * ld + h * HD;

  // K rows (16-byte chunks, swizzled) and V transposed: each thread takes 4 consecutive keys
  // of one 8-feature chunk and writes 4 keys x 8 features as eight 8-byte rows of Vt
  {
    const int c = tid & 7;
    const int r0 = (tid >> 3) * 4;
    uint32_t vw[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
      if (r < n) {
        kv = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + d + c * 8);
        vv = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + 2 * d + c * 8);
      }
      *reinterpret_cast<uint4*>(&Ks[r * HD + ((c ^ (r & 7)) * 8)]) = kv;
      vw[i][0] = vv.x; vw[i][1] = vv.y; vw[i][2] = vv.z; vw[i][3] = vv.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // feature c*8+e: keys r0..r0+3
      const int sh = (e & 1) * 16;
      const uint32_t k01 = ((vw[0][e >> 1] >> sh) & 0xffffu) | (((vw[1][e >> 1] >> sh) & 0xffffu) << 16);
      const uint32_t k23 = ((vw[2][e >> 1] >> sh) & 0xffffu) | (((vw[3][e >> 1] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<uint2*>(&Vt[(c * 8 + e) * VTS + r0]) = make_uint2(k01, k23);
    }
  }
  // Q as the B operand of S^T = K Q^T: lane -> query column l32, 8 features per K-step
  const int q = wv * 32 + l32;
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (q < n) v = *reinterpret_cast<const uint4*>(base + (int64_t)q * ld + ks * 16 + half * 8);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
  __syncthreads();

  // S^T blocks: rows = keys 32*kb + 8*(v/4) + 4*half + v%4, column = this lane's query
  f32x16_t S[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key = kb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = ks * 2 + half;
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[key * HD + ((ch ^ (key & 7)) * 8)]);
      S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? f32x16_t{} : S[kb], 0, 0, 0);
    }
  }
  // softmax over keys for this lane's query.  Keys past the valid length only exist in the
  // last blocks (the test is uniform over the workgroup), so full blocks skip the mask.  The
  // maximum is taken on the raw scores (the scale is positive), and exp(s/8 - m/8) is
  // exp2(s c - m c) with c = log2(e) / 8: one FMA and one v_exp_f32 per score.
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb * 32 + 32 <= n) {
#pragma unroll
      for (int v = 0; v < 16; v += 4)
        m = fmaxf(m, fmaxf(fmaxf(S[kb][v], S[kb][v + 1]), fmaxf(S[kb][v + 2], S[kb][v + 3])));
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        S[kb][v] = key < n ? S[kb][v] : -INFINITY;
        m = fmaxf(m, S[kb][v]);
      }
    }
  }
  // the other half of this query's keys sits in lane ^ 32: permlane32_swap hands each lane its
  // partner's value in one of the two results, the other being its own
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  constexpr float kC = 0.18033688011112042f;  // log2(e) / sqrt(64)
  const float mc = m * kC;
  float sum = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float e = __builtin_amdgcn_exp2f(fmaf(S[kb][v], kC, -mc));
      S[kb][v] = e;
      sum += e;
    }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    sum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float inv = 1.0f / sum;

  // P^T as the B operand of O^T = V^T P^T: K-step s covers keys 16s..16s+15 of block s/2; lane
  // half hh needs keys 16(s%2) + 8hh + (0..7) of that block, i.e. group g = 2(s%2) + hh (keys
  // 8g..8g+7).  A lane holds keys 8g + 4*half + (0..3) of every group, so the half-0 lane owns
  // the first four keys of each group and the half-1 lane the last four.  With X = group
  // 2(s%2) and Y = group 2(s%2)+1 (two packed words each), permlane32_swap exchanges the upper
  // half of X with the lower half of Y: afterwards every lane finds its eight keys as (X, Y).
  bf16x8_t pf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int kb = s >> 1, g0 = 2 * (s & 1);
    const uint32_t x0 = pack_bf16x2(S[kb][4 * g0 + 0], S[kb][4 * g0 + 1]);
    const uint32_t x1 = pack_bf16x2(S[kb][4 * g0 + 2], S[kb][4 * g0 + 3]);
    const uint32_t y0 = pack_bf16x2(S[kb][4 * g0 + 4], S[kb][4 * g0 + 5]);
    const uint32_t y1 = pack_bf16x2(S[kb][4 * g0 + 6], S[kb][4 * g0 + 7]);
    const auto r0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    pf[s] = __builtin_bit_cast(bf16x8_t, make_uint4(r0[0], r1[0], r0[1], r1[1]));
  }

  // O^T blocks: rows = features 32*db + 8*(v/4) + 4*half + v%4, column = this lane's query
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    f32x16_t O;
    const int feat = db * 32 + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(&Vt[feat * VTS + s * 16 + half * 8]);
      O = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], s == 0 ? f32x16_t{} : O, 0, 0, 0);
    }
    if (q < n) {
      bf16_t* o = out + (int64_t)(tok0 + q) * d + h * HD + db * 32 + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = pack_bf16x2(O[4 * g] * inv, O[4 * g + 1] * inv);
        const uint32_t hi = pack_bf16x2(O[4 * g + 2] * inv, O[4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(o + 8 * g) = make_uint2(lo, hi);
      }
    }
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
