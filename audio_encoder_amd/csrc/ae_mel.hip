// Log-mel front end: centred reflect-padded frames, periodic Hann window, one-sided power
// spectrum, Slaney mel filterbank, log10 with a 1e-10 floor and the per-clip maximum
// ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture" row "Audio": 128 mel bins,
// n_fft 400, hop 160, WhisperFeatureExtractor-compatible; "Non-obvious gotchas" item 2: the
// trailing STFT frame is dropped so a clip of N samples has N / 160 frames).
//
// Clips of one call may differ in length: clip c's samples start at clips[c].smp_off of the
// packed PCM and its frames at row clips[c].frame_off of the packed log-mel.
//
// One workgroup computes FB consecutive frames of one clip:
//   1. the FB*160 + 240 samples those frames touch are read once, coalesced, into LDS
//      (reflection at the clip edges is an index map, no padded copy in HBM);
//   2. each frame is windowed and folded about n = 200: with a[n] = w[n] x[n],
//      X[k] = sum_{n=0}^{200} u[n] cos(2 pi k n / 400) - i sum_{n=1}^{199} v[n] sin(2 pi k n / 400)
//      where u[n] = a[n] + a[400-n], v[n] = a[n] - a[400-n] (u[0] = a[0], u[200] = a[200]);
//      this halves the DFT work of a direct 400-point transform of real input;
//   3. the two real DFTs (cosine of u, sine of v) run as fp32 matrix products on MFMA, with the
//      twiddles from an LDS table;
//   4. the 128 sparse filters (<= 16 taps each) reduce the power spectrum, log10 is taken and
//      the block maximum joins the clip maximum through an ordered-integer atomicMax.
#include <algorithm>

#include "ae_internal.h"

namespace ae {
namespace {

constexpr int NFFT = 400;
constexpr int HOP = 160;
constexpr int NB = 201;  // one-sided bins
constexpr int NM = 128;  // mel bins
constexpr int FB = 16;   // frames per workgroup
constexpr int NSMP = (FB - 1) * HOP + NFFT;  // samples spanned by FB frames
constexpr int MAXTAP = 16;
constexpr int NKB = (NB + 15) / 16;    // 16-bin blocks of the DFT
constexpr int NSTEP = (NB + 3) / 4;    // 4-tap steps (the folded rows are zero-padded to 4*NSTEP)

__device__ inline uint32_t float_to_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void log_mel_kernel(const float* __restrict__ pcm,
                                                      const ClipSpan* __restrict__ clips,
                                                      const float* __restrict__ twid,
                                                      const float* __restrict__ hann,
                                                      const int32_t* __restrict__ fb_start,
                                                      const int32_t* __restrict__ fb_len,
                                                      const float* __restrict__ fb_w,
                                                      float* __restrict__ mel,
                                                      uint32_t* __restrict__ max_key) {
  __shared__ float xs[NSMP];
  __shared__ float2 tw[NFFT];
  __shared__ __attribute__((aligned(16))) float us[4 * NSTEP][FB];
  __shared__ __attribute__((aligned(16))) float vs[4 * NSTEP][FB];
  __shared__ float red[4];

  const int tid = threadIdx.x;
  const int clip = blockIdx.y;
  const ClipSpan cs = clips[clip];
  const int64_t N = cs.n, T = N / HOP;
  const int64_t t0 = (int64_t)blockIdx.x * FB;
  if (t0 >= T) return;  // grid spans the longest clip
  const float* x = pcm + cs.smp_off;

  // 1. samples [HOP*t0 - 200, HOP*t0 - 200 + NSMP) with reflection about both clip ends
  const int64_t g0 = HOP * t0 - NFFT / 2;
  for (int j = tid; j < NSMP; j += 256) {
    int64_t g = g0 + j;
    if (g < 0) g = -g;
    if (g >= N) g = 2 * (N - 1) - g;
    xs[j] = (g >= 0 && g < N) ? x[g] : 0.0f;  // out-of-range only for frames >= T
  }
  for (int j = tid; j < NFFT; j += 256) tw[j] = make_float2(twid[2 * j], twid[2 * j + 1]);
  __syncthreads();

  // 2. window and fold
  for (int idx = tid; idx < NB * FB; idx += 256) {
    const int f = idx / NB;
    const int n = idx - f * NB;
    const float* fr = xs + f * HOP;
    const float a = hann[n] * fr[n];
    float u, v;
    if (n == 0 || n == NFFT / 2) {
      u = a;
      v = 0.0f;
    } else {
      const float b = hann[NFFT - n] * fr[NFFT - n];
      u = a + b;
      v = a - b;
    }
    us[n][f] = u;
    vs[n][f] = v;
  }
  for (int idx = tid; idx < (4 * NSTEP - NB) * FB; idx += 256) {
    us[NB + idx / FB][idx % FB] = 0.0f;
    vs[NB + idx / FB][idx % FB] = 0.0f;
  }
  __syncthreads();

  // 3. DFT on fp32 MFMA.  As matrices, RE[f][k] = sum_n U[n][f] cos(2 pi k n / 400) and
  // IM[f][k] = sum_n V[n][f] sin(...).  v_mfma_f32_16x16x4_f32 takes A = 16 frames x 4 taps (lane
  // l: frame l%16, tap n0 + l/16), B = 4 taps x 16 bins (lane l: bin k0 + l%16, tap n0 + l/16)
  // and accumulates D = 16 frames x 16 bins (lane l: bin k0 + l%16, frames 4(l/16) + v).  Each
  // wave takes whole 16-bin blocks; a lane's twiddle index (k n) mod 400 advances by 4k per step.
  // Products and sums are fp32, as in a direct fp32 DFT (only the summation order differs).
  const int wave = tid >> 6, lane = tid & 63;
  const int lf = lane & 15, lq = lane >> 4;
  f32x4_t pwr[(NKB + 3) / 4];
#pragma unroll
  for (int b = 0; b < (NKB + 3) / 4; ++b) {
    const int kb = wave + 4 * b;
    if (kb < NKB) {  // uniform per wave
      const int k = kb * 16 + lf;  // bins past NB are computed and dropped
      const int dang = (4 * k) % NFFT;
      int ang = (k * lq) % NFFT;
      f32x4_t re = {0.0f, 0.0f, 0.0f, 0.0f}, im = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int st = 0; st < NSTEP; ++st) {
        const float2 c = tw[ang];
        re = __builtin_amdgcn_mfma_f32_16x16x4f32(us[4 * st + lq][lf], c.x, re, 0, 0, 0);
        im = __builtin_amdgcn_mfma_f32_16x16x4f32(vs[4 * st + lq][lf], c.y, im, 0, 0, 0);
        ang += dang;
        if (ang >= NFFT) ang -= NFFT;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) pwr[b][v] = re[v] * re[v] + im[v] * im[v];
    }
  }
  __syncthreads();  // us/vs are reused as the power table below
  float* P = &us[0][0];  // [FB][NB]
#pragma unroll
  for (int b = 0; b < (NKB + 3) / 4; ++b) {
    const int kb = wave + 4 * b;
    const int k = kb * 16 + lf;
    if (kb < NKB && k < NB) {
#pragma unroll
      for (int v = 0; v < 4; ++v) P[(4 * lq + v) * NB + k] = pwr[b][v];
    }
  }
  __syncthreads();

  // 4. mel filters, log10, maximum
  float lmax = -INFINITY;
  const int m = tid & (NM - 1);
  const int fh = tid >> 7;  // frames fh, fh+2, ...
  const int s0 = fb_start[m];
  const int nt = fb_len[m];
  for (int f = fh; f < FB; f += 2) {
    const int64_t t = t0 + f;
    if (t >= T) break;
    float acc = 0.0f;
    for (int j = 0; j < nt; ++j) acc = fmaf(fb_w[m * MAXTAP + j], P[f * NB + s0 + j], acc);
    const float l = log10f(fmaxf(acc, 1e-10f));
    mel[(cs.frame_off + t) * NM + m] = l;
    lmax = fmaxf(lmax, l);
  }
  for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
  if ((tid & 63) == 0) red[tid >> 6] = lmax;
  __syncthreads();
  if (tid == 0) {
    const float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (bm > -INFINITY) atomicMax(max_key + clip, float_to_key(bm));
  }
}

__global__ void clear_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__device__ inline float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// (max(L, max - 8) + 4) / 4; raw and out may be the same buffer (each element is read, then
// written, by one thread), so neither is declared restrict
__global__ void mel_normalize_kernel(const float* raw, const uint32_t* __restrict__ mk,
                                     int64_t T, int32_t nclip, float* out) {
  const int64_t total = (int64_t)nclip * T * NM;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t clip = i / (T * NM);
    const float lo = key_to_float(mk[clip]) - 8.0f;
    out[i] = (fmaxf(raw[i], lo) + 4.0f) * 0.25f;
  }
}

}  // namespace

hipError_t launch_log_mel(const float* pcm, const ClipSpan* clips, int32_t nclip, int64_t t_max,
                          const MelTables& t, float* mel, uint32_t* max_key, hipStream_t s) {
  if (nclip < 1 || t_max < 1) return hipSuccess;
  if (nclip > 65535 || (t_max + FB - 1) / FB >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  dim3 grid((unsigned)((t_max + FB - 1) / FB), (unsigned)nclip);
  hipLaunchKernelGGL(log_mel_kernel, grid, dim3(256), 0, s, pcm, clips, t.twiddle, t.window,
                     t.fb_start, t.fb_len, t.fb_w, mel, max_key);
  return hipGetLastError();
}

// spans of a [batch, n] call: clip b at samples b * n, frames b * (n / hop)
__global__ void batch_spans_kernel(ClipSpan* spans, int32_t batch, int64_t n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) spans[b] = ClipSpan{(int64_t)b * n, n, (int64_t)b * (n / HOP)};
}

hipError_t launch_batch_spans(ClipSpan* spans, int32_t batch, int64_t n, hipStream_t s) {
  if (batch < 1) return hipSuccess;
  hipLaunchKernelGGL(batch_spans_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, s, spans, batch, n);
  return hipGetLastError();
}

hipError_t launch_clear_u32(uint32_t* p, int64_t n, hipStream_t s) {
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(clear_u32_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_mel_normalize(const float* raw, const uint32_t* max_key, int64_t T,
                                int32_t nclip, float* out, hipStream_t s) {
  const int64_t total = (int64_t)nclip * T * NM;
  int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(mel_normalize_kernel, dim3(blocks), dim3(256), 0, s, raw, max_key, T, nclip,
                     out);
  return hipGetLastError();
}

}  // namespace ae
