// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/audio_encoder.h"

namespace ae {

// ------------------------------------------------------------------------------------------
// storage types
// ------------------------------------------------------------------------------------------
typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__host__ __device__ inline float bf16_to_f32(bf16_t h) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)h << 16;
  return c.f;
}
// Host conversion (weight packing): round to nearest even, NaN kept quiet.
inline bf16_t host_f32_to_bf16(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  if ((c.u & 0x7f800000u) == 0x7f800000u) return (bf16_t)((c.u >> 16) | ((c.u & 0xffff) ? 0x40 : 0));
  c.u += 0x7fffu + ((c.u >> 16) & 1u);
  return (bf16_t)(c.u >> 16);
}
// Device conversion: v_cvt_pk_bf16_f32 (round to nearest even), one instruction per pair.
__device__ inline bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct StoreT;
template <> struct StoreT<float> {
  __device__ static inline void put(float* p, float v) { *p = v; }
};
template <> struct StoreT<bf16_t> {
  __device__ static inline void put(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Exact-form GELU x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).  erfc(z) for z >= 0 is evaluated
// with Abramowitz & Stegun's formula 7.1.28, erfc(z) ~ (1 + a1 z + ... + a6 z^6)^-16
// (|error in erf| <= 3e-7; <= 2e-6 when evaluated in fp32), with no exponential.  Two constant
// factors are folded into the coefficients: z = |x| / sqrt 2 (a_i -> a_i 2^(-i/2), so the
// polynomial runs on t = |x|) and 2^(1/16) (the sixteenth power doubles, so its reciprocal is
// erfc(z) / 2 directly).  Since x Phi(x) = max(x, 0) - |x| erfc(|x| / sqrt 2) / 2 for either
// sign, one FMA finishes it: six FMAs, four squarings, one hardware reciprocal (v_rcp_f32,
// 1 ulp; a correctly rounded division costs ten instructions and buys nothing at this error),
// one max.  The left tail never forms 1 + erf, so it does not cancel; |GELU error| <= 1e-6.
__device__ inline float gelu_erf(float x) {
  const float t = fabsf(x);
  float p = fmaf(t, 5.62129966e-06f, 5.10552090e-05f);  // 2^(1/16) a6 / 8, 2^(1/16) a5 / 2^2.5
  p = fmaf(t, p, 3.96861370e-05f);                     // 2^(1/16) a4 / 4
  p = fmaf(t, p, 3.42273924e-03f);                     // 2^(1/16) a3 / 2^1.5
  p = fmaf(t, p, 2.20769985e-02f);                     // 2^(1/16) a2 / 2
  p = fmaf(t, p, 5.20751630e-02f);                     // 2^(1/16) a1 / 2^0.5
  p = fmaf(t, p, 1.04427378e+00f);                     // 2^(1/16)
  p *= p;
  p *= p;
  p *= p;
  p *= p;
  return fmaf(-t, __builtin_amdgcn_rcpf(p), fmaxf(x, 0.0f));
}
__device__ inline float silu(float x) { return x / (1.0f + expf(-x)); }

// ------------------------------------------------------------------------------------------
// window plan (one entry per attention window; all fields int32)
// ------------------------------------------------------------------------------------------
struct Win {
  int32_t clip;   // clip the window belongs to (its log-mel maximum)
  int32_t start;  // first mel frame within the clip
  int32_t L0, L1, L2, L3;  // valid lengths: frames, after conv1, conv2, conv3 (= tokens)
  int32_t tok;    // first token of the window within its pass
  int32_t mel_row;  // first frame of the window in the packed log-mel buffer (all clips)
};

// One clip of a call: its samples in the packed PCM buffer and its frames in the packed
// log-mel buffer (clips of one call may differ in length).
struct ClipSpan {
  int64_t smp_off;    // first sample
  int64_t n;          // samples
  int64_t frame_off;  // first log-mel frame (row)
};

// Geometry of one pass over a group of windows.  The conv activations hold every window of
// the pass at one time stride: act1 [n_win][L1s][64][C] and act2 [n_win][L2s][32][C], where
// L1s is at least the longest conv1 output of the pass (at most 4W) and L2s = ceil(L1s / 2).
// Windows of short clips thus take only the rows they use.
struct PassGeom {
  const Win* wins;     // device, n_win entries
  int32_t n_win;
  int32_t W;           // window tokens; window frames = 8W
  int32_t L1s, L2s;    // time rows per window of act1 and act2 in this pass
  int64_t n_tok;
  const int32_t* tok_pos;  // device, n_tok entries: position of each token within its window
};

// ------------------------------------------------------------------------------------------
// error plumbing
// ------------------------------------------------------------------------------------------
void set_error(const std::string& msg);
encoder_status hip_fail(hipError_t err, const char* what);

#define AE_HIP(call)                                              \
  do {                                                            \
    hipError_t _e = (call);                                       \
    if (_e != hipSuccess) return ::ae::hip_fail(_e, #call);       \
  } while (0)

// ------------------------------------------------------------------------------------------
// kernel launchers (each returns hipSuccess or the launch error)
// ------------------------------------------------------------------------------------------
struct MelTables {
  const float* twiddle;   // [400][2] cos, sin of 2*pi*j/400
  const float* window;    // [400] periodic Hann
  const int32_t* fb_start;  // [128] first bin of each mel filter
  const int32_t* fb_len;    // [128] taps (<= 16)
  const float* fb_w;        // [128][16] weights
};

// raw log10 mel of the clips in `clips` (device, nclip spans over the packed pcm) -> packed
// mel rows [frame_off + t][128]; per-clip max into max_key[clip] (ordered-uint encoding; must
// be cleared by launch_clear_u32 first).  t_max: frames of the longest clip.
hipError_t launch_log_mel(const float* pcm, const ClipSpan* clips, int32_t nclip, int64_t t_max,
                          const MelTables& t, float* mel, uint32_t* max_key, hipStream_t s);
hipError_t launch_clear_u32(uint32_t* p, int64_t n, hipStream_t s);
// the spans of a [batch, n] call written on the device (no host staging)
hipError_t launch_batch_spans(ClipSpan* spans, int32_t batch, int64_t n, hipStream_t s);
// normalised mel from raw + max keys (in place or out of place)
hipError_t launch_mel_normalize(const float* raw, const uint32_t* max_key, int64_t T,
                                int32_t nclip, float* out, hipStream_t s);

// conv1: raw packed mel (window rows at Win::mel_row) + the clip maxima -> act1
// [n_win][L1s][64][C].  The maxima come as ordered-integer keys (max_key, from the log-mel
// kernel) or, when max_f is not null, as floats.
template <typename T>
hipError_t launch_conv1(const PassGeom& g, const float* mel, const uint32_t* max_key, const float* max_f,
                        const float* w, const float* b, int32_t C, T* act1, hipStream_t s);

// GEMM epilogue kinds
enum Epi : int {
  EPI_BIAS = 0,        // C = acc + bias (dtype)
  EPI_BIAS_GELU = 1,   // C = gelu(acc + bias) (dtype)
  EPI_RESADD = 2,      // Cf32 += acc + bias
  EPI_SWIGLU = 3,      // C[:, n/2] = silu(gate) * up over 32-interleaved columns (dtype)
  EPI_PE = 4,          // Cf32 = acc + pe[pos(row)]
  EPI_STORE_F32 = 5    // Cf32 = acc + bias
};

struct LinearArgs {
  const void* A; int64_t lda;
  const void* W;            // [N, K]
  const float* bias;        // [N] or null
  void* C; int64_t ldc;
  int64_t M; int32_t N; int32_t K;
  // EPI_PE: pe table [window tokens][N] and each row's position within its window
  const float* pe; const int32_t* tok_pos;
  // int4 weight-only B (bf16 path, K % 128 == 0): W is then unused; q [N][K/2], s [N][K/128]
  const uint8_t* Wq = nullptr; const bf16_t* Ws = nullptr;
  // split-K scratch for GEMMs too small to fill the GPU (bf16 path; null: never split)
  float* ws = nullptr; int64_t ws_bytes = 0;
  // bf16 W in K-blocked layout (0: plain [N][K]; else its K block, see below)
  int32_t b_tiled = 0;
};
// split-K scratch each encoder keeps (fp32 partial products of the small-M GEMMs)
constexpr int64_t kSplitKScratchBytes = int64_t(64) << 20;
template <typename T>
hipError_t launch_linear(const LinearArgs& a, int epi, int tag, hipStream_t s);

// implicit-GEMM conv (conv2: level 2, conv3: level 3).  in: level 2 -> act1 [n_win][L1s][64][C],
// level 3 -> act2 [n_win][L2s][32][C]; out: level 2 -> act2; level 3 -> [n_tok][16][C].  wpk:
// [C][9][C] (w_tiled 0) or K-blocked (w_tiled 32: blocks of 16 rows x 32 k, bf16 only)
template <typename T>
hipError_t launch_conv_igemm(const PassGeom& g, int level, const T* in, const T* wpk,
                             const float* bias, int32_t C, T* out, hipStream_t s, int32_t w_tiled = 0);

// K-blocked weight layout read by the staged bf16 kernels (b_tiled / w_tiled = BK): W [N][K]
// stored as blocks of R = 512 / BK rows x BK columns, one kilobyte each, so that every LDS-DMA
// instruction of a K step reads one contiguous kilobyte instead of R row pieces.  Block
// (n / R, k / BK) starts at element ((n / R) * (K / BK) + k / BK) * 512; row n % R of it at
// (n % R) * BK.  Needs N % R == 0 and K % BK == 0.

template <typename T>
hipError_t launch_layernorm(const float* x, const float* g, const float* b, T* y, int64_t M,
                            int32_t D, float eps, hipStream_t s);

template <typename T>
hipError_t launch_attention(const T* qkv, const Win* wins, const int32_t* win2, int32_t n_win,
                            int32_t n_heads, int32_t d, T* out, hipStream_t s);

template <typename T>
hipError_t launch_swiglu_split(const T* gu, int64_t M, int32_t N2, T* out, hipStream_t s);

template <typename T>
hipError_t launch_to_f32(const T* src, int64_t n, float* dst, hipStream_t s);

// mono 16 kHz from interleaved [n_in][channels]: the mean of the channels, resampled with the
// L x 2K polyphase table `taps` (L = M = 1: downmix only)
hipError_t launch_resample(const float* in, int64_t n_in, int32_t channels, int32_t L, int32_t M,
                           int32_t K, const float* taps, float* out, int64_t n_out, hipStream_t s);

// table[pos[i]] = frames[i] for i < n (rows of dim elements); positions outside [0, rows) are
// skipped and counted into *n_skipped (device, may be null).  dim * sizeof(T) % 16 == 0.
template <typename T>
hipError_t launch_splice(const T* frames, int64_t n, int32_t dim, const int64_t* pos, T* table,
                         int64_t rows, int32_t* n_skipped, hipStream_t s);

}  // namespace ae
