// Host side of the C ABI (include/audio_encoder.h): configuration checks, the window planner,
// weight packing, workspace management and the order of kernel launches of one forward pass.
//
// Forward pass ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture"):
//   log-mel (+ per-clip max) -> conv1 -> conv2 -> conv3 -> conv_out + positions ->
//   n_layers x [LN1 -> QKV -> windowed attention -> out-proj + residual ->
//               LN2 -> FFN1 + GELU -> FFN2 + residual] ->
//   ln_post -> proj1 + GELU -> proj2 -> gate|up + SwiGLU -> down.
// Windows are the independent units (8*W mel frames each, zero time-padding at their own
// edges, positions restarting at 0), so a call is split into passes of whole windows that fit
// the workspace; the long-audio path groups whole 64 s pieces per pass ("SILVERTHRONE/Ossicle-4B"
// card, "Long Audio").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <mutex>
#include <thread>
#include <vector>

#include "ae_internal.h"

namespace ae {

// Scratch of the allocation-free entry point (encoder_log_mel_noalloc): clip spans and the
// per-clip maximum keys of up to kScratchClips clips.  One copy per GPU, held until the
// process ends; its device address is looked up once per device (scratch_on_device) and
// passed to the kernels; host code never uses the array's name as an address.
constexpr int32_t kScratchClips = 4096;
constexpr int64_t kScratchSpanBytes = ((int64_t)kScratchClips * (int64_t)sizeof(ClipSpan) + 255) & ~int64_t(255);
constexpr int64_t kScratchBytes = kScratchSpanBytes + (int64_t)kScratchClips * 4;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }
encoder_status hip_fail(hipError_t err, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(err));
  return err == hipErrorOutOfMemory ? ENC_E_OUT_OF_MEMORY : ENC_E_DEVICE;
}

static encoder_status invalid(const std::string& msg) {
  set_error(msg);
  return ENC_E_INVALID_ARG;
}

// ------------------------------------------------------------------------------------------
// configuration
// ------------------------------------------------------------------------------------------
// The GEMM and conv kernels address their operands through buffer descriptors with 32-bit
// byte offsets, so no operand of a pass may exceed this many bytes.
constexpr int64_t kMaxOperandBytes = 0x7fffffff;

static encoder_status check_cfg(const encoder_cfg* c) {
  if (!c) return invalid("cfg is NULL");
  if (c->n_fft != 400 || c->hop != 160 || c->n_mels != 128)
    return invalid("the front end is fixed at n_fft=400, hop=160, n_mels=128");
  if (c->conv_channels <= 0 || c->conv_channels % 32 != 0)
    return invalid("conv_channels must be a positive multiple of 32");
  if (c->head_dim != 64) return invalid("head_dim must be 64");
  if (c->n_heads <= 0 || c->n_heads * c->head_dim != c->d_model)
    return invalid("n_heads * head_dim must equal d_model");
  if (c->d_model % 64 || c->d_ffn <= 0 || c->d_ffn % 64 || c->d_out <= 0 || c->d_out % 64 ||
      c->d_adapter <= 0 || c->d_adapter % 64)
    return invalid("d_model, d_ffn, d_out and d_adapter must be positive multiples of 64");
  if (c->n_layers < 0) return invalid("n_layers must be >= 0");
  if (c->window_tokens < 1 || c->window_tokens > 128)
    return invalid("window_tokens must be in [1, 128]");
  if (c->piece_tokens < c->window_tokens || c->piece_tokens % c->window_tokens)
    return invalid("piece_tokens must be a positive multiple of window_tokens");
  if (c->dtype != ENC_BF16 && c->dtype != ENC_F32) return invalid("dtype must be ENC_BF16 or ENC_F32");
  if (!(c->ln_eps > 0.0f)) return invalid("ln_eps must be > 0");
  if (c->max_tokens_per_pass < 0) return invalid("max_tokens_per_pass must be >= 0");
  if (c->max_tokens_per_pass > 0 && c->max_tokens_per_pass < c->window_tokens)
    return invalid("max_tokens_per_pass must hold at least one window");
  if (c->weight_bits != 0 && c->weight_bits != 16 && c->weight_bits != 4)
    return invalid("weight_bits must be 16 (or 0) or 4");
  if (c->split_small_gemms != 0 && c->split_small_gemms != 1)
    return invalid("split_small_gemms must be 0 or 1");
  if (c->weight_bits == 4) {
    if (c->dtype != ENC_BF16) return invalid("int4 weights need dtype ENC_BF16");
    if (c->d_model % 128 || c->d_ffn % 128 || c->d_out % 128 || c->d_adapter % 128)
      return invalid("int4 weights need d_model, d_ffn, d_out and d_adapter multiples of 128");
  }
  {
    // one full window must fit one pass, and every weight matrix one buffer descriptor
    const int64_t es = c->dtype == ENC_BF16 ? 2 : 4;
    const int64_t C = c->conv_channels, d = c->d_model;
    const int64_t tb = std::max<int64_t>({16 * C * es, 3 * d * es, 4 * d, (int64_t)c->d_ffn * es,
                                          2 * (int64_t)c->d_adapter * es, (int64_t)c->d_out * es});
    if (4 * (int64_t)c->window_tokens * 64 * C * es > kMaxOperandBytes ||
        (int64_t)c->window_tokens * tb > kMaxOperandBytes)
      return invalid("one window's activations exceed 2^31 - 1 bytes");
    const int64_t wmax = std::max<int64_t>({9 * C * C, 16 * C * d, 3 * d * d, (int64_t)c->d_ffn * d,
                                            (int64_t)c->d_out * d, 2 * (int64_t)c->d_adapter * c->d_out});
    if (wmax * es > kMaxOperandBytes) return invalid("a weight matrix exceeds 2^31 - 1 bytes");
  }
  if (c->sample_rate != 16000) {
    set_error("only 16 kHz input is supported (no resampling)");
    return ENC_E_UNSUPPORTED;
  }
  return ENC_OK;
}

static int64_t max_tokens(const encoder_cfg& c) {
  return c.max_tokens_per_pass > 0 ? c.max_tokens_per_pass : 8192;
}
static int64_t elem_bytes(const encoder_cfg& c) { return c.dtype == ENC_BF16 ? 2 : 4; }

// Bytes per token of the largest per-token operand of a pass: conv3's output (16C), the qkv
// (3d), the fp32 residual, the FFN / head / adapter hidden rows and the output rows.
static int64_t token_bytes(const encoder_cfg& c) {
  const int64_t es = elem_bytes(c);
  return std::max<int64_t>({16 * (int64_t)c.conv_channels * es, 3 * (int64_t)c.d_model * es,
                            4 * (int64_t)c.d_model, (int64_t)c.d_ffn * es, 2 * (int64_t)c.d_adapter * es,
                            (int64_t)c.d_out * es});
}
// Bytes of one time row of conv1's output (64 frequencies x C channels); act1 of a pass is
// windows x L1s of them, the largest conv operand (conv2's A).
static int64_t act1_row_bytes(const encoder_cfg& c) { return 64 * (int64_t)c.conv_channels * elem_bytes(c); }
// tokens one pass may hold: the configured bound, capped by the per-token operands
static int64_t pass_token_cap(const encoder_cfg& c) {
  return std::min<int64_t>(max_tokens(c), kMaxOperandBytes / token_bytes(c));
}
// Passes of one call that run at once (each lane holds one pass's activations).  HIP maps
// streams onto four hardware queues by default; three lanes plus the caller's stream keep one
// queue each.  An hour at one 64 s piece per pass (57 passes) measured 160 ms with four lanes,
// 153 with two, 130 with three, 141 / 130 / 131 / 144 with five to eight.
constexpr int kLanes = 3;
// A single-pass call of at least this many tokens runs as two concurrent halves.  Measured on
// MI355X with 30 s clips: 12 clips (4500 tokens) 11.8 -> 11.1 ms, 16 clips 13.8 -> 13.2 ms;
// at 3750 tokens the halves are too small to gain (9.9 -> 10.1 ms).
constexpr int64_t kSplitTokens = 4000;

struct TensorSpec { const char* name; int64_t n; };

// blob order, see encoder_weight_count in the header
static std::vector<int64_t> blob_sizes(const encoder_cfg& c) {
  const int64_t C = c.conv_channels, d = c.d_model, f = c.d_ffn, o = c.d_out, a = c.d_adapter;
  std::vector<int64_t> s = {C * 9, C, C * C * 9, C, C * C * 9, C, d * C * 16};
  for (int i = 0; i < c.n_layers; ++i) {
    const int64_t L[] = {d, d, d * d, d, d * d, d, d * d, d, d * d, d, d, d, f * d, f, d * f, d};
    s.insert(s.end(), std::begin(L), std::end(L));
  }
  const int64_t H[] = {d, d, d * d, d, o * d, o, a * o, a * o, o * a};
  s.insert(s.end(), std::begin(H), std::end(H));
  return s;
}

// ------------------------------------------------------------------------------------------
// window plan
// ------------------------------------------------------------------------------------------
// Clips are laid out back to back: clip b's samples start at the sum of the earlier lengths,
// its log-mel frames at the sum of the earlier frame counts, and its windows follow those of
// clip b-1 in the token stream (so its output rows do too).
static void clip_spans(const encoder_cfg& c, const std::vector<int64_t>& lens,
                       std::vector<ClipSpan>& out) {
  out.clear();
  int64_t so = 0, fo = 0;
  for (int64_t n : lens) {
    out.push_back(ClipSpan{so, n, fo});
    so += n;
    fo += n / c.hop;
  }
}

static void plan_windows(const encoder_cfg& c, const std::vector<int64_t>& lens,
                         std::vector<Win>& out) {
  const int64_t wf = 8 * (int64_t)c.window_tokens;
  out.clear();
  int64_t tok = 0, fo = 0;
  for (size_t b = 0; b < lens.size(); ++b) {
    const int64_t T = lens[b] / c.hop;
    for (int64_t s = 0; s < T; s += wf) {
      Win w;
      w.clip = (int32_t)b;
      w.start = (int32_t)s;
      w.L0 = (int32_t)std::min<int64_t>(wf, T - s);
      w.L1 = (w.L0 + 1) / 2;
      w.L2 = (w.L1 + 1) / 2;
      w.L3 = (w.L2 + 1) / 2;
      w.tok = (int32_t)tok;
      w.mel_row = (int32_t)(fo + s);
      tok += w.L3;
      out.push_back(w);
    }
    fo += T;
  }
}

static int64_t frames_out(const encoder_cfg& c, int64_t n_samples) {
  const int64_t T = n_samples / c.hop;
  const int64_t wf = 8 * (int64_t)c.window_tokens;
  const int64_t full = T / wf, r = T % wf;
  int64_t f = full * c.window_tokens;
  if (r) f += (((r + 1) / 2 + 1) / 2 + 1) / 2;
  return f;
}

// ------------------------------------------------------------------------------------------
// input conditioning (resampling to 16 kHz; the filter is described in ae_resample.hip)
// ------------------------------------------------------------------------------------------
struct ResamplePlan { int32_t L = 1, M = 1, K = 0; };

static int64_t gcd64(int64_t a, int64_t b) {
  while (b) { const int64_t t = a % b; a = b; b = t; }
  return a;
}

// L/M = 16000/fs in lowest terms; K = taps on each side.  Returns false for rates this build
// does not handle (more than 4096 phases, or more than 32x downsampling).
static bool resample_plan(int32_t fs, ResamplePlan& r) {
  if (fs <= 0) return false;
  const int64_t g = gcd64(fs, 16000);
  r.L = (int32_t)(16000 / g);
  r.M = (int32_t)(fs / g);
  if (r.L == 1 && r.M == 1) { r.K = 0; return true; }
  if (r.L > 4096 || r.M > 32 * r.L) return false;
  const double fc = 0.5 * 0.945 * std::min(1.0, (double)r.L / r.M);
  const double R = 16.0 / (2.0 * fc);
  r.K = (int32_t)std::ceil(R);
  return true;
}

static std::vector<float> resample_taps(const ResamplePlan& r) {
  const double fc = 0.5 * 0.945 * std::min(1.0, (double)r.L / r.M);
  const double R = 16.0 / (2.0 * fc);
  const double pi = 3.14159265358979323846;
  std::vector<float> t((size_t)r.L * 2 * r.K);
  std::vector<double> h((size_t)2 * r.K);
  for (int32_t p = 0; p < r.L; ++p) {
    const double frac = (double)p / r.L;
    double sum = 0.0;
    for (int32_t k = 0; k < 2 * r.K; ++k) {
      const double dd = (double)(k - r.K + 1) - frac;  // input sample minus output position
      double v = 0.0;
      if (std::fabs(dd) <= R) {
        const double x = 2.0 * fc * dd;
        const double sinc = x == 0.0 ? 1.0 : std::sin(pi * x) / (pi * x);
        v = 2.0 * fc * sinc * 0.5 * (1.0 + std::cos(pi * dd / R));
      }
      h[k] = v;
      sum += v;
    }
    for (int32_t k = 0; k < 2 * r.K; ++k) t[(size_t)p * 2 * r.K + k] = (float)(h[k] / sum);
  }
  return t;
}

static int64_t conditioned_length(int64_t n_in, const ResamplePlan& r) {
  return (n_in * r.L + r.M - 1) / r.M;
}

// One pass: windows [win0, win0 + nwin) = tokens [tok0, tok0 + ntok) of the call, with the
// conv activations at time strides L1s / L2s (PassGeom).
struct Pass { int64_t win0, nwin, tok0, ntok; int32_t L1s, L2s; };

// Consecutive windows grouped into passes.  A pass ends where `boundary(window)` says so, where
// the next window would take it past `mt` tokens, or where its act1 (windows x L1s rows, L1s
// the longest conv1 output of the pass, or 4W for `full` strides) would exceed the bytes a
// buffer descriptor addresses; act2 and every per-token operand are then addressable too.
template <class F>
static std::vector<Pass> split_passes(const encoder_cfg& c, const std::vector<Win>& w, int64_t mt,
                                      bool full, F boundary) {
  const int32_t L1full = 4 * c.window_tokens;
  const int64_t rowb = act1_row_bytes(c);
  std::vector<Pass> ps;
  Pass cur{0, 0, 0, 0, 0, 0};
  for (size_t i = 0; i < w.size(); ++i) {
    const int32_t l1 = full ? L1full : std::max(cur.L1s, w[i].L1);
    const bool fits = cur.ntok + w[i].L3 <= mt && (cur.nwin + 1) * (int64_t)l1 * rowb <= kMaxOperandBytes;
    if (cur.nwin > 0 && (!fits || boundary((int64_t)i))) {
      ps.push_back(cur);
      cur = Pass{(int64_t)i, 0, w[i].tok, 0, 0, 0};
    }
    if (cur.nwin == 0) cur.tok0 = w[i].tok, cur.win0 = (int64_t)i;
    cur.nwin += 1;
    cur.ntok += w[i].L3;
    cur.L1s = full ? L1full : std::max(cur.L1s, w[i].L1);
    cur.L2s = (cur.L1s + 1) / 2;
  }
  if (cur.nwin) ps.push_back(cur);
  return ps;
}

// Passes a call runs in.  piece_windows > 0: long mode, passes start only at multiples of it.
// A call that fits one pass but holds at least kSplitTokens tokens runs as two halves of whole
// windows (whole pieces in long mode), unless `halves` is false.  `full`: act1/act2 keep the
// documented padded layout of 4W / 2W rows per window (the stage-wise debug exports).
static std::vector<Pass> plan_passes(const encoder_cfg& c, const std::vector<Win>& wins,
                                     int64_t piece_windows, bool halves, bool full) {
  const int64_t mt = pass_token_cap(c);
  std::vector<Pass> ps = split_passes(c, wins, mt, full, [&](int64_t i) {
    return piece_windows > 0 && i % piece_windows == 0;
  });
  // The passes of a call run concurrently on lanes, and two passes' kernels overlap where one
  // pass alone leaves the GPU partly idle (attention, LayerNorm, a GEMM's last round of tiles).
  // A window's rows are the same in any pass.
  if (halves && ps.size() == 1 && ps[0].ntok >= kSplitTokens) {
    std::vector<Pass> two;
    if (piece_windows > 0) {
      const int64_t pw = c.piece_tokens / c.window_tokens;  // windows per piece
      const int64_t np = (ps[0].nwin + pw - 1) / pw;
      if (np >= 2) {
        const int64_t b = (np / 2) * pw;
        two = split_passes(c, wins, mt, full, [&](int64_t i) { return i == b; });
      }
    } else {
      const int64_t half = (ps[0].ntok + 1) / 2;
      two = split_passes(c, wins, half + c.window_tokens - 1, full, [](int64_t) { return false; });
    }
    if (two.size() == 2) ps.swap(two);
  }
  return ps;
}

// ------------------------------------------------------------------------------------------
// host tables: twiddles, window, Slaney filterbank, positions
// ------------------------------------------------------------------------------------------
static void mel_host_tables(std::vector<float>& tw, std::vector<float>& win,
                            std::vector<int32_t>& fstart, std::vector<int32_t>& flen,
                            std::vector<float>& fw) {
  const double PI = 3.14159265358979323846;
  tw.resize(800);
  win.resize(400);
  for (int j = 0; j < 400; ++j) {
    tw[2 * j] = (float)std::cos(2.0 * PI * j / 400.0);
    tw[2 * j + 1] = (float)std::sin(2.0 * PI * j / 400.0);
    win[j] = (float)(0.5 - 0.5 * std::cos(2.0 * PI * j / 400.0));
  }
  // Slaney mel scale: 3 mel per 200 Hz below 1 kHz, then 27 mel per factor 6.4
  auto hz2mel = [](double f) {
    return f < 1000.0 ? f * 3.0 / 200.0 : 15.0 + std::log(f / 1000.0) * 27.0 / std::log(6.4);
  };
  auto mel2hz = [](double m) {
    return m < 15.0 ? m * 200.0 / 3.0 : 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0);
  };
  const double top = hz2mel(8000.0);
  double edge[130];
  for (int i = 0; i < 130; ++i) edge[i] = mel2hz(top * i / 129.0);
  fstart.assign(128, 0);
  flen.assign(128, 0);
  fw.assign(128 * 16, 0.0f);
  for (int m = 0; m < 128; ++m) {
    const double lo = edge[m], ce = edge[m + 1], hi = edge[m + 2];
    const double norm = 2.0 / (hi - lo);
    int first = -1, cnt = 0;
    for (int k = 0; k <= 200; ++k) {
      const double f = 40.0 * k;
      const double v = std::max(0.0, std::min((f - lo) / (ce - lo), (hi - f) / (hi - ce))) * norm;
      if (v > 0.0) {
        if (first < 0) first = k;
        const int j = k - first;
        if (j < 16) fw[m * 16 + j] = (float)v;
        cnt = j + 1;
      }
    }
    fstart[m] = first < 0 ? 0 : first;
    flen[m] = std::min(cnt, 16);
  }
}

static std::vector<float> pe_table(int W, int d) {
  std::vector<float> pe((size_t)W * d);
  const int h = d / 2;
  for (int p = 0; p < W; ++p)
    for (int i = 0; i < h; ++i) {
      const double om = std::exp(-std::log(10000.0) * i / (double)(h - 1));
      pe[(size_t)p * d + i] = (float)std::sin(p * om);
      pe[(size_t)p * d + h + i] = (float)std::cos(p * om);
    }
  return pe;
}

template <class F>
static void parallel_for(int64_t n, F fn) {
  const int nt = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < (1 << 20) || nt == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t step = (n + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    const int64_t a = t * step, b = std::min(n, a + step);
    if (a < b) th.emplace_back([=] { fn(a, b); });
  }
  for (auto& x : th) x.join();
}

// ------------------------------------------------------------------------------------------
// int4 weight-only quantisation (round to nearest, groups of 128 along K, bf16 scales)
// ------------------------------------------------------------------------------------------
// Row n, group g: s = bf16(max |w| / 7); q = clamp(rint(w / s), -8, 7) (0 when s == 0); the
// weight used on the GPU is bf16(q * s).  q is packed two per byte, even k in the low nibble.
static void quantize_int4_rows(const float* w, int64_t N, int64_t K, uint8_t* q, bf16_t* sc) {
  const int64_t G = K / 128;
  parallel_for(N, [&](int64_t a, int64_t b) {
    for (int64_t n = a; n < b; ++n) {
      const float* row = w + n * K;
      for (int64_t g = 0; g < G; ++g) {
        double mx = 0.0;
        for (int j = 0; j < 128; ++j) mx = std::max(mx, std::fabs((double)row[g * 128 + j]));
        const bf16_t sb = host_f32_to_bf16((float)(mx / 7.0));
        sc[n * G + g] = sb;
        const double sd = (double)bf16_to_f32(sb);
        for (int j = 0; j < 128; j += 2) {
          int v[2];
          for (int e = 0; e < 2; ++e) {
            const double x = sd > 0.0 ? std::nearbyint((double)row[g * 128 + j + e] / sd) : 0.0;
            v[e] = (int)std::min(7.0, std::max(-8.0, x));
          }
          q[n * (K / 2) + (g * 128 + j) / 2] = (uint8_t)((v[0] & 0xf) | ((v[1] & 0xf) << 4));
        }
      }
    }
  });
}


}  // namespace ae

using namespace ae;

// ------------------------------------------------------------------------------------------
// handle
// ------------------------------------------------------------------------------------------
// One linear weight [N, K] on the device: bf16/f32 (w) or int4 + bf16 scales (q, s).
struct WMat {
  void* w = nullptr;
  const uint8_t* q = nullptr;
  const bf16_t* s = nullptr;
  int32_t blk = 0;  // w in the K-blocked layout with this K block (0: plain [N][K])
};

struct LayerW {
  WMat wqkv, wo, w1, w2;
  float *bqkv, *bo, *b1, *b2, *ln1g, *ln1b, *ln2g, *ln2b;
};

struct TimedLaunch { int kid; hipEvent_t a, b; };

struct encoder {
  encoder_cfg cfg;
  int device = 0;
  bool bf16 = true;
  size_t esz = 2;
  // packed parameters
  void* wdev = nullptr;   // dtype weights
  uint8_t* qdev = nullptr;  // int4 weights and their scales (weight_bits = 4)
  float* fdev = nullptr;  // float32 parameters and tables
  int64_t wbytes = 0, fbytes = 0, qbytes = 0;
  float *conv1_w, *conv1_b, *conv2_b, *conv3_b;
  void *conv2_w, *conv3_w;
  int32_t conv_blk = 0;  // K block of conv2_w / conv3_w (0: plain [C][9][C])
  WMat conv_out_w;
  std::vector<LayerW> layers;
  float *lnp_g, *lnp_b, *proj1_b, *proj2_b;
  WMat proj1_w, proj2_w, gateup_w, down_w;
  float* pe;
  MelTables mel;
  // workspace (grown on demand)
  struct Buf { void* p = nullptr; int64_t bytes = 0; };
  Buf mel_raw, max_key, ctab, wtab, tpos, dbg;
  // Activation workspace of one pass.  The passes of a call are independent (windows are), so
  // they run round-robin on up to kLanes lanes at once, each with its own stream and buffers.
  struct Lane {
    Buf act1, act2, tokA, resid, xn, qkv, attn, hid, hid2, z;
    Buf splitk;                    // fp32 partial products of split-K GEMMs (bf16 path)
    hipStream_t stream = nullptr;  // created on first concurrent use
    hipEvent_t done = nullptr;
  };
  std::vector<Lane> lanes;
  hipEvent_t passes_ready = nullptr;
  // recorded on the caller's stream at the end of every call that used the workspace: a buffer
  // that must grow waits for it before the old one is freed (one call is in flight per handle)
  hipEvent_t call_done = nullptr;
  bool call_pending = false;
  // the allocation-free entry point's scratch on this handle's device (null: unavailable)
  void* scratch = nullptr;
  hipError_t scratch_err = hipSuccess;
  Buf rs_taps;            // polyphase table of the last input-conditioning rate
  int32_t rs_rate = 0;
  int64_t ws_bytes = 0, ws_peak = 0;
  // host staging for the plan upload
  void* pinned = nullptr;
  int64_t pinned_bytes = 0;
  hipEvent_t upload_done = nullptr;
  // timing: 0 off; 1 the passes of an untimed call, one after another on one lane; 2 as 1 but
  // a call that fits one pass is not split into halves
  int timing = 0;
  hipError_t timing_err = hipSuccess;  // first failed event record of the current call
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> event_pool;
  size_t event_next = 0;
};

namespace {

encoder_status ensure(encoder* e, encoder::Buf& b, int64_t bytes) {
  if (b.bytes >= bytes) return ENC_OK;
  if (b.p) {
    // the old buffer may still be read by the previous call's queued work
    if (e->call_pending) {
      AE_HIP(hipEventSynchronize(e->call_done));
      e->call_pending = false;
    }
    AE_HIP(hipFree(b.p));
    e->ws_bytes -= b.bytes;
    b.p = nullptr;
    b.bytes = 0;
  }
  const int64_t want = (bytes + 4095) & ~int64_t(4095);
  if (getenv("ENCODER_FAIL_ALLOC")) {
    set_error("allocation refused (ENCODER_FAIL_ALLOC is set)");
    return ENC_E_OUT_OF_MEMORY;
  }
  hipError_t err = hipMalloc(&b.p, want);
  if (err != hipSuccess) {
    b.p = nullptr;
    return hip_fail(err, "hipMalloc(workspace)");
  }
  b.bytes = want;
  e->ws_bytes += want;
  e->ws_peak = std::max(e->ws_peak, e->ws_bytes);
  return ENC_OK;
}

hipEvent_t next_event(encoder* e) {
  if (e->event_next == e->event_pool.size()) {
    hipEvent_t ev;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    e->event_pool.push_back(ev);
  }
  return e->event_pool[e->event_next++];
}

// Brackets one launch with events when timing is on.  A failed event creation or record is
// kept in e->timing_err (the first one of the call) and reported by LAUNCH.
struct Tm {
  encoder* e;
  int kid;
  hipStream_t s;
  hipEvent_t a = nullptr;
  void note(hipError_t err) {
    if (err != hipSuccess && e->timing_err == hipSuccess) e->timing_err = err;
  }
  Tm(encoder* e_, int k, hipStream_t s_) : e(e_), kid(k), s(s_) {
    if (!e->timing) return;
    a = next_event(e);
    if (!a) {
      note(hipErrorOutOfMemory);
      return;
    }
    const hipError_t err = hipEventRecord(a, s);
    if (err != hipSuccess) {
      a = nullptr;
      note(err);
    }
  }
  ~Tm() {
    if (!a) return;
    hipEvent_t b = next_event(e);
    const hipError_t err = b ? hipEventRecord(b, s) : hipErrorOutOfMemory;
    if (err != hipSuccess) {
      note(err);
      return;
    }
    e->timed.push_back({kid, a, b});
  }
};

#define LAUNCH(kid, call)                                                          \
  do {                                                                             \
    hipError_t _err;                                                               \
    {                                                                              \
      Tm _tm(e, kid, s);                                                           \
      _err = (call);                                                               \
    }                                                                              \
    if (_err != hipSuccess) return hip_fail(_err, #call);                          \
    if (e->timing_err != hipSuccess) return hip_fail(e->timing_err, "hipEventRecord"); \
  } while (0)

// log-mel of n_frames frames over nclip clips
encoder_status size_mel(encoder* e, int64_t nclip, int64_t n_frames) {
  encoder_status st;
  if ((st = ensure(e, e->mel_raw, std::max<int64_t>(n_frames, 1) * 128 * 4))) return st;
  if ((st = ensure(e, e->max_key, std::max<int64_t>(nclip, 1) * 4))) return st;
  return ensure(e, e->ctab, std::max<int64_t>(nclip, 1) * (int64_t)sizeof(ClipSpan));
}

// the log-mel, window table and token positions of a call
encoder_status size_call(encoder* e, int64_t nclip, int64_t n_frames, int64_t n_win_total,
                         int64_t n_tok_total) {
  encoder_status st;
  if ((st = size_mel(e, nclip, n_frames))) return st;
  if ((st = ensure(e, e->wtab, n_win_total * (int64_t)sizeof(Win)))) return st;
  return ensure(e, e->tpos, std::max<int64_t>(n_tok_total, 1) * 4);
}

// activation workspace of one lane for passes of up to mt tokens, rows1 act1 time rows
// (windows x L1s) and rows2 act2 time rows (windows x L2s)
encoder_status size_lane(encoder* e, encoder::Lane& ln, int64_t mt, int64_t rows1, int64_t rows2) {
  const encoder_cfg& c = e->cfg;
  const int64_t es = (int64_t)e->esz, C = c.conv_channels, d = c.d_model;
  encoder_status st;
  if ((st = ensure(e, ln.act1, rows1 * 64 * C * es))) return st;
  if ((st = ensure(e, ln.act2, rows2 * 32 * C * es))) return st;
  if ((st = ensure(e, ln.tokA, mt * 16 * C * es))) return st;
  if ((st = ensure(e, ln.resid, mt * d * 4))) return st;
  if ((st = ensure(e, ln.xn, mt * d * es))) return st;
  if ((st = ensure(e, ln.qkv, mt * 3 * d * es))) return st;
  if ((st = ensure(e, ln.attn, mt * d * es))) return st;
  const int64_t hidw = std::max<int64_t>({c.d_ffn, d, c.d_adapter});
  if ((st = ensure(e, ln.hid, mt * hidw * es))) return st;
  if (!e->bf16 && (st = ensure(e, ln.hid2, mt * 2 * c.d_adapter * es))) return st;
  if ((st = ensure(e, ln.z, mt * c.d_out * es))) return st;
  if (e->bf16 && c.split_small_gemms && (st = ensure(e, ln.splitk, kSplitKScratchBytes))) return st;
  return ENC_OK;
}

// clip spans, plan and per-pass relative token indices, uploaded once per call
encoder_status upload_plan(encoder* e, const std::vector<ClipSpan>& clips, const std::vector<Win>& wins,
                           const std::vector<Pass>& ps, hipStream_t s) {
  std::vector<Win> rel(wins);
  int64_t ntok = 0;
  for (const Pass& p : ps) ntok += p.ntok;
  std::vector<int32_t> tp((size_t)ntok);
  for (const Pass& p : ps)
    for (int64_t i = p.win0; i < p.win0 + p.nwin; ++i) {
      rel[i].tok = (int32_t)(wins[i].tok - p.tok0);
      for (int j = 0; j < wins[i].L3; ++j) tp[wins[i].tok + j] = j;
    }
  const int64_t wb = (int64_t)rel.size() * (int64_t)sizeof(Win), tb = ntok * 4;
  const int64_t cb = (int64_t)clips.size() * (int64_t)sizeof(ClipSpan);
  if (e->pinned_bytes < cb + wb + tb) {
    if (e->pinned) {
      AE_HIP(hipEventSynchronize(e->upload_done));
      AE_HIP(hipHostFree(e->pinned));
      e->pinned = nullptr;
      e->pinned_bytes = 0;
    }
    AE_HIP(hipHostMalloc(&e->pinned, cb + wb + tb, hipHostMallocDefault));
    e->pinned_bytes = cb + wb + tb;
  }
  AE_HIP(hipEventSynchronize(e->upload_done));  // the previous upload has left the staging area
  char* hp = (char*)e->pinned;
  if (cb) std::memcpy(hp, clips.data(), cb);
  if (wb) std::memcpy(hp + cb, rel.data(), wb);
  if (tb) std::memcpy(hp + cb + wb, tp.data(), tb);
  if (cb) AE_HIP(hipMemcpyAsync(e->ctab.p, hp, cb, hipMemcpyHostToDevice, s));
  if (wb) AE_HIP(hipMemcpyAsync(e->wtab.p, hp + cb, wb, hipMemcpyHostToDevice, s));
  if (tb) AE_HIP(hipMemcpyAsync(e->tpos.p, hp + cb + wb, tb, hipMemcpyHostToDevice, s));
  AE_HIP(hipEventRecord(e->upload_done, s));
  return ENC_OK;
}

template <typename T>
encoder_status launch_linear_t(encoder* e, encoder::Lane& ln, int kid, const void* A, int64_t lda, const WMat& Wt,
                               const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                               int epi, hipStream_t s, const float* pe = nullptr,
                               const int32_t* tok_pos = nullptr) {
  LinearArgs a{A, lda, Wt.w, bias, C, ldc, M, N, K, pe, tok_pos, Wt.q, Wt.s,
               (float*)ln.splitk.p, ln.splitk.bytes, Wt.blk};
  LAUNCH(kid, launch_linear<T>(a, epi, kid, s));
  return ENC_OK;
}

// stage ids of encoder_debug_stage
enum { ST_MEL = 0, ST_CONV1, ST_CONV2, ST_CONV3, ST_EMBED, ST_LAYER, ST_HEAD, ST_OUT };

// Residual-stream exports: after layer layers[t], rows [tok0, tok0 + ntok) of the pass go to
// dst[t][tok0 ..][d_model] (float32), ntok_total rows per tap.
struct TapReq {
  const int32_t* layers = nullptr;
  int32_t n = 0;
  float* dst = nullptr;
  int64_t ntok_total = 0;
};

// One pass over windows [p.win0, p.win0 + p.nwin): conv stack -> ... -> adapter, writing
// rows [p.tok0, p.tok0 + p.ntok) of `out`.  Stops after `stop` (debug) when stop >= 0.
template <typename T>
encoder_status run_pass(encoder* e, encoder::Lane& ln, const Pass& p, void* out, hipStream_t s,
                        int stop = -1, int stop_layer = -1, const TapReq* taps = nullptr) {
  const encoder_cfg& c = e->cfg;
  const int C = c.conv_channels, d = c.d_model, W = c.window_tokens;
  PassGeom g;
  g.wins = reinterpret_cast<const Win*>(e->wtab.p) + p.win0;
  g.n_win = (int32_t)p.nwin;
  g.W = W;
  g.L1s = p.L1s;
  g.L2s = p.L2s;
  g.n_tok = p.ntok;
  g.tok_pos = reinterpret_cast<const int32_t*>(e->tpos.p) + p.tok0;
  const int64_t M = p.ntok;
  T* act1 = (T*)ln.act1.p;
  T* act2 = (T*)ln.act2.p;
  T* tokA = (T*)ln.tokA.p;
  float* resid = (float*)ln.resid.p;
  T* xn = (T*)ln.xn.p;
  T* qkv = (T*)ln.qkv.p;
  T* attn = (T*)ln.attn.p;
  T* hid = (T*)ln.hid.p;
  T* z = (T*)ln.z.p;

  LAUNCH(ENC_K_CONV1, launch_conv1<T>(g, (const float*)e->mel_raw.p, (const uint32_t*)e->max_key.p,
                                      nullptr, e->conv1_w, e->conv1_b, C, act1, s));
  if (stop == ST_CONV1) return ENC_OK;
  LAUNCH(ENC_K_CONV2, launch_conv_igemm<T>(g, 2, act1, (const T*)e->conv2_w, e->conv2_b, C, act2, s, e->conv_blk));
  if (stop == ST_CONV2) return ENC_OK;
  LAUNCH(ENC_K_CONV3, launch_conv_igemm<T>(g, 3, act2, (const T*)e->conv3_w, e->conv3_b, C, tokA, s, e->conv_blk));
  if (stop == ST_CONV3) return ENC_OK;
  encoder_status st;
  if ((st = launch_linear_t<T>(e, ln, ENC_K_CONV_OUT, tokA, 16 * C, e->conv_out_w, nullptr, resid, d, M,
                               d, 16 * C, EPI_PE, s, e->pe, g.tok_pos)))
    return st;
  if (stop == ST_EMBED) return ENC_OK;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = e->layers[l];
    LAUNCH(ENC_K_LN, launch_layernorm<T>(resid, L.ln1g, L.ln1b, xn, M, d, c.ln_eps, s));
    if ((st = launch_linear_t<T>(e, ln, ENC_K_QKV, xn, d, L.wqkv, L.bqkv, qkv, 3 * d, M, 3 * d, d,
                                 EPI_BIAS, s)))
      return st;
    LAUNCH(ENC_K_ATTN, launch_attention<T>(qkv, g.wins, nullptr, g.n_win, c.n_heads, d, attn, s));
    if ((st = launch_linear_t<T>(e, ln, ENC_K_OPROJ, attn, d, L.wo, L.bo, resid, d, M, d, d, EPI_RESADD, s)))
      return st;
    LAUNCH(ENC_K_LN, launch_layernorm<T>(resid, L.ln2g, L.ln2b, xn, M, d, c.ln_eps, s));
    if ((st = launch_linear_t<T>(e, ln, ENC_K_FFN1, xn, d, L.w1, L.b1, hid, c.d_ffn, M, c.d_ffn, d,
                                 EPI_BIAS_GELU, s)))
      return st;
    if ((st = launch_linear_t<T>(e, ln, ENC_K_FFN2, hid, c.d_ffn, L.w2, L.b2, resid, d, M, d, c.d_ffn,
                                 EPI_RESADD, s)))
      return st;
    if (stop == ST_LAYER && stop_layer == l) return ENC_OK;
    if (taps)
      for (int32_t t = 0; t < taps->n; ++t)
        if (taps->layers[t] == l)
          AE_HIP(hipMemcpyAsync(taps->dst + (t * taps->ntok_total + p.tok0) * d, resid,
                                M * d * sizeof(float), hipMemcpyDeviceToDevice, s));
  }
  LAUNCH(ENC_K_LN, launch_layernorm<T>(resid, e->lnp_g, e->lnp_b, xn, M, d, c.ln_eps, s));
  if ((st = launch_linear_t<T>(e, ln, ENC_K_PROJ1, xn, d, e->proj1_w, e->proj1_b, hid, d, M, d, d,
                               EPI_BIAS_GELU, s)))
    return st;
  if ((st = launch_linear_t<T>(e, ln, ENC_K_PROJ2, hid, d, e->proj2_w, e->proj2_b, z, c.d_out, M,
                               c.d_out, d, EPI_BIAS, s)))
    return st;
  if (stop == ST_HEAD) return ENC_OK;
  const int da = c.d_adapter;
  if (e->bf16) {
    if ((st = launch_linear_t<T>(e, ln, ENC_K_GATE_UP, z, c.d_out, e->gateup_w, nullptr, hid, da, M,
                                 2 * da, c.d_out, EPI_SWIGLU, s)))
      return st;
  } else {
    T* hid2 = (T*)ln.hid2.p;
    if ((st = launch_linear_t<T>(e, ln, ENC_K_GATE_UP, z, c.d_out, e->gateup_w, nullptr, hid2, 2 * da,
                                 M, 2 * da, c.d_out, EPI_BIAS, s)))
      return st;
    LAUNCH(ENC_K_OTHER, launch_swiglu_split<T>(hid2, M, 2 * da, hid, s));
  }
  T* dst = (T*)out + p.tok0 * c.d_out;
  if ((st = launch_linear_t<T>(e, ln, ENC_K_DOWN, hid, da, e->down_w, nullptr, dst, c.d_out, M, c.d_out,
                               da, EPI_BIAS, s)))
    return st;
  return ENC_OK;
}

// log-mel of the clips (spans already uploaded to ctab) into mel_raw + max keys
encoder_status run_mel(encoder* e, const float* pcm, int32_t nclip, int64_t t_max, hipStream_t s) {
  LAUNCH(ENC_K_OTHER, launch_clear_u32((uint32_t*)e->max_key.p, nclip, s));
  LAUNCH(ENC_K_MEL, launch_log_mel(pcm, (const ClipSpan*)e->ctab.p, nclip, t_max, e->mel,
                                   (float*)e->mel_raw.p, (uint32_t*)e->max_key.p, s));
  return ENC_OK;
}

// clip lengths of a ragged call -> vector (validated)
encoder_status ragged_lengths(const encoder_cfg& c, const int64_t* lengths, int32_t n_clips,
                              std::vector<int64_t>& lens) {
  if (!lengths) return invalid("lengths is NULL");
  if (n_clips < 1) return invalid("n_clips must be >= 1");
  if (n_clips > 65535) return invalid("n_clips must be <= 65535");
  lens.assign(lengths, lengths + n_clips);
  int64_t frames = 0, tokens = 0;
  for (int32_t i = 0; i < n_clips; ++i) {
    if (lens[i] <= c.n_fft / 2)
      return invalid("clip " + std::to_string(i) + ": length must exceed n_fft/2 = 200 (reflect padding)");
    if (lens[i] / c.hop >= (int64_t(1) << 30)) return invalid("clip " + std::to_string(i) + " too long");
    frames += lens[i] / c.hop;
    tokens += frames_out(c, lens[i]);
  }
  if (frames >= (int64_t(1) << 31) || tokens >= (int64_t(1) << 31))
    return invalid("too many frames for one call");
  return ENC_OK;
}

encoder_status check_forward_args(encoder* e, const void* pcm, int64_t n_samples, int32_t batch,
                                  const void* out) {
  if (!e) return invalid("encoder handle is NULL");
  if (!pcm || !out) return invalid("pcm and output pointers must be non-NULL");
  if (batch < 1) return invalid("batch must be >= 1");
  if (batch > 65535) return invalid("batch must be <= 65535");
  if (n_samples <= e->cfg.n_fft / 2)
    return invalid("n_samples must exceed n_fft/2 = 200 (reflect padding)");
  if (n_samples / e->cfg.hop >= (int64_t(1) << 30)) return invalid("clip too long");
  if ((int64_t)batch * (n_samples / e->cfg.hop) >= (int64_t(1) << 31))
    return invalid("too many log-mel frames for one call");
  return ENC_OK;
}

// lens: samples of each clip of the call (packed back to back in pcm)
encoder_status forward_impl(encoder* e, const float* pcm, const std::vector<int64_t>& lens,
                            void* out, hipStream_t s, int64_t piece_windows, int stop = -1,
                            int stop_layer = -1, float* dst = nullptr, int64_t dst_elems = 0,
                            TapReq* taps = nullptr) {
  AE_HIP(hipSetDevice(e->device));
  e->timing_err = hipSuccess;
  const encoder_cfg& c = e->cfg;
  const int32_t batch = (int32_t)lens.size();
  std::vector<ClipSpan> clips;
  clip_spans(c, lens, clips);
  std::vector<Win> wins;
  plan_windows(c, lens, wins);
  // Debug stages export the padded conv layouts from a single pass; kernel-by-kernel timing
  // runs one lane, where halves help only when asked for (timing mode 1).
  const bool debug = stop >= 0;
  const std::vector<Pass> ps = plan_passes(c, wins, piece_windows, !debug && e->timing != 2, debug);
  if (debug && ps.size() > 1) return invalid("debug stages need a single pass");
  int64_t ntok = 0, n_frames = 0, t_max = 0;
  for (auto& p : ps) ntok += p.ntok;
  for (int64_t n : lens) {
    n_frames += n / c.hop;
    t_max = std::max<int64_t>(t_max, n / c.hop);
  }
  const int64_t T = t_max;  // equal to every clip's frame count on the debug paths
  // lanes: concurrent passes (bitwise the same as one after another), unless the call has a
  // single pass, stops at a debug stage or is timed kernel by kernel
  const int nl = (ps.size() > 1 && !debug && !e->timing)
                     ? (int)std::min<size_t>(ps.size(), (size_t)kLanes) : 1;
  int64_t mtp = 1, rows1 = 1, rows2 = 1;  // largest pass of the call
  for (const Pass& p : ps) {
    mtp = std::max<int64_t>(mtp, p.ntok);
    rows1 = std::max<int64_t>(rows1, p.nwin * p.L1s);
    rows2 = std::max<int64_t>(rows2, p.nwin * p.L2s);
  }
  if ((int)e->lanes.size() < nl) e->lanes.resize(nl);
  encoder_status st = size_call(e, batch, n_frames, (int64_t)wins.size(), ntok);
  if (st) return st;
  for (int i = 0; i < nl; ++i)
    if ((st = size_lane(e, e->lanes[i], mtp, rows1, rows2))) return st;
  if (nl > 1) {
    if (!e->passes_ready) AE_HIP(hipEventCreateWithFlags(&e->passes_ready, hipEventDisableTiming));
    for (int i = 0; i < nl; ++i) {
      encoder::Lane& ln = e->lanes[i];
      if (!ln.stream) AE_HIP(hipStreamCreateWithFlags(&ln.stream, hipStreamNonBlocking));
      if (!ln.done) AE_HIP(hipEventCreateWithFlags(&ln.done, hipEventDisableTiming));
    }
  }
  if ((st = upload_plan(e, clips, wins, ps, s))) return st;
  // from here on the call has work queued on s: its end is marked for the next workspace
  // growth, on every way out of this function
  struct CallDone {
    encoder* e;
    hipStream_t s;
    ~CallDone() { e->call_pending = hipEventRecord(e->call_done, s) == hipSuccess; }
  } call_done_guard{e, s};
  encoder_status body = ENC_OK;
  if ((body = run_mel(e, pcm, batch, t_max, s)) == ENC_OK && stop == ST_MEL) {
    LAUNCH(ENC_K_OTHER, launch_mel_normalize((const float*)e->mel_raw.p, (const uint32_t*)e->max_key.p,
                                             T, batch, dst, s));
  } else if (body == ENC_OK) {
    if (taps) taps->ntok_total = ntok;
    auto pass = [&](encoder::Lane& ln, const Pass& p, hipStream_t ps_) {
      return e->bf16 ? run_pass<bf16_t>(e, ln, p, out, ps_, stop, stop_layer, taps)
                     : run_pass<float>(e, ln, p, out, ps_, stop, stop_layer, taps);
    };
    if (nl == 1) {
      for (const Pass& p : ps)
        if ((body = pass(e->lanes[0], p, s))) break;
    } else {
      // fork after the log-mel, passes round-robin over the lanes, join on the caller's stream;
      // the join is enqueued even when a pass fails to enqueue, so that no lane's earlier work
      // is left running past the end of the call's work on s
      hipError_t err = hipEventRecord(e->passes_ready, s);
      for (int i = 0; i < nl && err == hipSuccess; ++i)
        err = hipStreamWaitEvent(e->lanes[i].stream, e->passes_ready, 0);
      if (err != hipSuccess) return hip_fail(err, "fork onto the lanes");
      for (size_t j = 0; j < ps.size() && body == ENC_OK; ++j) {
        encoder::Lane& ln = e->lanes[j % nl];
        body = pass(ln, ps[j], ln.stream);
      }
      for (int i = 0; i < nl; ++i) {
        err = hipEventRecord(e->lanes[i].done, e->lanes[i].stream);
        if (err == hipSuccess) err = hipStreamWaitEvent(s, e->lanes[i].done, 0);
        if (err != hipSuccess && body == ENC_OK) body = hip_fail(err, "join of the lanes");
      }
    }
  }
  if (body == ENC_OK && debug && stop != ST_MEL) {
    const Pass& p = ps[0];
    const int64_t W = c.window_tokens, C = c.conv_channels;
    const void* src = nullptr;
    int64_t n = 0;
    switch (stop) {
      case ST_CONV1: src = e->lanes[0].act1.p; n = p.nwin * 4 * W * 64 * C; break;
      case ST_CONV2: src = e->lanes[0].act2.p; n = p.nwin * 2 * W * 32 * C; break;
      case ST_CONV3: src = e->lanes[0].tokA.p; n = p.ntok * 16 * C; break;
      case ST_EMBED:
      case ST_LAYER:
        src = e->lanes[0].resid.p;
        n = p.ntok * c.d_model;
        break;
      case ST_HEAD: src = e->lanes[0].z.p; n = p.ntok * c.d_out; break;
      case ST_OUT: src = out; n = p.ntok * c.d_out; break;
      default: body = invalid("unknown stage");
    }
    if (body == ENC_OK && dst_elems < n) body = invalid("dst too small for this stage");
    if (body == ENC_OK) {
      if (stop == ST_EMBED || stop == ST_LAYER) {
        const hipError_t err = hipMemcpyAsync(dst, src, n * 4, hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) body = hip_fail(err, "hipMemcpyAsync(stage)");
      } else {
        auto cvt = [&]() -> encoder_status {
          if (e->bf16) LAUNCH(ENC_K_OTHER, launch_to_f32<bf16_t>((const bf16_t*)src, n, dst, s));
          else LAUNCH(ENC_K_OTHER, launch_to_f32<float>((const float*)src, n, dst, s));
          return ENC_OK;
        };
        body = cvt();
      }
    }
  }
  return body;
}

void free_all(encoder* e) {
  if (!e) return;
  hipSetDevice(e->device);
  hipDeviceSynchronize();
  encoder::Buf* bufs[] = {&e->mel_raw, &e->max_key, &e->ctab, &e->wtab, &e->tpos, &e->rs_taps, &e->dbg};
  for (auto* b : bufs)
    if (b->p) hipFree(b->p);
  for (auto& ln : e->lanes) {
    encoder::Buf* lb[] = {&ln.act1, &ln.act2, &ln.tokA, &ln.resid, &ln.xn, &ln.qkv, &ln.attn,
                          &ln.hid, &ln.hid2, &ln.z, &ln.splitk};
    for (auto* b : lb)
      if (b->p) hipFree(b->p);
    if (ln.stream) hipStreamDestroy(ln.stream);
    if (ln.done) hipEventDestroy(ln.done);
  }
  if (e->passes_ready) hipEventDestroy(e->passes_ready);
  if (e->call_done) hipEventDestroy(e->call_done);
  if (e->wdev) hipFree(e->wdev);
  if (e->qdev) hipFree(e->qdev);
  if (e->fdev) hipFree(e->fdev);
  if (e->pinned) hipHostFree(e->pinned);
  if (e->upload_done) hipEventDestroy(e->upload_done);
  for (auto ev : e->event_pool) hipEventDestroy(ev);
  delete e;
}

}  // namespace

// Device address of `scratch` on the current device, looked up once per device (the first
// lookup happens in encoder_create, with the handle's device current).  Null if the lookup
// failed (the error is in hip_err).
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};
static hipError_t g_scratch_err[kMaxDevices] = {};
static bool g_scratch_done[kMaxDevices] = {};

static void* scratch_on_device(int dev, hipError_t* hip_err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *hip_err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = err;
    g_scratch_done[dev] = true;
  }
  *hip_err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

// ==========================================================================================
// C ABI
// ==========================================================================================
extern "C" {

const char* encoder_last_error(void) { return g_err.c_str(); }

encoder_status encoder_validate_cfg(const encoder_cfg* cfg) { return check_cfg(cfg); }

encoder_status encoder_weight_count(const encoder_cfg* cfg, int64_t* n_floats) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!n_floats) return invalid("n_floats is NULL");
  int64_t n = 0;
  for (int64_t v : blob_sizes(*cfg)) n += v;
  *n_floats = n;
  return ENC_OK;
}

encoder_status encoder_output_frames(const encoder_cfg* cfg, int64_t n_samples, int64_t* n_frames) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!n_frames) return invalid("n_frames is NULL");
  if (n_samples <= cfg->n_fft / 2) return invalid("n_samples must exceed n_fft/2 = 200");
  *n_frames = frames_out(*cfg, n_samples);
  return ENC_OK;
}

encoder_status encoder_plan_windows(const encoder_cfg* cfg, int64_t n_samples, int32_t batch,
                                    int32_t* table, int32_t max_windows, int32_t* n_windows) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!n_windows) return invalid("n_windows is NULL");
  if (batch < 1) return invalid("batch must be >= 1");
  if (n_samples <= cfg->n_fft / 2) return invalid("n_samples must exceed n_fft/2 = 200");
  if (max_windows > 0 && !table) return invalid("table is NULL");
  std::vector<Win> w;
  plan_windows(*cfg, std::vector<int64_t>((size_t)batch, n_samples), w);
  *n_windows = (int32_t)w.size();
  for (int32_t i = 0; i < std::min<int32_t>(max_windows, (int32_t)w.size()); ++i) {
    int32_t* r = table + 7 * (int64_t)i;
    r[0] = w[i].clip; r[1] = w[i].start; r[2] = w[i].L0; r[3] = w[i].L1;
    r[4] = w[i].L2; r[5] = w[i].L3; r[6] = w[i].tok;
  }
  return ENC_OK;
}

encoder_status encoder_plan_windows_ragged(const encoder_cfg* cfg, const int64_t* lengths,
                                           int32_t n_clips, int32_t* table, int32_t max_windows,
                                           int32_t* n_windows) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!n_windows) return invalid("n_windows is NULL");
  if (max_windows > 0 && !table) return invalid("table is NULL");
  std::vector<int64_t> lens;
  if ((st = ragged_lengths(*cfg, lengths, n_clips, lens))) return st;
  std::vector<Win> w;
  plan_windows(*cfg, lens, w);
  *n_windows = (int32_t)w.size();
  for (int32_t i = 0; i < std::min<int32_t>(max_windows, (int32_t)w.size()); ++i) {
    int32_t* r = table + 7 * (int64_t)i;
    r[0] = w[i].clip; r[1] = w[i].start; r[2] = w[i].L0; r[3] = w[i].L1;
    r[4] = w[i].L2; r[5] = w[i].L3; r[6] = w[i].tok;
  }
  return ENC_OK;
}

encoder_status encoder_plan_passes(const encoder_cfg* cfg, const int64_t* lengths, int32_t n_clips,
                                   int32_t pieces_per_pass, int64_t* table, int32_t max_passes,
                                   int32_t* n_passes) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!n_passes) return invalid("n_passes is NULL");
  if (max_passes > 0 && !table) return invalid("table is NULL");
  if (pieces_per_pass < 0) return invalid("pieces_per_pass must be >= 0");
  if (pieces_per_pass > 0 && n_clips != 1) return invalid("long mode takes one recording (n_clips = 1)");
  std::vector<int64_t> lens;
  if ((st = ragged_lengths(*cfg, lengths, n_clips, lens))) return st;
  const int64_t pw = cfg->piece_tokens / cfg->window_tokens;
  if (pieces_per_pass > 0 && (int64_t)pieces_per_pass * cfg->piece_tokens > pass_token_cap(*cfg))
    return invalid("pieces_per_pass pieces exceed the tokens of one pass");
  std::vector<Win> w;
  plan_windows(*cfg, lens, w);
  const std::vector<Pass> ps = plan_passes(*cfg, w, pieces_per_pass > 0 ? pw * pieces_per_pass : 0, true, false);
  *n_passes = (int32_t)ps.size();
  for (int32_t i = 0; i < std::min<int32_t>(max_passes, (int32_t)ps.size()); ++i) {
    int64_t* r = table + 6 * (int64_t)i;
    r[0] = ps[i].win0; r[1] = ps[i].nwin; r[2] = ps[i].tok0; r[3] = ps[i].ntok;
    r[4] = ps[i].L1s; r[5] = ps[i].L2s;
  }
  return ENC_OK;
}

encoder_status encoder_create(const float* weights, int64_t n_floats, const encoder_cfg* cfg,
                              encoder** out) {
  encoder_status st = check_cfg(cfg);
  if (st) return st;
  if (!weights || !out) return invalid("weights and out must be non-NULL");
  const encoder_cfg& c = *cfg;
  const std::vector<int64_t> sizes = blob_sizes(c);
  int64_t need = 0;
  for (int64_t v : sizes) need += v;
  if (n_floats != need)
    return invalid("weight blob has " + std::to_string(n_floats) + " floats, config needs " +
                   std::to_string(need));
  if (getenv("ENCODER_FAIL_ALLOC")) {
    set_error("allocation refused (ENCODER_FAIL_ALLOC is set)");
    return ENC_E_OUT_OF_MEMORY;
  }
  int dev = 0;
  AE_HIP(hipGetDevice(&dev));

  encoder* e = new encoder();
  e->cfg = c;
  if (e->cfg.max_tokens_per_pass == 0) e->cfg.max_tokens_per_pass = 8192;
  e->device = dev;
  e->bf16 = c.dtype == ENC_BF16;
  e->esz = e->bf16 ? 2 : 4;

  const int64_t C = c.conv_channels, d = c.d_model, F = c.d_ffn, O = c.d_out, A = c.d_adapter;
  const int W = c.window_tokens;
  // blob offsets
  std::vector<const float*> src;
  {
    const float* p = weights;
    for (int64_t v : sizes) {
      src.push_back(p);
      p += v;
    }
  }
  // ---- layout of the dtype weight buffer (element offsets, 128-element aligned)
  int64_t woff = 0;
  auto wslot = [&](int64_t n) {
    const int64_t o = woff;
    woff += (n + 127) & ~int64_t(127);
    return o;
  };
  // with int4 weights the linear layers, head and adapter live in the int4 buffer instead
  const bool q4 = c.weight_bits == 4;
  auto lslot = [&](int64_t n) { return wslot(q4 ? 0 : n); };
  const int64_t o_conv2 = wslot(C * 9 * C), o_conv3 = wslot(C * 9 * C), o_co = wslot(d * 16 * C);
  std::vector<int64_t> o_qkv, o_o, o_1, o_2;
  for (int l = 0; l < c.n_layers; ++l) {
    o_qkv.push_back(lslot(3 * d * d));
    o_o.push_back(lslot(d * d));
    o_1.push_back(lslot(F * d));
    o_2.push_back(lslot(d * F));
  }
  const int64_t o_p1 = lslot(d * d), o_p2 = lslot(O * d), o_gu = lslot(2 * A * O), o_dn = lslot(O * A);
  // ---- int4 buffer: per matrix [N][K/2] bytes then [N][K/128] bf16 scales (256-byte aligned)
  int64_t qoff = 0;
  struct QSlot { int64_t q = 0, s = 0; };
  auto qslot = [&](int64_t N_, int64_t K_) {
    QSlot r;
    if (!q4) return r;
    r.q = qoff;
    qoff += ((N_ * K_ / 2) + 255) & ~int64_t(255);
    r.s = qoff;
    qoff += ((N_ * K_ / 128 * 2) + 255) & ~int64_t(255);
    return r;
  };
  std::vector<QSlot> q_qkv, q_o, q_1, q_2;
  for (int l = 0; l < c.n_layers; ++l) {
    q_qkv.push_back(qslot(3 * d, d));
    q_o.push_back(qslot(d, d));
    q_1.push_back(qslot(F, d));
    q_2.push_back(qslot(d, F));
  }
  const QSlot q_p1 = qslot(d, d), q_p2 = qslot(O, d), q_gu = qslot(2 * A, O), q_dn = qslot(O, A);
  // ---- float32 parameter buffer
  int64_t foff = 0;
  auto fslot = [&](int64_t n) {
    const int64_t o = foff;
    foff += (n + 63) & ~int64_t(63);
    return o;
  };
  const int64_t f_c1w = fslot(C * 9), f_c1b = fslot(C), f_c2b = fslot(C), f_c3b = fslot(C);
  std::vector<int64_t> f_bqkv, f_bo, f_b1, f_b2, f_l1g, f_l1b, f_l2g, f_l2b;
  for (int l = 0; l < c.n_layers; ++l) {
    f_bqkv.push_back(fslot(3 * d));
    f_bo.push_back(fslot(d));
    f_b1.push_back(fslot(F));
    f_b2.push_back(fslot(d));
    f_l1g.push_back(fslot(d));
    f_l1b.push_back(fslot(d));
    f_l2g.push_back(fslot(d));
    f_l2b.push_back(fslot(d));
  }
  const int64_t f_lpg = fslot(d), f_lpb = fslot(d), f_p1b = fslot(d), f_p2b = fslot(O);
  const int64_t f_pe = fslot((int64_t)W * d), f_tw = fslot(800), f_win = fslot(400);
  const int64_t f_fbw = fslot(128 * 16), f_fbs = fslot(128), f_fbl = fslot(128);

  std::vector<float> fh((size_t)foff, 0.0f);
  const size_t es = e->esz;
  std::vector<uint8_t> wh((size_t)(woff * (int64_t)es));
  auto put = [&](int64_t dst_el, int64_t idx, float v) {
    if (es == 2) reinterpret_cast<bf16_t*>(wh.data())[dst_el + idx] = host_f32_to_bf16(v);
    else reinterpret_cast<float*>(wh.data())[dst_el + idx] = v;
  };
  auto copy_plain = [&](int64_t dst_el, const float* s, int64_t n) {
    if (q4) return;  // quantised below instead
    parallel_for(n, [&](int64_t a, int64_t b) {
      for (int64_t i = a; i < b; ++i) put(dst_el, i, s[i]);
    });
  };
  std::vector<uint8_t> qh((size_t)qoff);
  // rows [row0, row0 + N_) of the int4 matrix at slot qs (K_ columns), from float32 rows src
  auto quant = [&](const QSlot& qs, int64_t row0, const float* src_rows, int64_t N_, int64_t K_) {
    quantize_int4_rows(src_rows, N_, K_, qh.data() + qs.q + row0 * K_ / 2,
                       reinterpret_cast<bf16_t*>(qh.data() + qs.s) + row0 * (K_ / 128));
  };
  auto fcopy = [&](int64_t dst_el, const float* s, int64_t n) {
    std::memcpy(fh.data() + dst_el, s, n * sizeof(float));
  };
  // conv1: [C][9] float32 as stored
  fcopy(f_c1w, src[0], C * 9);
  fcopy(f_c1b, src[1], C);
  // conv2/conv3: [co][ci][a][b] -> [co][a*3+b][ci]
  for (int which = 0; which < 2; ++which) {
    const float* s = src[2 + 2 * which];
    const int64_t o = which == 0 ? o_conv2 : o_conv3;
    parallel_for(C, [&](int64_t a0, int64_t a1) {
      for (int64_t co = a0; co < a1; ++co)
        for (int64_t ci = 0; ci < C; ++ci)
          for (int t = 0; t < 9; ++t) put(o, (co * 9 + t) * C + ci, s[(co * C + ci) * 9 + t]);
    });
    fcopy(which == 0 ? f_c2b : f_c3b, src[3 + 2 * which], C);
  }
  // conv_out: column c*16+f -> f*C+c
  parallel_for(d, [&](int64_t a0, int64_t a1) {
    for (int64_t n = a0; n < a1; ++n)
      for (int64_t ch = 0; ch < C; ++ch)
        for (int f = 0; f < 16; ++f) put(o_co, n * 16 * C + f * C + ch, src[6][n * 16 * C + ch * 16 + f]);
  });
  for (int l = 0; l < c.n_layers; ++l) {
    const float* const* s = src.data() + 7 + 16 * l;
    // s: ln1g ln1b qw qb kw kb vw vb ow ob ln2g ln2b fc1w fc1b fc2w fc2b
    fcopy(f_l1g[l], s[0], d);
    fcopy(f_l1b[l], s[1], d);
    copy_plain(o_qkv[l], s[2], d * d);
    copy_plain(o_qkv[l] + d * d, s[4], d * d);
    copy_plain(o_qkv[l] + 2 * d * d, s[6], d * d);
    if (q4) {
      quant(q_qkv[l], 0, s[2], d, d);
      quant(q_qkv[l], d, s[4], d, d);
      quant(q_qkv[l], 2 * d, s[6], d, d);
      quant(q_o[l], 0, s[8], d, d);
      quant(q_1[l], 0, s[12], F, d);
      quant(q_2[l], 0, s[14], d, F);
    }
    fcopy(f_bqkv[l], s[3], d);
    fcopy(f_bqkv[l] + d, s[5], d);
    fcopy(f_bqkv[l] + 2 * d, s[7], d);
    copy_plain(o_o[l], s[8], d * d);
    fcopy(f_bo[l], s[9], d);
    fcopy(f_l2g[l], s[10], d);
    fcopy(f_l2b[l], s[11], d);
    copy_plain(o_1[l], s[12], F * d);
    fcopy(f_b1[l], s[13], F);
    copy_plain(o_2[l], s[14], d * F);
    fcopy(f_b2[l], s[15], d);
  }
  const float* const* h = src.data() + 7 + 16 * c.n_layers;
  // h: lnpg lnpb p1w p1b p2w p2b gate up down
  fcopy(f_lpg, h[0], d);
  fcopy(f_lpb, h[1], d);
  copy_plain(o_p1, h[2], d * d);
  fcopy(f_p1b, h[3], d);
  copy_plain(o_p2, h[4], O * d);
  fcopy(f_p2b, h[5], O);
  // gate/up interleaved in groups of 32 rows: [gate 32 | up 32] per 64 rows
  if (!q4) {
    parallel_for(A, [&](int64_t a0, int64_t a1) {
      for (int64_t j = a0; j < a1; ++j) {
        const int64_t rg = 64 * (j / 32) + (j % 32);
        for (int64_t k = 0; k < O; ++k) {
          put(o_gu, rg * O + k, h[6][j * O + k]);
          put(o_gu, (rg + 32) * O + k, h[7][j * O + k]);
        }
      }
    });
  } else {
    quant(q_p1, 0, h[2], d, d);
    quant(q_p2, 0, h[4], O, d);
    std::vector<float> gu((size_t)(2 * A * O));  // the interleaved row order, then quantised
    parallel_for(A, [&](int64_t a0, int64_t a1) {
      for (int64_t j = a0; j < a1; ++j) {
        const int64_t rg = 64 * (j / 32) + (j % 32);
        std::memcpy(gu.data() + rg * O, h[6] + j * O, O * sizeof(float));
        std::memcpy(gu.data() + (rg + 32) * O, h[7] + j * O, O * sizeof(float));
      }
    });
    quant(q_gu, 0, gu.data(), 2 * A, O);
  }
  copy_plain(o_dn, h[8], O * A);
  if (q4) quant(q_dn, 0, h[8], O, A);
  // tables
  {
    std::vector<float> pe = pe_table(W, (int)d);
    fcopy(f_pe, pe.data(), (int64_t)pe.size());
    std::vector<float> tw, wn, fw;
    std::vector<int32_t> fs, fl;
    mel_host_tables(tw, wn, fs, fl, fw);
    fcopy(f_tw, tw.data(), 800);
    fcopy(f_win, wn.data(), 400);
    fcopy(f_fbw, fw.data(), 128 * 16);
    std::memcpy(fh.data() + f_fbs, fs.data(), 128 * 4);
    std::memcpy(fh.data() + f_fbl, fl.data(), 128 * 4);
  }

  // bf16 matrices read by the staged kernels go to the K-blocked layout (conv2/conv3 with the
  // conv tiles' 32-wide K steps, the linear layers with 64); a shape that does not divide into
  // blocks stays plain
  auto blockify = [&](int64_t o, int64_t N_, int64_t K_, int BK) -> int32_t {
    const int64_t R = 512 / BK;
    if (es != 2 || N_ % R != 0 || K_ % BK != 0) return 0;
    bf16_t* p = reinterpret_cast<bf16_t*>(wh.data()) + o;
    std::vector<bf16_t> plain(p, p + N_ * K_);
    const int64_t kb = K_ / BK;
    parallel_for(N_ / R, [&](int64_t g0, int64_t g1) {
      for (int64_t g = g0; g < g1; ++g)
        for (int64_t r = 0; r < R; ++r)
          for (int64_t k = 0; k < K_; ++k)
            p[(g * kb + k / BK) * 512 + r * BK + k % BK] = plain[(g * R + r) * K_ + k];
    });
    return BK;
  };
  // conv2 and conv3 have the same shape, hence the same layout (one flag for both)
  const int32_t b_conv = blockify(o_conv2, C, 9 * C, 32);
  blockify(o_conv3, C, 9 * C, 32);
  const int32_t b_co = blockify(o_co, d, 16 * C, 64);
  std::vector<int32_t> b_qkv, b_o, b_1, b_2;
  for (int l = 0; l < c.n_layers; ++l) {
    b_qkv.push_back(q4 ? 0 : blockify(o_qkv[l], 3 * d, d, 64));
    b_o.push_back(q4 ? 0 : blockify(o_o[l], d, d, 64));
    b_1.push_back(q4 ? 0 : blockify(o_1[l], F, d, 64));
    b_2.push_back(q4 ? 0 : blockify(o_2[l], d, F, 64));
  }
  const int32_t b_p1 = q4 ? 0 : blockify(o_p1, d, d, 64), b_p2 = q4 ? 0 : blockify(o_p2, O, d, 64);
  const int32_t b_gu = q4 ? 0 : blockify(o_gu, 2 * A, O, 64), b_dn = q4 ? 0 : blockify(o_dn, O, A, 64);

  hipError_t err = hipMalloc(&e->wdev, woff * (int64_t)es);
  if (err == hipSuccess) err = hipMalloc((void**)&e->fdev, foff * 4);
  if (err == hipSuccess && q4) err = hipMalloc((void**)&e->qdev, qoff);
  if (err == hipSuccess && q4) err = hipMemcpy(e->qdev, qh.data(), qoff, hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipMemcpy(e->wdev, wh.data(), woff * (int64_t)es, hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipMemcpy(e->fdev, fh.data(), foff * 4, hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&e->upload_done, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&e->call_done, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventRecord(e->upload_done, nullptr);
  if (err != hipSuccess) {
    encoder_status r = hip_fail(err, "encoder_create");
    free_all(e);
    return r;
  }
  e->scratch = scratch_on_device(dev, &e->scratch_err);
  e->wbytes = woff * (int64_t)es;
  e->fbytes = foff * 4;
  e->qbytes = qoff;
  auto W_ = [&](int64_t o) { return (void*)((uint8_t*)e->wdev + o * (int64_t)es); };
  auto M_ = [&](int64_t o, const QSlot& qs, int32_t blk) {
    WMat m;
    if (q4) {
      m.q = e->qdev + qs.q;
      m.s = reinterpret_cast<const bf16_t*>(e->qdev + qs.s);
    } else {
      m.w = W_(o);
      m.blk = blk;
    }
    return m;
  };
  auto F_ = [&](int64_t o) { return e->fdev + o; };
  e->conv1_w = F_(f_c1w); e->conv1_b = F_(f_c1b); e->conv2_b = F_(f_c2b); e->conv3_b = F_(f_c3b);
  e->conv2_w = W_(o_conv2); e->conv3_w = W_(o_conv3);
  e->conv_blk = b_conv;
  e->conv_out_w.w = W_(o_co);
  e->conv_out_w.blk = b_co;
  for (int l = 0; l < c.n_layers; ++l) {
    LayerW L;
    L.wqkv = M_(o_qkv[l], q_qkv[l], b_qkv[l]); L.wo = M_(o_o[l], q_o[l], b_o[l]);
    L.w1 = M_(o_1[l], q_1[l], b_1[l]); L.w2 = M_(o_2[l], q_2[l], b_2[l]);
    L.bqkv = F_(f_bqkv[l]); L.bo = F_(f_bo[l]); L.b1 = F_(f_b1[l]); L.b2 = F_(f_b2[l]);
    L.ln1g = F_(f_l1g[l]); L.ln1b = F_(f_l1b[l]); L.ln2g = F_(f_l2g[l]); L.ln2b = F_(f_l2b[l]);
    e->layers.push_back(L);
  }
  e->lnp_g = F_(f_lpg); e->lnp_b = F_(f_lpb); e->proj1_b = F_(f_p1b); e->proj2_b = F_(f_p2b);
  e->proj1_w = M_(o_p1, q_p1, b_p1); e->proj2_w = M_(o_p2, q_p2, b_p2);
  e->gateup_w = M_(o_gu, q_gu, b_gu); e->down_w = M_(o_dn, q_dn, b_dn);
  e->pe = F_(f_pe);
  e->mel.twiddle = F_(f_tw);
  e->mel.window = F_(f_win);
  e->mel.fb_w = F_(f_fbw);
  e->mel.fb_start = reinterpret_cast<const int32_t*>(F_(f_fbs));
  e->mel.fb_len = reinterpret_cast<const int32_t*>(F_(f_fbl));
  *out = e;
  return ENC_OK;
}

void encoder_destroy(encoder* e) { free_all(e); }

encoder_status encoder_memory_stats(const encoder* e, int64_t* weight_bytes, int64_t* workspace_bytes) {
  if (!e) return invalid("encoder handle is NULL");
  if (weight_bytes) *weight_bytes = e->wbytes + e->fbytes + e->qbytes;
  if (workspace_bytes) *workspace_bytes = e->ws_peak;
  return ENC_OK;
}

encoder_status encoder_forward(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                               void* out, void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, batch, out);
  if (st) return st;
  return forward_impl(e, pcm, std::vector<int64_t>((size_t)batch, n_samples), out,
                      (hipStream_t)stream, 0);
}

encoder_status encoder_forward_long(encoder* e, const float* pcm, int64_t n_samples,
                                    int32_t pieces_per_pass, void* out, void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, 1, out);
  if (st) return st;
  if (pieces_per_pass < 1) return invalid("pieces_per_pass must be >= 1");
  const int64_t pw = e->cfg.piece_tokens / e->cfg.window_tokens;  // windows per piece
  if ((int64_t)pieces_per_pass * e->cfg.piece_tokens > max_tokens(e->cfg))
    return invalid("pieces_per_pass * piece_tokens exceeds max_tokens_per_pass");
  if ((int64_t)pieces_per_pass * e->cfg.piece_tokens > pass_token_cap(e->cfg) ||
      (int64_t)pieces_per_pass * pw * 4 * e->cfg.window_tokens * act1_row_bytes(e->cfg) > kMaxOperandBytes)
    return invalid("pieces_per_pass pieces exceed what one pass can address (2^31 - 1 bytes per operand)");
  return forward_impl(e, pcm, std::vector<int64_t>(1, n_samples), out, (hipStream_t)stream,
                      pw * pieces_per_pass);
}

encoder_status encoder_forward_ragged(encoder* e, const float* pcm, const int64_t* lengths,
                                      int32_t n_clips, void* out, void* stream) {
  if (!e) return invalid("encoder handle is NULL");
  if (!pcm || !out) return invalid("pcm and output pointers must be non-NULL");
  std::vector<int64_t> lens;
  encoder_status st = ragged_lengths(e->cfg, lengths, n_clips, lens);
  if (st) return st;
  return forward_impl(e, pcm, lens, out, (hipStream_t)stream, 0);
}

encoder_status encoder_forward_taps(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                    void* out, const int32_t* layers, int32_t n_taps, float* taps,
                                    void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, batch, out);
  if (st) return st;
  if (n_taps < 0) return invalid("n_taps must be >= 0");
  if (n_taps > 0 && (!layers || !taps)) return invalid("layers and taps must be non-NULL");
  for (int32_t t = 0; t < n_taps; ++t)
    if (layers[t] < 0 || layers[t] >= e->cfg.n_layers)
      return invalid("tap " + std::to_string(t) + ": layer out of range");
  TapReq req;
  req.layers = layers;
  req.n = n_taps;
  req.dst = taps;
  return forward_impl(e, pcm, std::vector<int64_t>((size_t)batch, n_samples), out,
                      (hipStream_t)stream, 0, -1, -1, nullptr, 0, &req);
}

encoder_status encoder_splice(const void* frames, int64_t n_frames, int32_t dim,
                              const int64_t* positions, void* table, int64_t table_rows,
                              int32_t dtype, int32_t* n_skipped, void* stream) {
  if (n_frames < 0 || table_rows < 0 || dim <= 0) return invalid("bad sizes");
  if (n_frames > 0 && (!frames || !positions || !table))
    return invalid("frames, positions and table must be non-NULL");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  if (dim % 8) return invalid("dim must be a multiple of 8");
  hipError_t err;
  if (dtype == ENC_BF16)
    err = launch_splice<bf16_t>((const bf16_t*)frames, n_frames, dim, positions, (bf16_t*)table,
                                table_rows, n_skipped, (hipStream_t)stream);
  else
    err = launch_splice<float>((const float*)frames, n_frames, dim, positions, (float*)table,
                               table_rows, n_skipped, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_splice");
  return ENC_OK;
}

encoder_status encoder_conditioned_length(int64_t n_in, int32_t sample_rate, int64_t* n_out) {
  if (!n_out) return invalid("n_out is NULL");
  if (n_in < 1) return invalid("n_in must be >= 1");
  ResamplePlan r;
  if (!resample_plan(sample_rate, r)) {
    set_error("sample rate " + std::to_string(sample_rate) + " is not supported");
    return ENC_E_UNSUPPORTED;
  }
  if (n_in > (int64_t(1) << 40)) return invalid("n_in too large");
  *n_out = conditioned_length(n_in, r);
  return ENC_OK;
}

encoder_status encoder_condition_audio(encoder* e, const float* in, int64_t n_in, int32_t channels,
                                       int32_t sample_rate, float* out, void* stream) {
  if (!e) return invalid("encoder handle is NULL");
  if (!in || !out) return invalid("in and out must be non-NULL");
  if (n_in < 1) return invalid("n_in must be >= 1");
  if (channels < 1 || channels > 64) return invalid("channels must be in [1, 64]");
  if (n_in > (int64_t(1) << 40)) return invalid("n_in too large");
  ResamplePlan r;
  if (!resample_plan(sample_rate, r)) {
    set_error("sample rate " + std::to_string(sample_rate) + " is not supported");
    return ENC_E_UNSUPPORTED;
  }
  AE_HIP(hipSetDevice(e->device));
  hipStream_t s = (hipStream_t)stream;
  encoder_status st;
  if (r.K > 0 && e->rs_rate != sample_rate) {
    const std::vector<float> taps = resample_taps(r);
    const int64_t tb = (int64_t)taps.size() * 4;
    if ((st = ensure(e, e->rs_taps, tb))) return st;
    AE_HIP(hipEventSynchronize(e->upload_done));
    if (e->pinned_bytes < tb) {
      if (e->pinned) AE_HIP(hipHostFree(e->pinned));
      e->pinned = nullptr;
      e->pinned_bytes = 0;
      AE_HIP(hipHostMalloc(&e->pinned, tb, hipHostMallocDefault));
      e->pinned_bytes = tb;
    }
    std::memcpy(e->pinned, taps.data(), tb);
    AE_HIP(hipMemcpyAsync(e->rs_taps.p, e->pinned, tb, hipMemcpyHostToDevice, s));
    AE_HIP(hipEventRecord(e->upload_done, s));
    e->rs_rate = sample_rate;
  }
  LAUNCH(ENC_K_OTHER, launch_resample(in, n_in, channels, r.L, r.M, r.K, (const float*)e->rs_taps.p,
                                      out, conditioned_length(n_in, r), s));
  AE_HIP(hipEventRecord(e->call_done, s));  // the filter table is read until here
  e->call_pending = true;
  return ENC_OK;
}

encoder_status encoder_log_mel(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                               float* mel, void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, batch, mel);
  if (st) return st;
  AE_HIP(hipSetDevice(e->device));
  hipStream_t s = (hipStream_t)stream;
  const int64_t T = n_samples / e->cfg.hop;
  if ((st = size_mel(e, batch, (int64_t)batch * T))) return st;
  std::vector<ClipSpan> clips;
  clip_spans(e->cfg, std::vector<int64_t>((size_t)batch, n_samples), clips);
  if ((st = upload_plan(e, clips, {}, {}, s))) return st;
  st = run_mel(e, pcm, batch, T, s);
  if (st == ENC_OK) {
    const hipError_t err = launch_mel_normalize((const float*)e->mel_raw.p, (const uint32_t*)e->max_key.p,
                                                T, batch, mel, s);
    if (err != hipSuccess) st = hip_fail(err, "launch_mel_normalize");
  }
  // the workspace is read until here
  e->call_pending = hipEventRecord(e->call_done, s) == hipSuccess;
  return st;
}

encoder_status encoder_log_mel_noalloc(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                       float* mel, void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, batch, mel);
  if (st) return st;
  if (batch > kScratchClips)
    return invalid("encoder_log_mel_noalloc takes at most " + std::to_string(kScratchClips) +
                   " clips (its scratch holds that many); use encoder_log_mel");
  if (!e->scratch) return hip_fail(e->scratch_err, "hipGetSymbolAddress(scratch)");
  AE_HIP(hipSetDevice(e->device));
  hipStream_t s = (hipStream_t)stream;
  const int64_t T = n_samples / e->cfg.hop;
  ClipSpan* spans = reinterpret_cast<ClipSpan*>(e->scratch);
  uint32_t* keys = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(e->scratch) + kScratchSpanBytes);
  // spans written by a kernel and keys cleared by a kernel (no host staging, no memset); the
  // raw log10 mel goes straight into the output and is normalised there
  AE_HIP(launch_batch_spans(spans, batch, n_samples, s));
  AE_HIP(launch_clear_u32(keys, batch, s));
  AE_HIP(launch_log_mel(pcm, spans, batch, T, e->mel, mel, keys, s));
  AE_HIP(launch_mel_normalize(mel, keys, T, batch, mel, s));
  return ENC_OK;
}

encoder_status encoder_debug_stage(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                   int32_t stage, int32_t layer, float* dst, int64_t dst_elems,
                                   void* stream) {
  encoder_status st = check_forward_args(e, pcm, n_samples, batch, dst);
  if (st) return st;
  if (stage < ST_MEL || stage > ST_OUT) return invalid("unknown stage");
  if (stage == ST_LAYER && (layer < 0 || layer >= e->cfg.n_layers)) return invalid("layer out of range");
  if (stage == ST_MEL && dst_elems < (int64_t)batch * (n_samples / e->cfg.hop) * 128)
    return invalid("dst too small for this stage");
  const int64_t F = frames_out(e->cfg, n_samples) * batch;
  if (F > max_tokens(e->cfg)) return invalid("debug stages need a single pass");
  if ((st = ensure(e, e->dbg, F * e->cfg.d_out * (int64_t)e->esz))) return st;
  return forward_impl(e, pcm, std::vector<int64_t>((size_t)batch, n_samples), e->dbg.p,
                      (hipStream_t)stream, 0, stage, layer, dst, dst_elems);
}

encoder_status encoder_timing_enable(encoder* e, int32_t enable) {
  if (!e) return invalid("encoder handle is NULL");
  if (enable < 0 || enable > 2) return invalid("timing mode must be 0, 1 or 2");
  e->timing = enable;
  return ENC_OK;
}

encoder_status encoder_timing_read(encoder* e, double* ms, int64_t* launches, int32_t reset) {
  if (!e) return invalid("encoder handle is NULL");
  AE_HIP(hipSetDevice(e->device));
  if (ms) std::fill(ms, ms + ENC_K_COUNT, 0.0);
  if (launches) std::fill(launches, launches + ENC_K_COUNT, int64_t(0));
  for (const TimedLaunch& t : e->timed) {
    AE_HIP(hipEventSynchronize(t.b));
    float v = 0.0f;
    AE_HIP(hipEventElapsedTime(&v, t.a, t.b));
    if (ms) ms[t.kid] += v;
    if (launches) launches[t.kid] += 1;
  }
  if (reset) {
    e->timed.clear();
    e->event_next = 0;
  }
  return ENC_OK;
}

encoder_status encoder_op_linear(const void* A, const void* W, const float* bias, void* C,
                                 int64_t M, int32_t N, int32_t K, int32_t epi, int32_t dtype,
                                 void* stream) {
  if (!A || !W || !C) return invalid("A, W and C must be non-NULL");
  // the epilogue writes four consecutive columns per lane
  if (M < 0 || N <= 0 || N % 4 || K <= 0 || K % 8)
    return invalid("need M >= 0, N > 0, N % 4 == 0, K > 0, K % 8 == 0");
  if (epi < 0 || epi > 3) return invalid("epi must be 0..3");
  if (epi == 3 && N % 64) return invalid("SwiGLU needs N % 64 == 0");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  // bf16 outputs leave as eight columns per lane
  if (dtype == ENC_BF16 && (epi == 0 || epi == 1) && N % 8) return invalid("bf16 output needs N % 8 == 0");
  hipStream_t s = (hipStream_t)stream;
  static const int map[4] = {EPI_BIAS, EPI_BIAS_GELU, EPI_RESADD, EPI_SWIGLU};
  const int64_t ldc = epi == 3 ? N / 2 : N;
  LinearArgs a{A, K, W, bias, C, ldc, M, N, K, nullptr, nullptr};
  hipError_t err;
  if (dtype == ENC_BF16) {
    err = launch_linear<bf16_t>(a, map[epi], ENC_K_OTHER, s);
  } else if (epi == 3) {
    float* tmp = nullptr;
    AE_HIP(hipMallocAsync((void**)&tmp, M * N * 4, s));
    LinearArgs t = a;
    t.C = tmp;
    t.ldc = N;
    err = launch_linear<float>(t, EPI_BIAS, ENC_K_OTHER, s);
    if (err == hipSuccess) err = launch_swiglu_split<float>(tmp, M, N, (float*)C, s);
    hipFreeAsync(tmp, s);
  } else {
    err = launch_linear<float>(a, map[epi], ENC_K_OTHER, s);
  }
  if (err != hipSuccess) return hip_fail(err, "encoder_op_linear");
  return ENC_OK;
}

encoder_status encoder_quantize_int4(const float* w, int64_t N, int64_t K, uint8_t* q,
                                     uint16_t* scales) {
  if (!w || !q || !scales) return invalid("w, q and scales must be non-NULL");
  if (N < 1 || K < 128 || K % 128) return invalid("need N >= 1 and K a positive multiple of 128");
  quantize_int4_rows(w, N, K, q, scales);
  return ENC_OK;
}

encoder_status encoder_op_linear_int4(const void* A, const uint8_t* q, const uint16_t* scales,
                                      const float* bias, void* C, int64_t M, int32_t N, int32_t K,
                                      int32_t epi, void* stream) {
  if (!A || !q || !scales || !C) return invalid("A, q, scales and C must be non-NULL");
  if (M < 0 || N <= 0 || N % 4 || K < 128 || K % 128)
    return invalid("need M >= 0, N > 0, N % 4 == 0, K % 128 == 0");
  if (epi < 0 || epi > 3) return invalid("epi must be 0..3");
  if (epi == 3 && N % 64) return invalid("SwiGLU needs N % 64 == 0");
  if ((epi == 0 || epi == 1) && N % 8) return invalid("bf16 output needs N % 8 == 0");
  static const int map[4] = {EPI_BIAS, EPI_BIAS_GELU, EPI_RESADD, EPI_SWIGLU};
  const int64_t ldc = epi == 3 ? N / 2 : N;
  LinearArgs a{A, K, nullptr, bias, C, ldc, M, N, K, nullptr, nullptr, q, (const bf16_t*)scales};
  const hipError_t err = launch_linear<bf16_t>(a, map[epi], ENC_K_OTHER, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_op_linear_int4");
  return ENC_OK;
}

encoder_status encoder_op_attention(const void* qkv, const int32_t* windows, int32_t n_windows,
                                    int32_t n_heads, int64_t ntok, void* out, int32_t dtype,
                                    void* stream) {
  if (!qkv || !windows || !out) return invalid("qkv, windows and out must be non-NULL");
  if (n_windows < 0 || n_heads <= 0 || ntok < 0) return invalid("bad sizes");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  {
    std::vector<int32_t> h((size_t)n_windows * 2);
    if (n_windows) AE_HIP(hipMemcpy(h.data(), windows, h.size() * 4, hipMemcpyDeviceToHost));
    for (int32_t i = 0; i < n_windows; ++i)
      if (h[2 * i + 1] < 1 || h[2 * i + 1] > 128 || h[2 * i] < 0 || h[2 * i] + h[2 * i + 1] > ntok)
        return invalid("window " + std::to_string(i) + " is empty, longer than 128 or outside ntok");
  }
  hipError_t err;
  if (dtype == ENC_BF16)
    err = launch_attention<bf16_t>((const bf16_t*)qkv, nullptr, windows, n_windows, n_heads,
                                   n_heads * 64, (bf16_t*)out, (hipStream_t)stream);
  else
    err = launch_attention<float>((const float*)qkv, nullptr, windows, n_windows, n_heads,
                                  n_heads * 64, (float*)out, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_op_attention");
  return ENC_OK;
}

// Window tables of the kernel-level conv entries: copied to the host and checked before any
// launch, so that no kernel reads or writes outside the buffers the caller described.
static encoder_status check_conv_windows(const int32_t* windows, int32_t n_windows, int32_t W, int32_t L1s,
                                         int64_t n_tok, int64_t mel_rows, int32_t n_clips, bool conv1) {
  if (n_windows < 1) return invalid("n_windows must be >= 1");
  if (W < 1 || W > 128) return invalid("window_tokens must be in [1, 128]");
  if (L1s < 1 || L1s > 4 * W) return invalid("L1s must be in [1, 4 * window_tokens]");
  std::vector<Win> h((size_t)n_windows);
  AE_HIP(hipMemcpy(h.data(), windows, h.size() * sizeof(Win), hipMemcpyDeviceToHost));
  for (int32_t i = 0; i < n_windows; ++i) {
    const Win& w = h[i];
    const std::string at = "window " + std::to_string(i) + ": ";
    if (w.L0 < 1 || w.L0 > 8 * W || w.L1 != (w.L0 + 1) / 2 || w.L2 != (w.L1 + 1) / 2 ||
        w.L3 != (w.L2 + 1) / 2)
      return invalid(at + "lengths must be 1 <= L0 <= 8W and the ceil chain L1..L3");
    if (w.L1 > L1s) return invalid(at + "L1 exceeds L1s");
    if (!conv1 && (w.tok < 0 || (int64_t)w.tok + w.L3 > n_tok)) return invalid(at + "tokens outside n_tok");
    if (conv1 && (w.clip < 0 || w.clip >= n_clips || w.mel_row < 0 || (int64_t)w.mel_row + w.L0 > mel_rows))
      return invalid(at + "clip or mel rows outside the inputs");
  }
  return ENC_OK;
}

encoder_status encoder_op_conv1(const float* mel, int64_t mel_rows, const float* clip_max, int32_t n_clips,
                                const int32_t* windows, int32_t n_windows, int32_t window_tokens,
                                int32_t L1s, const float* w, const float* b, int32_t C, void* act1,
                                int32_t dtype, void* stream) {
  if (!mel || !clip_max || !windows || !w || !b || !act1) return invalid("pointers must be non-NULL");
  if (C < 32 || C % 32 || C > 2048) return invalid("C must be a multiple of 32 in [32, 2048]");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  if (n_clips < 1 || mel_rows < 1) return invalid("n_clips and mel_rows must be >= 1");
  encoder_status st = check_conv_windows(windows, n_windows, window_tokens, L1s, 0, mel_rows, n_clips, true);
  if (st) return st;
  PassGeom g{reinterpret_cast<const Win*>(windows), n_windows, window_tokens, L1s, (L1s + 1) / 2, 0, nullptr};
  hipError_t err;
  if (dtype == ENC_BF16)
    err = launch_conv1<bf16_t>(g, mel, nullptr, clip_max, w, b, C, (bf16_t*)act1, (hipStream_t)stream);
  else
    err = launch_conv1<float>(g, mel, nullptr, clip_max, w, b, C, (float*)act1, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_op_conv1");
  return ENC_OK;
}

encoder_status encoder_op_conv(int32_t level, const void* in, const int32_t* windows, int32_t n_windows,
                               int32_t window_tokens, int32_t L1s, int64_t n_tok, const void* w_packed,
                               const float* bias, int32_t C, void* out, int32_t dtype, void* stream) {
  if (!in || !windows || !w_packed || !bias || !out) return invalid("pointers must be non-NULL");
  if (level != 2 && level != 3) return invalid("level must be 2 (conv2) or 3 (conv3)");
  if (C < 32 || C % 32 || C > 4096) return invalid("C must be a multiple of 32 in [32, 4096]");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  if (n_tok < 0) return invalid("n_tok must be >= 0");
  encoder_status st = check_conv_windows(windows, n_windows, window_tokens, L1s, n_tok, 0, 0, false);
  if (st) return st;
  const int64_t es = dtype == ENC_BF16 ? 2 : 4;
  const int32_t L2s = (L1s + 1) / 2;
  if ((int64_t)n_windows * L1s * 64 * C * es > kMaxOperandBytes || n_tok * 16 * C * es > kMaxOperandBytes)
    return invalid("an operand exceeds 2^31 - 1 bytes");
  PassGeom g{reinterpret_cast<const Win*>(windows), n_windows, window_tokens, L1s, L2s, n_tok, nullptr};
  hipError_t err;
  if (dtype == ENC_BF16)
    err = launch_conv_igemm<bf16_t>(g, level, (const bf16_t*)in, (const bf16_t*)w_packed, bias, C, (bf16_t*)out,
                                    (hipStream_t)stream);
  else
    err = launch_conv_igemm<float>(g, level, (const float*)in, (const float*)w_packed, bias, C, (float*)out,
                                   (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_op_conv");
  return ENC_OK;
}

encoder_status encoder_op_layernorm(const float* x, const float* gamma, const float* beta, void* y,
                                    int64_t M, int32_t D, float eps, int32_t dtype, void* stream) {
  if (!x || !gamma || !beta || !y) return invalid("x, gamma, beta and y must be non-NULL");
  if (M < 0 || D <= 0 || D % 64) return invalid("need M >= 0 and D % 64 == 0");
  if (dtype != ENC_BF16 && dtype != ENC_F32) return invalid("bad dtype");
  hipError_t err;
  if (dtype == ENC_BF16)
    err = launch_layernorm<bf16_t>(x, gamma, beta, (bf16_t*)y, M, D, eps, (hipStream_t)stream);
  else
    err = launch_layernorm<float>(x, gamma, beta, (float*)y, M, D, eps, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "encoder_op_layernorm");
  return ENC_OK;
}

}  // extern "C"
