/*
 * audio_encoder.h - C ABI of the MI355X (gfx950) audio-tower library.
 *
 * The library computes the audio tower described on the "cstr/MOSS-Transcribe-preview-2B-GGUF"
 * card (section "Architecture"): 16 kHz mono PCM -> 128-bin Whisper-style log-mel (n_fft 400,
 * hop 160) -> 3 x Conv2D 3x3 stride 2 with GELU (1 -> C -> C -> C) -> conv_out (16*C -> d,
 * no bias) + sinusoidal positions -> pre-LN Transformer layers with windowed (block-diagonal)
 * self-attention -> ln_post -> proj1 -> GELU -> proj2 -> SwiGLU adapter.  It emits 12.5
 * embeddings per second of audio ("SILVERTHRONE/Ossicle-4B" card, "Model Overview").  The
 * long-audio entry point encodes a recording in 64 s pieces whose log-mel equals the whole-clip
 * log-mel (Ossicle card, "Long Audio").
 *
 * Conventions (all readings of points the cards leave open):
 *  - The encoder is window-local.  An attention window of W tokens covers 8*W mel frames.  Each
 *    window is convolved with zero padding at its own time edges, and its sinusoidal positions
 *    restart at 0.  The last window of a clip holds the remaining frames.
 *  - The log-mel has T = n_samples / 160 frames: centred reflect-padded frames, a periodic Hann
 *    window and the power spectrum; the trailing STFT frame is dropped (Transcribe card,
 *    "Non-obvious gotchas", item 2).  The filterbank is Slaney-normalised.  The mel is
 *    log10(max(., 1e-10)), clamped at (max - 8) and mapped to (x + 4) / 4.  The max runs over
 *    one clip, or over the whole recording in long-audio mode.
 *  - GELU is the exact erf form; LayerNorm uses eps = cfg.ln_eps with a biased variance.
 *    Attention has biases on q, k, v, o and scale 1/sqrt(head_dim).  The adapter has no biases
 *    and applies SiLU to the gate branch.
 *
 * Errors: every call returns an encoder_status; no C++ exception crosses the ABI.  On failure,
 * encoder_last_error() returns a thread-local message.  A call that fails validation enqueues
 * no GPU work.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream).  Forward calls
 * are asynchronous on that stream, and device faults surface at the caller's next
 * synchronisation.  One forward may be in flight per handle (the workspace is shared).
 */
#ifndef AUDIO_ENCODER_H
#define AUDIO_ENCODER_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ENC_API __attribute__((visibility("default")))
#else
#define ENC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ENC_OK = 0,
  ENC_E_INVALID_ARG = -1,   /* null pointer, bad size or inconsistent config; nothing enqueued */
  ENC_E_OUT_OF_MEMORY = -2, /* a device or pinned-host allocation failed                         */
  ENC_E_DEVICE = -3,        /* a HIP runtime call failed; message in encoder_last_error()       */
  ENC_E_UNSUPPORTED = -4,   /* valid request this build does not handle (e.g. sample_rate != 16 kHz) */
  ENC_E_INTERNAL = -5
} encoder_status;

typedef enum { ENC_BF16 = 0, ENC_F32 = 1 } encoder_dtype;

/* Model and runtime configuration.  Full-size tower: 16000,400,160,128 | 480 | 1280,32,20,64,5120 |
 * 100 | 2048,8192 | 800 | ENC_BF16 | 1e-5.  Dimension constraints (checked by
 * encoder_validate_cfg): n_heads*head_dim == d_model, head_dim == 64, conv_channels % 32 == 0,
 * d_model, d_ffn, d_out and d_adapter multiples of 64, 1 <= window_tokens <= 128,
 * piece_tokens a multiple of window_tokens. */
typedef struct {
  int32_t sample_rate;    /* must be 16000 (no resampling)                                  */
  int32_t n_fft;          /* 400                                                            */
  int32_t hop;            /* 160                                                            */
  int32_t n_mels;         /* 128                                                            */
  int32_t conv_channels;  /* C: conv1..conv3 output channels                                */
  int32_t d_model;        /* Transformer width d                                            */
  int32_t n_layers;
  int32_t n_heads;
  int32_t head_dim;
  int32_t d_ffn;
  int32_t window_tokens;  /* W: attention window (tokens); a window covers 8*W mel frames   */
  int32_t d_out;          /* proj2 output and adapter in/out width                          */
  int32_t d_adapter;      /* SwiGLU hidden width                                            */
  int32_t piece_tokens;   /* long-audio piece length in tokens (800 = 64 s)                 */
  int32_t dtype;          /* encoder_dtype: weights, GEMM operands and output storage      */
  float ln_eps;
  int64_t max_tokens_per_pass; /* bounds the activation workspace; larger inputs run in several
                                  window-aligned passes.  0 selects 8192.                    */
  int32_t weight_bits;    /* 16 (or 0): weights in dtype.  4: int4 weight-only for the layer
                             linears, head and adapter (encoder_quantize_int4 at create; "to_4bit"
                             of the "SILVERTHRONE/Ossicle-4B" card), dequantised to bf16 in the
                             GEMM loader; needs ENC_BF16 and d_model, d_ffn, d_out, d_adapter
                             multiples of 128.  Convs and conv_out stay in dtype.           */
  int32_t split_small_gemms; /* 0 (default): every GEMM accumulates K in one order, so a clip's
                             embeddings are bitwise independent of what else shares its call
                             or pass.  1 (bf16): GEMMs too small to fill the GPU (a single
                             clip) with K >= 4096 split K over workgroups and sum the fp32
                             partial products in a second kernel, in K-range order - faster
                             for small calls, but rounded differently from the same rows in a
                             large call.  Needs 64 MiB of extra workspace.                  */
} encoder_cfg;

typedef struct encoder encoder; /* opaque handle */

/* ---- host-only calls (no GPU work) ----------------------------------------------------- */

/* Checks the dimension constraints above.  ENC_OK, ENC_E_INVALID_ARG or ENC_E_UNSUPPORTED. */
ENC_API encoder_status encoder_validate_cfg(const encoder_cfg* cfg);

/* Number of float32 values the weight blob for `cfg` must hold.  Blob order (each tensor
 * row-major, PyTorch [out, in] layout): conv1.w[C,1,3,3] conv1.b[C] conv2.w[C,C,3,3] conv2.b
 * conv3.w conv3.b conv_out.w[d,16C] (column c*16+f: channel-major flatten); per layer: ln1.g[d]
 * ln1.b q.w[d,d] q.b k.w k.b v.w v.b o.w o.b ln2.g ln2.b fc1.w[ffn,d] fc1.b fc2.w[d,ffn] fc2.b;
 * then ln_post.g ln_post.b proj1.w[d,d] proj1.b proj2.w[dout,d] proj2.b gate.w[da,dout]
 * up.w[da,dout] down.w[dout,da].  Conv taps: [out][in][freq][time]. */
ENC_API encoder_status encoder_weight_count(const encoder_cfg* cfg, int64_t* n_floats);

/* Embeddings per clip: the sum over windows of the 3 x stride-2 ceil chain of each window's
 * frame count = ceil((n_samples/160)/8): 12.5 embeddings per second of audio
 * ("SILVERTHRONE/Ossicle-4B" card, "Model Overview"; frame count from the
 * "cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Non-obvious gotchas" item 2).  n_samples must
 * exceed n_fft/2, else ENC_E_INVALID_ARG. */
ENC_API encoder_status encoder_output_frames(const encoder_cfg* cfg, int64_t n_samples, int64_t* n_frames);

/* The window plan of a [batch, n_samples] call: for each window, 7 int32 values
 * {clip, first mel frame within the clip, L0 (frames), L1, L2, L3 (valid lengths after each
 * stride-2 conv; L3 = tokens), first output token (row of the [batch*F, d_out] output)}.
 * Writes min(n_windows, max_windows) entries to `table` (may be NULL when max_windows is 0)
 * and the total count to *n_windows. */
ENC_API encoder_status encoder_plan_windows(const encoder_cfg* cfg, int64_t n_samples, int32_t batch,
                                    int32_t* table, int32_t max_windows, int32_t* n_windows);

/* The window plan of a ragged call (see encoder_forward_ragged): the same 7 values per window,
 * clips in order, each clip's frames counted from its own start; the token column runs over
 * the whole call (row of the [sum F_c, d_out] output). */
ENC_API encoder_status encoder_plan_windows_ragged(const encoder_cfg* cfg, const int64_t* lengths,
                                           int32_t n_clips, int32_t* table, int32_t max_windows,
                                           int32_t* n_windows);

/* The passes a forward call runs in (windows are the independent units of the tower, so a call
 * is encoded as passes of consecutive whole windows; "SILVERTHRONE/Ossicle-4B" card, "Many clips
 * in one question" and "Long Audio").  lengths: host int64 [n_clips] sample counts of the clips
 * (as encoder_forward_ragged takes them; a [batch, n] call is n_clips = batch equal lengths).
 * pieces_per_pass: 0 for the whole-clip and ragged paths; >= 1 for encoder_forward_long, which
 * takes n_clips = 1 and starts a pass only at a multiple of pieces_per_pass 64 s pieces.  For
 * each pass, 6 int64 values: {first window, windows, first token, tokens, act1 time rows per
 * window L1s, act2 time rows per window L2s = ceil(L1s / 2)}; windows and tokens index the plan
 * of encoder_plan_windows(_ragged).  The conv activations of a pass hold windows x L1s x 64 x C
 * (act1) and windows x L2s x 32 x C (act2) elements, L1s being the longest conv1 output of the
 * pass.  A pass never holds more than max_tokens_per_pass tokens, and none of its operands
 * exceeds 2^31 - 1 bytes (the kernels address operands with 32-bit byte offsets): act1, and
 * tokens x max(16C, 3 d_model, d_ffn, 2 d_adapter, d_out) elements or tokens x d_model float32
 * (the residual).  A call of 4000 tokens or more that fits one pass is split into two halves of
 * whole windows (whole pieces in long mode), which run concurrently.  Writes
 * min(n_passes, max_passes) entries (table may be NULL when max_passes is 0). */
ENC_API encoder_status encoder_plan_passes(const encoder_cfg* cfg, const int64_t* lengths, int32_t n_clips,
                                   int32_t pieces_per_pass, int64_t* table, int32_t max_passes,
                                   int32_t* n_passes);

/* ---- handle lifecycle -------------------------------------------------------------------- */

/* Packs the host float32 weight blob (n_floats values, order above) for the current HIP device:
 * bf16 weights for ENC_BF16 (round-to-nearest-even), float32 for ENC_F32.  The caller keeps
 * ownership of `weights` and may free it when the call returns.  The handle owns the packed
 * weights, tables and workspace.  Synchronous. */
ENC_API encoder_status encoder_create(const float* weights, int64_t n_floats, const encoder_cfg* cfg,
                              encoder** out);
ENC_API void encoder_destroy(encoder* e);

/* Bytes of packed weights and tables, and the workspace high-water mark so far. */
ENC_API encoder_status encoder_memory_stats(const encoder* e, int64_t* weight_bytes,
                                    int64_t* workspace_bytes);

/* ---- forward passes ------------------------------------------------------------------------ */

/* Whole-clip path: the forward pass of the tower ("cstr/MOSS-Transcribe-preview-2B-GGUF" card,
 * "Architecture": 16 kHz mono PCM in, 12.5 Hz embeddings of width d_out out, in time order).
 * pcm: device float32 [batch, n_samples] (independent equal-length clips; each
 * is normalised by its own log-mel maximum).  out: device [batch, F, d_out] with F from
 * encoder_output_frames, bf16 for ENC_BF16 and float32 for ENC_F32.  n_samples > n_fft/2,
 * batch >= 1.  Inputs above max_tokens_per_pass run in several window-aligned passes.  Passes of
 * one call run concurrently on up to three internal streams (joined back onto `stream` before
 * the call's work ends), and a single-pass call of 4000 tokens or more runs as two concurrent
 * halves; every window's output rows are the same whatever pass it lands in. */
ENC_API encoder_status encoder_forward(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                               void* out, void* stream);

/* Long-audio path for one recording (Ossicle card, "Long Audio").  The log-mel and its maximum
 * are computed over the whole recording, which is then encoded in pieces of piece_tokens tokens
 * (8*piece_tokens frames), pieces_per_pass pieces per pass (passes run concurrently as for
 * encoder_forward; a single pass of 4000 tokens or more runs as two halves of whole pieces).
 * The last piece may be partial.
 * Output rows are written in time order: out [F, d_out].  Equals encoder_forward(batch = 1) up to
 * summation order. */
ENC_API encoder_status encoder_forward_long(encoder* e, const float* pcm, int64_t n_samples,
                                    int32_t pieces_per_pass, void* out, void* stream);

/* Ragged batch: several clips of different lengths in one call ("SILVERTHRONE/Ossicle-4B"
 * card: the audio-input line of the model summary, and "Many clips in one question").
 * pcm: device float32, the clips back to back (clip c at samples [off_c, off_c + lengths[c]),
 * off_c = sum of the earlier lengths).  lengths: host int64 [n_clips], each > n_fft/2;
 * 1 <= n_clips <= 65535.  out: device [sum_c F_c, d_out] with F_c = encoder_output_frames of
 * lengths[c], clips in order, bf16 for ENC_BF16 and float32 for ENC_F32.  Each clip is
 * normalised by its own log-mel maximum and encoded window by window, so its rows equal those
 * of encoder_forward on that clip alone.  `lengths` is read before the call returns. */
ENC_API encoder_status encoder_forward_ragged(encoder* e, const float* pcm, const int64_t* lengths,
                                      int32_t n_clips, void* out, void* stream);

/* Whole-clip path that also exports the residual stream (float32, after the layer's FFN
 * residual add) after each layer listed in `layers` (host int32 [n_taps], each in
 * [0, n_layers), repeats allowed): taps device float32 [n_taps, batch*F, d_model], row order as
 * `out`.  For cross-layer adapters that read intermediate encoder states ("DeepStack"-style
 * wiring named by the MOSS-Audio recipe page and the "scragnog/MOSS-Music-8B-Instruct-GGUF"
 * card; the pages do not say which layers are read).  `layers` is read before the call returns. */
ENC_API encoder_status encoder_forward_taps(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                    void* out, const int32_t* layers, int32_t n_taps, float* taps,
                                    void* stream);

/* Audio injection ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture", row "Audio
 * injection"): the embedding-table rows at the prompt's audio placeholder positions are
 * replaced by the adapter frames, in order: table[positions[i]] = frames[i], i < n_frames.
 * frames: device [n_frames, dim]; positions: device int64 [n_frames]; table: device
 * [table_rows, dim]; one dtype for both (ENC_BF16 or ENC_F32); dim % 8 == 0.  Positions outside
 * [0, table_rows) are skipped and counted into *n_skipped (device int32, may be NULL; the caller
 * clears it).  Positions should be distinct: a repeated row receives one of its frames.
 * Asynchronous on `stream`. */
ENC_API encoder_status encoder_splice(const void* frames, int64_t n_frames, int32_t dim,
                              const int64_t* positions, void* table, int64_t table_rows,
                              int32_t dtype, int32_t* n_skipped, void* stream);

/* ---- input conditioning ("SILVERTHRONE/Ossicle-4B" card: mono or stereo at any rate;
 * "cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Quick Start": the tower takes 16 kHz mono) --- */

/* Samples after conditioning n_in input frames at sample_rate: ceil(n_in * 16000 / rate) (n_in
 * at 16 kHz).  ENC_E_UNSUPPORTED for rates whose ratio to 16 kHz needs more than 4096 filter
 * phases (16000 / gcd(rate, 16000) > 4096) or more than 32x downsampling. */
ENC_API encoder_status encoder_conditioned_length(int64_t n_in, int32_t sample_rate, int64_t* n_out);

/* 16 kHz mono from interleaved float32 PCM in (device [n_in][channels], 1 <= channels <= 64):
 * the mean of the channels, then (rates other than 16 kHz) band-limited resampling with a
 * Hann-windowed sinc: cutoff 0.945 x the lower Nyquist, 16 zero crossings per side, each
 * polyphase phase normalised to unit DC gain, zeros outside the signal.  out: device float32
 * [n_out] (encoder_conditioned_length).  The pages name no filter; this one is the documented
 * reading.  The filter table is built on the host and cached per rate in the handle. */
ENC_API encoder_status encoder_condition_audio(encoder* e, const float* in, int64_t n_in, int32_t channels,
                                       int32_t sample_rate, float* out, void* stream);

/* Normalised log-mel only ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture" row
 * "Audio": 128 Whisper-style mel bins, n_fft 400, hop 160; "Non-obvious gotchas" item 2):
 * mel device float32 [batch, n_samples/160, 128], each clip normalised by its own maximum.
 * Same argument checks as encoder_forward; the workspace grows on demand. */
ENC_API encoder_status encoder_log_mel(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                               float* mel, void* stream);

/* encoder_log_mel for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid hipMalloc): same arguments, same result, and no
 * allocation of any kind in the call.  Its per-call scratch (clip spans and per-clip maximum
 * keys) lives in a fixed 128 KiB array of device memory per GPU, held until the process ends,
 * so batch is at most 4096 (larger calls return ENC_E_INVALID_ARG).  Every call on one GPU
 * shares that array: calls that overlap on one GPU (from several threads or streams) race and
 * must be serialised by the caller.  The raw log-mel is written into `mel` and normalised in
 * place. */
ENC_API encoder_status encoder_log_mel_noalloc(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                       float* mel, void* stream);

/* Stage-wise check point: runs the whole-clip path up to `stage` and writes that stage's output
 * as float32 to dst (dst_elems values available).  Single pass only (batch*F <=
 * max_tokens_per_pass).  Stages and layouts (nw = windows, ntok = batch*F):
 *   0 log-mel [batch, T, 128]      1 conv1 [nw, 4W, 64, C]   2 conv2 [nw, 2W, 32, C]
 *   3 conv3 [ntok, 16, C]          4 conv_out + positions [ntok, d]
 *   5 residual after layer `layer` [ntok, d]     6 head (proj2) [ntok, d_out]
 *   7 adapter output [ntok, d_out]
 * Conv stages are padded per window; positions at or beyond a window's valid length are
 * undefined.  Conv channels are innermost (c fastest, then frequency, then time). */
ENC_API encoder_status encoder_debug_stage(encoder* e, const float* pcm, int64_t n_samples, int32_t batch,
                                   int32_t stage, int32_t layer, float* dst, int64_t dst_elems,
                                   void* stream);

/* ---- per-kernel timing (HIP events on the forward's stream) -------------------------------- */

enum {
  ENC_K_MEL = 0, ENC_K_CONV1, ENC_K_CONV2, ENC_K_CONV3, ENC_K_CONV_OUT, ENC_K_LN, ENC_K_QKV,
  ENC_K_ATTN, ENC_K_OPROJ, ENC_K_FFN1, ENC_K_FFN2, ENC_K_PROJ1, ENC_K_PROJ2, ENC_K_GATE_UP,
  ENC_K_DOWN, ENC_K_OTHER, ENC_K_COUNT
};
/* mode 0: off.  mode 1: forward calls bracket each kernel launch with events on the call's
 * stream and run their passes one after another there (the passes of an untimed call: a call of
 * 4000 tokens or more that fits one pass still runs as its two halves).  mode 2: as mode 1, but
 * a call that fits one pass runs as that single pass.  Other modes return ENC_E_INVALID_ARG.
 * encoder_timing_read synchronises on the recorded events and returns, per ENC_K_* id, the
 * summed milliseconds and the launch count since the last reset (arrays of ENC_K_COUNT
 * entries). */
ENC_API encoder_status encoder_timing_enable(encoder* e, int32_t enable);
ENC_API encoder_status encoder_timing_read(encoder* e, double* ms, int64_t* launches, int32_t reset);

/* ---- single-kernel entry points (kernel-level tests) --------------------------------------- */

/* C = epi(A . W^T).  A device [M, K] row-major, W device [N, K] row-major, both bf16 (dtype
 * ENC_BF16) or float32 (ENC_F32).  bias: device float32 [N] or NULL.  N % 4 == 0 (N % 8 == 0
 * for bf16 output, epi 0 and 1), K % 8 == 0; other shapes return ENC_E_INVALID_ARG before any
 * launch.
 * epi 0: C[M,N] = acc + bias, stored in dtype.   epi 1: C = GELU(acc + bias), stored in dtype.
 * epi 2: C[M,N] float32 += acc + bias (residual update).
 * epi 3: SwiGLU over 32-column interleaved gate/up rows of W (rows 64j..64j+31 gate, 64j+32..64j+63
 *        up, N % 64 == 0): C[M, N/2] = SiLU(gate) * up, stored in dtype. */
ENC_API encoder_status encoder_op_linear(const void* A, const void* W, const float* bias, void* C,
                                 int64_t M, int32_t N, int32_t K, int32_t epi, int32_t dtype,
                                 void* stream);

/* int4 weight-only quantisation of a float32 [N, K] weight (host; K % 128 == 0): per row and
 * group of 128 inputs, scale s = bf16(max |w| / 7) and q = clamp(rint(w / s), -8, 7) (0 for an
 * all-zero group); q packed two per byte [N, K/2] (even k in the low nibble, two's complement),
 * scales bf16 bit patterns [N, K/128].  The GPU multiplies q by s in fp32 (exact) and rounds the
 * weight to bf16.  Storage for the "to_4bit" option of the "SILVERTHRONE/Ossicle-4B" card
 * (round-to-nearest, groups of 128). */
ENC_API encoder_status encoder_quantize_int4(const float* w, int64_t N, int64_t K, uint8_t* q,
                                     uint16_t* scales);

/* encoder_op_linear with int4 weights (q, scales from encoder_quantize_int4, on the device) and
 * bf16 A / C; N % 4 == 0 (N % 8 == 0 for epi 0 and 1), K % 128 == 0. */
ENC_API encoder_status encoder_op_linear_int4(const void* A, const uint8_t* q, const uint16_t* scales,
                                      const float* bias, void* C, int64_t M, int32_t N, int32_t K,
                                      int32_t epi, void* stream);

/* Windowed (block-diagonal) self-attention ("cstr/MOSS-Transcribe-preview-2B-GGUF" card,
 * "Architecture", row "Audio encoder": each token attends to the tokens of its own window only).
 * qkv device [ntok, 3*n_heads*64] (q | k | v, head h = columns 64h..64h+63 of each part), windows
 * device int32 [n_windows, 2] = {first token, length 1..128} (copied to the host and checked
 * before the launch).  out device [ntok, n_heads*64]; rows outside every window are not
 * written.  Scores scaled by 1/8, softmax in float32.  dtype ENC_BF16 or ENC_F32. */
ENC_API encoder_status encoder_op_attention(const void* qkv, const int32_t* windows, int32_t n_windows,
                                    int32_t n_heads, int64_t ntok, void* out, int32_t dtype,
                                    void* stream);

/* Window table of the kernel-level conv entries: device int32 [n_windows][8] per window
 * {clip, first frame within the clip (unused here), L0, L1, L2, L3, first token, first mel row}.
 * L0 (1..8W) is the window's frame count and L1..L3 its valid lengths after each stride-2 conv:
 * L1 = ceil(L0/2), L2 = ceil(L1/2), L3 = ceil(L2/2) (checked on the host before any launch).
 * Each window is an independent image: zero padding at its own time edges and at the frequency
 * edges (the window-local reading of the "cstr/MOSS-Transcribe-preview-2B-GGUF" card's conv
 * front end, which the "SILVERTHRONE/Ossicle-4B" card's "Long Audio" equality needs). */

/* conv1 of the conv front end ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture", row
 * "Conv front-end": Conv2D 1 -> C, 3x3, stride 2, pad 1, + bias, exact GELU) on the windows of
 * one pass.  mel: device float32 [mel_rows][128] raw log10 mel (window i reads rows
 * mel_row .. mel_row + L0 - 1); clip_max: device float32 [n_clips], each clip's maximum raw
 * value; the input image is the normalised mel (max(L, clip_max - 8) + 4) / 4.  w: device
 * float32 [C][3][3] (taps [freq][time]), b: device float32 [C].  act1: device [n_windows][L1s]
 * [64][C] in dtype (channels innermost), L1s >= every window's L1 (at most 4W); rows at or past
 * a window's L1 are not written.  C a multiple of 32, at most 2048.  Kernel-level test entry. */
ENC_API encoder_status encoder_op_conv1(const float* mel, int64_t mel_rows, const float* clip_max,
                                int32_t n_clips, const int32_t* windows, int32_t n_windows,
                                int32_t window_tokens, int32_t L1s, const float* w, const float* b,
                                int32_t C, void* act1, int32_t dtype, void* stream);

/* conv2 (level 2) or conv3 (level 3) of the conv front end (same card and row: Conv2D C -> C,
 * 3x3, stride 2, pad 1, + bias, exact GELU) as the library's implicit GEMM on the windows of one
 * pass.  L2s = ceil(L1s / 2).  level 2: in = act1 [n_windows][L1s][64][C], out = act2
 * [n_windows][L2s][32][C]; level 3: in = act2, out = token rows [n_tok][16][C] (window i's L3
 * rows from its first token on).  w_packed: device [C_out][9][C_in] in dtype, tap index
 * 3*freq + time (the [out][in][freq][time] weight with its taps moved outside the input
 * channels); bias: device float32 [C].  Rows at or past a window's output length are not
 * written.  C a multiple of 32, at most 4096; no operand above 2^31 - 1 bytes.  Kernel-level
 * test entry. */
ENC_API encoder_status encoder_op_conv(int32_t level, const void* in, const int32_t* windows,
                               int32_t n_windows, int32_t window_tokens, int32_t L1s, int64_t n_tok,
                               const void* w_packed, const float* bias, int32_t C, void* out,
                               int32_t dtype, void* stream);

/* LayerNorm of float32 rows x [M, D] -> y [M, D] in dtype; D % 256 == 0 or D % 64 == 0. */
ENC_API encoder_status encoder_op_layernorm(const float* x, const float* gamma, const float* beta,
                                    void* y, int64_t M, int32_t D, float eps, int32_t dtype,
                                    void* stream);

ENC_API const char* encoder_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AUDIO_ENCODER_H */
