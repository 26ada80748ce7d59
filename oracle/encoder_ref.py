"""Float64 CPU oracle of the audio-tower forward pass (log-mel -> conv stack -> windowed
pre-LN Transformer -> head -> SwiGLU adapter).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Written from the model cards.  "Card T" below is the "cstr/MOSS-Transcribe-preview-2B-GGUF"
card, "card O" is the "SILVERTHRONE/Ossicle-4B" card, and "card M" is the
"scragnog/MOSS-Music-8B-Instruct-GGUF" card.  The method reaches its result directly, with no
approximation and no iteration, so every function here is the plain definition of its step in
float64, with numpy matmul as the only library primitive.  Where the cards leave a step open,
the docstring states the reading taken.

Pinned by ``tests/test_oracle_pins.py``: closed forms, invariants, brute force on tiny inputs
and independent library routines.  No function here is marked "parity unpinned".  The values
of the end-to-end output have no printed example to compare against; they are pinned stage by
stage instead.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

# Audio front end: 16 kHz mono, 128 mel bins, n_fft=400, hop=160 (card T, "Architecture",
# row "Audio").
SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160
N_MELS = 128
N_BINS = N_FFT // 2 + 1  # 201 one-sided DFT bins

# Full-size tower (card T, "Architecture": 32-layer pre-LN Transformer, d=1280, 20 heads x 64,
# FFN 5120; conv 1->480->480->480; conv_out 480*16 -> 1280; head 1280->1280->2048;
# SwiGLU adapter 2048->8192->2048).  The attention window is 100 tokens (8 s at 12.5 Hz).
FULL = dict(conv_channels=480, d_model=1280, n_layers=32, n_heads=20, head_dim=64, d_ffn=5120,
            window_tokens=100, d_out=2048, d_adapter=8192, n_mels=N_MELS, piece_tokens=800,
            dtype="bf16")
# Tiny stand-in used for fast end-to-end checks: channels 32, d 256, 2 layers, 4 heads x 64,
# FFN 1024, window 25 tokens, head 256->256->512, adapter 512->1024->512, fp32.
TINY = dict(conv_channels=32, d_model=256, n_layers=2, n_heads=4, head_dim=64, d_ffn=1024,
            window_tokens=25, d_out=512, d_adapter=1024, n_mels=N_MELS, piece_tokens=800,
            dtype="f32")

LN_EPS = 1e-5


# ============================================================================================
# O1  framing
# ============================================================================================
def n_mel_frames(n_samples: int) -> int:
    """Number of log-mel frames: one per hop.  The trailing STFT frame is dropped, which gives
    exactly ``n_samples // hop`` frames (card T, "Non-obvious gotchas", item 2)."""
    return int(n_samples) // HOP


def reflect_pad(x: np.ndarray, pad: int) -> np.ndarray:
    """Mirror ``pad`` samples about each end without repeating the edge sample:
    xp[-k] = x[k] and xp[N-1+k] = x[N-1-k] for k = 1..pad (Whisper's centred STFT; reading:
    reflect, the WhisperFeatureExtractor convention card T names).  Needs N > pad."""
    n = x.shape[0]
    if n <= pad:
        raise ValueError("reflect padding needs more samples than the pad width")
    left = x[1:pad + 1][::-1]
    right = x[n - 1 - pad:n - 1][::-1]
    return np.concatenate([left, x, right])


def frames(x: np.ndarray) -> np.ndarray:
    """Centred frames: frame t covers padded samples [hop*t, hop*t + n_fft), i.e. it is centred
    on original sample hop*t.  Frames 0..n_samples//hop-1 are kept."""
    x = np.asarray(x, dtype=np.float64)
    xp = reflect_pad(x, N_FFT // 2)
    T = n_mel_frames(x.shape[0])
    idx = HOP * np.arange(T)[:, None] + np.arange(N_FFT)[None, :]
    return xp[idx]


# ============================================================================================
# O2  STFT power
# ============================================================================================
def hann_periodic(n: int = N_FFT) -> np.ndarray:
    """Periodic Hann window w[n] = 0.5 - 0.5 cos(2 pi n / N) (reading: periodic, as Whisper)."""
    k = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * k / n)


def dft_basis() -> tuple[np.ndarray, np.ndarray]:
    """cos/sin of 2 pi k n / N for n < 400, k <= 200; the angle index k*n is reduced mod N
    in integers first so every entry is one correctly rounded fp64 cos or sin."""
    n = np.arange(N_FFT)[:, None]
    k = np.arange(N_BINS)[None, :]
    ang = 2.0 * np.pi * ((n * k) % N_FFT).astype(np.float64) / N_FFT
    return np.cos(ang), np.sin(ang)


def stft_power(fr: np.ndarray) -> np.ndarray:
    """|X_t[k]|^2 with X_t[k] = sum_n w[n] frame_t[n] exp(-2 pi i k n / 400), k = 0..200
    (reading: power spectrum, Whisper convention).  Direct DFT, fp64."""
    c, s = dft_basis()
    wf = fr * hann_periodic()[None, :]
    re = wf @ c
    im = -(wf @ s)
    return re * re + im * im


# ============================================================================================
# O3  Slaney mel filterbank
# ============================================================================================
_F_SP = 200.0 / 3.0           # Hz per mel below 1 kHz
_MIN_LOG_HZ = 1000.0
_MIN_LOG_MEL = _MIN_LOG_HZ / _F_SP   # 15
_LOGSTEP = math.log(6.4) / 27.0


def hz_to_mel(f):
    """Slaney (1998) mel scale: linear below 1 kHz, logarithmic above."""
    f = np.asarray(f, dtype=np.float64)
    lin = f / _F_SP
    logp = _MIN_LOG_MEL + np.log(np.maximum(f, 1e-300) / _MIN_LOG_HZ) / _LOGSTEP
    return np.where(f >= _MIN_LOG_HZ, logp, lin)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    lin = _F_SP * m
    logp = _MIN_LOG_HZ * np.exp(_LOGSTEP * (m - _MIN_LOG_MEL))
    return np.where(m >= _MIN_LOG_MEL, logp, lin)


def mel_points(n_mels: int = N_MELS, fmax: float = SAMPLE_RATE / 2) -> np.ndarray:
    """n_mels + 2 edge frequencies equally spaced in mel on [0, mel(fmax)], in Hz."""
    return mel_to_hz(np.linspace(0.0, float(hz_to_mel(fmax)), n_mels + 2))


def mel_filterbank(n_mels: int = N_MELS) -> np.ndarray:
    """[n_mels, 201] triangular filters on the DFT bin centres k*16000/400 Hz.

    Row m rises from f_m to f_{m+1} and falls to f_{m+2}, scaled by 2/(f_{m+2}-f_m) so each
    continuous triangle has unit area (Slaney area normalisation; reading of the standard
    construction the Whisper front end uses, fmin 0, fmax 8 kHz, no HTK scale).
    """
    f = mel_points(n_mels)
    fb = np.arange(N_BINS, dtype=np.float64) * SAMPLE_RATE / N_FFT
    W = np.zeros((n_mels, N_BINS))
    for m in range(n_mels):
        lo, ce, hi = f[m], f[m + 1], f[m + 2]
        rise = (fb - lo) / (ce - lo)
        fall = (hi - fb) / (hi - ce)
        W[m] = np.maximum(0.0, np.minimum(rise, fall)) * (2.0 / (hi - lo))
    return W


# ============================================================================================
# O4  log-mel and its normalisation
# ============================================================================================
def log_mel_raw(x: np.ndarray, chunk: int = 20000) -> np.ndarray:
    """log10(max(mel power, 1e-10)) per frame, [T, 128] (before the dynamic-range clamp)."""
    x = np.asarray(x, dtype=np.float64)
    T = n_mel_frames(x.shape[0])
    fb = mel_filterbank()
    xp = reflect_pad(x, N_FFT // 2)
    out = np.empty((T, N_MELS))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        idx = HOP * np.arange(t0, t1)[:, None] + np.arange(N_FFT)[None, :]
        P = stft_power(xp[idx])
        out[t0:t1] = np.log10(np.maximum(P @ fb.T, 1e-10))
    return out


def normalize_log_mel(L: np.ndarray, lmax: float) -> np.ndarray:
    """Clamp to (max - 8) then map x -> (x + 4) / 4.  ``lmax`` is the maximum over the clip
    (over the whole recording in long-audio mode, whose log-mel must equal the whole-clip
    one: card O, "Long Audio")."""
    return (np.maximum(L, lmax - 8.0) + 4.0) / 4.0


def log_mel(x: np.ndarray) -> np.ndarray:
    """Whisper-style normalised log-mel of one clip, [T, 128]."""
    L = log_mel_raw(x)
    return normalize_log_mel(L, float(L.max()))


# ============================================================================================
# O5  windows (the encoder's independent units)
# ============================================================================================
def ceil_half(n: int) -> int:
    return (int(n) + 1) // 2


def window_plan(T: int, window_tokens: int) -> list[dict]:
    """Split T mel frames into consecutive windows of 8*W frames; the last holds the remainder.

    Reading: the encoder is window-local.  Each attention window (W tokens = 8*W mel frames)
    is convolved with zero padding at its own time edges and its positions restart at 0.  This
    is the reading under which a piece encoder that sees only its 64 s piece reproduces the
    whole-clip output (card O, "Long Audio"); windowed block-diagonal attention is from card T,
    "Architecture".  Per window: start frame, valid lengths after 0..3 stride-2 convs (ceil
    chain), and the window's first output token.
    """
    wf = 8 * window_tokens
    out = []
    tok = 0
    for s in range(0, T, wf):
        L0 = min(wf, T - s)
        L1 = ceil_half(L0)
        L2 = ceil_half(L1)
        L3 = ceil_half(L2)
        out.append(dict(start=s, L0=L0, L1=L1, L2=L2, L3=L3, tok=tok))
        tok += L3
    return out


def n_output_frames(n_samples: int, window_tokens: int = 100) -> int:
    """Embeddings per clip: sum over windows of the 3x stride-2 ceil chain."""
    return sum(w["L3"] for w in window_plan(n_mel_frames(n_samples), window_tokens))


# ============================================================================================
# O6  conv stack
# ============================================================================================
def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) (reading: erf form; card T lists
    GELU without saying which)."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def conv2d_s2(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """3x3 stride-2 cross-correlation with zero padding 1 (card T, "Architecture": 3 x Conv2D
    stride-2).  x [Cin, H, T], w [Cout, Cin, 3, 3] (taps a along H = frequency, b along T =
    time), b [Cout].  y[o, i, j] = b[o] + sum_{c,a,b} w[o,c,a,b] x[c, 2i+a-1, 2j+b-1]."""
    Cin, H, Tn = x.shape
    Ho, To = ceil_half(H), ceil_half(Tn)
    xp = np.zeros((Cin, H + 2, Tn + 2))
    xp[:, 1:H + 1, 1:Tn + 1] = x
    y = np.empty((w.shape[0], Ho, To))
    y[...] = b[:, None, None]
    for a in range(3):
        for bb in range(3):
            patch = xp[:, a:a + 2 * Ho:2, bb:bb + 2 * To:2].reshape(Cin, Ho * To)
            tap = np.ascontiguousarray(w[:, :, a, bb])  # contiguous, so matmul uses BLAS
            y += (tap @ patch).reshape(-1, Ho, To)
    return y


def conv_stack(melw: np.ndarray, Wt: dict) -> list[np.ndarray]:
    """Three conv+GELU layers on one window's normalised log-mel melw [L0, 128].
    Returns the three activations, each [C, freq, time]."""
    x = melw.T[None, :, :]
    outs = []
    for i in (1, 2, 3):
        x = gelu(conv2d_s2(x, Wt[f"conv{i}.w"], Wt[f"conv{i}.b"]))
        outs.append(x)
    return outs


# ============================================================================================
# O7  flatten, conv_out, sinusoidal positions
# ============================================================================================
def flatten_tokens(y3: np.ndarray) -> np.ndarray:
    """h[j, c*F + f] = y3[c, f, j]: channel-major flatten to 480*16 = 7680 features per token
    (card T, "Architecture")."""
    C, F, L = y3.shape
    return y3.transpose(2, 0, 1).reshape(L, C * F)


def inv_timescales(d: int) -> np.ndarray:
    """omega_i = 10000^(-i/(d/2 - 1)), i < d/2 (the recomputed ``inv_timescales`` buffer,
    card M, "Conversion provenance")."""
    h = d // 2
    return np.exp(-math.log(10000.0) * np.arange(h, dtype=np.float64) / (h - 1))


def sinusoids(length: int, d: int) -> np.ndarray:
    """PE[p] = [sin(p*omega), cos(p*omega)] (sinusoidal positions, card T, "Architecture")."""
    ang = np.arange(length, dtype=np.float64)[:, None] * inv_timescales(d)[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


# ============================================================================================
# O8  pre-LN Transformer layer with windowed attention
# ============================================================================================
def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the feature axis, biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = np.square(x - mu).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def softmax(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int) -> np.ndarray:
    """Full (non-causal) softmax attention among the tokens of ONE window; head h uses features
    [64h, 64h+64); scores scaled by 1/sqrt(head_dim)."""
    n, d = q.shape
    hd = d // n_heads
    o = np.empty_like(q)
    for h in range(n_heads):
        sl = slice(h * hd, (h + 1) * hd)
        p = softmax((q[:, sl] @ k[:, sl].T) / math.sqrt(hd))
        o[:, sl] = p @ v[:, sl]
    return o


def encoder_layer(x: np.ndarray, Wt: dict, i: int, windows: list[tuple[int, int]],
                  n_heads: int) -> np.ndarray:
    """x += Attn(LN1(x)); x += FFN(LN2(x)).  Attention is block-diagonal: each window
    (token offset, length) attends only to itself (card T, "Architecture": pre-LN,
    windowed (block-diagonal) attention)."""
    p = f"layers.{i}."
    a = layer_norm(x, Wt[p + "ln1.g"], Wt[p + "ln1.b"])
    q = a @ Wt[p + "q.w"].T + Wt[p + "q.b"]
    k = a @ Wt[p + "k.w"].T + Wt[p + "k.b"]
    v = a @ Wt[p + "v.w"].T + Wt[p + "v.b"]
    o = np.empty_like(q)
    for t0, n in windows:
        o[t0:t0 + n] = window_attention(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], n_heads)
    x = x + o @ Wt[p + "o.w"].T + Wt[p + "o.b"]
    hdn = gelu(layer_norm(x, Wt[p + "ln2.g"], Wt[p + "ln2.b"]) @ Wt[p + "fc1.w"].T
               + Wt[p + "fc1.b"])
    return x + hdn @ Wt[p + "fc2.w"].T + Wt[p + "fc2.b"]


# ============================================================================================
# O9 / O10  head and adapter
# ============================================================================================
def head(x: np.ndarray, Wt: dict) -> np.ndarray:
    """ln_post -> proj1 -> GELU -> proj2 (card T, "Architecture", row "Encoder head")."""
    z = layer_norm(x, Wt["ln_post.g"], Wt["ln_post.b"])
    z = gelu(z @ Wt["proj1.w"].T + Wt["proj1.b"])
    return z @ Wt["proj2.w"].T + Wt["proj2.b"]


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def adapter(z: np.ndarray, Wt: dict) -> np.ndarray:
    """Gated MLP (SwiGLU): down(SiLU(gate z) * up z), no biases (card T, "Architecture",
    row "Adapter"; reading: bias-free, SiLU on the gate branch)."""
    return (silu(z @ Wt["gate.w"].T) * (z @ Wt["up.w"].T)) @ Wt["down.w"].T


# ============================================================================================
# weights
# ============================================================================================
def tensor_shapes(cfg: dict) -> list[tuple[str, tuple[int, ...]]]:
    """The flat blob's tensor order and shapes ([out, in] for linears, [out, in, 3, 3] for
    convs).  Written independently of the input generator; tests assert both agree."""
    C, d, f = cfg["conv_channels"], cfg["d_model"], cfg["d_ffn"]
    do, da = cfg["d_out"], cfg["d_adapter"]
    sh = [("conv1.w", (C, 1, 3, 3)), ("conv1.b", (C,)), ("conv2.w", (C, C, 3, 3)),
          ("conv2.b", (C,)), ("conv3.w", (C, C, 3, 3)), ("conv3.b", (C,)),
          ("conv_out.w", (d, C * (cfg["n_mels"] // 8)))]
    for i in range(cfg["n_layers"]):
        p = f"layers.{i}."
        for nm, s in (("ln1.g", (d,)), ("ln1.b", (d,)), ("q.w", (d, d)), ("q.b", (d,)),
                      ("k.w", (d, d)), ("k.b", (d,)), ("v.w", (d, d)), ("v.b", (d,)),
                      ("o.w", (d, d)), ("o.b", (d,)), ("ln2.g", (d,)), ("ln2.b", (d,)),
                      ("fc1.w", (f, d)), ("fc1.b", (f,)), ("fc2.w", (d, f)), ("fc2.b", (d,))):
            sh.append((p + nm, s))
    sh += [("ln_post.g", (d,)), ("ln_post.b", (d,)), ("proj1.w", (d, d)), ("proj1.b", (d,)),
           ("proj2.w", (do, d)), ("proj2.b", (do,)), ("gate.w", (da, do)), ("up.w", (da, do)),
           ("down.w", (do, da))]
    return sh


def unpack_weights(blob: np.ndarray, cfg: dict) -> dict:
    """Slice the flat float32 blob into float64 tensors."""
    out = {}
    off = 0
    for name, s in tensor_shapes(cfg):
        n = int(np.prod(s))
        out[name] = np.asarray(blob[off:off + n], dtype=np.float64).reshape(s)
        off += n
    if off != blob.size:
        raise ValueError(f"weight blob has {blob.size} floats, config needs {off}")
    return out


def tower_parameter_count(cfg: dict) -> int:
    """Parameters of conv stack + Transformer + head (the adapter excluded)."""
    return sum(int(np.prod(s)) for n, s in tensor_shapes(cfg)
               if not n.startswith(("gate", "up.", "down")))


# ============================================================================================
# whole forward
# ============================================================================================
def embed_windows(mel: np.ndarray, Wt: dict, cfg: dict, stages: dict | None = None):
    """Conv stack, flatten, conv_out and positions for every window of a normalised log-mel
    [T, 128].  Returns (tokens [F, d], [(token offset, length)] per window)."""
    W = cfg["window_tokens"]
    plan = window_plan(mel.shape[0], W)
    rows = []
    wins = []
    for wi in plan:
        ys = conv_stack(mel[wi["start"]:wi["start"] + wi["L0"]], Wt)
        if stages is not None:
            for i, y in enumerate(ys, 1):
                stages.setdefault(f"conv{i}", []).append(y)
        h = flatten_tokens(ys[2])
        e = h @ Wt["conv_out.w"].T + sinusoids(h.shape[0], cfg["d_model"])
        rows.append(e)
        wins.append((wi["tok"], wi["L3"]))
    return np.concatenate(rows, axis=0), wins


def encode_mel(mel: np.ndarray, Wt: dict, cfg: dict, stages: dict | None = None) -> np.ndarray:
    """Encoder + head + adapter on a normalised log-mel [T, 128] -> [F, d_out]."""
    x, wins = embed_windows(mel, Wt, cfg, stages)
    if stages is not None:
        stages["embed"] = x.copy()
    for i in range(cfg["n_layers"]):
        x = encoder_layer(x, Wt, i, wins, cfg["n_heads"])
        if stages is not None:
            stages[f"layer{i}"] = x.copy()
    z = head(x, Wt)
    if stages is not None:
        stages["head"] = z.copy()
    y = adapter(z, Wt)
    if stages is not None:
        stages["out"] = y.copy()
    return y


def encode(pcm: np.ndarray, Wt: dict, cfg: dict) -> np.ndarray:
    """Whole-clip path for one clip: log-mel normalised by the clip's own maximum, then
    ``encode_mel``.  Output [F, d_out] at 12.5 frames per second."""
    return encode_mel(log_mel(pcm), Wt, cfg)


def encode_batch(pcm: np.ndarray, Wt: dict, cfg: dict) -> np.ndarray:
    """[B, N] equal-length independent clips -> [B, F, d_out]."""
    return np.stack([encode(c, Wt, cfg) for c in np.atleast_2d(pcm)])


def encode_ragged(clips: list, Wt: dict, cfg: dict) -> np.ndarray:
    """Several clips of different lengths in one call (card O: the audio-input line of the
    model summary, and "Many clips in one question"): each clip is its own recording with its
    own log-mel maximum, encoded by ``encode``; the outputs are concatenated in clip order."""
    return np.concatenate([encode(np.asarray(c), Wt, cfg) for c in clips], axis=0)


# ---- input conditioning ---------------------------------------------------------------------
# Card O's model summary accepts mono or stereo at any sample rate; card T's "Quick Start" feeds
# the tower 16 kHz mono.  The pages name no resampling filter.  Reading (R29): the mean of the
# channels; 16 kHz passes through; otherwise band-limited interpolation with a Hann-windowed
# sinc (cutoff 0.945 x the lower Nyquist, 16 zero crossings per side), each output sample's
# weights normalised to sum to 1 over the full window (zeros outside the signal).
RS_ROLLOFF = 0.945
RS_ZEROS = 16


def downmix(x: np.ndarray) -> np.ndarray:
    """[n] or interleaved [n, channels] -> mono [n]: the mean over channels."""
    x = np.asarray(x, dtype=np.float64)
    return x if x.ndim == 1 else x.mean(axis=1)


def resample_ratio(fs: int) -> tuple[int, int]:
    """(L, M) with L / M = 16000 / fs in lowest terms."""
    g = math.gcd(int(fs), 16000)
    return 16000 // g, int(fs) // g


def conditioned_length(n_in: int, fs: int) -> int:
    L, M = resample_ratio(fs)
    return -(-n_in * L // M)


def resample_to_16k(x: np.ndarray, fs: int) -> np.ndarray:
    """Mono x at fs -> 16 kHz (R29), output sample j at input position t_j = j * fs / 16000:
    y[j] = sum_i x[i] h(i - t_j) / sum_k h(k - t_j) with the sums over the integers i, k with
    |i - t_j| <= R (x = 0 outside [0, n)), h(u) = 2 fc sinc(2 fc u) (1 + cos(pi u / R)) / 2,
    fc = 0.945 min(1, 16000/fs) / 2 cycles per input sample, R = 16 / (2 fc)."""
    x = np.asarray(x, dtype=np.float64)
    L, M = resample_ratio(fs)
    if L == 1 and M == 1:
        return x.copy()
    fc = 0.5 * RS_ROLLOFF * min(1.0, L / M)
    R = RS_ZEROS / (2.0 * fc)
    n_out = conditioned_length(x.size, fs)
    y = np.zeros(n_out)
    for j in range(n_out):
        t = j * M / L
        i = np.arange(math.ceil(t - R), math.floor(t + R) + 1)
        u = i - t
        h = 2.0 * fc * np.sinc(2.0 * fc * u) * 0.5 * (1.0 + np.cos(np.pi * u / R))
        xi = np.where((i >= 0) & (i < x.size), x[np.clip(i, 0, x.size - 1)], 0.0)
        y[j] = (h * xi).sum() / h.sum()
    return y


def condition_audio(x: np.ndarray, fs: int) -> np.ndarray:
    """Any channel count and rate -> 16 kHz mono (R29)."""
    return resample_to_16k(downmix(x), fs)


# ---- int4 weight-only (card O: to_4bit, round to nearest; groups of 128; R32) -----------------
def bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quantize_int4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """[N, K] (K a multiple of 128) -> (q int8 [N, K] in [-8, 7], s float32 [N, K/128]).
    Per row and group of 128 inputs: s = bf16(float32(max |w| / 7)), q = clip(rint(w / s), -8, 7)
    (q = 0 where s = 0)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    g = w.reshape(N, K // 128, 128)
    s = bf16((np.abs(g).max(axis=2) / 7.0).astype(np.float32))
    sd = s.astype(np.float64)[:, :, None]
    q = np.where(sd > 0, np.clip(np.rint(g / np.where(sd > 0, sd, 1.0)), -8, 7), 0.0)
    return q.reshape(N, K).astype(np.int8), s


def dequant_int4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The weight the GPU multiplies with: bf16(q * s) (the product is exact in float32)."""
    N, K = q.shape
    prod = (q.reshape(N, K // 128, 128).astype(np.float32) * s[:, :, None]).reshape(N, K)
    return bf16(prod).astype(np.float64)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two weights per byte, even k in the low nibble (two's complement)."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


INT4_MATRICES = ("q.w", "k.w", "v.w", "o.w", "fc1.w", "fc2.w")
INT4_HEAD = ("proj1.w", "proj2.w", "gate.w", "up.w", "down.w")


def int4_weights(Wt: dict, cfg: dict) -> dict:
    """The weights of an int4 configuration: every layer linear, the head projections and the
    adapter replaced by their dequantised int4 versions; convs, conv_out, biases and norms as
    they are."""
    out = dict(Wt)
    names = [f"layers.{i}.{m}" for i in range(cfg["n_layers"]) for m in INT4_MATRICES]
    for name in names + list(INT4_HEAD):
        out[name] = dequant_int4(*quantize_int4(Wt[name]))
    return out


def splice(table: np.ndarray, positions, frames: np.ndarray) -> tuple[np.ndarray, int]:
    """Audio injection (card T, "Architecture", row "Audio injection"): the embedding rows at
    the audio placeholder positions are replaced by the adapter frames, in order.  Returns the
    new table and the number of positions outside the table (left alone)."""
    out = table.copy()
    skipped = 0
    for i, p in enumerate(positions):
        if 0 <= p < out.shape[0]:
            out[p] = frames[i]
        else:
            skipped += 1
    return out, skipped


def encode_taps(pcm: np.ndarray, Wt: dict, cfg: dict, layers: list) -> tuple[np.ndarray, list]:
    """Whole-clip encoding plus the residual stream after each listed layer (the states a
    cross-layer adapter would read; which layers is not stated on the pages)."""
    st = {}
    y = encode_mel(log_mel(pcm), Wt, cfg, st)
    return y, [st[f"layer{l}"] for l in layers]


def ragged_window_plan(lengths: list, window_tokens: int) -> list[dict]:
    """Window plan of a ragged call: each clip's ``window_plan`` in clip order, tagged with the
    clip index, with the first output token counted over the whole call."""
    out, tok0 = [], 0
    for c, n in enumerate(lengths):
        plan = window_plan(n_mel_frames(int(n)), window_tokens)
        for w in plan:
            out.append(dict(w, clip=c, tok=w["tok"] + tok0))
        tok0 += sum(w["L3"] for w in plan)
    return out


def encode_long(pcm: np.ndarray, Wt: dict, cfg: dict) -> np.ndarray:
    """Long-audio mode: the log-mel of the whole recording (one maximum for all of it), cut at
    64 s piece boundaries (800 tokens = 6400 frames); each piece is encoded on its own and
    the outputs are concatenated (card O, "Long Audio")."""
    mel = log_mel(pcm)
    pf = 8 * cfg["piece_tokens"]
    return np.concatenate([encode_mel(mel[s:s + pf], Wt, cfg)
                           for s in range(0, mel.shape[0], pf)], axis=0)
