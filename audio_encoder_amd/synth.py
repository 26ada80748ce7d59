"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle's tests.

This module holds none of the encoder's arithmetic. It only draws random numbers and
synthesises test signals:

* PCM: 16 kHz mono float32 clips shaped like the workloads the model cards talk about
  (30 s question clips, 64 s long-audio pieces, hour-long recordings; "SILVERTHRONE/Ossicle-4B"
  card, sections "Model Overview" and "Long Audio").  The content (pink noise, speech-like
  harmonic bursts, chords, tones) is made up here; no dataset item is reproduced.
* Weights: one flat little-endian float32 blob, every tensor drawn N(0, 0.02) (LayerNorm gains
  1 + N(0, 0.02)) from ``numpy.random.default_rng(seed)`` in a fixed tensor order.  bf16
  configurations round each drawn value to bf16 (round-to-nearest-even) once, so both the oracle
  and the GPU library read exactly the same weight values.

The tensor order (``weight_spec``) is the blob interface that both implementations parse on
their own; it is documented in ``include/audio_encoder.h``.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000


# --------------------------------------------------------------------------------------------
# weight blob
# --------------------------------------------------------------------------------------------
def weight_spec(cfg: dict) -> list[tuple[str, tuple[int, ...]]]:
    """Names and shapes of the blob's tensors, in blob order (PyTorch [out, in] layouts)."""
    C = cfg["conv_channels"]
    d = cfg["d_model"]
    f = cfg["d_ffn"]
    do = cfg["d_out"]
    da = cfg["d_adapter"]
    freq3 = cfg["n_mels"] // 8
    spec: list[tuple[str, tuple[int, ...]]] = [
        ("conv1.w", (C, 1, 3, 3)), ("conv1.b", (C,)),
        ("conv2.w", (C, C, 3, 3)), ("conv2.b", (C,)),
        ("conv3.w", (C, C, 3, 3)), ("conv3.b", (C,)),
        ("conv_out.w", (d, C * freq3)),
    ]
    for i in range(cfg["n_layers"]):
        p = f"layers.{i}."
        spec += [
            (p + "ln1.g", (d,)), (p + "ln1.b", (d,)),
            (p + "q.w", (d, d)), (p + "q.b", (d,)),
            (p + "k.w", (d, d)), (p + "k.b", (d,)),
            (p + "v.w", (d, d)), (p + "v.b", (d,)),
            (p + "o.w", (d, d)), (p + "o.b", (d,)),
            (p + "ln2.g", (d,)), (p + "ln2.b", (d,)),
            (p + "fc1.w", (f, d)), (p + "fc1.b", (f,)),
            (p + "fc2.w", (d, f)), (p + "fc2.b", (d,)),
        ]
    spec += [
        ("ln_post.g", (d,)), ("ln_post.b", (d,)),
        ("proj1.w", (d, d)), ("proj1.b", (d,)),
        ("proj2.w", (do, d)), ("proj2.b", (do,)),
        ("gate.w", (da, do)), ("up.w", (da, do)), ("down.w", (do, da)),
    ]
    return spec


def weight_count(cfg: dict) -> int:
    return int(sum(int(np.prod(s)) for _, s in weight_spec(cfg)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returned as float32."""
    x = np.array(x, dtype=np.float32, copy=True)
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)  # finite values only: no carry out of the exponent
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def make_weights(cfg: dict, seed: int = 0) -> np.ndarray:
    """Flat float32 blob, tensors in ``weight_spec`` order, N(0, 0.02) draws.

    LayerNorm gains are 1 + N(0, 0.02) (a pure N(0, 0.02) gain would squash every normalised
    row towards zero); LayerNorm shifts and all biases are N(0, 0.02) so every bias path is live.
    """
    rng = np.random.default_rng(seed)
    blob = np.empty(weight_count(cfg), dtype=np.float32)
    off = 0
    for name, shape in weight_spec(cfg):
        n = int(np.prod(shape))
        v = rng.standard_normal(n, dtype=np.float32)
        v *= np.float32(0.02)
        if name.endswith(".g"):
            v += np.float32(1.0)
        blob[off:off + n] = v
        off += n
    if cfg.get("dtype", "bf16") == "bf16":
        # chunked so the full-size blob never needs a second full-size uint64 temporary
        step = 1 << 24
        for s in range(0, blob.size, step):
            blob[s:s + step] = round_to_bf16(blob[s:s + step])
    return blob


# --------------------------------------------------------------------------------------------
# PCM primitives
# --------------------------------------------------------------------------------------------
def _t(n: int) -> np.ndarray:
    return np.arange(n, dtype=np.float64) / SAMPLE_RATE


def rms_normalize(x: np.ndarray) -> np.ndarray:
    r = float(np.sqrt(np.mean(np.square(x))))
    return x / r if r > 0 else x


def peak_normalize(x: np.ndarray, peak: float) -> np.ndarray:
    m = float(np.max(np.abs(x)))
    return x * (peak / m) if m > 0 else x


def pink(rng: np.random.Generator, n: int) -> np.ndarray:
    """White N(0,1) shaped by 1/sqrt(k) in the rfft domain (DC removed), unit RMS."""
    w = rng.standard_normal(n)
    X = np.fft.rfft(w)
    k = np.arange(X.size, dtype=np.float64)
    X[0] = 0.0
    X[1:] /= np.sqrt(k[1:])
    return rms_normalize(np.fft.irfft(X, n))


def bursts(rng: np.random.Generator, n: int) -> np.ndarray:
    """Speech-like harmonic bursts separated by exact-zero gaps.

    Gaps last U(0.05, 0.30) s, bursts U(0.08, 0.40) s.  A burst has f0 ~ U(100, 300) Hz gliding
    linearly to f0*U(0.9, 1.1), harmonics up to 4 kHz with amplitude 1/h and random phase, and a
    Hann envelope.
    """
    y = np.zeros(n, dtype=np.float64)
    pos = 0
    while True:
        pos += int(rng.uniform(0.05, 0.30) * SAMPLE_RATE)
        blen = int(rng.uniform(0.08, 0.40) * SAMPLE_RATE)
        if pos >= n:
            break
        blen = min(blen, n - pos)
        f0 = rng.uniform(100.0, 300.0)
        f1 = f0 * rng.uniform(0.9, 1.1)
        freq = np.linspace(f0, f1, blen)
        phase = 2.0 * np.pi * np.cumsum(freq) / SAMPLE_RATE
        nh = int(4000.0 // max(f0, f1))
        ph = rng.uniform(0.0, 2.0 * np.pi, size=nh)
        s = np.zeros(blen)
        for h in range(1, nh + 1):
            s += np.sin(h * phase + ph[h - 1]) / h
        if blen > 1:
            env = 0.5 - 0.5 * np.cos(2.0 * np.pi * np.arange(blen) / (blen - 1))
        else:
            env = np.zeros(1)
        y[pos:pos + blen] = s * env
        pos += blen
    return y


def chords(rng: np.random.Generator, n: int, change_s: float = 2.0) -> np.ndarray:
    """Major triads (ratios 1, 5/4, 3/2) on a root ~ U(110, 440) Hz, re-drawn every 2 s."""
    y = np.zeros(n, dtype=np.float64)
    step = int(change_s * SAMPLE_RATE)
    for s in range(0, n, step):
        m = min(step, n - s)
        root = rng.uniform(110.0, 440.0)
        t = _t(m)
        ph = rng.uniform(0.0, 2.0 * np.pi, size=3)
        for r, p in zip((1.0, 1.25, 1.5), ph):
            y[s:s + m] += np.sin(2.0 * np.pi * root * r * t + p)
    return y


def tone(rng: np.random.Generator, n: int) -> np.ndarray:
    f = rng.uniform(100.0, 1000.0)
    return np.sin(2.0 * np.pi * f * _t(n))


# --------------------------------------------------------------------------------------------
# workload clips
# --------------------------------------------------------------------------------------------
def three_sines(seed: int = 0, n: int = 64000) -> np.ndarray:
    """Tiny-encoder clip: 0.3*sin at 220, 440 and 1000 Hz (zero phase) + N(0, 0.01^2) noise."""
    rng = np.random.default_rng(seed)
    t = _t(n)
    x = sum(0.3 * np.sin(2.0 * np.pi * f * t) for f in (220.0, 440.0, 1000.0))
    x = x + rng.normal(0.0, 0.01, n)
    return x.astype(np.float32)


def pink_plus_bursts(seed: int = 1, n: int = 480000) -> np.ndarray:
    """30 s clip: 0.25 x unit-RMS pink noise plus harmonic bursts, peak 0.5."""
    rng = np.random.default_rng(seed)
    x = 0.25 * pink(rng, n) + bursts(rng, n)
    return peak_normalize(x, 0.5).astype(np.float32)


def mixed_clip(seed: int, n: int = 480000) -> np.ndarray:
    """Pink noise, a tone or chords, and bursts mixed with Dirichlet(1,1,1) weights, peak 0.5."""
    rng = np.random.default_rng(seed)
    w = rng.dirichlet([1.0, 1.0, 1.0])
    tonal = tone(rng, n) if rng.uniform() < 0.5 else chords(rng, n)
    x = (w[0] * pink(rng, n) + w[1] * rms_normalize(tonal)
         + w[2] * rms_normalize(bursts(rng, n)))
    return peak_normalize(x, 0.5).astype(np.float32)


def mixed_batch(seeds, n: int = 480000) -> np.ndarray:
    return np.stack([mixed_clip(s, n) for s in seeds])


def segment_stream(seed: int, seconds: float, seg_s=None, per_segment_peak: bool = False,
                   peak: float = 0.5) -> np.ndarray:
    """A recording made of consecutive segments cycling bursts -> pink noise -> chords.

    ``seg_s=None`` draws each segment length from U(5, 20) s; a number fixes it.
    With ``per_segment_peak`` each segment is peak-normalised on its own, otherwise the
    whole stream is.
    """
    rng = np.random.default_rng(seed)
    n = int(round(seconds * SAMPLE_RATE))
    out = np.zeros(n, dtype=np.float64)
    pos = 0
    kind = 0
    while pos < n:
        sl = rng.uniform(5.0, 20.0) if seg_s is None else float(seg_s)
        m = min(int(round(sl * SAMPLE_RATE)), n - pos)
        if kind == 0:
            s = bursts(rng, m)
        elif kind == 1:
            s = pink(rng, m)
        else:
            s = chords(rng, m)
        if per_segment_peak:
            s = peak_normalize(s, peak)
        out[pos:pos + m] = s
        pos += m
        kind = (kind + 1) % 3
    if not per_segment_peak:
        out = peak_normalize(out, peak)
    return out.astype(np.float32)


def long_stream_512s(seed: int = 200) -> np.ndarray:
    """512 s stream (8 pieces of 64 s), U(5, 20) s segments, peak 0.5."""
    return segment_stream(seed, 512.0)


def hour_stream(seed: int = 300, seconds: float = 3600.0) -> np.ndarray:
    """60-minute recording: 20 s segments bursts -> pink -> chords, each peak 0.5."""
    return segment_stream(seed, seconds, seg_s=20.0, per_segment_peak=True)


def pure_tone_bin(k: int, amp: float, n: int) -> np.ndarray:
    """A sine exactly on STFT bin k (k*40 Hz at 16 kHz with a 400-point frame), no noise."""
    return (amp * np.sin(2.0 * np.pi * 40.0 * k * _t(n))).astype(np.float32)
