"""ctypes binding of ``libaudio_encoder.so`` (declared in ``include/audio_encoder.h``).

Argument marshalling only: every step of the forward pass runs in the library's HIP kernels.
PyTorch is used for device memory and the current stream.  There is no fallback: if the library
is missing or the GPU is absent, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_int64, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaudio_encoder.so")

ENC_OK = 0
ENC_E_INVALID_ARG = -1
ENC_E_OUT_OF_MEMORY = -2
ENC_E_DEVICE = -3
ENC_E_UNSUPPORTED = -4
ENC_BF16 = 0
ENC_F32 = 1

# kernel ids of encoder_timing_read
KERNELS = ["mel", "conv1", "conv2", "conv3", "conv_out", "layernorm", "qkv", "attention", "o_proj",
           "ffn1", "ffn2", "proj1", "proj2", "gate_up", "down", "other"]

STAGE_MEL, STAGE_CONV1, STAGE_CONV2, STAGE_CONV3, STAGE_EMBED, STAGE_LAYER, STAGE_HEAD, \
    STAGE_OUT = range(8)

# Full-size tower ("cstr/MOSS-Transcribe-preview-2B-GGUF" card, "Architecture"), and a tiny
# fp32 stand-in of the same structure for fast end-to-end checks.
FULL = dict(sample_rate=16000, n_fft=400, hop=160, n_mels=128, conv_channels=480, d_model=1280,
            n_layers=32, n_heads=20, head_dim=64, d_ffn=5120, window_tokens=100, d_out=2048,
            d_adapter=8192, piece_tokens=800, dtype="bf16", ln_eps=1e-5, max_tokens_per_pass=8192)
TINY = dict(FULL, conv_channels=32, d_model=256, n_layers=2, n_heads=4, d_ffn=1024,
            window_tokens=25, d_out=512, d_adapter=1024, dtype="f32")


class EncoderCfg(ctypes.Structure):
    _fields_ = [("sample_rate", c_int32), ("n_fft", c_int32), ("hop", c_int32),
                ("n_mels", c_int32), ("conv_channels", c_int32), ("d_model", c_int32),
                ("n_layers", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("d_ffn", c_int32), ("window_tokens", c_int32), ("d_out", c_int32),
                ("d_adapter", c_int32), ("piece_tokens", c_int32), ("dtype", c_int32),
                ("ln_eps", c_float), ("max_tokens_per_pass", c_int64), ("weight_bits", c_int32),
                ("split_small_gemms", c_int32)]


def make_cfg(cfg: dict) -> EncoderCfg:
    c = EncoderCfg()
    for name, _ in EncoderCfg._fields_:
        if name == "weight_bits":
            v = cfg.get(name, 16)
        elif name == "split_small_gemms":
            v = cfg.get(name, 0)
        else:
            v = cfg[name]
        if name == "dtype":
            v = {"bf16": ENC_BF16, "f32": ENC_F32}.get(v, v)
        setattr(c, name, v)
    return c


class EncoderError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None

_SIGS = {
    "encoder_validate_cfg": [POINTER(EncoderCfg)],
    "encoder_weight_count": [POINTER(EncoderCfg), POINTER(c_int64)],
    "encoder_output_frames": [POINTER(EncoderCfg), c_int64, POINTER(c_int64)],
    "encoder_plan_windows": [POINTER(EncoderCfg), c_int64, c_int32, POINTER(c_int32), c_int32,
                             POINTER(c_int32)],
    "encoder_plan_windows_ragged": [POINTER(EncoderCfg), POINTER(c_int64), c_int32, POINTER(c_int32),
                                    c_int32, POINTER(c_int32)],
    "encoder_plan_passes": [POINTER(EncoderCfg), POINTER(c_int64), c_int32, c_int32, POINTER(c_int64),
                            c_int32, POINTER(c_int32)],
    "encoder_create": [POINTER(c_float), c_int64, POINTER(EncoderCfg), POINTER(c_void_p)],
    "encoder_destroy": [c_void_p],
    "encoder_memory_stats": [c_void_p, POINTER(c_int64), POINTER(c_int64)],
    "encoder_forward": [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p],
    "encoder_forward_long": [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p],
    "encoder_forward_ragged": [c_void_p, c_void_p, POINTER(c_int64), c_int32, c_void_p, c_void_p],
    "encoder_forward_taps": [c_void_p, c_void_p, c_int64, c_int32, c_void_p, POINTER(c_int32),
                             c_int32, c_void_p, c_void_p],
    "encoder_conditioned_length": [c_int64, c_int32, POINTER(c_int64)],
    "encoder_condition_audio": [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p],
    "encoder_splice": [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_int64, c_int32, c_void_p,
                       c_void_p],
    "encoder_log_mel": [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p],
    "encoder_log_mel_noalloc": [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p],
    "encoder_debug_stage": [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_int32, c_void_p,
                            c_int64, c_void_p],
    "encoder_timing_enable": [c_void_p, c_int32],
    "encoder_timing_read": [c_void_p, POINTER(c_double), POINTER(c_int64), c_int32],
    "encoder_op_linear": [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32,
                          c_int32, c_int32, c_void_p],
    "encoder_quantize_int4": [POINTER(c_float), c_int64, c_int64, c_void_p, c_void_p],
    "encoder_op_linear_int4": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                               c_int32, c_int32, c_void_p],
    "encoder_op_attention": [c_void_p, c_void_p, c_int32, c_int32, c_int64, c_void_p, c_int32,
                             c_void_p],
    "encoder_op_conv1": [c_void_p, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                         c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "encoder_op_conv": [c_int32, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p,
                        c_void_p, c_int32, c_void_p, c_int32, c_void_p],
    "encoder_op_layernorm": [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_float,
                             c_int32, c_void_p],
    "encoder_last_error": [],
}


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m audio_encoder_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = None if name == "encoder_destroy" else c_int32
        L.encoder_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st: int):
    if st != ENC_OK:
        raise EncoderError(st, lib().encoder_last_error().decode())


# ---- host-only calls ---------------------------------------------------------------------------
def encoder_validate_cfg(cfg: dict) -> int:
    c = make_cfg(cfg)
    return lib().encoder_validate_cfg(ctypes.byref(c))


def encoder_weight_count(cfg: dict) -> int:
    c, n = make_cfg(cfg), c_int64()
    _check(lib().encoder_weight_count(ctypes.byref(c), ctypes.byref(n)))
    return n.value


def encoder_output_frames(cfg: dict, n_samples: int) -> int:
    c, n = make_cfg(cfg), c_int64()
    _check(lib().encoder_output_frames(ctypes.byref(c), n_samples, ctypes.byref(n)))
    return n.value


def encoder_plan_windows(cfg: dict, n_samples: int, batch: int) -> np.ndarray:
    c, nw = make_cfg(cfg), c_int32()
    _check(lib().encoder_plan_windows(ctypes.byref(c), n_samples, batch, None, 0, ctypes.byref(nw)))
    tab = np.zeros((nw.value, 7), dtype=np.int32)
    _check(lib().encoder_plan_windows(ctypes.byref(c), n_samples, batch,
                                      tab.ctypes.data_as(POINTER(c_int32)), nw.value,
                                      ctypes.byref(nw)))
    return tab


def encoder_conditioned_length(n_in: int, sample_rate: int) -> int:
    n = c_int64()
    _check(lib().encoder_conditioned_length(n_in, sample_rate, ctypes.byref(n)))
    return n.value


def _lengths(lengths) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(lengths, dtype=np.int64).ravel())


def encoder_plan_windows_ragged(cfg: dict, lengths) -> np.ndarray:
    """Window plan of a ragged call (clips of the given sample lengths, back to back)."""
    c, nw, L = make_cfg(cfg), c_int32(), _lengths(lengths)
    lp = L.ctypes.data_as(POINTER(c_int64))
    _check(lib().encoder_plan_windows_ragged(ctypes.byref(c), lp, L.size, None, 0, ctypes.byref(nw)))
    tab = np.zeros((nw.value, 7), dtype=np.int32)
    _check(lib().encoder_plan_windows_ragged(ctypes.byref(c), lp, L.size,
                                             tab.ctypes.data_as(POINTER(c_int32)), nw.value,
                                             ctypes.byref(nw)))
    return tab


def encoder_plan_passes(cfg: dict, lengths, pieces_per_pass: int = 0) -> np.ndarray:
    """Passes of a forward call over clips of the given sample lengths: int64 [n_passes, 6] =
    {first window, windows, first token, tokens, act1 rows per window, act2 rows per window}."""
    c, n, L = make_cfg(cfg), c_int32(), _lengths(lengths)
    lp = L.ctypes.data_as(POINTER(c_int64))
    _check(lib().encoder_plan_passes(ctypes.byref(c), lp, L.size, pieces_per_pass, None, 0,
                                     ctypes.byref(n)))
    tab = np.zeros((n.value, 6), dtype=np.int64)
    _check(lib().encoder_plan_passes(ctypes.byref(c), lp, L.size, pieces_per_pass,
                                     tab.ctypes.data_as(POINTER(c_int64)), n.value,
                                     ctypes.byref(n)))
    return tab


# ---- device calls (torch tensors for memory and stream) ---------------------------------------
def _stream():
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> c_void_p:
    return c_void_p(t.data_ptr()) if t is not None else c_void_p(0)


def _dtype_code(dt) -> int:
    import torch
    return ENC_BF16 if dt == torch.bfloat16 else ENC_F32


class Encoder:
    """One packed copy of the weights on the current GPU plus its workspace."""

    def __init__(self, weights: np.ndarray, cfg: dict):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("audio_encoder_amd needs a GPU; none is visible")
        self.cfg = dict(cfg)
        self._c = make_cfg(self.cfg)
        w = np.ascontiguousarray(weights, dtype=np.float32)
        h = c_void_p()
        _check(lib().encoder_create(w.ctypes.data_as(POINTER(c_float)), w.size,
                                    ctypes.byref(self._c), ctypes.byref(h)))
        self._h = h
        self.out_dtype = torch.bfloat16 if self.cfg["dtype"] == "bf16" else torch.float32

    def close(self):
        if getattr(self, "_h", None):
            lib().encoder_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def output_frames(self, n_samples: int) -> int:
        return encoder_output_frames(self.cfg, n_samples)

    def forward(self, pcm, out=None):
        """pcm: float32 CUDA tensor [batch, n_samples] -> [batch, F, d_out]."""
        import torch
        assert pcm.is_cuda and pcm.dtype == torch.float32 and pcm.is_contiguous()
        B, N = pcm.shape
        F = self.output_frames(N)
        if out is None:
            out = torch.empty((B, F, self.cfg["d_out"]), dtype=self.out_dtype, device=pcm.device)
        _check(lib().encoder_forward(self._h, _ptr(pcm), N, B, _ptr(out), _stream()))
        return out

    def forward_long(self, pcm, pieces_per_pass: int = 1, out=None):
        """pcm: float32 CUDA tensor [n_samples] (one recording) -> [F, d_out]."""
        import torch
        assert pcm.is_cuda and pcm.dtype == torch.float32 and pcm.is_contiguous()
        N = pcm.numel()
        F = self.output_frames(N)
        if out is None:
            out = torch.empty((F, self.cfg["d_out"]), dtype=self.out_dtype, device=pcm.device)
        _check(lib().encoder_forward_long(self._h, _ptr(pcm), N, pieces_per_pass, _ptr(out),
                                          _stream()))
        return out

    def forward_ragged(self, pcm, lengths, out=None):
        """pcm: float32 CUDA tensor of the clips back to back (sum(lengths) samples);
        lengths: per-clip sample counts -> [sum_c F_c, d_out], clips in order."""
        import torch
        assert pcm.is_cuda and pcm.dtype == torch.float32 and pcm.is_contiguous()
        L = _lengths(lengths)
        if int(L.sum()) != pcm.numel():
            raise ValueError(f"lengths add up to {int(L.sum())} samples, pcm has {pcm.numel()}")
        F = sum(self.output_frames(int(n)) for n in L) if all(n > 200 for n in L) else 0
        if out is None:
            out = torch.empty((max(F, 1), self.cfg["d_out"]), dtype=self.out_dtype,
                              device=pcm.device)[:F]
        _check(lib().encoder_forward_ragged(self._h, _ptr(pcm), L.ctypes.data_as(POINTER(c_int64)),
                                            L.size, _ptr(out), _stream()))
        return out

    def forward_taps(self, pcm, layers, out=None):
        """Whole-clip forward that also returns the residual stream after each layer in
        `layers`: (out [batch, F, d_out], taps float32 [len(layers), batch*F, d_model])."""
        import torch
        assert pcm.is_cuda and pcm.dtype == torch.float32 and pcm.is_contiguous()
        B_, N = pcm.shape
        F = self.output_frames(N)
        if out is None:
            out = torch.empty((B_, F, self.cfg["d_out"]), dtype=self.out_dtype, device=pcm.device)
        L = np.ascontiguousarray(np.asarray(layers, dtype=np.int32).ravel())
        taps = torch.empty((L.size, B_ * F, self.cfg["d_model"]), dtype=torch.float32,
                           device=pcm.device)
        _check(lib().encoder_forward_taps(self._h, _ptr(pcm), N, B_, _ptr(out),
                                          L.ctypes.data_as(POINTER(c_int32)), L.size, _ptr(taps),
                                          _stream()))
        return out, taps

    def condition_audio(self, pcm, sample_rate: int, out=None):
        """pcm: float32 CUDA tensor [n] (mono) or [n, channels] (interleaved) at sample_rate ->
        16 kHz mono float32 [n_out] (channel mean, windowed-sinc resampling)."""
        import torch
        assert pcm.is_cuda and pcm.dtype == torch.float32 and pcm.is_contiguous()
        n, ch = (pcm.shape[0], 1) if pcm.dim() == 1 else (pcm.shape[0], pcm.shape[1])
        n_out = encoder_conditioned_length(n, sample_rate)
        if out is None:
            out = torch.empty(n_out, dtype=torch.float32, device=pcm.device)
        _check(lib().encoder_condition_audio(self._h, _ptr(pcm), n, ch, sample_rate, _ptr(out),
                                             _stream()))
        return out

    def log_mel(self, pcm):
        import torch
        B, N = pcm.shape
        mel = torch.empty((B, N // 160, 128), dtype=torch.float32, device=pcm.device)
        _check(lib().encoder_log_mel(self._h, _ptr(pcm), N, B, _ptr(mel), _stream()))
        return mel

    def log_mel_noalloc(self, pcm, mel=None):
        """encoder_log_mel_noalloc: the log-mel with no allocation in the library (batch <= 4096);
        `mel` float32 [batch, n_samples/160, 128] may be passed in."""
        import torch
        B_, N = pcm.shape
        if mel is None:
            mel = torch.empty((B_, N // 160, 128), dtype=torch.float32, device=pcm.device)
        _check(lib().encoder_log_mel_noalloc(self._h, _ptr(pcm), N, B_, _ptr(mel), _stream()))
        return mel

    def debug_stage(self, pcm, stage: int, layer: int = 0):
        """float32 copy of one stage's output (layouts in include/audio_encoder.h)."""
        import torch
        B, N = pcm.shape
        cfg = self.cfg
        T = N // 160
        F = self.output_frames(N) * B
        nw = len(encoder_plan_windows(cfg, N, B))
        W, C = cfg["window_tokens"], cfg["conv_channels"]
        shape = {STAGE_MEL: (B, T, 128), STAGE_CONV1: (nw, 4 * W, 64, C),
                 STAGE_CONV2: (nw, 2 * W, 32, C), STAGE_CONV3: (F, 16, C),
                 STAGE_EMBED: (F, cfg["d_model"]), STAGE_LAYER: (F, cfg["d_model"]),
                 STAGE_HEAD: (F, cfg["d_out"]), STAGE_OUT: (F, cfg["d_out"])}[stage]
        dst = torch.empty(shape, dtype=torch.float32, device=pcm.device)
        _check(lib().encoder_debug_stage(self._h, _ptr(pcm), N, B, stage, layer, _ptr(dst),
                                         dst.numel(), _stream()))
        return dst

    def memory_stats(self) -> tuple[int, int]:
        w, ws = c_int64(), c_int64()
        _check(lib().encoder_memory_stats(self._h, ctypes.byref(w), ctypes.byref(ws)))
        return w.value, ws.value

    def timing_enable(self, mode: int = 1):
        """0 off; 1 time each kernel launch, running the passes of an untimed call one after
        another on one stream; 2 as 1, with a call that fits one pass run as that one pass."""
        _check(lib().encoder_timing_enable(self._h, int(mode)))

    def timing_read(self, reset: bool = True) -> dict:
        ms = (c_double * len(KERNELS))()
        n = (c_int64 * len(KERNELS))()
        _check(lib().encoder_timing_read(self._h, ms, n, 1 if reset else 0))
        return {k: (ms[i], n[i]) for i, k in enumerate(KERNELS)}


# ---- single-kernel entry points ------------------------------------------------------------------
def splice(frames, positions, table, n_skipped=None):
    """table[positions[i]] = frames[i] on the GPU (audio injection); positions int64 CUDA tensor.
    Out-of-range positions are skipped and counted into n_skipped (int32 CUDA tensor [1])."""
    import torch
    assert frames.dtype == table.dtype and frames.shape[-1] == table.shape[-1]
    assert positions.dtype == torch.int64 and positions.numel() == frames.shape[0]
    _check(lib().encoder_splice(_ptr(frames), frames.shape[0], frames.shape[-1], _ptr(positions),
                                _ptr(table), table.shape[0], _dtype_code(table.dtype),
                                _ptr(n_skipped), _stream()))
    return table


def encoder_quantize_int4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 [N, K] -> (q uint8 [N, K/2], scales uint16 bf16 bits [N, K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.zeros((N, K // 2), dtype=np.uint8)
    sc = np.zeros((N, max(K // 128, 1)), dtype=np.uint16)
    _check(lib().encoder_quantize_int4(w.ctypes.data_as(POINTER(c_float)), N, K,
                                       c_void_p(q.ctypes.data), c_void_p(sc.ctypes.data)))
    return q, sc


def op_linear_int4(A, q, scales, bias, C, epi: int):
    """C = epi(A @ dequant(q, scales)^T + bias) on the GPU; A/C bf16 CUDA tensors, q uint8 and
    scales int16 (bf16 bits) CUDA tensors from encoder_quantize_int4."""
    M, K = A.shape
    N = q.shape[0]
    _check(lib().encoder_op_linear_int4(_ptr(A), _ptr(q), _ptr(scales), _ptr(bias), _ptr(C), M, N,
                                        K, epi, _stream()))


def op_linear(A, W, bias, C, epi: int):
    """C = epi(A W^T) (see encoder_op_linear)."""
    M, K = A.shape
    N = W.shape[0]
    _check(lib().encoder_op_linear(_ptr(A), _ptr(W), _ptr(bias), _ptr(C), M, N, K, epi,
                                   _dtype_code(A.dtype), _stream()))
    return C


def op_attention(qkv, windows, n_heads: int, out):
    _check(lib().encoder_op_attention(_ptr(qkv), _ptr(windows), windows.shape[0], n_heads,
                                      qkv.shape[0], _ptr(out), _dtype_code(qkv.dtype), _stream()))
    return out


def op_conv1(mel, clip_max, windows, window_tokens: int, L1s: int, w, b, act1):
    """conv1 on the windows of one pass (see encoder_op_conv1): mel float32 [rows, 128], clip_max
    float32 [n_clips], windows int32 [n_windows, 8], w float32 [C, 3, 3], b float32 [C] and
    act1 [n_windows, L1s, 64, C] (bf16 or float32), all CUDA tensors."""
    C = b.shape[0]
    _check(lib().encoder_op_conv1(_ptr(mel), mel.shape[0], _ptr(clip_max), clip_max.shape[0],
                                  _ptr(windows), windows.shape[0], window_tokens, L1s, _ptr(w),
                                  _ptr(b), C, _ptr(act1), _dtype_code(act1.dtype), _stream()))
    return act1


def op_conv(level: int, inp, windows, window_tokens: int, L1s: int, n_tok: int, w_packed, bias, out):
    """conv2 (level 2) or conv3 (level 3) implicit GEMM (see encoder_op_conv); w_packed
    [C_out, 9, C_in] in the dtype of inp and out."""
    C = bias.shape[0]
    _check(lib().encoder_op_conv(level, _ptr(inp), _ptr(windows), windows.shape[0], window_tokens,
                                 L1s, n_tok, _ptr(w_packed), _ptr(bias), C, _ptr(out),
                                 _dtype_code(out.dtype), _stream()))
    return out


def op_layernorm(x, gamma, beta, y, eps: float = 1e-5):
    M, D = x.shape
    _check(lib().encoder_op_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), M, D, eps,
                                      _dtype_code(y.dtype), _stream()))
    return y
