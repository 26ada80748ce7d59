"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function
include/audio_encoder.h declares, validates configurations, and its integer window plan equals
the oracle's window plan exactly."""
import os
import re

import numpy as np
import pytest

import oracle as O
from audio_encoder_amd import binding as B
from audio_encoder_amd import synth as S

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "audio_encoder.h")


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"ENC_API\s+[\w\s\*]+?\b(encoder_\w+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("encoder_create", "encoder_forward", "encoder_forward_long", "encoder_log_mel",
              "encoder_destroy", "encoder_output_frames", "encoder_last_error"):
        assert n in names


def test_library_exports_every_declared_function():
    L = B.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(B._SIGS)


def oracle_cfg(cfg):
    return {k: cfg[k] for k in O.FULL}


def test_product_presets_match_oracle_presets():
    assert oracle_cfg(B.FULL) == O.FULL
    assert oracle_cfg(B.TINY) == O.TINY


@pytest.mark.parametrize("cfg", [B.FULL, B.TINY])
def test_weight_count_matches_blob_layout(cfg):
    assert B.encoder_weight_count(cfg) == S.weight_count(cfg)


def test_validate_cfg():
    assert B.encoder_validate_cfg(B.FULL) == B.ENC_OK
    assert B.encoder_validate_cfg(B.TINY) == B.ENC_OK
    bad = [dict(B.FULL, n_heads=19), dict(B.FULL, head_dim=32, n_heads=40),
           dict(B.FULL, conv_channels=100), dict(B.FULL, window_tokens=129),
           dict(B.FULL, window_tokens=0), dict(B.FULL, piece_tokens=850),
           dict(B.FULL, d_ffn=5000), dict(B.FULL, n_fft=512), dict(B.FULL, ln_eps=0.0),
           dict(B.FULL, dtype=7), dict(B.FULL, max_tokens_per_pass=50)]
    for c in bad:
        assert B.encoder_validate_cfg(c) == B.ENC_E_INVALID_ARG, c
    assert B.encoder_validate_cfg(dict(B.FULL, sample_rate=44100)) == B.ENC_E_UNSUPPORTED


@pytest.mark.parametrize("n", [201, 16000, 64000, 480000, 1024000, 2560000, 57600000, 480160,
                               127999, 128001])
def test_output_frames_match_oracle(n):
    assert B.encoder_output_frames(B.FULL, n) == O.n_output_frames(n, 100)
    assert B.encoder_output_frames(B.TINY, n) == O.n_output_frames(n, 25)


def test_output_frames_rejects_short_input():
    with pytest.raises(B.EncoderError):
        B.encoder_output_frames(B.FULL, 200)


@pytest.mark.parametrize("cfg,W", [(B.FULL, 100), (B.TINY, 25)])
@pytest.mark.parametrize("n,batch", [(480000, 16), (64000, 1), (8192000, 1), (57600000, 1),
                                     (129760, 3), (201, 2)])
def test_window_plan_is_bit_exact_with_oracle(cfg, W, n, batch):
    got = B.encoder_plan_windows(cfg, n, batch)
    T = O.n_mel_frames(n)
    F = O.n_output_frames(n, W)
    rows = []
    for b in range(batch):
        for w in O.window_plan(T, W):
            rows.append([b, w["start"], w["L0"], w["L1"], w["L2"], w["L3"], b * F + w["tok"]])
    assert np.array_equal(got, np.array(rows, dtype=np.int32).reshape(-1, 7))


RAGGED_LENGTHS = [[480000, 64000, 1_030_000], [201, 201], [129760, 201, 53920, 8192000],
                  [480000] * 4, [1000, 127999, 128001, 16000]]


@pytest.mark.parametrize("cfg,W", [(B.FULL, 100), (B.TINY, 25)])
@pytest.mark.parametrize("lengths", RAGGED_LENGTHS)
def test_ragged_window_plan_is_bit_exact_with_oracle(cfg, W, lengths):
    got = B.encoder_plan_windows_ragged(cfg, lengths)
    rows = [[w["clip"], w["start"], w["L0"], w["L1"], w["L2"], w["L3"], w["tok"]]
            for w in O.ragged_window_plan(lengths, W)]
    assert np.array_equal(got, np.array(rows, dtype=np.int32).reshape(-1, 7))
    # tokens of the call = the sum of the clips' output frames
    assert got[:, 5].sum() == sum(O.n_output_frames(n, W) for n in lengths)


def test_ragged_plan_of_equal_clips_is_the_batch_plan():
    a = B.encoder_plan_windows_ragged(B.FULL, [480000] * 5)
    b = B.encoder_plan_windows(B.FULL, 480000, 5)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("lengths", [[], [480000, 200], [200], [480000, -5]])
def test_ragged_plan_rejects_bad_lengths(lengths):
    with pytest.raises(B.EncoderError) as ei:
        B.encoder_plan_windows_ragged(B.FULL, lengths)
    assert ei.value.status == B.ENC_E_INVALID_ARG


@pytest.mark.parametrize("fs", [8000, 11025, 16000, 22050, 32000, 44100, 48000, 88200, 96000, 192000])
@pytest.mark.parametrize("n", [1, 3, 44100, 1_234_567])
def test_conditioned_length_matches_oracle(fs, n):
    assert B.encoder_conditioned_length(n, fs) == O.conditioned_length(n, fs)


@pytest.mark.parametrize("fs", [44101, 7, 0, -16000, 600000])
def test_conditioning_rejects_unsupported_rates(fs):
    with pytest.raises(B.EncoderError) as ei:
        B.encoder_conditioned_length(1000, fs)
    assert ei.value.status in (B.ENC_E_UNSUPPORTED, B.ENC_E_INVALID_ARG)


@pytest.mark.parametrize("N,K", [(3, 128), (37, 1280), (64, 2048)])
def test_library_int4_quantiser_is_bit_exact_with_oracle(N, K):
    rng = np.random.default_rng(N + K)
    w = (rng.standard_normal((N, K)) * rng.uniform(0.001, 0.1, size=(N, 1))).astype(np.float32)
    w[0, :128] = 0.0
    w[-1, -128:] *= 1e4
    q, sc = B.encoder_quantize_int4(w)
    q0, s0 = O.quantize_int4(w)
    assert np.array_equal(q, O.pack_int4(q0))
    assert np.array_equal(sc, s0.view(np.uint32) >> 16)


def test_int4_config_checks():
    assert B.encoder_validate_cfg(dict(B.FULL, weight_bits=4)) == B.ENC_OK
    assert B.encoder_validate_cfg(dict(B.TINY, weight_bits=4)) == B.ENC_E_INVALID_ARG  # fp32
    assert B.encoder_validate_cfg(dict(B.TINY, dtype="bf16", weight_bits=4)) == B.ENC_OK
    assert B.encoder_validate_cfg(dict(B.FULL, weight_bits=8)) == B.ENC_E_INVALID_ARG


def test_plan_of_hour_stream_has_45000_tokens():
    tab = B.encoder_plan_windows(B.FULL, 57_600_000, 1)
    assert len(tab) == 450 and tab[:, 5].sum() == 45000
    # 64 s pieces are 8 whole windows each: every 8th window starts a piece
    assert np.all(tab[::8, 1] % 6400 == 0)


def test_create_rejects_bad_blob_without_touching_the_gpu():
    import ctypes
    c = B.make_cfg(B.TINY)
    h = ctypes.c_void_p()
    w = np.zeros(10, dtype=np.float32)
    st = B.lib().encoder_create(w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 10,
                                ctypes.byref(c), ctypes.byref(h))
    assert st == B.ENC_E_INVALID_ARG
    assert b"config needs" in B.lib().encoder_last_error()


def test_forward_argument_checks():
    import ctypes
    L = B.lib()
    assert L.encoder_forward(None, None, 1000, 1, None, None) == B.ENC_E_INVALID_ARG
    assert L.encoder_op_linear(None, None, None, None, 1, 1, 1, 0, 0, None) == B.ENC_E_INVALID_ARG
    # shape checks come before any device access: the pointers below are never dereferenced
    p = ctypes.c_void_p(256)
    for N, K in ((6, 64), (2, 64), (64, 12), (64, 0), (0, 64)):
        assert L.encoder_op_linear(p, p, None, p, 8, N, K, 0, 0, None) == B.ENC_E_INVALID_ARG, (N, K)
        if N == 6:
            assert b"N % 4" in L.encoder_last_error()
    for N, K in ((6, 128), (64, 64), (12, 128)):
        assert L.encoder_op_linear_int4(p, p, p, None, p, 8, N, K, 0, None) == B.ENC_E_INVALID_ARG, (N, K)
    # bf16 outputs (epi 0 and 1) leave eight columns per lane: N % 8 == 0
    assert L.encoder_op_linear(p, p, None, p, 8, 12, 64, 1, B.ENC_BF16, None) == B.ENC_E_INVALID_ARG
    assert b"N % 8" in L.encoder_last_error()


def test_kernel_gelu_constants_follow_abramowitz_stegun_7_1_28():
    """The device GELU (csrc/ae_internal.h, gelu_erf) folds 1/sqrt(2) and 2^(1/16) into the
    coefficients of Abramowitz & Stegun 7.1.28, erfc(z) ~ (1 + a1 z + ... + a6 z^6)^-16.  Its seven
    constants must be 2^(1/16) a_i 2^(-i/2) (a_0 = 1), and the formula, evaluated in float32 as
    written, must stay within 1e-6 of x Phi(x) (float64 erf)."""
    import math
    src = open(os.path.join(os.path.dirname(HEADER), "..", "audio_encoder_amd", "csrc",
                            "ae_internal.h")).read()
    body = src[src.index("inline float gelu_erf"):src.index("inline float silu")]
    consts = [float(c) for c in re.findall(r"([0-9]\.[0-9]+e[+-][0-9]+)f", body)]
    # in Horner order: c6, c5, c4, c3, c2, c1, c0
    a = [1.0, 0.0705230784, 0.0422820123, 0.0092705272, 0.0001520143, 0.0002765672, 0.0000430638]
    want = [2 ** (1 / 16) * a[i] * 2 ** (-i / 2) for i in (6, 5, 4, 3, 2, 1, 0)]
    assert len(consts) == 7
    np.testing.assert_allclose(consts, want, rtol=2e-8)

    f32 = np.float32
    c = [f32(v) for v in consts]
    x = np.linspace(-12, 12, 480001).astype(f32)
    t = np.abs(x)
    p = f32(np.float64(t) * c[0] + c[1])
    for ci in c[2:]:
        p = (np.float64(t) * p + ci).astype(f32)  # fmaf: one rounding
    for _ in range(4):
        p = (p * p).astype(f32)
    with np.errstate(over="ignore", divide="ignore"):
        r = (f32(1) / p).astype(f32)
    g = (np.maximum(x, 0).astype(np.float64) - np.float64(t) * r).astype(f32)
    exact = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in x.astype(np.float64)])
    assert np.max(np.abs(g - exact)) < 1e-6


def test_conv_tap_from_float_reciprocal_is_exact():
    """The implicit-GEMM conv gather (csrc/ae_gemm.hip, AConv::kc) takes the tap of a K index k
    as trunc((float(k) + 0.5) * float(1 / C)) instead of an integer division; the launcher allows
    C <= 65536 (C % 32 == 0 from the config).  Exhaustive over k < 9C for every such C up to 8192
    and for the largest ones."""
    Cs = list(range(32, 8193, 32)) + list(range(65536 - 32 * 64, 65537, 32))
    for C in Cs:
        k = np.arange(9 * C, dtype=np.int64)
        inv = np.float32(1.0) / np.float32(C)
        tap = ((k.astype(np.float32) + np.float32(0.5)) * inv).astype(np.int64)
        assert np.array_equal(tap, k // C), C


def test_kernel_gelu_is_the_identity_from_16_up():
    """The conv index probes of the GPU suite (bias 16, integer inputs) rely on the device GELU
    returning x unchanged for x >= 16.  The formula of csrc/ae_internal.h, evaluated in float32
    as written (the reciprocal correctly rounded or flushed to zero alike), returns x exactly on
    every integer 16..1024 and on every float32 value of [16, 32) with a bf16 pattern."""
    src = open(os.path.join(os.path.dirname(HEADER), "..", "audio_encoder_amd", "csrc",
                            "ae_internal.h")).read()
    body = src[src.index("inline float gelu_erf"):src.index("inline float silu")]
    c = [np.float32(float(v)) for v in re.findall(r"([0-9]\.[0-9]+e[+-][0-9]+)f", body)]
    assert len(c) == 7
    f32 = np.float32
    ints = np.arange(16, 1025, dtype=f32)
    bf = (np.arange(0x4180, 0x4200, dtype=np.uint32) << 16).view(f32)  # [16, 32) in bf16 steps
    for x in (ints, bf):
        t = np.abs(x)
        p = f32(np.float64(t) * c[0] + c[1])
        for ci in c[2:]:
            p = (np.float64(t) * p + ci).astype(f32)
        with np.errstate(over="ignore", divide="ignore"):  # the 16th power overflows to inf
            for _ in range(4):
                p = (p * p).astype(f32)
            r = (f32(1) / p).astype(f32)
        for rr in (r, np.where(np.abs(r) < np.finfo(f32).tiny, f32(0), r)):  # with denormals flushed
            g = (np.maximum(x, 0).astype(np.float64) - np.float64(t) * rr).astype(f32)  # one fma
            assert np.array_equal(g, x)


def test_create_reports_a_failed_allocation(monkeypatch):
    """encoder_create with allocations refused (ENCODER_FAIL_ALLOC) returns ENC_E_OUT_OF_MEMORY
    before touching the GPU and leaves the handle unset."""
    import ctypes
    c = B.make_cfg(B.TINY)
    w = np.zeros(S.weight_count(B.TINY), dtype=np.float32)
    h = ctypes.c_void_p()
    monkeypatch.setenv("ENCODER_FAIL_ALLOC", "1")
    st = B.lib().encoder_create(w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), w.size,
                                ctypes.byref(c), ctypes.byref(h))
    assert st == B.ENC_E_OUT_OF_MEMORY and h.value is None
    assert b"ENCODER_FAIL_ALLOC" in B.lib().encoder_last_error()

