"""The pass plan (encoder_plan_passes, host only): a call is encoded as passes of consecutive
whole windows, and no pass may hold an operand the kernels cannot address (32-bit byte offsets
of their buffer descriptors) or more tokens than max_tokens_per_pass.  Many clips per call is
the workload of the "SILVERTHRONE/Ossicle-4B" card ("Many clips in one question"); long-audio
passes hold whole 64 s pieces (same card, "Long Audio").  Each operand size below is computed
here from the configuration, independently of the library."""
import numpy as np
import pytest

from audio_encoder_amd import binding as B

LIMIT = 2 ** 31 - 1


def es(cfg):
    return 2 if cfg["dtype"] == "bf16" else 4


def check_plan(cfg, lengths, ppp=0):
    """Every pass fits, and the passes tile the window plan in order."""
    wins = B.encoder_plan_windows_ragged(cfg, lengths)
    ps = B.encoder_plan_passes(cfg, lengths, ppp)
    C, d, W = cfg["conv_channels"], cfg["d_model"], cfg["window_tokens"]
    e = es(cfg)
    per_token = max(16 * C * e, 3 * d * e, 4 * d, cfg["d_ffn"] * e, 2 * cfg["d_adapter"] * e,
                    cfg["d_out"] * e)
    mt = cfg.get("max_tokens_per_pass") or 8192
    w0 = t0 = 0
    for win0, nwin, tok0, ntok, L1s, L2s in ps:
        assert win0 == w0 and tok0 == t0 and nwin >= 1
        sel = wins[win0:win0 + nwin]
        assert tok0 == sel[0, 6] and ntok == sel[:, 5].sum()
        assert L1s == sel[:, 3].max() and L2s == (L1s + 1) // 2 and L1s <= 4 * W
        # conv operands: act1 (conv1 out, conv2 A), act2 (conv2 out, conv3 A), conv3 out
        assert nwin * L1s * 64 * C * e <= LIMIT
        assert nwin * L2s * 32 * C * e <= LIMIT
        # per-token operands of the linear layers, and the configured token bound
        assert ntok * per_token <= LIMIT
        assert ntok <= mt
        if ppp:
            assert win0 % (cfg["piece_tokens"] // W) == 0  # passes start on whole pieces
        w0 += nwin
        t0 += ntok
    assert w0 == len(wins) and t0 == wins[:, 5].sum()
    return ps


SR = 16000


@pytest.mark.parametrize("n_clips,seconds", [(100, 2), (90, 3), (113, 1), (200, 5), (65535, 0.0126),
                                             (24, 30), (16, 30), (1, 30), (300, 0.5), (4000, 1.3)])
def test_equal_clip_batches_fit(n_clips, seconds):
    n = max(201, int(round(seconds * SR)))
    ps = check_plan(B.FULL, [n] * n_clips)
    # passes stay large: no pass of a multi-pass call falls below half the fullest one's tokens
    # except the last
    if len(ps) > 2:
        assert ps[:-1, 3].min() * 2 >= ps[:, 3].max() or ps[:-1, 1].min() > 1


def test_short_clips_share_passes():
    # 100 clips of 2 s: 25 frames of conv1 per window, so a pass holds every clip at act1
    # rows of 25 each (no 400-row padding) and runs as the two halves of a one-pass call
    ps = check_plan(B.FULL, [2 * SR] * 100)
    assert ps[:, 1].sum() == 100
    assert len(ps) == 1 or ps[:, 4].max() == 100  # L1s = ceil(200 / 2) = 100


def test_full_windows_are_bounded_by_act1():
    # with the token bound lifted, 30 s clips would put 12 windows each in a pass; act1 (24.6 MB
    # per full window) then caps a pass at 87 windows
    cfg = dict(B.FULL, max_tokens_per_pass=10 ** 6)
    ps = check_plan(cfg, [480000] * 40)
    assert ps[:, 1].max() <= (LIMIT // (400 * 64 * 480 * 2))
    assert ps[:, 1].max() == 87


def test_token_bound_caps_passes():
    cfg = dict(B.FULL, max_tokens_per_pass=1000)
    ps = check_plan(cfg, [480000] * 5)
    assert ps[:, 3].max() <= 1000


@pytest.mark.parametrize("seed", range(6))
def test_random_ragged_calls_fit(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    lengths = [int(v) for v in rng.integers(201, 40 * SR, size=n)]
    mt = int(rng.choice([0, 500, 3000, 8192, 50000]))
    cfg = dict(B.FULL, max_tokens_per_pass=mt)
    check_plan(cfg, lengths)
    check_plan(dict(B.TINY, max_tokens_per_pass=mt if mt == 0 or mt >= 25 else 25), lengths)


@pytest.mark.parametrize("seconds,ppp", [(3600, 1), (3600, 8), (512, 8), (150.37, 1), (150.37, 2),
                                         (64 * 10, 10)])
def test_long_mode_passes_hold_whole_pieces(seconds, ppp):
    n = int(round(seconds * SR))
    ps = check_plan(B.FULL, [n], ppp)
    # ppp pieces per pass except where the two-halves split of a one-pass call applies
    pw = B.FULL["piece_tokens"] // B.FULL["window_tokens"]
    assert ps[:, 1].max() <= ppp * pw


def test_one_pass_calls_split_into_halves():
    ps = check_plan(B.FULL, [480000] * 16)
    assert ps[:, 3].tolist() == [3000, 3000]
    ps = check_plan(B.FULL, [480000] * 8)  # 3000 tokens: one pass
    assert len(ps) == 1


def test_plan_rejects_bad_calls():
    with pytest.raises(B.EncoderError):
        B.encoder_plan_passes(B.FULL, [480000, 480000], 1)  # long mode takes one recording
    with pytest.raises(B.EncoderError):
        B.encoder_plan_passes(B.FULL, [480000], -1)
    with pytest.raises(B.EncoderError):
        B.encoder_plan_passes(B.FULL, [200])


def test_configs_whose_window_cannot_be_addressed_are_rejected():
    # one full window's act1 above 2^31 - 1 bytes (C = 16384 in fp32), and a weight matrix above
    # it (FFN 32768 x 16384 bf16)
    assert B.encoder_validate_cfg(dict(B.FULL, conv_channels=16384, dtype="f32")) == B.ENC_E_INVALID_ARG
    assert B.encoder_validate_cfg(dict(B.FULL, d_ffn=65536, d_model=16384, n_heads=256)) == B.ENC_E_INVALID_ARG
