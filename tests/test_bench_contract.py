"""bench.py's host-side contract (CPU): the one-GPU guard and the algorithmic work it divides by.

The FLOP count is checked against a per-token tally written from the layer shapes of the
"cstr/MOSS-Transcribe-preview-2B-GGUF" card ("Architecture" table): for a full 100-token window
every token owns 4 x 64 conv1 outputs, 2 x 32 conv2 outputs and 16 conv3 outputs, and attends to
the 100 tokens of its window.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_work_model_matches_per_token_tally():
    import bench
    from audio_encoder_amd import binding as B
    cfg = dict(B.FULL)
    w = bench.work_model(cfg, [30 * 16000] * 16)
    assert w["ntok"] == 16 * 375
    C, d, F, O, A, W = 480, 1280, 5120, 2048, 8192, 100
    per_tok_conv = 2 * 9 * (4 * 64 * 1 * C + 2 * 32 * C * C + 16 * C * C)
    per_tok_layer = 2 * (3 * d * d + d * d + 2 * d * F) + 2 * 2 * W * d
    per_tok_rest = 2 * (16 * C * d + d * d + d * O + O * 2 * A + A * O)
    # 30 s = 375 tokens: three full windows and one of 75 tokens, whose tokens attend to 75 keys
    ntok = 16 * 375
    attn_short = 16 * 32 * 2 * 2 * 75 * (W - 75) * d
    expect = ntok * (per_tok_conv + 32 * per_tok_layer + per_tok_rest) - attn_short
    # conv1 and conv2 of the short window cover its valid frames only: 375 tokens of 30 s have
    # exactly 4 * 375 conv1 and 2 * 375 conv2 time rows, as for whole windows
    assert w["total_flops"] == pytest.approx(expect, rel=1e-12)
    assert w["total_flops"] / ntok == pytest.approx(1.7375e9, rel=2e-3)


def test_work_model_layernorm_bytes():
    import bench
    from audio_encoder_amd import binding as B
    w = bench.work_model(dict(B.FULL), [30 * 16000] * 16)
    # 65 LayerNorms (two per layer and ln_post), each reading fp32 rows and writing bf16 rows
    assert w["bytes"]["layernorm"] == 65 * 6000 * 1280 * 6
