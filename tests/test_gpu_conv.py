"""Conv front end at kernel level, through the C ABI (encoder_op_conv1 / encoder_op_conv).

Index probes: with one-hot 3x3 kernels (channel c reads only tap c % 9 of its own channel, or of
the single mel channel for conv1), bias 16 and small-integer inputs, every output is the shifted
input + 16, or 16 where the tap falls outside the window's valid image.  All values are
integers below 256, so they are exact in bf16, the products and sums are exact in fp32, and the
GELU returns x unchanged for x >= 16 (pinned on the CPU in test_host_abi.py): the comparison is
bit for bit.  This pins the window indexing of the conv kernels: taps at time and frequency
edges, windows shorter than the pass stride (L0 = 601 and 137, and one- and two-frame windows),
rows past a window's valid length (never read, never written) and GEMM tiles that straddle
windows.  The conv front end is the one the "cstr/MOSS-Transcribe-preview-2B-GGUF" card's
"Architecture" table describes; windows are independent images (the window-local reading).

Random-data cases compare the same entries with the float64 oracle's conv (oracle.conv2d_s2 +
oracle.gelu) within one bf16 rounding of the output."""
import sys

import numpy as np
import pytest
import torch

import oracle as O

from audio_encoder_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -3.0  # output rows the kernels must leave untouched


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ceil_half(n):
    return (n + 1) // 2


def window_table(L0s, clips=None, tok_gap=0):
    """int32 [n, 8] {clip, start, L0, L1, L2, L3, tok, mel_row}; mel rows and tokens are laid
    out window after window, with tok_gap unused token rows after each window."""
    rows = []
    tok = mel = 0
    for i, L0 in enumerate(L0s):
        L1 = ceil_half(L0)
        L2 = ceil_half(L1)
        L3 = ceil_half(L2)
        rows.append([0 if clips is None else clips[i], 0, L0, L1, L2, L3, tok, mel])
        tok += L3 + tok_gap
        mel += L0 + 3  # three unused mel rows between windows
    return np.array(rows, dtype=np.int32), tok, mel


def probe_values(shape, seed):
    """Integers in [1, 239] from a multiplicative hash of every index (distinct neighbours)."""
    grids = np.ogrid[tuple(slice(0, n) for n in shape)]
    h = np.uint64(seed)
    for k, a in enumerate(grids):
        h = h + a.astype(np.uint64) * np.uint64([1000003, 7919, 104729, 31337, 65537][k])
    h = (h * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    return (1 + (h >> np.uint64(7)) % np.uint64(239)).astype(np.float32)


def tap_of(c):
    q = c % 9
    return q // 3, q % 3  # (frequency tap a, time tap b)


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


# ---------------------------------------------------------------------------------------------
# conv1
# ---------------------------------------------------------------------------------------------
CONV1_CASES = [("bf16", 480, 100, [800, 601, 137, 1, 2, 800]), ("f32", 32, 25, [200, 151, 37, 1, 2])]


@pytest.mark.parametrize("dtype,C,W,L0s", CONV1_CASES)
def test_conv1_index_probe_is_bit_exact(dtype, C, W, L0s):
    tab, _, mel_rows = window_table(L0s, clips=[i % 2 for i in range(len(L0s))])
    L1s = int(tab[:, 3].max())
    v = probe_values((mel_rows, 128), 11)
    # rows outside every window hold 200: a read of them would show
    inside = np.zeros(mel_rows, bool)
    for r in tab:
        inside[r[7]:r[7] + r[2]] = True
    v[~inside] = 200.0
    mel = 4.0 * v - 4.0  # raw log10 values whose normalised form (max 8: no clamp) is v
    w = np.zeros((C, 3, 3), np.float32)
    for c in range(C):
        a, b = tap_of(c)
        w[c, a, b] = 1.0
    act1 = torch.full((len(L0s), L1s, 64, C), SENTINEL, dtype=torch_dtype(dtype), device=DEV)
    B.op_conv1(torch.from_numpy(mel).to(DEV), torch.full((2,), 8.0, device=DEV),
               torch.from_numpy(tab).to(DEV), W, L1s, torch.from_numpy(w).to(DEV),
               torch.full((C,), 16.0, device=DEV), act1)
    got = act1.float().cpu().numpy()
    for i, r in enumerate(tab):
        L0, L1, row = int(r[2]), int(r[3]), int(r[7])
        img = np.zeros((L0 + 2 * L1 + 2, 130), np.float32)  # zero-padded [time, freq] image
        img[1:L0 + 1, 1:129] = v[row:row + L0]
        want = np.empty((L1, 64, C), np.float32)
        for c in range(C):
            a, b = tap_of(c)
            want[:, :, c] = img[b:b + 2 * L1:2, a:a + 128:2] + 16.0
        assert np.array_equal(got[i, :L1], want), (dtype, i)
        assert np.all(got[i, L1:] == SENTINEL), (dtype, i, "rows past L1 written")


@pytest.mark.parametrize("dtype,C,W,L0s", CONV1_CASES)
def test_conv1_random_matches_oracle(dtype, C, W, L0s):
    rng = np.random.default_rng(C)
    tab, _, mel_rows = window_table(L0s, clips=[i % 2 for i in range(len(L0s))])
    L1s = int(tab[:, 3].max())
    raw = rng.uniform(-6.0, 1.5, size=(mel_rows, 128)).astype(np.float32)
    cmax = np.array([1.2, 0.5], np.float32)  # clip 1's clamp is active (max - 8 = -7.5)
    w = rng.standard_normal((C, 3, 3)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    act1 = torch.full((len(L0s), L1s, 64, C), SENTINEL, dtype=torch_dtype(dtype), device=DEV)
    B.op_conv1(torch.from_numpy(raw).to(DEV), torch.from_numpy(cmax).to(DEV), torch.from_numpy(tab).to(DEV),
               W, L1s, torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV), act1)
    got = act1.float().cpu().numpy()
    for i, r in enumerate(tab):
        L0, L1, row, clip = int(r[2]), int(r[3]), int(r[7]), int(r[0])
        melw = O.normalize_log_mel(raw[row:row + L0].astype(np.float64), float(cmax[clip]))
        ref = O.gelu(O.conv2d_s2(melw.T[None], w[:, None].astype(np.float64), b.astype(np.float64)))
        ref = ref.transpose(2, 1, 0)  # [time, freq, channel]
        err = np.abs(got[i, :L1] - ref)
        if dtype == "f32":
            assert err.max() <= 1e-5 * max(1.0, np.abs(ref).max()), (i, err.max())
        else:
            assert np.all(err <= 2 ** -8 * np.abs(ref) + 1e-5), (i, err.max())


# ---------------------------------------------------------------------------------------------
# conv2 / conv3 (implicit GEMM)
# ---------------------------------------------------------------------------------------------
CONV_CASES = [("bf16", 480, 100, [800, 601, 137, 1, 2]), ("bf16", 480, 100, [601, 137, 601]),
              ("bf16", 64, 100, [800] * 3 + [5, 3, 799]), ("f32", 32, 25, [200, 151, 37, 1, 2])]


def one_hot_weights(C):
    wp = np.zeros((C, 9, C), np.float32)
    for c in range(C):
        a, b = tap_of(c)
        wp[c, 3 * a + b, c] = 1.0
    return wp


def conv_probe_expect(inp, Lin, Lout, Fin):
    """[Lout, Fin/2, C] one-hot conv of one window's [rows, Fin, C] input (valid rows < Lin)."""
    C = inp.shape[-1]
    img = np.zeros((2 * Lout + 2, Fin + 2, C), np.float32)
    img[1:Lin + 1, 1:Fin + 1] = inp[:Lin]
    want = np.empty((Lout, Fin // 2, C), np.float32)
    for q in range(9):
        a, b = q // 3, q % 3
        cs = np.arange(q, C, 9)
        want[:, :, cs] = img[b:b + 2 * Lout:2, a:a + Fin:2][:, :, cs] + 16.0
    return want


@pytest.mark.parametrize("dtype,C,W,L0s", CONV_CASES)
def test_conv_index_probe_is_bit_exact(dtype, C, W, L0s):
    tab, n_tok, _ = window_table(L0s, tok_gap=2)
    nw = len(L0s)
    L1s = int(tab[:, 3].max())
    L2s = ceil_half(L1s)
    td = torch_dtype(dtype)
    wp = torch.from_numpy(one_hot_weights(C)).to(DEV).to(td)
    bias = torch.full((C,), 16.0, device=DEV)
    tabd = torch.from_numpy(tab).to(DEV)
    # conv2: act1 rows past each window's L1 hold 7 (never to be read)
    a1 = probe_values((nw, L1s, 64, C), 5)
    for i, r in enumerate(tab):
        a1[i, r[3]:] = 7.0
    act2 = torch.full((nw, L2s, 32, C), SENTINEL, dtype=td, device=DEV)
    B.op_conv(2, torch.from_numpy(a1).to(DEV).to(td), tabd, W, L1s, n_tok, wp, bias, act2)
    g2 = act2.float().cpu().numpy()
    for i, r in enumerate(tab):
        L1, L2 = int(r[3]), int(r[4])
        assert np.array_equal(g2[i, :L2], conv_probe_expect(a1[i], L1, L2, 64)), (dtype, "conv2", i)
        assert np.all(g2[i, L2:] == SENTINEL), (dtype, "conv2", i, "rows past L2 written")
    # conv3 on fresh probe values (act2 rows past L2 hold 7), into token rows with gaps
    a2 = probe_values((nw, L2s, 32, C), 9)
    for i, r in enumerate(tab):
        a2[i, r[4]:] = 7.0
    tok = torch.full((n_tok, 16, C), SENTINEL, dtype=td, device=DEV)
    B.op_conv(3, torch.from_numpy(a2).to(DEV).to(td), tabd, W, L1s, n_tok, wp, bias, tok)
    g3 = tok.float().cpu().numpy()
    written = np.zeros(n_tok, bool)
    for i, r in enumerate(tab):
        L2, L3, t0 = int(r[4]), int(r[5]), int(r[6])
        assert np.array_equal(g3[t0:t0 + L3], conv_probe_expect(a2[i], L2, L3, 32)), (dtype, "conv3", i)
        written[t0:t0 + L3] = True
    assert np.all(g3[~written] == SENTINEL), (dtype, "conv3 wrote a gap row")


@pytest.mark.parametrize("dtype,C,W,L0s", [CONV_CASES[0], CONV_CASES[3]])
def test_conv_random_matches_oracle(dtype, C, W, L0s):
    rng = np.random.default_rng(C + len(L0s))
    tab, n_tok, _ = window_table(L0s)
    nw = len(L0s)
    L1s = int(tab[:, 3].max())
    L2s = ceil_half(L1s)
    td = torch_dtype(dtype)
    rnd = (lambda a: O.bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    w = rnd((rng.standard_normal((C, C, 3, 3)) / np.sqrt(9 * C)).astype(np.float32))
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    wp = torch.from_numpy(np.ascontiguousarray(w.reshape(C, C, 9).transpose(0, 2, 1))).to(DEV).to(td)
    bias = torch.from_numpy(b).to(DEV)
    tabd = torch.from_numpy(tab).to(DEV)
    a1 = rnd(rng.uniform(-0.2, 1.5, size=(nw, L1s, 64, C)).astype(np.float32))
    act2 = torch.zeros((nw, L2s, 32, C), dtype=td, device=DEV)
    B.op_conv(2, torch.from_numpy(a1).to(DEV).to(td), tabd, W, L1s, n_tok, wp, bias, act2)
    tok = torch.zeros((n_tok, 16, C), dtype=td, device=DEV)
    B.op_conv(3, act2, tabd, W, L1s, n_tok, wp, bias, tok)
    g2 = act2.float().cpu().numpy()
    g3 = tok.float().cpu().numpy()
    w64, b64 = w.astype(np.float64), b.astype(np.float64)
    for i, r in enumerate(tab):
        L1, L2, L3, t0 = int(r[3]), int(r[4]), int(r[5]), int(r[6])
        x = a1[i, :L1].astype(np.float64).transpose(2, 1, 0)  # [C, freq, time]
        ref2 = O.gelu(O.conv2d_s2(x, w64, b64))
        got2 = g2[i, :L2].transpose(2, 1, 0)
        # conv3 runs on the library's own conv2 output (one rounding per layer)
        ref3 = O.gelu(O.conv2d_s2(g2[i, :L2].astype(np.float64).transpose(2, 1, 0), w64, b64))
        got3 = g3[t0:t0 + L3].transpose(2, 1, 0)
        for got, ref, what in ((got2, ref2, "conv2"), (got3, ref3, "conv3")):
            err = np.abs(got - ref)
            scale = np.abs(ref).max()
            if dtype == "f32":
                assert err.max() <= 1e-5 * max(1.0, scale), (what, i, err.max())
            else:
                assert np.all(err <= 2 ** -8 * np.abs(ref) + 1e-4 * scale), (what, i, err.max())


def test_conv_entries_reject_bad_tables():
    C, W = 32, 25
    tab, n_tok, mel_rows = window_table([200, 37])
    bad = tab.copy()
    bad[1, 3] += 1  # L1 not ceil(L0 / 2)
    z = torch.zeros(4096, device=DEV)
    for t in (bad,):
        with pytest.raises(B.EncoderError) as ei:
            B.op_conv(2, z, torch.from_numpy(t).to(DEV), W, 100, n_tok, z, torch.zeros(C, device=DEV), z)
        assert ei.value.status == B.ENC_E_INVALID_ARG
    with pytest.raises(B.EncoderError):  # L1s below a window's L1
        B.op_conv(2, z, torch.from_numpy(tab).to(DEV), W, 50, n_tok, z, torch.zeros(C, device=DEV), z)
    with pytest.raises(B.EncoderError):  # tokens past n_tok
        B.op_conv(3, z, torch.from_numpy(tab).to(DEV), W, 100, n_tok - 1, z, torch.zeros(C, device=DEV), z)
    with pytest.raises(B.EncoderError):  # mel rows past the input
        B.op_conv1(torch.zeros((239, 128), device=DEV), torch.zeros(1, device=DEV),
                   torch.from_numpy(tab).to(DEV), W, 100, torch.zeros((C, 3, 3), device=DEV),
                   torch.zeros(C, device=DEV), z)
