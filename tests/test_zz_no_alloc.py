"""encoder_log_mel_noalloc: the log-mel entry for callers that cannot allocate, through the C ABI.
Its output equals encoder_log_mel's bit for bit (the same kernels) on two calls in a row, the
second with a smaller input, whose scratch then holds the first call's leftovers; the call
leaves the device's free memory and the library's workspace unchanged; a batch above its scratch
is rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from audio_encoder_amd import binding as B
from audio_encoder_amd import synth as S

pytestmark = pytest.mark.gpu


def call(enc, pcm, mel):
    B_, N = pcm.shape
    return B.lib().encoder_log_mel_noalloc(enc._h, ctypes.c_void_p(pcm.data_ptr()), N, B_,
                                           ctypes.c_void_p(mel.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_log_mel_noalloc_equals_log_mel_on_two_calls():
    enc = B.Encoder(S.make_weights(B.TINY, seed=0), B.TINY)
    big = np.stack([S.mixed_clip(800 + i, 480000 + 159) for i in range(6)])
    small = np.stack([S.three_sines(seed=1), 0.01 * S.three_sines(seed=2)])  # 2 x 4 s
    for x in (big, small):
        pcm = torch.from_numpy(x).cuda()
        ref = enc.log_mel(pcm)
        mel = torch.full(ref.shape, float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        ws0 = enc.memory_stats()[1]
        assert call(enc, pcm, mel) == B.ENC_OK
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        assert enc.memory_stats()[1] == ws0
        assert torch.equal(mel, ref)
        got = mel.cpu().numpy()
        for b in range(x.shape[0]):
            assert np.abs(got[b] - O.log_mel(x[b])).max() <= 1e-3
    enc.close()


def test_log_mel_noalloc_rejects_a_batch_above_its_scratch():
    enc = B.Encoder(S.make_weights(B.TINY, seed=0), B.TINY)
    pcm = torch.zeros((4097, 201), dtype=torch.float32, device="cuda")
    mel = torch.full((4097, 1, 128), 3.0, device="cuda")
    assert call(enc, pcm, mel) == B.ENC_E_INVALID_ARG
    assert b"4096" in B.lib().encoder_last_error()
    torch.cuda.synchronize()
    assert bool((mel == 3.0).all())
    # at the limit it runs, and equals the allocating entry
    pcm = torch.from_numpy(np.random.default_rng(3).standard_normal((4096, 401)).astype(np.float32)).cuda()
    mel = torch.empty((4096, 2, 128), device="cuda")
    assert call(enc, pcm, mel) == B.ENC_OK
    assert torch.equal(mel, enc.log_mel(pcm))
    enc.close()
