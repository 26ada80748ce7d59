"""CPU oracle of the audio-tower forward pass (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the ``audio_encoder_amd`` package.
"""
from .encoder_ref import *  # noqa: F401,F403
from . import encoder_ref  # noqa: F401
