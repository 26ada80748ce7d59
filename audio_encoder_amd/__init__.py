"""MI355X-native audio-tower forward pass (log-mel -> conv stack -> windowed Transformer ->
head -> SwiGLU adapter) behind a C-ABI HIP library.

``audio_encoder_amd.synth`` holds the seeded synthetic inputs; ``audio_encoder_amd.binding``
loads the built library (``libaudio_encoder.so``) and fails loudly if it is missing.
"""
