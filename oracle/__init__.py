"""Oracle for the log-mel + Conformer audio encoder forward.

TEST INFRASTRUCTURE. This package is a plain, slow, obviously correct CPU
statement of what the encoder computes, in float64 storage and accumulation
(numpy). It exists only to check the HIP path: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import or call it. The HIP
path shares no code, table or constant generator with it, and neither side
imports the other.

Source of the method: the docs.rs source page of cortiq-engine 0.8.49,
``cortiq_engine/egemma2_audio.rs`` (the ``gemma4_audio`` tower of
EmbeddingGemma 2), cited below as "egemma2_audio.rs" with the item it
defines; the RMS-norm form comes from the cortiq-engine 0.5.94
``ltxdit.rs`` page (``rms_plain`` / ``rms_w``). The same egemma2_audio.rs
page defines the step ahead of the log-mel, mixdown and resampling to
16 kHz (``oracle.resample``). The second encoder, the LFM2A Conformer of
the docs.rs source page of cera 0.5.3 (``src/model/audio_encoder_gpu.rs``),
is ``oracle.lfm2a``.

Every function is pinned by a CPU test (values the pages print, closed
forms, invariants, library cross-checks or brute force); the one result with
no external pin is the whole encoder against the trained release, for
which no weights exist here ("parity unpinned", recorded in the design
notes).
"""
from .frontend import (num_frames, num_tokens, hann_window, linspace,
                       mel_filter_bank, frames_of, dft_magnitude, log_mel)
from .tower import (layer_norm_relu, subsample, rms_norm, clip_linear, silu,
                    sigmoid, softplus, rel_pos_table, relative_keys, ffn,
                    local_attention, attention_block, glu, causal_dwconv,
                    light_conv, conformer_layer, head, encode_clips,
                    tower_constants)
from . import resample  # the module: oracle.resample.resample, .mixdown, ...
from . import lfm2a     # the module: oracle.lfm2a.encode, .log_mel, ...
