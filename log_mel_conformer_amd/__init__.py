"""log_mel_conformer_amd: the log-mel + Conformer audio-encoder forward on
MI355X (gfx950), hand-written HIP kernels behind the C-ABI library
``libae.so``; ``ae`` is its thin Python binding."""
