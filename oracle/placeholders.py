"""Oracle for the soft-token placement around the encoder: placeholder
expansion of a token-id sequence and the merge of soft tokens into the text
embedding rows.

TEST INFRASTRUCTURE (see the package docstring). Integer bookkeeping and row
copies only (bit-exact). Source: egemma2_audio.rs (cortiq-engine 0.8.49),
``input_ids`` and ``embed_audio_inputs`` (the rows whose id is the audio
token receive the soft tokens in order), with the release's token ids
among the page's constants.
"""
from __future__ import annotations

import numpy as np

AUDIO_TOKEN = 258881   # <|audio|>
BOA_TOKEN = 256000     # <|audio>
EOA_TOKEN = 258883     # <audio|>


class PlacementError(ValueError):
    pass


def expand_ids(body, n_soft, bos, eos, max_tokens, audio=AUDIO_TOKEN, boa=BOA_TOKEN,
               eoa=EOA_TOKEN):
    """[bos] + body with each audio placeholder k replaced by
    [boa] + [audio] * n_soft[k] + [eoa], + [eos] (egemma2_audio.rs,
    ``input_ids``). The body must hold exactly one placeholder per clip, and
    the result at most max_tokens ids."""
    body = [int(x) for x in body]
    found = sum(1 for x in body if x == audio)
    if found != len(n_soft):
        raise PlacementError(f"{found} placeholders for {len(n_soft)} clips")
    out = [bos]
    k = 0
    for x in body:
        if x == audio:
            out.append(boa)
            out.extend([audio] * int(n_soft[k]))
            out.append(eoa)
            k += 1
        else:
            out.append(x)
    out.append(eos)
    if len(out) > max_tokens:
        raise PlacementError(f"{len(out)} tokens > {max_tokens}")
    return out


def merge_soft_tokens(x, ids, soft, audio=AUDIO_TOKEN):
    """Rows of x (one per id) whose id is the audio token, in order, take the
    rows of soft (egemma2_audio.rs, ``embed_audio_inputs``). The number of
    such rows must equal the number of soft tokens."""
    x = np.array(x, copy=True)
    rows = [i for i, t in enumerate(ids) if int(t) == audio]
    if len(rows) != len(soft):
        raise PlacementError(f"{len(rows)} audio rows for {len(soft)} soft tokens")
    for r, s in zip(rows, soft):
        x[r] = s
    return x
