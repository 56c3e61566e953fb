"""Pins for the soft-token placement oracle: the page's token ids
(tests/golden/placement_printed.json), a worked example written out by
hand from the page's rule, and invariants of the expansion."""
import json
import os

import numpy as np
import pytest

from oracle import placeholders as ph

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "placement_printed.json")))


def test_token_ids_printed():
    assert (ph.AUDIO_TOKEN, ph.BOA_TOKEN, ph.EOA_TOKEN) == tuple(GOLD["ids"]["audio_boa_eoa"])


def test_worked_example_by_hand():
    A, S, E = ph.AUDIO_TOKEN, ph.BOA_TOKEN, ph.EOA_TOKEN
    out = ph.expand_ids([10, A, 11, A], [2, 0], bos=2, eos=1, max_tokens=100)
    assert out == [2, 10, S, A, A, E, 11, S, E, 1]
    # no text: the clips between BOS and EOS (one placeholder per clip)
    assert ph.expand_ids([A, A], [1, 1], bos=2, eos=1, max_tokens=100) == [2, S, A, E, S, A, E, 1]


def test_expansion_invariants_random():
    rng = np.random.default_rng(0)
    A = ph.AUDIO_TOKEN
    for _ in range(200):
        k = int(rng.integers(0, 5))
        body = list(rng.integers(3, 1000, int(rng.integers(0, 12))))
        for _ in range(k):
            body.insert(int(rng.integers(0, len(body) + 1)), A)
        n = list(rng.integers(0, 40, k))
        out = ph.expand_ids(body, n, bos=2, eos=1, max_tokens=10 ** 6)
        assert len(out) == len(body) + 2 + sum(n) + k
        assert out.count(A) == sum(n)
        assert out.count(ph.BOA_TOKEN) == k and out.count(ph.EOA_TOKEN) == k
        # removing the expansions gives back the body
        back, skip = [], False
        for t in out[1:-1]:
            if t == ph.BOA_TOKEN:
                skip = True
                back.append(A)
            elif t == ph.EOA_TOKEN:
                skip = False
            elif not skip:
                back.append(t)
        assert back == [int(b) for b in body]


def test_errors():
    A = ph.AUDIO_TOKEN
    with pytest.raises(ph.PlacementError):
        ph.expand_ids([A], [1, 2], bos=2, eos=1, max_tokens=100)
    with pytest.raises(ph.PlacementError):
        ph.expand_ids([A], [200], bos=2, eos=1, max_tokens=100)
    assert len(ph.expand_ids([A], [96], bos=2, eos=1, max_tokens=100)) == 100


def test_merge_places_rows_in_order():
    A = ph.AUDIO_TOKEN
    ids = [2, 7, A, A, 9, A, 1]
    x = np.arange(7 * 3, dtype=np.float32).reshape(7, 3)
    soft = -np.arange(3 * 3, dtype=np.float32).reshape(3, 3) - 1
    m = ph.merge_soft_tokens(x, ids, soft)
    assert np.array_equal(m[[2, 3, 5]], soft)
    assert np.array_equal(m[[0, 1, 4, 6]], x[[0, 1, 4, 6]])
    with pytest.raises(ph.PlacementError):
        ph.merge_soft_tokens(x, ids, soft[:2])
