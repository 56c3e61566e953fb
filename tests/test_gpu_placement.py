"""GPU parity of the soft-token merge (ae_merge_soft_tokens) against the
oracle: row copies, so bit-exact, with the audio-row count exact."""
import numpy as np
import pytest

from oracle import placeholders as ph
from _util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from log_mel_conformer_amd import ae  # noqa: E402


def packed_inputs(n_inputs, n_soft, text_len, seed):
    """Expanded id sequences of n_inputs inputs (one clip each), packed."""
    rng = np.random.default_rng(seed)
    seqs = []
    for i in range(n_inputs):
        body = list(rng.integers(3, 250000, text_len))
        body.insert(int(rng.integers(0, text_len + 1)), ph.AUDIO_TOKEN)
        seqs.append(ph.expand_ids(body, [n_soft[i]], bos=2, eos=1, max_tokens=10 ** 6))
    return np.concatenate([np.asarray(s, np.int32) for s in seqs])


@pytest.mark.parametrize("case", [
    ("ragged", [5, 0, 300, 1, 77], 9),
    ("block edges", [255, 256, 257], 0),
    ("single", [1], 0),
])
def test_merge_matches_oracle(case):
    name, n_soft, text_len = case
    say(f"[gpu] merge soft tokens: {name}")
    ids = packed_inputs(len(n_soft), n_soft, text_len, seed=len(name))
    L, d, S = len(ids), 64, int(sum(n_soft))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((L, d)).astype(np.float32)
    soft = rng.standard_normal((S, d)).astype(np.float32)
    xg = torch.from_numpy(x).cuda()
    cnt = ae.merge_soft_tokens(torch.from_numpy(ids).cuda(), xg, torch.from_numpy(soft).cuda())
    assert int(cnt.item()) == S
    assert np.array_equal(xg.cpu().numpy(), ph.merge_soft_tokens(x, ids, soft))


def test_merge_without_audio_rows_and_with_fewer_soft_rows():
    say("[gpu] merge: no audio rows; fewer soft rows than audio rows")
    rng = np.random.default_rng(2)
    ids = rng.integers(3, 1000, 700).astype(np.int32)
    x = rng.standard_normal((700, 8)).astype(np.float32)
    xg = torch.from_numpy(x).cuda()
    cnt = ae.merge_soft_tokens(torch.from_numpy(ids).cuda(), xg,
                               torch.zeros((0, 8), dtype=torch.float32, device="cuda"))
    assert int(cnt.item()) == 0 and np.array_equal(xg.cpu().numpy(), x)
    ids[[3, 300, 699]] = ph.AUDIO_TOKEN
    soft = rng.standard_normal((2, 8)).astype(np.float32)
    xg = torch.from_numpy(x).cuda()
    cnt = ae.merge_soft_tokens(torch.from_numpy(ids).cuda(), xg, torch.from_numpy(soft).cuda())
    got = xg.cpu().numpy()
    assert int(cnt.item()) == 3
    assert np.array_equal(got[[3, 300]], soft) and np.array_equal(got[699], x[699])


def test_merge_full_size_batch32():
    """The encoder's batch: 32 inputs of 750 soft tokens, d = 512."""
    say("[gpu] merge: 32 inputs x 750 soft tokens, d 512")
    ids = packed_inputs(32, [750] * 32, 16, seed=7)
    L, d, S = len(ids), 512, 32 * 750
    rng = np.random.default_rng(3)
    x = rng.standard_normal((L, d)).astype(np.float32)
    soft = rng.standard_normal((S, d)).astype(np.float32)
    xg = torch.from_numpy(x).cuda()
    cnt = ae.merge_soft_tokens(torch.from_numpy(ids).cuda(), xg, torch.from_numpy(soft).cuda())
    assert int(cnt.item()) == S
    assert np.array_equal(xg.cpu().numpy(), ph.merge_soft_tokens(x, ids, soft))
