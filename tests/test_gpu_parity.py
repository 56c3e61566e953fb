"""GPU parity: the HIP path (through the C ABI) against the oracle.

Tolerances: log-mel elementwise |d| <= 1e-4 * max(1, |o|); every fp32
stage ||g - o||_2 / ||o||_2 <= 1e-4 per clip; bf16 final embeddings
<= 2e-2 per clip. Integer quantities (frame and token counts) are exact.
Full-size workloads compare sampled clips (clips are independent, so the
oracle runs those clips alone).
"""
import math

import numpy as np
import pytest

import oracle
from log_mel_conformer_amd import synth
from _util import bf16_gate, rel_l2, rel_max, say, weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from log_mel_conformer_amd import ae  # noqa: E402

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def cuda(x, dtype=torch.float32):
    return torch.as_tensor(np.asarray(x)).to("cuda", dtype)


def logmel_ok(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape
    bound = 1e-4 * np.maximum(1.0, np.abs(o))
    bad = np.abs(g - o) > bound
    assert not bad.any(), f"{bad.sum()} log-mel values off, worst {np.max(np.abs(g - o))}"


# ------------------------------------------------------------------ log-mel

def test_logmel_tone_clip():
    say("[gpu] logmel: 1 s tone, seed 0")
    x = synth.tone_clip(0)
    wave, so = synth.pack([x])
    g = ae.logmel(cuda(wave), so).cpu().numpy()
    assert g.shape == (99, 128)
    logmel_ok(g, oracle.log_mel(x))


def test_logmel_ragged_batch_and_edges():
    say("[gpu] logmel: ragged batch with odd offsets, tiny and over-long clips")
    rng = np.random.default_rng(5)
    clips = [rng.uniform(-1, 1, n).astype(np.float32)
             for n in (161, 100, 321, 481, 1001, 160, 4000, 3)]
    clips.append(synth.white_clip(9, 480000 + 777))   # truncated at 30 s
    wave, so = synth.pack(clips)
    g = ae.logmel(cuda(wave), so).cpu().numpy()
    F = [oracle.num_frames(len(c)) for c in clips]
    assert g.shape[0] == sum(F)
    off = 0
    for c, f in zip(clips, F):
        if f:
            logmel_ok(g[off:off + f], oracle.log_mel(c))
        off += f


def test_more_clips_than_the_lds_offset_tables():
    """700 short clips: past the 512 clips whose offsets the kernels stage in
    LDS, so the clip lookups go through global memory. The log-mel of every
    seventh clip and of those around index 512 against the oracle, then the
    encoder (one layer and the head, bf16) on a sample of the clips. Besides
    every seventh clip, each clip next to a clip with no frames is checked:
    the front end's per-lane clip tracking must step over those."""
    say("[gpu] 700 ragged short clips: log-mel of ~180, encoder (1 layer, bf16) on 6")
    rng = np.random.default_rng(21)
    lens = rng.integers(0, 3000, 700)
    lens[[3, 400, 699]] = [0, 160, 161]
    clips = [synth.white_clip(1000 + i, int(n)) if n else np.zeros(0, np.float32)
             for i, n in enumerate(lens)]
    wave, so = synth.pack(clips)
    wd = cuda(wave)
    g = ae.logmel(wd, so).cpu().numpy()
    F = [oracle.num_frames(len(c)) for c in clips]
    assert g.shape[0] == sum(F)
    fo = np.concatenate([[0], np.cumsum(F)])
    assert sum(1 for f in F if f == 0) >= 20, "the batch should hold many frameless clips"
    near_empty = {i for i in range(700) if (i > 0 and F[i - 1] == 0) or (i < 699 and F[i + 1] == 0)}
    for i in sorted(set(range(0, 700, 7)) | {3, 400, 511, 512, 513, 699} | near_empty):
        if F[i]:
            logmel_ok(g[fo[i]:fo[i + 1]], oracle.log_mel(clips[i]))
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    out = ae.encode(m, wd, so).cpu().numpy()
    T = [oracle.num_tokens(len(c)) for c in clips]
    to = np.concatenate([[0], np.cumsum(T)])
    assert out.shape[0] == to[-1]
    for i in (0, 1, 401, 650, 698, 699):
        if T[i]:
            bf16_gate(out[to[i]:to[i + 1]], oracle.encode_clips([clips[i]], W)[0], f"clip {i}")


def test_logmel_silence_and_impulse():
    say("[gpu] logmel: silence and impulse")
    z = np.zeros(16000, np.float32)
    imp = np.zeros(1000, np.float32)
    imp[80] = 1.0
    wave, so = synth.pack([z, imp])
    g = ae.logmel(cuda(wave), so).cpu().numpy()
    assert np.all(np.abs(g[:99] - math.log(1e-3)) < 1e-6)
    logmel_ok(g[99:], oracle.log_mel(imp))


def test_logmel_full_batch_sampled():
    """256 clips x 30 s of white noise; sampled clips checked in full."""
    say("[gpu] logmel: 256 x 30 s white noise (full size), sampled clips")
    clips = synth.white_batch(256)
    wave, so = synth.pack(clips)
    g = ae.logmel(cuda(wave), so).cpu().numpy()
    assert g.shape == (256 * 2999, 128)
    for i in (0, 137, 255):
        logmel_ok(g[i * 2999:(i + 1) * 2999], oracle.log_mel(clips[i]))


# --------------------------------------------------------- fp32 tower stages

@pytest.fixture(scope="module")
def model1_f32():
    return ae.Model(weights(1), dtype="f32")


def test_subsample_tone_fp32(model1_f32):
    say("[gpu] subsample: 1 s tone, fp32")
    x = synth.tone_clip(0)
    mel_o = oracle.log_mel(x)
    mel = cuda(mel_o)
    g = ae.subsample(model1_f32, mel, np.array([0, 99])).cpu().numpy()
    want = oracle.subsample(mel_o.astype(np.float32), weights(1))
    assert g.shape == (25, 1024)
    assert rel_l2(g, want) <= FP32_TOL, rel_l2(g, want)


def test_subsample_ragged_fp32(model1_f32):
    say("[gpu] subsample: ragged frame counts (1, 2, 3, 5, 99, 2999), fp32")
    rng = np.random.default_rng(11)
    Fs = [1, 2, 3, 5, 99, 2999, 0, 4]
    mels = [rng.standard_normal((f, 128)).astype(np.float32) for f in Fs]
    fo = np.concatenate([[0], np.cumsum(Fs)])
    g = ae.subsample(model1_f32, cuda(np.concatenate(mels)), fo).cpu().numpy()
    off = 0
    for m, f in zip(mels, Fs):
        t = -(-(-(-f // 2)) // 2)
        if t:
            want = oracle.subsample(m, weights(1))
            assert rel_l2(g[off:off + t], want) <= FP32_TOL, (f, rel_l2(g[off:off + t], want))
        off += t
    assert off == g.shape[0]


def test_subsample_ragged_bf16():
    """bf16 subsampler (conv0 on the matrix cores with split operands, conv1
    and in_proj in bf16) on ragged frame counts, including clips shorter
    than one token window and an empty one."""
    say("[gpu] subsample: ragged frame counts (1, 2, 3, 5, 99, 2999, 0, 4), bf16")
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    rng = np.random.default_rng(13)
    Fs = [1, 2, 3, 5, 99, 2999, 0, 4]
    mels = [(rng.standard_normal((f, 128)) - 3.0).astype(np.float32) for f in Fs]
    fo = np.concatenate([[0], np.cumsum(Fs)])
    g = ae.subsample(m, cuda(np.concatenate(mels)), fo).float().cpu().numpy()
    off = 0
    for mm, f in zip(mels, Fs):
        t = -(-(-(-f // 2)) // 2)
        if t:
            r = rel_l2(g[off:off + t], oracle.subsample(mm, W))
            say(f"    {f} frames: rel {r:.3e}")
            assert r <= BF16_TOL, (f, r)
        off += t
    assert off == g.shape[0]


def test_subsample_many_short_clips_bf16():
    """The bf16 subsampler walks runs of consecutive tokens (about
    tokens / 512 a block) with a three-row window of conv0 rows: 400 clips
    of 1-200 frames (about 10^4 tokens, runs of about 20 tokens, most of
    them crossing clip boundaries), each clip against the oracle."""
    say("[gpu] subsample: 400 clips of 1-200 frames, bf16")
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    rng = np.random.default_rng(400)
    Fs = [int(f) for f in rng.integers(1, 201, 400)]
    mels = [(rng.standard_normal((f, 128)) - 3.0).astype(np.float32) for f in Fs]
    fo = np.concatenate([[0], np.cumsum(Fs)])
    g = ae.subsample(m, cuda(np.concatenate(mels)), fo).float().cpu().numpy()
    off, worst = 0, 0.0
    for mm, f in zip(mels, Fs):
        want = oracle.subsample(mm, W)
        t = want.shape[0]
        r = rel_l2(g[off:off + t], want)
        worst = max(worst, r)
        assert r <= BF16_TOL, (f, r)
        off += t
    assert off == g.shape[0]
    say(f"    worst clip rel {worst:.3e}")


def test_layer_tone_fp32(model1_f32):
    say("[gpu] conformer_layer: 1 layer on the tone clip's tokens, fp32")
    W = weights(1)
    x = synth.tone_clip(0)
    h0 = oracle.subsample(oracle.log_mel(x), W).astype(np.float32)
    pos = np.arange(25, dtype=np.int32)
    h = cuda(h0)
    ae.conformer_layer(model1_f32, 0, h, cuda(pos, torch.int32))
    want = oracle.conformer_layer(h0, W["layers"][0], pos)
    assert rel_l2(h.cpu().numpy(), want) <= FP32_TOL, rel_l2(h.cpu().numpy(), want)


def test_layer_packed_positions_fp32(model1_f32):
    """Two clips packed: masks must not cross the boundary."""
    say("[gpu] conformer_layer: packed clips of 7 and 30 tokens, fp32")
    W = weights(1)
    rng = np.random.default_rng(12)
    h0 = rng.standard_normal((37, 1024)).astype(np.float32)
    pos = np.concatenate([np.arange(7), np.arange(30)]).astype(np.int32)
    h = cuda(h0)
    ae.conformer_layer(model1_f32, 0, h, cuda(pos, torch.int32))
    want = oracle.conformer_layer(h0, W["layers"][0], pos)
    g = h.cpu().numpy()
    assert rel_l2(g[:7], want[:7]) <= FP32_TOL and rel_l2(g[7:], want[7:]) <= FP32_TOL


def test_layer_packed_positions_bf16():
    """One bf16 layer (bf16 GEMMs and epilogues, the packed-bf16 dot
    products of the attention logits, bf16 light conv) on three packed
    clips of 1, 11 and 300 tokens: a clip shorter than the window, one
    that just fills it, and a long one; each against the oracle with the
    same bf16-rounded weights."""
    say("[gpu] conformer_layer: packed clips of 1, 11 and 300 tokens, bf16")
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    rng = np.random.default_rng(14)
    lens = [1, 11, 300]
    h0 = rng.standard_normal((sum(lens), 1024)).astype(np.float32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    h = cuda(h0)
    ae.conformer_layer(m, 0, h, cuda(pos, torch.int32))
    g = h.cpu().numpy()
    off = 0
    for n in lens:
        want = oracle.conformer_layer(h0[off:off + n], W["layers"][0], np.arange(n, dtype=np.int32))
        bf16_gate(g[off:off + n], want, f"{n} tokens")
        off += n


def test_layer_attention_block_edges_bf16():
    """The bf16 attention takes 128 tokens a block: clips of 127, 128 and
    129 tokens, then clips of 12 and 13 (one just fills the window, one
    just exceeds it), one of 256 and a single token, packed so that clip
    starts fall at varied offsets inside the blocks and a block's staged
    keys reach back into the previous clip; each clip against the oracle."""
    say("[gpu] conformer_layer: clips of 127/128/129/12/13/256/1 tokens at block edges, bf16")
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    rng = np.random.default_rng(128)
    lens = [127, 128, 129, 12, 13, 256, 1]
    h0 = rng.standard_normal((sum(lens), 1024)).astype(np.float32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    h = cuda(h0)
    ae.conformer_layer(m, 0, h, cuda(pos, torch.int32))
    g = h.cpu().numpy()
    off = 0
    for n in lens:
        want = oracle.conformer_layer(h0[off:off + n], W["layers"][0], np.arange(n, dtype=np.int32))
        bf16_gate(g[off:off + n], want, f"{n} tokens at {off}")
        off += n


@pytest.mark.parametrize("total", [16383, 16384, 16385])
def test_layer_row_count_across_tile_rules_bf16(total):
    """The bf16 projections pick their tiles by row count: below 16384 rows
    128x128 tiles of eight wavefronts, from 16384 rows 384x256 tiles,
    paired 192x256 blocks or 256x128 blocks (the residual add). One layer
    on packed clips totalling 16383, 16384 and 16385 rows (ragged tails in
    every tile shape); the short clips and the last one, whose rows sit in
    the final partial row tile, against the oracle."""
    say(f"[gpu] conformer_layer: {total} packed rows around the 16384-row tile rule, bf16")
    W = weights(1, bf16=True)
    m = ae.Model(W, dtype="bf16")
    rng = np.random.default_rng(total)
    lens = [3, 40, total - 3 - 40 - 57, 57]
    h0 = (0.5 * rng.standard_normal((total, 1024))).astype(np.float32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    h = cuda(h0)
    ae.conformer_layer(m, 0, h, cuda(pos, torch.int32))
    g = h.cpu().numpy()
    offs = np.concatenate([[0], np.cumsum(lens)])
    for i in (0, 1, 3):
        a, b = offs[i], offs[i + 1]
        want = oracle.conformer_layer(h0[a:b], W["layers"][0], np.arange(b - a, dtype=np.int32))
        bf16_gate(g[a:b], want, f"clip of {b - a} rows at {a}")
    assert np.all(np.isfinite(g))


def test_layer_clamps_and_softcap_bind_fp32():
    """Bounds of +-0.5 make every clamp bind; large q weights and
    per_dim_scale above 20 (softplus pass-through) push logits past the
    cap; q, k, v get different input bounds."""
    say("[gpu] conformer_layer: clamps +-0.5, softcap binding, distinct q/k/v input clamps")
    W = synth.make_weights(layers=1, clip=(-0.5, 0.5, -0.5, 0.5))
    L = W["layers"][0]
    L["q"] = (L["q"] * 40).astype(np.float32)
    L["q_clip"] = (-3.0, 3.0, -math.inf, math.inf)
    L["k_clip"] = (-2.0, 2.0, -math.inf, math.inf)
    L["v_clip"] = (-1.0, 1.0, -0.25, 0.25)
    pds = L["per_dim_scale"].copy()
    pds[::2] = 21.0 + np.arange(64) * 0.1
    L["per_dim_scale"] = pds
    m = ae.Model(W, dtype="f32")
    rng = np.random.default_rng(13)
    h0 = rng.standard_normal((40, 1024)).astype(np.float32)
    pos = np.arange(40, dtype=np.int32)
    h = cuda(h0)
    ae.conformer_layer(m, 0, h, cuda(pos, torch.int32))
    want = oracle.conformer_layer(h0, L, pos)
    assert rel_l2(h.cpu().numpy(), want) <= FP32_TOL, rel_l2(h.cpu().numpy(), want)


# ----------------------------------------------------------- whole encoder

def test_encode_tone_one_layer_fp32():
    say("[gpu] encode: 1 s tone, 1 layer + head, fp32, per-stage trace")
    W = weights(1)
    m = ae.Model(W, dtype="f32")
    x = synth.tone_clip(0)
    wave, so = synth.pack([x])
    out, tr = ae.encode(m, cuda(wave), so, trace=True)
    otr = []
    want = oracle.encode_clips([x], W, trace=otr)[0]
    assert rel_l2(tr[0].cpu().numpy(), otr[0]) <= FP32_TOL
    assert rel_l2(tr[1].cpu().numpy(), otr[1]) <= FP32_TOL
    assert rel_l2(out.cpu().numpy(), want) <= FP32_TOL, rel_l2(out.cpu().numpy(), want)


def test_encode_30s_twelve_layers_fp32():
    say("[gpu] encode: one 30 s multisine clip, 12 layers + head, fp32")
    W = weights(12)
    m = ae.Model(W, dtype="f32")
    x = synth.multisine_clip(0)
    wave, so = synth.pack([x])
    out, tr = ae.encode(m, cuda(wave), so, trace=True)
    otr = []
    want = oracle.encode_clips([x], W, trace=otr)[0]
    assert out.shape == (750, 512)
    for i in range(13):
        r = rel_l2(tr[i].cpu().numpy(), otr[i])
        say(f"    stage {i}: rel {r:.3e}")
        assert r <= FP32_TOL, (i, r)
    r = rel_l2(out.cpu().numpy(), want)
    say(f"    output: rel {r:.3e}")
    assert r <= FP32_TOL


def test_encode_batch32_bf16_sampled():
    """The benchmark workload: 32 x 30 s, bf16 weights and operands."""
    say("[gpu] encode: 32 x 30 s multisine, bf16, clips 0, 5, 13, 20, 27, 31 vs oracle")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    clips = synth.multisine_batch(32)
    wave, so = synth.pack(clips)
    out, tr = ae.encode(m, cuda(wave), so, trace=True)
    out = out.cpu().numpy()
    assert out.shape == (24000, 512)
    otr = []
    oracle.encode_clips([clips[0]], W, trace=otr)
    for k in range(13):
        say(f"    clip 0 stage {k}: rel {rel_l2(tr[k][:750].cpu().numpy(), otr[k]):.3e}")
    for i in (0, 5, 13, 20, 27, 31):
        want = oracle.encode_clips([clips[i]], W)[0]
        bf16_gate(out[i * 750:(i + 1) * 750], want, f"clip {i}")


def test_encode_batch256_bf16_sampled():
    """256 clips x 30 s through the whole bf16 encoder in one call: 192,000
    tokens, eight times the benchmark's rows (every projection's M, the
    conv0 plane of 384,256 rows, offsets past 2^17 rows). The first, a
    middle and the last clip against the oracle."""
    say("[gpu] encode: 256 x 30 s white noise, bf16, 192000 tokens, clips 0, 128, 255 vs oracle")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    clips = synth.white_batch(256)
    wave, so = synth.pack(clips)
    out = ae.encode(m, cuda(wave), so).cpu().numpy()
    assert out.shape == (256 * 750, 512)
    assert np.all(np.isfinite(out))
    for i in (0, 128, 255):
        bf16_gate(out[i * 750:(i + 1) * 750], oracle.encode_clips([clips[i]], W)[0], f"clip {i}")


def test_encode_ragged64_bf16_sampled():
    say("[gpu] encode: 64 ragged pink-noise clips, bf16, 8 clips (shortest, longest, last) vs oracle")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    clips = synth.ragged_batch(64)
    wave, so = synth.pack(clips)
    out = ae.encode(m, cuda(wave), so).cpu().numpy()
    T = [oracle.num_tokens(len(c)) for c in clips]
    toff = np.concatenate([[0], np.cumsum(T)])
    assert out.shape[0] == toff[-1]
    lens = [len(c) for c in clips]
    # 23900 tokens: the last clip's rows fill the final, partial row tile of
    # every projection (92 rows of a 192- or 256-row tile; the rows past the
    # end are read as zeros and never stored)
    for i in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7, 19, 32, 45, 58, len(clips) - 1}):
        want = oracle.encode_clips([clips[i]], W)[0]
        bf16_gate(out[toff[i]:toff[i + 1]], want, f"clip {i} ({lens[i]} samples)")


# -------------------------------------------------------------- invariants

def test_causality_bf16():
    """Token j reads samples <= 640 j + 639: perturbing later samples
    leaves tokens 0..j bit-identical on the GPU."""
    say("[gpu] invariant: causality, bf16")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    x = synth.multisine_clip(3, 64000)
    j = 40
    y = x.copy()
    y[640 * j + 640:] += np.float32(0.25)
    a = ae.encode(m, cuda(x), np.array([0, len(x)])).cpu().numpy()
    b = ae.encode(m, cuda(y), np.array([0, len(y)])).cpu().numpy()
    assert np.array_equal(a[:j + 1], b[:j + 1])
    assert not np.array_equal(a[j + 1], b[j + 1])


def test_clip_isolation_and_determinism_bf16():
    say("[gpu] invariant: clip isolation in a pack, determinism, bf16")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    clips = [synth.pink_clip(1, 30000), synth.tone_clip(2, 150), synth.multisine_clip(4, 50000)]
    wave, so = synth.pack(clips)
    packed = ae.encode(m, cuda(wave), so).cpu().numpy()
    again = ae.encode(m, cuda(wave), so).cpu().numpy()
    assert np.array_equal(packed, again)
    T = [ae.num_tokens(len(c)) for c in clips]
    assert T[1] == 0
    off = 0
    for c, t in zip(clips, T):
        alone = ae.encode(m, cuda(c), np.array([0, len(c)])).cpu().numpy() if t else np.zeros((0, 512))
        assert np.array_equal(alone, packed[off:off + t])
        off += t


def test_clip_isolation_fp32():
    """The fp32 path keeps a clip's output bit-identical alone and packed
    too (its attention sums the window in a fixed order, its GEMMs
    accumulate every output in the same k order whatever its row and
    whichever tile shape the row count selects)."""
    say("[gpu] invariant: clip isolation in a pack, fp32, 2 layers + head")
    W = weights(2)
    m = ae.Model(W, dtype="f32")
    clips = [synth.pink_clip(3, 30000), synth.multisine_clip(7, 50000), synth.tone_clip(8, 12000)]
    wave, so = synth.pack(clips)
    packed = ae.encode(m, cuda(wave), so).cpu().numpy()
    off = 0
    for c in clips:
        t = ae.num_tokens(len(c))
        alone = ae.encode(m, cuda(c), np.array([0, len(c)])).cpu().numpy()
        assert np.array_equal(alone, packed[off:off + t])
        off += t
    assert off == packed.shape[0]
    # a pack past 4096 rows runs its GEMMs in the large-row tiles: the same
    # bits again for the clip that also ran alone
    big = [synth.multisine_clip(20 + i) for i in range(6)] + [clips[1]]
    wave, so = synth.pack(big)
    packed = ae.encode(m, cuda(wave), so).cpu().numpy()
    assert packed.shape[0] == 6 * 750 + ae.num_tokens(len(clips[1]))
    alone = ae.encode(m, cuda(clips[1]), np.array([0, len(clips[1])])).cpu().numpy()
    assert np.array_equal(alone, packed[6 * 750:])


def test_encode_matches_layer_by_layer_bf16():
    """ae_encode fuses each layer's FFN 1 pre-norm into the previous layer's
    last row kernel and runs the row kernels in pairs; ae_conformer_layer
    called once per layer on the subsampler's output gives the same bits
    for every layer's h (two packed clips, three layers)."""
    say("[gpu] invariant: ae_encode's layer outputs = ae_conformer_layer layer by layer, bf16")
    W = weights(3, bf16=True)
    m = ae.Model(W, dtype="bf16")
    clips = [synth.multisine_clip(40, 64000), synth.pink_clip(41, 37000)]
    wave, so = synth.pack(clips)
    _, tr = ae.encode(m, cuda(wave), so, trace=True)
    T = [ae.num_tokens(len(c)) for c in clips]
    pos = cuda(np.concatenate([np.arange(t) for t in T]).astype(np.int32), torch.int32)
    h = tr[0].clone()
    for layer in range(3):
        ae.conformer_layer(m, layer, h, pos)
        assert torch.equal(h, tr[layer + 1]), layer


def test_overlong_clip_truncated_bf16():
    """A clip past 30 s is encoded as its first 480000 samples: the 31 s
    clip, alone and packed between two short clips, gives the bits of its
    30 s prefix."""
    say("[gpu] invariant: a 31 s clip encodes as its first 30 s, bf16")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    x = synth.multisine_clip(31, 496000)
    a = ae.encode(m, cuda(x), np.array([0, len(x)])).cpu().numpy()
    b = ae.encode(m, cuda(x[:480000].copy()), np.array([0, 480000])).cpu().numpy()
    assert a.shape == (750, 512) and np.array_equal(a, b)
    clips = [synth.tone_clip(5, 20000), x, synth.tone_clip(6, 9000)]
    wave, so = synth.pack(clips)
    packed = ae.encode(m, cuda(wave), so).cpu().numpy()
    t0 = ae.num_tokens(20000)
    assert np.array_equal(packed[t0:t0 + 750], b)


def test_empty_batches():
    say("[gpu] edge: empty batch, clips without tokens")
    W = weights(1)
    m = ae.Model(W, dtype="f32")
    out = ae.encode(m, cuda(np.zeros(0, np.float32)), np.array([0]))
    assert out.shape == (0, 512)
    out = ae.encode(m, cuda(np.zeros(300, np.float32)), np.array([0, 100, 260, 300]))
    assert out.shape == (0, 512)
    x = synth.tone_clip(0, 161)
    out = ae.encode(m, cuda(x), np.array([0, 161]))
    want = oracle.encode_clips([x], W)[0]
    assert out.shape == (1, 512) and rel_l2(out.cpu().numpy(), want) <= FP32_TOL
