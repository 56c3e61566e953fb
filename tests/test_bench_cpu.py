"""CPU checks of the benchmark's host logic: the one-GPU refusal, the FLOP
counts behind the roofline, and the rule that a stored HBM-traffic record
counts only while the kernel sources it was measured on are unchanged."""
import json
import os
import subprocess
import sys
import types


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "asked for 2" in r.stderr


def test_gemm_flops_per_launch():
    cfg = types.SimpleNamespace(hidden=1024, ff=4096)
    T = 24000
    # 2 M N K for each projection of a layer
    assert bench.gemm_flops_per_launch("gemm_ffn1", T, cfg) == 2.0 * T * 4096 * 1024
    assert bench.gemm_flops_per_launch("gemm_ffn2", T, cfg) == 2.0 * T * 1024 * 4096
    assert bench.gemm_flops_per_launch("gemm_qkv", T, cfg) == 2.0 * T * 3072 * 1024
    assert bench.gemm_flops_per_launch("gemm_lcstart", T, cfg) == 2.0 * T * 2048 * 1024
    # 201.3 GFLOP for the 32 x 30 s workload's FFN W1
    assert abs(bench.gemm_flops_per_launch("gemm_ffn1", T, cfg) / 1e9 - 201.3) < 0.05


def _record(tmp_path, kclass, workload, sha, hbm):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    rec = {"kernel_class": kclass, "workload": workload, "hbm_bytes_per_launch": hbm,
           "sources_sha256": sha}
    (prof / f"traffic_{kclass}_{workload}.md").write_text(
        "# record\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "log_mel_conformer_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES["gemm"]:
        (csrc / f).write_text(f"// {f}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.sources_sha256("gemm_ffn1")
    _record(tmp_path, "gemm_ffn1", "batch32", sha, 12345)
    assert bench.recorded_traffic("gemm_ffn1", "batch32") == 12345.0
    # no record for another workload
    assert bench.recorded_traffic("gemm_ffn1", "lfm2a32") is None
    # any change to a source the kernel is built from voids the record
    (csrc / "common.h").write_text("// common.h, edited\n")
    assert bench.recorded_traffic("gemm_ffn1", "batch32") is None


def test_committed_records_name_their_kernel():
    """Every committed traffic record parses and names its kernel class and
    workload (whether it is still valid depends on the sources)."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith("traffic_") and n.endswith(".md")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        blocks = text.split("```json")[1:]
        assert blocks, n
        rec = json.loads(blocks[-1].split("```")[0])
        assert n == f"traffic_{rec['kernel_class']}_{rec['workload']}.md"
        assert rec["hbm_bytes_per_launch"] > 0 and len(rec["sources_sha256"]) == 64


def test_encoder_work_matches_independent_counts():
    """The per-kernel work of the 32 x 30 s step: the projection GEMMs and
    conv1 total 588.0 MFLOP per token (48.23 per layer x 12, in_proj 2.10,
    out_proj 3.15, embed 1.57, conv1 2 (32 T) 32 1152 / T = 2.36), 1.411e13
    FLOP for 24000 tokens; the row kernels' bytes from a per-launch count of
    what each one reads and writes, in bf16 (paired launches) and in fp32."""
    cfg = types.SimpleNamespace(hidden=1024, ff=4096, out_hidden=1536, out_dim=512)
    T, F, T1, S = 24000, 32 * 2999, 32 * 1500, 32 * 480000
    pl = {"token_off": [0, T], "frame_off": [0, F], "row_off": [0, T1], "sample_off": [0, S]}
    w = bench.encoder_work(pl, cfg, 2, 12)
    # bf16: the conv1 class is the fused subsampler, conv0's flops included
    conv0 = 2.0 * T1 * 64 * 128 * 9
    assert "conv0" not in w and w["conv1"][1] == 2.0 * 32 * T * 32 * 1152 + conv0
    gemm = sum(v for k, (b, v) in w.items() if k.startswith("gemm_") or k == "conv1") - conv0
    assert abs(gemm / T / 1e6 - 588.0) < 0.05
    assert abs(gemm / 1e13 - 1.411) < 0.001
    wf = bench.encoder_work(pl, cfg, 4, 12)
    assert wf["conv1"][1] == 2.0 * 32 * T * 32 * 1152
    assert wf["conv0"][1] == 4.0 * 128 * F + 4 * T1 * 64 * 128
    # row kernels, launch by launch (bf16 activations, fp32 h, d = 1024)
    d, es = 1024, 2
    launches = [(4 + es) * d]                       # layer 0's FFN 1 pre-norm
    for layer in range(12):
        # pairs: post FFN 1 (h, y1 in; q|k|v input out; h left unwritten),
        # post attention (h, y1, y2 in; h, lc input out), lc add + FFN 2 pre
        # (h, y3 in; FFN 2 input out), post FFN 2 + norm_out (h, y3, y4 in;
        # h, next layer's input out)
        launches += [(4 + es) * d + es * d, (4 + 2 * es) * d + (4 + es) * d] * 2
    # the last layer's last launch writes the head's bf16 copy in place of a
    # next input (the same bytes); FFN 2's pre-norm sits in the lc add
    # launch and each later layer's FFN 1 pre-norm in the previous layer's
    # last launch: 49 launches, plus the head's
    launches.append((4 + es) * 1536)
    assert len(launches) == 50
    assert abs(w["rownorm"][1] - T * sum(launches)) < 1.0
    # float models: four launches a layer, each y and h in, h and the next
    # input out; the last writes no next input
    wf_rows = [(4 + 4) * d] + [(4 + 8 + 4) * d] * 48
    wf_rows[-1] -= 4 * d
    wf_rows.append((4 + 4) * 1536)
    assert abs(wf["rownorm"][1] - T * sum(wf_rows)) < 1.0
    assert w["logmel"][1] == 4.0 * S + 512.0 * F
    assert w["attn"][1] == 12 * T * 4 * es * d and w["lconv"][1] == 12 * T * 2 * es * d


def test_lfm2a_work_matches_independent_counts():
    """The LFM2A work model against a launch-by-launch count built from the
    oracle's geometry (frames, conv_out, tokens): 32 clips of 30 s."""
    from oracle import lfm2a as olfm
    n = [480000] * 31 + [123457]
    F = [olfm.num_frames(x) for x in n]
    T = [olfm.num_tokens(x) for x in n]
    w = bench.lfm2a_work(n, F, T)
    d, ff, L = 512, 2048, 17
    r1 = [olfm.conv_out(f, 3, 2, 1) for f in F]
    r2 = [olfm.conv_out(r, 3, 2, 1) for r in r1]
    assert [olfm.conv_out(r, 3, 2, 1) for r in r2] == T
    Tn, R1, R2 = sum(T), sum(r1), sum(r2)
    assert T[0] == 376 and Tn == 31 * 376 + T[-1]
    mm = lambda m, nn, k: 2.0 * m * nn * k  # noqa: E731
    # stem: three 3x3 layers, 9 multiply-adds per output value, 256 channels
    assert w["lfm_stem"] == ("alu", 2 * 9 * 256 * (R1 * 64 + R2 * 32 + Tn * 16.0))
    assert w["lfm_gemm_stem"][1] == mm(R2 * 32, 256, 256) + mm(Tn * 16, 256, 256) + mm(Tn, 512, 4096)
    # per block: ffn, attention (q|k|v, position rows, output), conv (pw1, pw2), ffn
    launches = {"lfm_gemm_ffn1": 0.0, "lfm_gemm_ffn2": 0.0, "lfm_gemm_attn": 0.0,
                "lfm_gemm_conv": 0.0}
    for _ in range(L):
        for _half in range(2):
            launches["lfm_gemm_ffn1"] += mm(Tn, ff, d)
            launches["lfm_gemm_ffn2"] += mm(Tn, d, ff)
        launches["lfm_gemm_attn"] += mm(Tn, 3 * d, d) + mm(2 * max(T) - 1, d, d) + mm(Tn, d, d)
        launches["lfm_gemm_conv"] += mm(Tn, 2 * d, d) + mm(Tn, d, d)
    for k, v in launches.items():
        assert abs(w[k][1] - v) <= 1e-9 * v, k
    assert w["lfm_gemm_adapter"][1] == mm(Tn, 2048, 512) + mm(Tn, 2048, 2048)
    assert w["lfm_attn"][1] == L * sum(3 * 2.0 * t * t * d for t in T)
    # 69 LayerNorm launches: one before block 0, four per block; the last of
    # each block writes x back besides the next norm's bf16 output
    ln = [(4 + 2) * d]
    for _ in range(L):
        ln += [(4 + 2) * d] * 3 + [(4 + 4 + 2) * d]
    assert len(ln) == 69 and w["lfm_ln"] == ("hbm", Tn * float(sum(ln)))
    assert w["lfm_dwconv"] == ("hbm", L * Tn * (2 + 2) * d * 1.0)
    # front end: samples in; every frame written twice (features, then the
    # normalised or zeroed plane); the statistics frames read twice
    E = [olfm.effective_frames(x) for x in n]
    assert all(e == f - 1 for e, f in zip(E, F))
    assert w["lfm_front"] == ("hbm", 4.0 * sum(n) + 512.0 * (2 * sum(F) + 2 * sum(E)))
