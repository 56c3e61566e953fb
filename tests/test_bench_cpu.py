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
    what each one reads and writes."""
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
        launches += [(es + 8 + es) * d] * 3         # post FFN 1, post attention, lc add + FFN 2 pre
        launches += [(es + 8 + es) * d]             # post FFN 2 + norm_out + next pre / bf16 copy
    launches[-1] = (es + 8 + es) * d                # the last layer writes the head's bf16 copy
    # FFN 2's pre-norm of each layer (h in, a out) is inside the lc add launch,
    # and each layer's first FFN 1 pre-norm after layer 0 is inside the
    # previous layer's last launch: 49 launches, plus the head's
    launches.append((4 + es) * 1536)
    assert len(launches) == 50
    assert abs(w["rownorm"][1] - T * sum(launches)) < 1.0
    assert w["logmel"][1] == 4.0 * S + 512.0 * F
    assert w["attn"][1] == 12 * T * 4 * es * d and w["lconv"][1] == 12 * T * 2 * es * d
