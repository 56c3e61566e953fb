"""Throughput of the audio-encoder forward on one MI355X.

Default workload: 32 clips x 30 s (multisine + noise, seeds 0..31), the
whole encoder (log-mel, subsampler, 12 Conformer layers, head) with bf16
weights and projection operands on MFMA, fp32 accumulation, norms and
residual stream; random-init weights. A step is one ae_encode over the
batch, inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                  [--workload batch32|batch32q8|frontend256|ragged64|resample48k|merge32|
                              lfm2a32]
                  [--kernel gemm_ffn1] [--no-cpu-baseline] [--copy-probe]

--copy-probe runs one plain 256 MiB device-to-device copy after the timed
region; under rocprofv3 --pmc it is the calibration for FETCH_SIZE and
WRITE_SIZE (the counters' reading for a known byte count).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "audio-seconds encoded/sec (log-mel + 12-layer Conformer, batch 32); % roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_F64_TFLOPS = 78.6   # fp64 vector FMA: 256 CUs x 64 lanes x 2 flops x 2.4 GHz

# HBM traffic per launch measured with rocprofv3 counters, one record per
# kernel class and workload (profiles/traffic_<class>_<workload>.md); valid
# only while the kernel sources hash to what they were when the counters
# were taken.
KERNEL_SOURCES = {
    "logmel": ["logmel.hip", "common.h"],
    "gemm": ["gemm.hip", "launch.h", "common.h"],
    "resample": ["resample.hip", "launch.h", "common.h"],
    "merge": ["placement.hip", "launch.h", "common.h"],
}
COPY_PROBE_BYTES = 256 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_flops_per_launch(cls, tokens, cfg):
    d, ff = cfg.hidden, cfg.ff
    return {
        "gemm_ffn1": 2.0 * tokens * ff * d,
        "gemm_ffn2": 2.0 * tokens * d * ff,
        "gemm_qkv": 2.0 * tokens * 3 * d * d,
        "gemm_post": 2.0 * tokens * d * d,
        "gemm_lcstart": 2.0 * tokens * 2 * d * d,
        "gemm_lcend": 2.0 * tokens * d * d,
    }[cls]


def sources_sha256(kclass):
    files = KERNEL_SOURCES[kclass if kclass in KERNEL_SOURCES else "gemm"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "log_mel_conformer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kclass, workload):
    """Bytes per launch from the committed counter record, or None when there
    is no record for this kernel and workload or its sources have changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kclass}_{workload}.md")
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return None
    for block in text.split("```json")[1:]:
        rec = json.loads(block.split("```")[0])
        if rec.get("kernel_class") == kclass and rec.get("workload") == workload:
            if rec.get("sources_sha256") != sources_sha256(kclass):
                return None
            return float(rec["hbm_bytes_per_launch"])
    return None


def cpu_baseline(clip, W, seconds):
    """The oracle (f64 numpy) on one clip of the workload, timed on the host."""
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    t0 = time.perf_counter()
    oracle.encode_clips([clip], W)
    dt = time.perf_counter() - t0
    return {"value": seconds / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
            "sample": f"1 clip of the workload ({seconds:.0f} s, {len(clip)} samples), full "
                      f"encoder in float64 numpy, {dt:.1f} s wall"}


def copy_probe(torch):
    """One plain device-to-device copy of COPY_PROBE_BYTES: the counters'
    calibration under rocprofv3 --pmc."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def copy_bandwidth(torch):
    """Measured device-to-device copy bandwidth (bytes read + written per
    second, GB/s) of a COPY_PROBE_BYTES copy, best of 6, timed with events
    after the timed region: a second HBM denominator beside the nominal
    peak."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2.0 * COPY_PROBE_BYTES / (best / 1e3) / 1e9


def add_copy_denominator(roof, torch):
    """The measured copy bandwidth, and for an HBM-bound kernel its
    achieved bandwidth as a fraction of it."""
    bw = copy_bandwidth(torch)
    roof["measured_copy_GBps"] = bw
    if roof.get("bound") == "hbm":
        roof["frac_of_copy"] = roof["achieved"] / bw
    return roof


def bench_resample(args, torch, ae, synth):
    """32 clips x 30 s of stereo at 48 kHz -> mono 16 kHz (mixdown and the
    Kaiser-sinc resampler, float64 accumulation)."""
    clips = synth.recorded_batch(32, 48000, 30.0)
    data_np, off = synth.pack_frames(clips)
    data = torch.from_numpy(data_np).cuda()
    r = ae.Resampler(48000, 16000)
    oo = r.out_offsets(off)
    y = torch.empty(int(oo[-1]), dtype=torch.float32, device="cuda")
    step = lambda: ae.to_mono_16k(r, data, off, 2, out=y)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ae.timing_enable("resample")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches, kms = ae.timing_read()
    ae.timing_enable(None)
    ms = (t1 - t0) * 1e3 / args.steps
    if args.copy_probe:
        copy_probe(torch)
    audio_s = float(off[-1]) / 48000.0
    info = r.info()
    # the method's multiply-adds: the taps inside the window of every output
    macs = info["nonzero_taps_per_cycle"] / info["phases"] * float(oo[-1])
    avg_ms = kms / max(launches, 1)
    achieved = 2.0 * macs / (avg_ms / 1e3) / 1e12
    roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_F64_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_F64_TFLOPS,
            "traffic": recorded_traffic("resample", args.workload), "kernel": "k_resample",
            "avg_ms": avg_ms, "launches": launches}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.resample as ors
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        c0 = clips[0]
        t0 = time.perf_counter()
        ors.to_mono_16k([c0[:, 0], c0[:, 1]], 48000)
        dt = time.perf_counter() - t0
        cpu = {"value": 30.0 / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
               "sample": f"1 clip of the workload (30 s stereo at 48 kHz) through the oracle's "
                         f"mixdown and resampler, float64 numpy, {dt:.1f} s wall"}
    r.close()
    rec = {"metric": "audio-seconds resampled/sec (stereo 48 kHz -> mono 16 kHz, batch 32)",
           "value": audio_s / (ms / 1e3), "unit": "audio-s/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f64",
           "data": "synthetic (seeded multisine + noise, two channels)",
           "config": {"workload": "32 clips x 30 s stereo 48 kHz: mixdown + Kaiser-sinc "
                                  "resampling to 16 kHz (float64 accumulation)",
                      "global_batch": 32, "audio_seconds": audio_s,
                      "output_samples": int(oo[-1]), "parallelism": "none (1 GPU)"},
           "roofline": roof, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


def bench_merge(args, torch, ae, synth):
    """The soft tokens of 32 inputs (750 each, 512-d) merged into their
    text embedding rows: ids expanded on the host (ae_expand_ids), rows
    placed on the GPU (ae_merge_soft_tokens)."""
    rng = np.random.default_rng(7)
    seqs = []
    for _ in range(32):
        body = list(rng.integers(3, 250000, 16))
        body.insert(int(rng.integers(0, 17)), ae.RELEASE_AUDIO)
        seqs.append(ae.expand_ids(body, [750], bos=2, eos=1, max_tokens=4096))
    ids_np = np.concatenate(seqs)
    L, d, S = len(ids_np), 512, 32 * 750
    ids = torch.from_numpy(ids_np).cuda()
    x = torch.randn((L, d), dtype=torch.float32, device="cuda")
    soft = torch.randn((S, d), dtype=torch.float32, device="cuda")
    step = lambda: ae.merge_soft_tokens(ids, x, soft)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ae.timing_enable("merge")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches, kms = ae.timing_read()
    ae.timing_enable(None)
    ms = (t1 - t0) * 1e3 / args.steps
    if args.copy_probe:
        copy_probe(torch)
    avg_ms = kms / max(launches, 1)
    # algorithmic bytes: every id read once, every soft row read and written once
    per_launch = 4.0 * L + 2.0 * 4.0 * S * d
    achieved = per_launch / (avg_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": recorded_traffic("merge", args.workload), "kernel": "merge (3 kernels)",
            "avg_ms": avg_ms, "launches": launches}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.placeholders as oph
        xs, ss = x.cpu().numpy(), soft.cpu().numpy()
        t0 = time.perf_counter()
        oph.merge_soft_tokens(xs, ids_np, ss)
        dt = time.perf_counter() - t0
        cpu = {"value": S / dt, "unit": "soft tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"the whole workload through the oracle's merge (numpy rows), {dt:.2f} s"}
    rec = {"metric": "soft tokens merged/sec (32 inputs x 750 soft tokens, 512-d)",
           "value": S / (ms / 1e3), "unit": "soft tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded ids, random rows)",
           "config": {"workload": "32 inputs x (16 text ids + 1 clip of 750 soft tokens), d 512: "
                                  "soft-token merge into the embedding rows",
                      "global_batch": 32, "ids": L, "soft_tokens": S, "parallelism": "none (1 GPU)"},
           "roofline": roof, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


def lfm2a_flops_per_launch(kclass, token_counts):
    """Algorithmic flops of one launch of an LFM2A kernel class over the
    batch: the feed-forward GEMMs are 2 T d n_ff; the attention per clip
    and head takes q.k, (q + v).p on the t x t (query, key) pairs and
    softmax.v, 2 t^2 head_dim each."""
    T = float(sum(token_counts))
    d, ff = 512, 2048
    if kclass in ("lfm_gemm_ffn1", "lfm_gemm_ffn2"):
        return 2.0 * T * d * ff
    if kclass == "lfm_attn":
        return sum(6.0 * t * t * d for t in token_counts)
    raise SystemExit(f"bench.py: no flop count for kernel class {kclass}")


def bench_lfm2a(args, torch, ae, synth):
    """The LFM2A encoder (front end, stem, 17 blocks, adapter) on 32 clips
    of 30 s; one lfm2a_encode per step."""
    from log_mel_conformer_amd import lfm2a
    clips = synth.multisine_batch(32)
    wave_np, so = synth.pack(clips)
    wave = torch.from_numpy(wave_np).cuda()
    pl = lfm2a.plan(np.diff(so))
    toks = [int(t) for t in np.diff(pl["token_off"])]
    tokens, frames = int(pl["token_off"][-1]), int(pl["frame_off"][-1])
    audio_s = float(so[-1]) / 16000.0
    log("[bench] generating weights (LFM2A, 17 blocks, bf16)")
    W = synth.make_lfm2a_weights(17)
    model = lfm2a.Model(W)
    out = torch.empty((tokens, 2048), dtype=torch.float32, device="cuda")
    model.workspace(len(clips), frames, tokens, max(toks))
    kclass = args.kernel if args.kernel.startswith("lfm_") else "lfm_gemm_ffn1"
    step = lambda: lfm2a.encode(model, wave, so, out=out)  # noqa: E731
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps (events around {kclass})")
    ae.timing_enable(kclass)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches, kms = ae.timing_read()
    ae.timing_enable(None)
    ms = (t1 - t0) * 1e3 / args.steps
    if args.copy_probe:
        copy_probe(torch)
    avg_ms = kms / max(launches, 1)
    achieved = lfm2a_flops_per_launch(kclass, toks) / (avg_ms / 1e3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": recorded_traffic(kclass, args.workload),
            "kernel": kclass, "avg_ms": avg_ms, "launches": launches}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: the LFM2A oracle on one clip")
        from oracle import lfm2a as olfm
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        c0 = time.perf_counter()
        olfm.encode(clips[0], W)
        dt = time.perf_counter() - c0
        cpu = {"value": 30.0 / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
               "sample": f"1 clip of the workload (30 s), the whole LFM2A encoder in float64 "
                         f"numpy, {dt:.1f} s wall"}
    rec = {"metric": "audio-seconds encoded/sec (LFM2A Conformer: front end, stem, 17 blocks, "
                     "adapter; batch 32)",
           "value": audio_s / (ms / 1e3), "unit": "audio-s/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded waveforms, random-init weights)",
           "config": {"workload": "32 clips x 30 s multisine+noise through the LFM2A encoder: "
                                  "log-mel (pre-emphasis, power, Slaney, per-bin norm), 8x "
                                  "conv stem, 17 relative-position Conformer blocks, adapter "
                                  "to 2048 (bf16 MFMA, fp32 accumulation and norms)",
                      "global_batch": len(clips), "seq_len": max(toks), "tokens": tokens,
                      "frames": frames, "audio_seconds": audio_s,
                      "tokens_per_s": tokens / (ms / 1e3), "parallelism": "none (1 GPU)"},
           "roofline": roof, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch32",
                    choices=["batch32", "batch32q8", "frontend256", "ragged64", "resample48k",
                             "merge32", "lfm2a32"])
    ap.add_argument("--kernel", default="gemm_ffn1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for {args.gpus}); "
              "clips are independent, so more GPUs would each encode their own share.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from log_mel_conformer_amd import ae, synth

    torch.cuda.set_device(0)
    log(f"[bench] workload {args.workload}: generating inputs")
    if args.workload == "resample48k":
        return bench_resample(args, torch, ae, synth)
    if args.workload == "merge32":
        return bench_merge(args, torch, ae, synth)
    if args.workload == "lfm2a32":
        return bench_lfm2a(args, torch, ae, synth)
    if args.workload in ("batch32", "batch32q8"):
        clips = synth.multisine_batch(32)
    elif args.workload == "ragged64":
        clips = synth.ragged_batch(64)
    else:
        clips = synth.white_batch(256)
    wave_np, so = synth.pack(clips)
    wave = torch.from_numpy(wave_np).cuda()
    pl = ae.plan(np.diff(so))
    audio_s = float(pl["sample_off"][-1]) / 16000.0
    tokens = int(pl["token_off"][-1])
    frames = int(pl["frame_off"][-1])

    W = None
    if args.workload == "frontend256":
        mel = torch.empty((frames, 128), dtype=torch.float32, device="cuda")
        step = lambda: ae.logmel(wave, so, out=mel)  # noqa: E731
        kclass = "logmel"
        dtype = "f32"
    else:
        if args.workload == "batch32q8":
            log("[bench] generating weights (12 layers, int8 projections)")
            W, S = synth.make_weights_q8(layers=12)
            model = ae.Model(W, dtype="bf16", scales=S)
        else:
            log("[bench] generating weights (12 layers, bf16)")
            W = synth.make_weights(layers=12, bf16=True)
            model = ae.Model(W, dtype="bf16")
        out = torch.empty((tokens, 512), dtype=torch.float32, device="cuda")
        model.workspace(len(clips), frames, tokens)
        step = lambda: ae.encode(model, wave, so, out=out)  # noqa: E731
        kclass = args.kernel
        dtype = "bf16"

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps (events around {kclass})")
    ae.timing_enable(kclass)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches, kms = ae.timing_read()
    ae.timing_enable(None)
    ms = (t1 - t0) * 1e3 / args.steps
    if args.copy_probe:
        copy_probe(torch)
    value = audio_s / (ms / 1e3)
    avg_ms = kms / max(launches, 1)

    if kclass == "logmel":
        # algorithmic bytes: every input sample read once, every log-mel value written once
        per_launch = 4.0 * float(pl["sample_off"][-1]) + 4.0 * 128 * frames
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS,
                "traffic": recorded_traffic(kclass, args.workload), "kernel": "k_logmel",
                "avg_ms": avg_ms, "launches": launches}
    else:
        flops = gemm_flops_per_launch(kclass, tokens, model.cfg)
        achieved = flops / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": recorded_traffic(kclass, args.workload),
                "kernel": kclass, "avg_ms": avg_ms, "launches": launches}

    cpu = None
    if not args.no_cpu_baseline and W is not None:
        log("[bench] cpu baseline: oracle on one clip")
        if args.workload == "batch32q8":
            # the oracle runs the widened weights bf16(float32(q) * s)
            from oracle import quant
            W = {**W, "layers": [{**L, **{k: quant.dequantize_rows(L[k], sc[k]) for k in sc}}
                                 for L, sc in zip(W["layers"], S)]}
        cpu = cpu_baseline(clips[0], W, len(clips[0]) / 16000.0)
    elif not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 10.0 and n < len(clips):
            oracle.log_mel(clips[n])
            n += 1
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        cpu = {"value": n * 30.0 / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
               "sample": f"log-mel of {n} of the 256 clips in float64 numpy"}

    names = {"batch32": "32 clips x 30 s multisine+noise: log-mel, subsampler, 12 Conformer "
                        "layers, head (bf16 MFMA, fp32 accumulation and norms)",
             "batch32q8": "32 clips x 30 s multisine+noise, the encoder with int8 projections "
                          "(per-row scales) widened to bf16 per layer per forward",
             "ragged64": "64 clips, 1-30 s pink noise, packed ragged: full encoder, bf16",
             "frontend256": "256 clips x 30 s white noise: log-mel front end only, fp32"}
    rec = {"metric": METRIC, "value": value, "unit": "audio-s/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded waveforms, random-init weights)",
           "config": {"workload": names[args.workload], "global_batch": len(clips),
                      "seq_len": int(max(np.diff(pl["token_off"]))) if tokens else 0,
                      "tokens": tokens, "frames": frames, "audio_seconds": audio_s,
                      "tokens_per_s": tokens / (ms / 1e3), "parallelism": "none (1 GPU)"},
           "roofline": roof, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
