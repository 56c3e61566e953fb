"""Throughput of the audio-encoder forward on one MI355X.

Default workload: 32 clips x 30 s (multisine + noise, seeds 0..31), the
whole encoder (log-mel, subsampler, 12 Conformer layers, head) with bf16
weights and projection operands on MFMA, fp32 accumulation, norms and
residual stream; random-init weights. A step is one ae_encode over the
batch, inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                  [--workload batch32|batch32q8|ragged64|frontend256|tone1s|clip30f32|
                              resample48k|merge32|lfm2a32]
                  [--kernel gemm_ffn1] [--no-cpu-baseline] [--cpu-threads N]
                  [--no-kernel-table] [--copy-probe]

Workloads of the encoder: batch32 (32 x 30 s, bf16), ragged64 (64 clips of
1-30 s, bf16), frontend256 (the log-mel front end over 256 x 30 s, fp32),
tone1s (1 s tone: log-mel, subsampler and one Conformer layer, fp32),
clip30f32 (one 30 s clip, 12 layers and the head, fp32), batch32q8
(batch32 with int8 projections).

The timed region carries HIP events around the launches of one kernel
class (--kernel; the roofline object). After it: the same steps with no
events (ms_per_step_no_events), and for the encoder workloads one short
pass per kernel class with events around that class alone, for the
per-kernel roofline table ("kernels"). --copy-probe runs one plain 256 MiB
device-to-device copy after the timed region; under rocprofv3 --pmc it is
the calibration for FETCH_SIZE and WRITE_SIZE. --cpu-threads sets the BLAS
threads of the oracle baseline (default: every core this process may use).
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
    "logmel": ["logmel.hip", "fft16.h", "launch.h", "common.h"],
    "gemm": ["gemm.hip", "lds_dma.h", "launch.h", "common.h"],
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


def host_cpu():
    """The host CPU's model name and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def oracle_run(fn, threads):
    """fn() under a BLAS thread limit; returns (seconds, threads used, CPU)."""
    from threadpoolctl import threadpool_limits
    model, avail = host_cpu()
    n = threads or avail
    with threadpool_limits(limits=n):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
    return dt, n, model


def cpu_baseline(clips, W, seconds, threads, layers=None, with_head=True, what=None):
    """The oracle (f64 numpy) on a sample of the workload's clips."""
    import oracle
    dt, n, model = oracle_run(lambda: oracle.encode_clips(clips, W, layers=layers,
                                                          with_head=with_head), threads)
    return {"value": seconds / dt, "unit": "audio-s/s", "cores": n, "kind": "oracle",
            "cpu": model,
            "sample": what or (f"{len(clips)} clip(s) of the workload ({seconds:.1f} s of audio), "
                               f"full encoder in float64 numpy, {dt:.1f} s wall")}


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


def mfma_rate(torch):
    """The device's sustained bf16 matrix-core rate (TFLOP/s): the
    library's probe kernel (independent matrix instructions on register
    operands, no memory traffic; about 5 ms a run, long enough for the
    clock to settle), best of 3, timed with events after the timed region:
    a second denominator beside the nominal 2.5 PFLOP/s."""
    from log_mel_conformer_amd import ae
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ae.probe_mfma(100, sink)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = ae.probe_mfma(10000, sink)
        e1.record()
        torch.cuda.synchronize()
        rate = flops / (e0.elapsed_time(e1) / 1e3) / 1e12
        best = rate if best is None else max(best, rate)
    return best


def add_copy_denominator(roof, torch):
    """The measured copy bandwidth, and for an HBM-bound kernel its
    achieved bandwidth as a fraction of it; for a bf16 matrix-core kernel
    the measured matrix-core rate and the fraction of it."""
    bw = copy_bandwidth(torch)
    roof["measured_copy_GBps"] = bw
    if roof.get("bound") == "hbm":
        roof["frac_of_copy"] = roof["achieved"] / bw
    if roof.get("bound") == "mfma" and roof.get("peak") == PEAK_BF16_TFLOPS:
        rate = mfma_rate(torch)
        roof["measured_mfma_TFLOPs"] = rate
        roof["frac_of_measured_mfma"] = roof["achieved"] / rate
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
        c0 = clips[0]
        dt, threads, model = oracle_run(lambda: ors.to_mono_16k([c0[:, 0], c0[:, 1]], 48000),
                                        args.cpu_threads)
        cpu = {"value": 30.0 / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
               "cpu": model,
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


def lfm2a_work(sample_counts, frame_counts, token_counts, blocks=17):
    """Algorithmic work per step of each LFM2A kernel class: (bound, amount)
    with flops for the matrix-core and vector classes and bytes for the
    memory-bound ones.
    - front end: the samples read once (4 B); the 128-band feature plane
      (512 B a frame) written; the frames the statistics cover (n // 160 of
      a clip's 1 + n // 160) read for them and read again to normalise;
      every frame written by the normalisation (the rest as zeros);
    - stem convolutions (vector units): 9 multiply-adds per output value of
      the 3x3 layer 0 (one input channel, 256 out) and of the two depthwise
      layers; a 3x3 stride-2 layer with one row of padding maps h rows to
      ceil(h / 2), and frequencies go 128 -> 64 -> 32 -> 16;
    - GEMMs 2 M N K: the stem's two pointwise layers (256 -> 256 over
      (rows, frequency)) and pre_encode_out (4096 -> 512); per block two
      feed-forward pairs (512 -> 2048 -> 512), q|k|v (512 -> 1536), the
      position projection of the 2 t_max - 1 table rows, the attention
      output (512 -> 512), pw1 (512 -> 1024) and pw2 (512 -> 512); the
      adapter (512 -> 2048 -> 2048);
    - attention per clip of t tokens and block: q.k, (q + v).p and
      softmax.v over the t x t pairs, 2 t^2 512 flops each;
    - LayerNorms: one ahead of block 0 (x in, bf16 out: 6 B a value), three
      of that kind per block and the block's closing norm, which writes x
      back and the next norm's bf16 output (10 B);
    - depthwise convolution: the GLU output in, its output out (bf16)."""
    S, F = float(sum(sample_counts)), float(sum(frame_counts))
    E = float(sum(int(n) // 160 for n in sample_counts))
    T = float(sum(token_counts))
    up = lambda h: (h + 1) // 2  # noqa: E731
    r1 = [up(f) for f in frame_counts]
    r2 = [up(r) for r in r1]
    R1, R2 = float(sum(r1)), float(sum(r2))
    t_max = max(token_counts) if token_counts else 0
    d, ff, ch, L = 512, 2048, 256, blocks
    gemm = lambda m, n, k: 2.0 * m * n * k  # noqa: E731
    return {
        "lfm_front": ("hbm", 4.0 * S + 512.0 * (2 * F + 2 * E)),
        "lfm_stem": ("alu", 2.0 * 9 * ch * (R1 * 64 + R2 * 32 + T * 16)),
        "lfm_gemm_stem": ("mfma", gemm(R2 * 32, ch, ch) + gemm(T * 16, ch, ch)
                          + gemm(T, d, 16 * ch)),
        "lfm_gemm_ffn1": ("mfma", L * 2 * gemm(T, ff, d)),
        "lfm_gemm_ffn2": ("mfma", L * 2 * gemm(T, d, ff)),
        "lfm_gemm_attn": ("mfma", L * (gemm(T, 3 * d, d) + gemm(2 * t_max - 1, d, d)
                                       + gemm(T, d, d))),
        "lfm_gemm_conv": ("mfma", L * (gemm(T, 2 * d, d) + gemm(T, d, d))),
        "lfm_gemm_adapter": ("mfma", gemm(T, 2048, d) + gemm(T, 2048, 2048)),
        "lfm_attn": ("mfma", L * sum(6.0 * t * t * d for t in token_counts)),
        "lfm_ln": ("hbm", T * d * (6.0 + L * (3 * 6.0 + 10.0))),
        "lfm_dwconv": ("hbm", L * T * d * 2 * 2.0),
    }


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
    log("[bench] the same steps without events")
    ms_plain = time_steps(step, torch, args.steps)
    if args.copy_probe:
        copy_probe(torch)
    avg_ms = kms / max(launches, 1)
    work = lfm2a_work(np.diff(so), np.diff(pl["frame_off"]), toks)
    bound, amount = work[kclass]
    per_launch = amount / max(launches // args.steps, 1)
    if bound == "hbm":
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_F32_TFLOPS if bound == "alu" else PEAK_BF16_TFLOPS
        achieved = per_launch / (avg_ms / 1e3) / 1e12
        roof = {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    roof.update({"frac": achieved / roof["peak"],
                 "traffic": recorded_traffic(kclass, args.workload), "kernel": kclass,
                 "work_per_launch": per_launch, "avg_ms": avg_ms, "launches": launches})
    table = None
    if not args.no_kernel_table:
        log("[bench] per-kernel events, one class at a time")
        table = kernel_table(ae, torch, step, work, 3, PEAK_BF16_TFLOPS)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: the LFM2A oracle on one clip")
        from oracle import lfm2a as olfm
        dt, threads, model = oracle_run(lambda: olfm.encode(clips[0], W), args.cpu_threads)
        cpu = {"value": 30.0 / dt, "unit": "audio-s/s", "cores": threads, "kind": "oracle",
               "cpu": model,
               "sample": f"1 clip of the workload (30 s), the whole LFM2A encoder in float64 "
                         f"numpy, {dt:.1f} s wall"}
    rec = {"metric": "audio-seconds encoded/sec (LFM2A Conformer: front end, stem, 17 blocks, "
                     "adapter; batch 32)",
           "value": audio_s / (ms / 1e3), "unit": "audio-s/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "ms_per_step_no_events": ms_plain,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded waveforms, random-init weights)",
           "config": {"workload": "32 clips x 30 s multisine+noise through the LFM2A encoder: "
                                  "log-mel (pre-emphasis, power, Slaney, per-bin norm), 8x "
                                  "conv stem, 17 relative-position Conformer blocks, adapter "
                                  "to 2048 (bf16 MFMA, fp32 accumulation and norms)",
                      "global_batch": len(clips), "seq_len": max(toks), "tokens": tokens,
                      "frames": frames, "audio_seconds": audio_s,
                      "tokens_per_s": tokens / (ms / 1e3), "parallelism": "none (1 GPU)"},
           "roofline": roof, "kernels": table, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


ENCODER_NAMES = {
    "batch32": "32 clips x 30 s multisine+noise: log-mel, subsampler, 12 Conformer layers, head "
               "(bf16 MFMA, fp32 accumulation and norms)",
    "batch32q8": "32 clips x 30 s multisine+noise, the encoder with int8 projections (per-row "
                 "scales) widened to bf16",
    "ragged64": "64 clips, 1-30 s pink noise, packed ragged: full encoder, bf16",
    "frontend256": "256 clips x 30 s white noise: log-mel front end only, fp32",
    "tone1s": "one 1 s tone (440 Hz + noise): log-mel, subsampler, one Conformer layer, fp32",
    "clip30f32": "one 30 s multisine clip: full encoder (12 layers + head), fp32",
}


def encoder_work(pl, cfg, es, layers, q8=False, head=True):
    """Algorithmic work per step of each kernel class of ae_encode: (bound,
    amount) with flops for the matrix-core classes and bytes for the
    memory-bound ones. es = bytes per stored activation (2 bf16, 4 fp32).
    Row kernels per layer: four launches (after FFN 1, after attention,
    the light conv's residual add with FFN 2's pre-norm, after FFN 2 with
    norm_out). In fp32 each reads a GEMM output y and h and writes h and
    the next normed input. In bf16 they run in pairs: the first reads h and
    its y and writes only the next input; the second reads h, the first's
    y and its own, and writes h and the next input. The first layer's
    FFN 1 pre-norm reads h and writes its input; the last launch writes the
    head's bf16 copy of h instead of a next input (nothing in fp32); the
    head's norm reads and writes 1536 columns."""
    T = float(pl["token_off"][-1])
    F = float(pl["frame_off"][-1])
    T1 = float(pl["row_off"][-1])
    S = float(pl["sample_off"][-1])
    d, ff, oh, od = cfg.hidden, cfg.ff, cfg.out_hidden, cfg.out_dim
    L = layers
    pre = (4 + es) * d                  # h in, normed input out
    if es == 2:
        first = (4 + 2 * es) * d        # h and y in, next input out
        second = (8 + 3 * es) * d       # h, y0 and y in; h and next input (or head copy) out
        rows = pre + L * 2 * (first + second) - (0 if head else es * d)
    else:
        post = (es + 8 + es) * d        # y in, h read and written, next input out
        rows = pre + L * 4 * post - es * d   # the last launch writes no next input
    rows += (4 + es) * oh if head else 0
    w = {
        "logmel": ("hbm", 4.0 * S + 4.0 * 128 * F),
        "conv0": ("hbm", 4.0 * 128 * F + es * T1 * 64 * 128),
        "conv1": ("mfma", 2.0 * (32 * T) * 32 * 1152),
        "gemm_ffn1": ("mfma", L * 2 * 2.0 * T * ff * d),
        "gemm_ffn2": ("mfma", L * 2 * 2.0 * T * d * ff),
        "gemm_qkv": ("mfma", L * 2.0 * T * 3 * d * d),
        "gemm_post": ("mfma", L * 2.0 * T * d * d),
        "gemm_lcstart": ("mfma", L * 2.0 * T * 2 * d * d),
        "gemm_lcend": ("mfma", L * 2.0 * T * d * d),
        "gemm_head": ("mfma", 2.0 * T * d * 1024 + (2.0 * T * oh * d + 2.0 * T * od * oh
                                                    if head else 0.0)),
        "rownorm": ("hbm", T * rows),
        "attn": ("hbm", L * T * 4 * es * d),
        "lconv": ("hbm", L * T * 2 * es * d),
    }
    if es == 2:
        # bf16 models run both convolutions in one kernel (timed as conv1):
        # conv0's 64 x 128 x 9 multiply-adds per conv0 row join conv1's
        del w["conv0"]
        w["conv1"] = ("mfma", w["conv1"][1] + 2.0 * T1 * 64 * 128 * 9)
    if q8:
        w["dequant"] = ("hbm", L * 3.0 * (2 * ff * d * 2 + 7 * d * d) * 1.0)
    return w


def kernel_table(ae, torch, step, work, steps, peak_mm):
    """One pass per kernel class with HIP events around its launches alone:
    average launch time, achieved rate and fraction of the roofline (the
    matrix cores' peak for "mfma", the fp32 vector peak for "alu", HBM for
    "hbm")."""
    out = []
    for cls, (bound, amount) in work.items():
        ae.timing_enable(cls)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        launches, kms = ae.timing_read()
        ae.timing_enable(None)
        if launches == 0:
            continue
        per_step_ms = kms / steps
        if bound in ("mfma", "alu"):
            ach = amount / (per_step_ms / 1e3) / 1e12
            peak, unit = (peak_mm if bound == "mfma" else PEAK_F32_TFLOPS), "TFLOP/s"
        else:
            ach = amount / (per_step_ms / 1e3) / 1e9
            peak, unit = PEAK_HBM_GBS, "GB/s"
        out.append({"kernel": cls, "bound": bound, "launches_per_step": launches // steps,
                    "avg_us": 1e3 * kms / launches, "ms_per_step": per_step_ms,
                    "work_per_step": amount, "achieved": ach, "peak": peak, "unit": unit,
                    "frac": ach / peak})
    return out


def time_steps(step, torch, steps):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch32",
                    choices=["batch32", "batch32q8", "ragged64", "frontend256", "tone1s",
                             "clip30f32", "resample48k", "merge32", "lfm2a32"])
    ap.add_argument("--kernel", default=None,
                    help="kernel class of the roofline object (default: the workload's largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--no-kernel-table", action="store_true")
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
        args.kernel = args.kernel or "lfm_gemm_ffn1"
        return bench_lfm2a(args, torch, ae, synth)
    wl = args.workload
    clips = {"batch32": lambda: synth.multisine_batch(32),
             "batch32q8": lambda: synth.multisine_batch(32),
             "ragged64": lambda: synth.ragged_batch(64),
             "frontend256": lambda: synth.white_batch(256),
             "tone1s": lambda: [synth.tone_clip(0)],
             "clip30f32": lambda: [synth.multisine_clip(0)]}[wl]()
    wave_np, so = synth.pack(clips)
    wave = torch.from_numpy(wave_np).cuda()
    pl = ae.plan(np.diff(so))
    audio_s = float(pl["sample_off"][-1]) / 16000.0
    tokens = int(pl["token_off"][-1])
    frames = int(pl["frame_off"][-1])

    W = None
    model = None
    work = {}
    layers = 12
    if wl == "frontend256":
        mel = torch.empty((frames, 128), dtype=torch.float32, device="cuda")
        step = lambda: ae.logmel(wave, so, out=mel)  # noqa: E731
        kclass = args.kernel or "logmel"
        dtype = "f32"
        work = {"logmel": ("hbm", 4.0 * float(pl["sample_off"][-1]) + 4.0 * 128 * frames)}
        peak_mm = PEAK_F32_TFLOPS
    else:
        f32 = wl in ("tone1s", "clip30f32")
        layers = 1 if wl == "tone1s" else 12
        if wl == "batch32q8":
            log("[bench] generating weights (12 layers, int8 projections)")
            W, S = synth.make_weights_q8(layers=12)
            model = ae.Model(W, dtype="bf16", scales=S)
        else:
            log(f"[bench] generating weights ({layers} layers, {'fp32' if f32 else 'bf16'})")
            W = synth.make_weights(layers=layers, bf16=not f32)
            model = ae.Model(W, dtype="f32" if f32 else "bf16")
        dtype = "f32" if f32 else "bf16"
        peak_mm = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
        model.workspace(len(clips), frames, tokens)
        if wl == "tone1s":
            # the configuration's three stages: log-mel, subsampler, one layer
            mel = torch.empty((frames, 128), dtype=torch.float32, device="cuda")
            h = torch.empty((tokens, model.cfg.hidden), dtype=torch.float32, device="cuda")
            pos = torch.arange(tokens, dtype=torch.int32, device="cuda")

            def step():
                ae.logmel(wave, so, out=mel)
                ae.subsample(model, mel, pl["frame_off"], out=h)
                ae.conformer_layer(model, 0, h, pos)
            work = encoder_work(pl, model.cfg, 4, 1, head=False)
        else:
            out = torch.empty((tokens, 512), dtype=torch.float32, device="cuda")
            step = lambda: ae.encode(model, wave, so, out=out)  # noqa: E731
            work = encoder_work(pl, model.cfg, 4 if f32 else 2, layers, q8=(wl == "batch32q8"))
        kclass = args.kernel or "gemm_ffn1"

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps (events around {kclass})")
    ae.timing_enable(kclass)
    ms = time_steps(step, torch, args.steps)
    launches, kms = ae.timing_read()
    ae.timing_enable(None)
    log("[bench] the same steps without events")
    ms_plain = time_steps(step, torch, args.steps)
    if args.copy_probe:
        copy_probe(torch)
    value = audio_s / (ms / 1e3)
    avg_ms = kms / max(launches, 1)

    bound, amount = work[kclass]
    per_launch = amount / max(launches // args.steps, 1)
    if bound == "hbm":
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = per_launch / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_mm, "unit": "TFLOP/s"}
    roof.update({"frac": achieved / roof["peak"],
                 "traffic": recorded_traffic(kclass, wl), "kernel": kclass,
                 "work_per_launch": per_launch, "avg_ms": avg_ms, "launches": launches})

    table = None
    if not args.no_kernel_table and len(work) > 1:
        log("[bench] per-kernel events, one class at a time")
        table = kernel_table(ae, torch, step, work, 3, peak_mm)

    cpu = None
    if not args.no_cpu_baseline:
        if wl == "frontend256":
            import oracle
            log("[bench] cpu baseline: oracle log-mel on a sample of the clips")
            n = 128   # about 10 s of host work
            dt, threads, cpu_model = oracle_run(lambda: [oracle.log_mel(c) for c in clips[:n]],
                                                args.cpu_threads)
            cpu = {"value": n * 30.0 / dt, "unit": "audio-s/s", "cores": threads,
                   "kind": "oracle", "cpu": cpu_model,
                   "sample": f"log-mel of {n} of the 256 clips in float64 numpy, {dt:.1f} s wall"}
        else:
            Wo = W
            if wl == "batch32q8":
                # the oracle runs the widened weights bf16(float32(q) * s)
                from oracle import quant
                Wo = {**W, "layers": [{**L, **{k: quant.dequantize_rows(L[k], sc[k]) for k in sc}}
                                      for L, sc in zip(W["layers"], S)]}
            # a bounded sample of about 10-20 s of host work
            if wl == "ragged64":
                # the clips nearest the batch's mean length
                order = np.argsort(np.abs(np.diff(so) - np.mean(np.diff(so))))
                sample = [clips[i] for i in order[:6]]
            else:
                sample = clips[:3]
            secs = sum(len(c) for c in sample) / 16000.0
            log(f"[bench] cpu baseline: oracle on {len(sample)} clip(s), {secs:.1f} s of audio")
            cpu = cpu_baseline(sample, Wo, secs, args.cpu_threads,
                               layers=layers, with_head=(wl != "tone1s"))
            if wl == "tone1s":
                cpu["sample"] = ("the whole workload (1 s clip: log-mel, subsampler, one layer) "
                                 "in float64 numpy")

    rec = {"metric": METRIC, "value": value, "unit": "audio-s/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "ms_per_step_no_events": ms_plain,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded waveforms, random-init weights)",
           "config": {"workload": ENCODER_NAMES[wl], "global_batch": len(clips),
                      "seq_len": int(max(np.diff(pl["token_off"]))) if tokens else 0,
                      "tokens": tokens, "frames": frames, "audio_seconds": audio_s,
                      "tokens_per_s": tokens / (ms / 1e3), "parallelism": "none (1 GPU)"},
           "roofline": roof, "kernels": table, "cpu_baseline": cpu}
    add_copy_denominator(rec["roofline"], torch)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
