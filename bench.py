"""Throughput of the cache-aware streaming Conformer chunk step on one MI355X.

A step is one push of one chunk for every stream of the workload through the whole path
(front end if any, 17 blocks, joint projection), inputs already resident in HBM. The headline
workload is the largest one-GPU configuration: 1024 streams at staggered positions, each
pushing 16 log-mel frames through the front end and the 17-layer d=512 encoder in bf16 (fp32
accumulate). The one-stream float32 encoder (the weight-bandwidth-bound case) and greedy
RNNT + EOU decoding of 1024 streams, the streaming log-mel front, and batched beam search over
64 utterances are measured in the same run and reported in the same JSON line under
"secondary". Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload C4|C2|C3|C5] [--secondary C2|none]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoder frames/sec (streams×frames) per chunk step; % HBM or MFMA peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 100 for C4/C3/C5, 1000 for C2)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--secondary", default="C2,C2Q,C4S",
                    help="comma-separated workloads reported in the same line, or 'none'")
    ap.add_argument("--decode", default="D2", help="greedy-decoding workload reported in the same line, or 'none'")
    ap.add_argument("--mel", default="A4", help="streaming log-mel workload reported in the same line, or 'none'")
    ap.add_argument("--beam", default="B8", help="beam-search workload reported in the same line, or 'none'")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="oracle time per CPU-baseline mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy a 256 MiB device buffer 4 times (the reference dispatches for "
                         "scaling hardware byte counters)")
    return ap.parse_args()


def source_hash(files) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "cache_aware_conformer_amd", "csrc")
    for name in sorted(files):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch (read + write) from the committed counter summary of this kernel
    family on this workload, if it was taken on the current source of that kernel; else None."""
    path = os.path.join(PROFILES, "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(f"{workload}:{kernel}")
    if not ent or ent.get("source_hash") != source_hash(ent.get("sources", [])):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def usable_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(cfg, W, seconds: float):
    """The float64 oracle's cached chunk step as it stands, timed on the host cores, once with
    one BLAS thread and once with every usable core, on a bounded sample of the workload: for
    many-stream workloads 32 streams from their staggered states (streams are independent, so
    the per-stream rate scales to the batch), for one stream that stream; as many chunks as
    fit in ``seconds`` per mode (at least one)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import Oracle
    from synth import make_inputs, make_state
    orc = Oracle(cfg, W)
    n_s = min(cfg.streams, 32)
    ids = list(np.linspace(0, cfg.streams - 1, n_s).astype(int))
    xs = np.stack([make_inputs(cfg, s, min(cfg.chunks, 200)) for s in ids])
    modes = {}
    for name, threads in (("1_thread", 1), ("all_cores", usable_cores())):
        sts = [orc.state_from(make_state(cfg, s)) if cfg.staggered else orc.new_state() for s in ids]
        with threadpool_limits(threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            t0 = time.perf_counter()
            chunks = 0
            while chunks < xs.shape[1] and (chunks < 1 or time.perf_counter() - t0 < seconds):
                orc.push(sts, xs[:, chunks].astype(np.float64))
                chunks += 1
            dt = time.perf_counter() - t0
        frames = n_s * cfg.n_emit * chunks
        modes[name] = {"value": frames / dt, "threads": int(used), "chunks": chunks, "seconds": dt}
    best = modes["all_cores"]
    return {"value": best["value"], "unit": "frames/s", "cores": best["threads"], "kind": "oracle",
            "cpu_model": cpu_model(), "usable_cores": usable_cores(),
            "single_thread": {"value": modes["1_thread"]["value"], "cores": 1},
            "sample": (f"{cfg.name}: {n_s} stream(s){' from staggered states' if cfg.staggered else ''} x "
                       f"{best['chunks']} chunk(s), float64 cached step; {best['seconds']:.1f} s all-core "
                       f"({best['threads']} threads), {modes['1_thread']['seconds']:.1f} s on one thread "
                       f"({modes['1_thread']['chunks']} chunk(s))")}


def roofline_of(enc, fam: str, workload: str, reps: int = 20) -> dict:
    """Back-to-back launch duration of one kernel family (its launches of the last recorded
    step, replayed as a graph between HIP events on the library's stream) against its
    algorithmic work: MFMA-bound when its flops per algorithmic byte exceed the bf16 ridge
    (312 flop/B), otherwise HBM-bound."""
    rep = enc.profile_replay(fam, reps=reps)
    us, kbytes, kflops = rep["us_per_launch"], rep["bytes_per_launch"], rep["flops_per_launch"]
    if "mfma" in fam and kbytes and kflops / kbytes > 312.0:
        roof = {"bound": "mfma", "achieved": kflops / (us * 1e-6) / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kbytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(fam, workload)
    roof["kernel"] = fam
    roof["avg_launch_us"] = us
    roof["launches_per_step"] = rep["launches"]
    roof["algorithmic_bytes_per_launch"] = kbytes
    roof["algorithmic_flops_per_launch"] = kflops
    return roof


def run_workload(key: str, steps, warmup: int, profile_steps: int, want_cpu: bool, cpu_seconds: float,
                 extra_families=()):
    import torch

    from cache_aware_conformer_amd import StreamingEncoder
    from synth import CONFIGS, make_inputs, make_state, make_weights

    cfg = CONFIGS[key]
    if steps is None:
        steps = min(cfg.chunks, 1000) if cfg.streams == 1 else 100
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    W = make_weights(cfg)
    S = cfg.streams
    enc = StreamingEncoder(cfg, W, max_streams=S)
    if cfg.staggered:
        for g0 in range(0, S, 64):
            grp = list(range(g0, min(S, g0 + 64)))
            enc.import_state_dicts(grp, [make_state(cfg, s) for s in grp])
    # distinct inputs for every pushed chunk up to the workload's length, then cycled
    per_stream = min(cfg.chunks, warmup + steps + profile_steps + 1)
    # chunk-major [chunks, S, frames, width]: each step's input is one contiguous slab in HBM
    xs = np.ascontiguousarray(np.stack([make_inputs(cfg, s, per_stream) for s in range(S)]).swapaxes(0, 1))
    x_dev = torch.from_numpy(xs).to(dev).to(tdt)
    del xs
    out = torch.empty((S, cfg.n_emit, cfg.joint_dim or cfg.d_model), dtype=torch.float32, device=dev)
    ids = list(range(S))
    k = 0

    def step():
        nonlocal k
        enc.push_chunk(ids, x_dev[k % per_stream], out)
        k += 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the library enqueues on torch's current stream (given at create time), so events recorded
    # there bracket exactly the pushes
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    frames = S * cfg.n_emit * steps
    value = frames / (ms / 1e3)
    ms_step = ms / steps

    # per-kernel timing over a second window of the same workload
    enc.profile(True)
    for _ in range(profile_steps):
        step()
    torch.cuda.synchronize()
    prof = enc.profile_read()
    enc.profile(False)
    # kernel families ("gemm_mfma_bf16/qkv" -> "gemm_mfma_bf16"); the roofline covers the family
    # that takes the most time, the others named in extra_families get their own figure
    fam = {}
    for n, v in prof.items():
        f = fam.setdefault(n.split("/")[0], [0, 0.0, 0.0, 0.0])
        for i in range(4):
            f[i] += v[i]
    dom = max(fam, key=lambda n: fam[n][1])
    step()                       # a graph replay: the family replays use its recorded launches
    torch.cuda.synchronize()
    others = {f: roofline_of(enc, f, cfg.name) for f in extra_families if f in fam and f != dom}
    roof = roofline_of(enc, dom, cfg.name)   # leaves the streams' state unspecified
    step_bytes = sum(v[2] for v in prof.values()) / profile_steps
    step_flops = sum(v[3] for v in prof.values()) / profile_steps
    res = {
        "value": value, "ms_per_step": ms_step, "steps": steps, "warmup": warmup,
        "dtype": {"f32": "f32", "bf16": "bf16", "i8w": "f32 (int8 weights)"}[cfg.dtype],
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "d_model": cfg.d_model, "heads": cfg.n_heads,
                   "d_ff": cfg.d_ff, "att_left": cfg.att_left, "streams": S, "frames_per_chunk": cfg.n_emit,
                   "frames_computed_per_chunk": cfg.n_compute, "joint_dim": cfg.joint_dim,
                   "frontend": cfg.frontend, "staggered_start": cfg.staggered, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step": {"algorithmic_bytes": step_bytes, "algorithmic_flops": step_flops,
                 "hbm_frac_of_peak": step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "mfma_frac_of_peak": step_flops / (ms_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                 "kernels_note": "dispatch-bound HIP events per launch (include the event markers)",
                 "kernels": {n: {"launches_per_step": v[0] / profile_steps,
                                 "us_per_step": v[1] / profile_steps * 1e3} for n, v in
                             sorted(prof.items(), key=lambda kv: -kv[1][1])}},
    }
    if others:
        res["rooflines_other"] = others
    enc.close()
    del x_dev, out, enc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, W, cpu_seconds)
    return res


FP32_MFMA_PEAK_TFLOPS = 157.3  # dense fp32 matrix


def run_decode(key: str, steps, warmup: int, profile_steps: int):
    """Greedy decoding throughput of one decode workload: every stream decodes its next
    ``frames`` projected frames per call (inputs resident in HBM), state carried across calls."""
    import torch

    from cache_aware_conformer_amd import StreamingDecoder
    from synth import DEC_CONFIGS, make_dec_inputs, make_dec_weights

    cfg = DEC_CONFIGS[key]
    steps = steps if steps is not None else 100
    S = cfg.streams
    dev = torch.device("cuda:0")
    dec = StreamingDecoder(cfg, make_dec_weights(cfg), max_streams=S)
    per = min(cfg.calls, warmup + steps + profile_steps + 1)
    xs = np.ascontiguousarray(np.stack([make_dec_inputs(cfg, s, per) for s in range(S)]).swapaxes(0, 1))
    z = torch.from_numpy(xs).to(dev)
    del xs
    ids = list(range(S))
    tok = torch.empty((S, cfg.frames * cfg.max_symbols), dtype=torch.int32, device=dev)
    frm = torch.empty_like(tok)
    cnt = torch.empty(S, dtype=torch.int32, device=dev)
    k = 0

    def call():
        nonlocal k
        dec.decode(ids, z[k % per], tok, frm, cnt)
        k += 1

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    dec.profile(True)
    emitted = 0
    for _ in range(profile_steps):
        call()
        emitted += int(cnt.sum().item())
    torch.cuda.synchronize()
    prof = dec.profile_read()
    dec.profile(False)
    busy = {n: v for n, v in prof.items() if not n.endswith("/idle")}
    dom = max(busy, key=lambda n: busy[n][1])
    launches, tms, by, fl = busy[dom]
    us = tms / launches * 1e3
    roof = {"bound": "mfma", "achieved": fl / launches / (us * 1e-6) / 1e12, "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "traffic": None, "kernel": dom, "avg_launch_us": us,
            "launches_per_step": launches / profile_steps, "algorithmic_flops_per_launch": fl / launches,
            "algorithmic_bytes_per_launch": by / launches,
            "timing": "per-launch HIP events bound to each dispatch (include the event markers)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    res = {"value": S * cfg.frames * steps / (ms / 1e3), "unit": "frames/s", "ms_per_step": ms / steps,
           "steps": steps, "dtype": "f32",
           "emitted_classes_per_step": emitted / profile_steps,
           "config": {"workload": cfg.name, "streams": S, "frames_per_call": cfg.frames,
                      "pred_layers": cfg.pred_layers, "pred_hidden": cfg.pred_hidden, "joint_dim": cfg.joint_dim,
                      "classes": cfg.classes, "max_symbols": cfg.max_symbols,
                      "rounds_per_call": 1 + cfg.frames * cfg.max_symbols},
           "roofline": roof,
           "kernels": {n: {"launches_per_step": v[0] / profile_steps, "us_per_step": v[1] / profile_steps * 1e3}
                       for n, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}}
    dec.close()
    return res


def run_beam(key: str, steps, warmup: int):
    """Batched MALSD beam search: one call decodes every utterance of the workload (frames
    resident in HBM) to its K best transcripts; the call returns once the search has ended."""
    import torch

    from cache_aware_conformer_amd import BeamSearch
    from synth import BEAM_CONFIGS, make_beam_inputs, make_dec_weights

    cfg = BEAM_CONFIGS[key]
    steps = steps if steps is not None else 10
    steps = min(steps, 20)
    n = cfg.streams
    dev = torch.device("cuda:0")
    W = make_dec_weights(cfg)
    zs, lens = zip(*(make_beam_inputs(cfg, s, W) for s in range(n)))
    z = torch.from_numpy(np.stack(zs)).to(dev)
    lens = np.array(lens, np.int32)
    bs = BeamSearch(cfg, W, max_streams=n, max_frames=cfg.frames)
    out = bs.decode(z, lens)
    iters = out[4]
    for _ in range(warmup):
        bs.decode(z, lens, out=out[:4])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        bs.decode(z, lens, out=out[:4])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    bs.profile(True)
    bs.decode(z, lens, out=out[:4])
    torch.cuda.synchronize()
    prof = bs.profile_read()
    bs.profile(False)
    busy = {k: v for k, v in prof.items() if not k.endswith("/idle") and v[3] > 0}
    dom = max(busy, key=lambda k: busy[k][1])
    launches, tms, by, fl = busy[dom]
    us = tms / launches * 1e3
    roof = {"bound": "mfma", "achieved": fl / launches / (us * 1e-6) / 1e12, "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "traffic": None, "kernel": dom, "avg_launch_us": us,
            "launches_per_step": launches, "algorithmic_flops_per_launch": fl / launches,
            "algorithmic_bytes_per_launch": by / launches,
            "timing": "per-launch HIP events bound to each dispatch (include the event markers)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tl = out[1].cpu().numpy()
    res = {"value": float(lens.sum()) * steps / (ms / 1e3), "unit": "frames/s", "ms_per_step": ms / steps,
           "utterances_per_s": n * steps / (ms / 1e3), "steps": steps, "dtype": "f32",
           "iterations_per_call": iters, "best_transcript_tokens_mean": float(tl[:, 0].mean()),
           "config": {"workload": cfg.name, "utterances": n, "frames_max": cfg.frames,
                      "frames_total": int(lens.sum()), "beam": cfg.beam, "max_symbols": cfg.max_symbols,
                      "pred_layers": cfg.pred_layers, "pred_hidden": cfg.pred_hidden, "joint_dim": cfg.joint_dim,
                      "classes": cfg.classes},
           "roofline": roof,
           "kernels": {k: {"launches_per_step": v[0], "us_per_step": v[1] * 1e3}
                       for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}}
    bs.close()
    return res


FP64_VECTOR_PEAK_TFLOPS = 78.6


def run_mel(key: str, steps, warmup: int):
    """Streaming log-mel throughput: every stream pushes one chunk of raw audio (16 hops of 10 ms)
    per step, inputs resident in HBM."""
    import torch

    from cache_aware_conformer_amd import StreamingMel
    from synth import MEL_CONFIGS, make_audio

    cfg = MEL_CONFIGS[key]
    steps = steps if steps is not None else 100
    S = cfg.streams
    dev = torch.device("cuda:0")
    mel = StreamingMel(cfg)
    per = min(cfg.chunks, warmup + steps + 1)
    xs = np.ascontiguousarray(np.stack([make_audio(cfg, s, per) for s in range(S)]).swapaxes(0, 1))
    x = torch.from_numpy(xs).to(dev)
    del xs
    ids = list(range(S))
    out = torch.empty((S, cfg.hops, cfg.n_mels), dtype=torch.bfloat16 if cfg.out_dtype == "bf16" else torch.float32,
                      device=dev)
    k = 0

    def call():
        nonlocal k
        mel.push(ids, x[k % per], out)
        k += 1

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    frames = S * cfg.hops
    n2 = cfg.n_fft // 2
    # float64 operations per frame: the complex FFT (5 N2 log2 N2), the real split (~10 per
    # bin), the filter sums (2 per filter weight, about 2 bins per filter on average here)
    flops = frames * (5.0 * n2 * np.log2(n2) + 10.0 * (n2 + 1) + 2.0 * 2 * cfg.n_mels)
    res = {"value": frames / (ms / 1e3), "unit": "frames/s", "ms_per_step": ms, "steps": steps, "dtype": "f64 transform, "
           + cfg.out_dtype + " out",
           "config": {"workload": cfg.name, "streams": S, "hops_per_chunk": cfg.hops, "n_fft": cfg.n_fft,
                      "win_length": cfg.win_length, "hop": cfg.hop, "n_mels": cfg.n_mels},
           "roofline": {"bound": "alu", "achieved": flops / (ms * 1e-3) / 1e12, "peak": FP64_VECTOR_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "kernel": "logmel + mel_tail (one push)", "avg_launch_us": ms * 1e3,
                        "traffic": None, "timing": "HIP events around each push (both kernels)",
                        "hbm_bytes_per_push": S * cfg.hops * cfg.hop * 4.0 + frames * cfg.n_mels * 2.0}}
    res["roofline"]["frac"] = res["roofline"]["achieved"] / res["roofline"]["peak"]
    mel.close()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the chunk step shards by stream with no "
                                   "collectives, so N GPUs would run N independent copies; --gpus must be 1"}))
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    head = run_workload(args.workload, args.steps, args.warmup, args.profile_steps, not args.no_cpu_baseline,
                        args.cpu_seconds, extra_families=("attention", "gemm_mfma_bf16_dwconv"))
    res = {"metric": METRIC, "value": head["value"], "unit": "frames/s", "n_gpus": 1, "steps": head["steps"],
           "warmup": head["warmup"], "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
           "config": head["config"], "roofline": head["roofline"]}
    for key in ("rooflines_other", "cpu_baseline", "step"):
        if key in head:
            res[key] = head[key]
    for key in (args.secondary or "none").split(","):
        if key.lower() == "none" or key == args.workload:
            continue
        sec = run_workload(key, args.steps, args.warmup, args.profile_steps, False, 0.0)
        rec = {k: sec[k] for k in ("value", "ms_per_step", "steps", "dtype", "config", "roofline", "step")}
        rec["unit"] = "frames/s"
        res.setdefault("secondary", {})[sec["config"]["workload"]] = rec
    if args.mel and args.mel.lower() != "none":
        mres = run_mel(args.mel, args.steps, args.warmup)
        res.setdefault("secondary", {})[mres["config"]["workload"]] = mres
    if args.decode and args.decode.lower() != "none":
        dres = run_decode(args.decode, args.steps, args.warmup, args.profile_steps)
        res.setdefault("secondary", {})[dres["config"]["workload"]] = dres
    if args.beam and args.beam.lower() != "none":
        bres = run_beam(args.beam, None, min(args.warmup, 3))
        res.setdefault("secondary", {})[bres["config"]["workload"]] = bres
    print(json.dumps(res))


if __name__ == "__main__":
    main()
