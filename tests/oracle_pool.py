"""Oracle runs of many independent streams in worker processes.

The float64 oracle spends most of its time in per-stream Python work (attention and the
depthwise conv run stream by stream), so whole-workload parity (every stream of a
256- or 1024-stream batch) splits the streams into groups and runs the groups in parallel.
The workers are started with the "spawn" method: fresh interpreters that import only numpy,
``oracle`` and ``synth``, never a copy of a process that holds the GPU. Each worker keeps the
oracle of the last configuration it saw.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time
from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait

import numpy as np

_POOL = None
_WORKERS = max(1, min(8, os.cpu_count() or 1))
_CACHE = {}


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(2)
    except Exception:  # pragma: no cover
        pass


def pool() -> ProcessPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ProcessPoolExecutor(max_workers=_WORKERS, mp_context=mp.get_context("spawn"), initializer=_init)
    return _POOL


def _oracle(cfg):
    from oracle import Oracle
    from oracle.decoder import GreedyDecoder
    from synth import BeamConfig, DecConfig, make_dec_weights, make_weights
    from oracle.quant import compress_weights
    if cfg not in _CACHE:
        _CACHE.clear()
        if isinstance(cfg, (DecConfig, BeamConfig)):
            _CACHE[cfg] = GreedyDecoder(cfg, make_dec_weights(cfg))
        elif cfg.dtype == "i8w":   # int8 dense weights: the oracle runs on their reconstruction
            _CACHE[cfg] = Oracle(cfg, compress_weights(make_weights(cfg)))
        else:
            _CACHE[cfg] = Oracle(cfg, make_weights(cfg))
    return _CACHE[cfg]


def _run_group(cfg, ids, chunks, staggered, flush):
    """Oracle outputs of streams ``ids`` (their seeded inputs) over ``chunks`` pushes, from
    their injected states or fresh; optionally followed by a flush of each stream."""
    from synth import make_inputs, make_state
    orc = _oracle(cfg)
    sts = [orc.state_from(make_state(cfg, s)) if staggered else orc.new_state() for s in ids]
    xs = np.stack([make_inputs(cfg, s, chunks) for s in ids])
    outs = [orc.push(sts, xs[:, c].astype(np.float64)) for c in range(chunks)]
    fl = [orc.flush(st) for st in sts] if flush else None
    return outs, fl


def submit_streams(cfg, ids, chunks, staggered=True, flush=False, group=None):
    """Start the oracle runs of ``ids``; returns a handle for ``collect``."""
    ids = list(ids)
    if group is None:
        group = max(1, -(-len(ids) // (2 * _WORKERS)))
    groups = [ids[i:i + group] for i in range(0, len(ids), group)]
    futs = [pool().submit(_run_group, cfg, g, chunks, staggered, flush) for g in groups]
    return groups, futs, chunks, flush


def collect(handle):
    """Per-chunk oracle outputs [len(ids), m, P] (m = frames emitted by that push) in the order
    of the submitted ids, and the flush outputs (a list, or None)."""
    groups, futs, chunks, flush = handle
    t0, pending = time.time(), set(futs)
    while pending:
        _, pending = wait(pending, timeout=30, return_when=FIRST_COMPLETED)
        print(f"oracle: {len(futs) - len(pending)}/{len(futs)} stream groups done after {time.time() - t0:.0f} s",
              flush=True)
        sys.stdout.flush()
    per_chunk = [[] for _ in range(chunks)]
    flushed = [] if flush else None
    for fut in futs:
        outs, fl = fut.result()
        for c in range(chunks):
            per_chunk[c].append(outs[c])
        if flush:
            flushed += fl
    return [np.concatenate(p, axis=0) for p in per_chunk], flushed


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None


def _dec_group(cfg, ids, calls):
    """Greedy decoding of streams ``ids`` over their seeded projected frames, ``calls`` calls of
    cfg.frames frames each from fresh states; per call, per stream, the (frame, class) list."""
    from synth import make_dec_inputs
    dec = _oracle(cfg)
    out = []
    for s in ids:
        st = dec.new_state()
        xs = make_dec_inputs(cfg, s, calls)
        out.append([dec.decode(st, xs[c]) for c in range(calls)])
    return out


def submit_decode(cfg, ids, calls, group=None):
    ids = list(ids)
    if group is None:
        group = max(1, -(-len(ids) // (2 * _WORKERS)))
    groups = [ids[i:i + group] for i in range(0, len(ids), group)]
    return groups, [pool().submit(_dec_group, cfg, g, calls) for g in groups]


def collect_decode(handle):
    """{stream id: [per call: [(frame, class), ...]]}."""
    groups, futs = handle
    t0, pending = time.time(), set(futs)
    while pending:
        _, pending = wait(pending, timeout=30, return_when=FIRST_COMPLETED)
        print(f"oracle decode: {len(futs) - len(pending)}/{len(futs)} stream groups done after {time.time() - t0:.0f} s",
              flush=True)
    res = {}
    for g, fut in zip(groups, futs):
        for s, calls in zip(g, fut.result()):
            res[s] = calls
    return res


def _beam_group(cfg, ids, steps):
    """Beam search of utterances ``ids`` (their seeded frames and lengths): per utterance the
    final live hypotheses [(transcript, score, frame)], the per-iteration decision gaps and
    score scales, the iteration count, and the live hypotheses after each iteration count in
    ``steps`` (when the search ran that long)."""
    from oracle.beam import BeamTrace, malsd, ModelScorer
    from synth import make_beam_inputs, make_dec_weights
    dec = _oracle(cfg)
    W = _CACHE.setdefault(("weights", cfg), make_dec_weights(cfg))
    out = []
    for s in ids:
        z, n = make_beam_inputs(cfg, s, W)
        tr = BeamTrace()
        slots = malsd(ModelScorer(dec, z), n, cfg.beam, cfg.max_symbols, dec.blank, tr, keep_beams=True)
        live = lambda sl: [(h.prefix, h.score, h.t) for h in sl if h.live]  # noqa: E731
        out.append({"final": live(slots), "gaps": tr.gaps, "scale": tr.scale, "iterations": tr.iterations,
                    "length": n, "at": {m: live(tr.beams[m - 1]) for m in steps if 0 < m <= len(tr.beams)}})
    return out


def submit_beam(cfg, ids, steps=(), group=None):
    ids = list(ids)
    if group is None:
        group = max(1, -(-len(ids) // (2 * _WORKERS)))
    groups = [ids[i:i + group] for i in range(0, len(ids), group)]
    return groups, [pool().submit(_beam_group, cfg, g, tuple(steps)) for g in groups]


def collect_beam(handle):
    """{utterance id: result of _beam_group}."""
    groups, futs = handle
    t0, pending = time.time(), set(futs)
    while pending:
        _, pending = wait(pending, timeout=30, return_when=FIRST_COMPLETED)
        print(f"oracle beam: {len(futs) - len(pending)}/{len(futs)} groups done after {time.time() - t0:.0f} s",
              flush=True)
    res = {}
    for g, fut in zip(groups, futs):
        for s, r in zip(g, fut.result()):
            res[s] = r
    return res
