"""Helpers for the GPU parity tests: device tensors of the seeded draws, staggered-state
import, and the oracle runs of sampled streams."""
from __future__ import annotations

import sys

import numpy as np
import torch

from synth import make_state


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, cfg) -> torch.Tensor:
    """float32 host values (bf16-representable for bf16 workloads) -> device compute dtype."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0").to(dev_dtype(cfg))


def import_staggered(enc, cfg, n_streams: int, group: int = 64) -> list:
    """Inject the seeded mid-stream state of every stream; returns the positions."""
    positions = []
    for g0 in range(0, n_streams, group):
        ids = list(range(g0, min(n_streams, g0 + group)))
        sts = [make_state(cfg, s) for s in ids]
        enc.import_state_dicts(ids, sts)
        positions += [st["pos"] for st in sts]
    torch.cuda.synchronize()
    return positions


def rel_inf(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
