"""Check-only greedy token head, applied in float64 to each path's joint outputs z.

TEST INFRASTRUCTURE ONLY. The pages put a joint over vocabulary + blank + EOU after the
encoder projection ("Parakeet-EOU-120M — Streaming ASR Model", "Joint" and "Vocabulary"; the
projected joint form add -> ReLU -> linear in "Fast Accuracy-Preserving RNNT Beam Search on
Apple Silicon", "NeMo's source already shows the split"). There is no trained decoder here,
so a fixed seeded stand-in p0 replaces the predictor projection (reading A20):
``tok = argmax_c (ReLU(z + p0) @ Wout + bout)[c]``, ties to the lowest index.
"""
from __future__ import annotations

import numpy as np


def logits(z: np.ndarray, head: dict) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z + head["p0"], 0.0) @ head["wout"] + head["bout"]


def greedy_tokens(z: np.ndarray, head: dict):
    """Returns (tokens, margin): argmax per frame and the top-1 minus top-2 logit gap."""
    lg = logits(z, head)
    tok = np.argmax(lg, axis=-1)
    part = np.partition(lg, -2, axis=-1)
    return tok, part[..., -1] - part[..., -2]


def ambiguous_frames(z_ref: np.ndarray, z_test: np.ndarray, head: dict) -> np.ndarray:
    """Frames whose argmax may legitimately differ: the reference margin is below
    2 * max|dz| * max_c ||Wout[:, c]||_1, the most any logit can move under a perturbation dz
    of z (ReLU is 1-Lipschitz)."""
    _, margin = greedy_tokens(z_ref, head)
    dz = np.abs(np.asarray(z_test, np.float64) - np.asarray(z_ref, np.float64)).max(axis=-1)
    col_l1 = np.abs(head["wout"]).sum(axis=0).max()
    return margin < 2.0 * dz * col_l1
