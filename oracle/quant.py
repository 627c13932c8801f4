"""Int8 weight compression of the encoder's dense matrices, for the one-stream
weight-bandwidth-bound path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name compressed encoder weights as a deployment step ("Fast Accuracy-Preserving RNNT
Beam Search on Apple Silicon", §1.3: 6-bit palettized encoder weights; "True streaming encode
— implementation spec", "Status", Nemotron bullet: measurements with int8 weights) but give no
scheme. Reading Q1: symmetric per-output-channel int8. For the weights W [in][out] of a dense
layer, output column n has the scale s_n = max_k |W[k, n]| / 127 and the codes
q[k, n] = round_half_even(W[k, n] / s_n) clamped to [-127, 127] (0 for an all-zero column),
both computed in float32 (the weights' precision); the layer then computes with
W'[k, n] = q[k, n] * s_n. The encoder is otherwise unchanged, so the oracle of the compressed
path is the float64 oracle run on W'.

Compressed: every dense matrix of the blocks (FF1 and FF2 w1, w2; wq, wk, wv, wo; pw1, pw2)
and the joint projection. Not compressed: LayerNorm parameters, biases, the depthwise taps,
the position biases u, v and the position projection (used once at setup).

Parity status: pinned in ``tests/test_oracle_quant_pins.py`` (scalar loops, the half-LSB error
bound, idempotence, and ties to even).
"""
from __future__ import annotations

import numpy as np

COMPRESSED = ("ff1.w1", "ff1.w2", "att.wq", "att.wk", "att.wv", "att.wo", "conv.pw1", "conv.pw2", "ff2.w1", "ff2.w2")


def quantize_columns(w: np.ndarray):
    """Codes (int8) and per-column scales (float32) of a float32 matrix [in][out]."""
    w = np.asarray(w, dtype=np.float32)
    s = (np.abs(w).max(axis=0) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(w / safe)                          # float32 division, round half to even
    q = np.where(s > 0, np.clip(q, -127, 127), 0).astype(np.int8)
    return q, s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return q.astype(np.float64) * s.astype(np.float64)


def compressed_name(name: str) -> bool:
    if name == "joint.w":
        return True
    parts = name.split(".", 1)
    return len(parts) == 2 and parts[0].startswith("l") and parts[0][1:].isdigit() and parts[1] in COMPRESSED


def compress_weights(weights: dict) -> dict:
    """The workload's weights with every compressed matrix replaced by its int8 reconstruction
    (float64); everything else unchanged."""
    out = {}
    for name, w in weights.items():
        if compressed_name(name):
            out[name] = dequantize(*quantize_columns(w))
        else:
            out[name] = w
    return out
