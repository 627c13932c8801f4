"""Float64 oracle of the 2-D time x frequency subsampling front (the variant of the encoder's
conv front end that treats the log-mel frames as an image).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe the front end as three causal stride-2 convolutions with kernel 3 in time
and a 14-frame mel tail ("True streaming encode — implementation spec", "State" and "Per-chunk
flow" step 2; "Status": padTop at the first chunk only, padBottom at flush, which hints at a
2-D time x frequency layout) and the model's encoder as NeMo's cache-aware Conformer with its
mel loopback cache ("Parakeet-EOU-120M — Streaming ASR Model", "Encoder"). Reading S1-S4 for
the 2-D variant, the depthwise-striding stack:
  S1 stage 1: a 3 x 3 convolution from 1 to C channels, stride 2 in time and frequency, then
     ReLU; stages 2 and 3: a depthwise 3 x 3 convolution (stride 2 in both) followed by a
     pointwise C -> C convolution, then ReLU.
  S2 time is causal as in the 1-D front end (output t reads input rows 2t-2 .. 2t; at the first
     chunk each stage's input is padded with two zero rows before the stream start, later chunks
     run over [14-frame mel tail || 16 new frames] without padding); frequency is padded with one
     zero column on each side (F -> F/2 per stage: 128 -> 64 -> 32 -> 16).
  S3 the C x F/8 map of each output frame is flattened channel-major (index c * F/8 + f) and
     projected to d_model by a linear layer with bias.
  S4 C = 256 channels; weights: c1 [C][3][3], dw2 / dw3 [C][3][3], pw2 / pw3 [C_out][C_in],
     lin [C * F/8][D] ([in][out]), each with a bias.

Parity status: pinned in ``tests/test_oracle_subsample2d_pins.py`` (each stage against torch's
conv2d, and chunked streaming against the offline computation of a whole mel sequence).
"""
from __future__ import annotations

import numpy as np


def _conv3x3_s2(x, w, b, time_pad):
    """x [Cin, T, F] -> [Cout, T', F'] for a full (groups 1) 3 x 3 convolution, or a depthwise
    one when w is [C, 3, 3] and x has C channels (then Cout = Cin); stride 2 in both axes,
    frequency padded by one zero column on each side, time padded by ``time_pad`` zero rows in
    front (0: valid in time)."""
    Cin, T, F = x.shape
    xp = np.zeros((Cin, T + time_pad, F + 2))
    xp[:, time_pad:, 1:F + 1] = x
    To = (T + time_pad - 3) // 2 + 1
    Fo = (F + 2 - 3) // 2 + 1
    depthwise = w.ndim == 3
    out = np.zeros((Cin if depthwise else w.shape[0], To, Fo)) + b[:, None, None]
    for i in range(3):
        for j in range(3):
            patch = xp[:, i: i + 2 * To - 1: 2, j: j + 2 * Fo - 1: 2]   # [Cin, To, Fo]
            if depthwise:
                out += w[:, i, j][:, None, None] * patch
            else:
                out += np.einsum("oc,ctf->otf", w[:, :, i, j], patch)
    return out


def stages(W, mel, time_pad):
    """The three stages and the projection on a mel block [T, F]; returns [T/8, D]."""
    x = mel[None]                                                        # [1, T, F]
    x = np.maximum(_conv3x3_s2(x, W["fe2.c1.w"][:, None], W["fe2.c1.b"], time_pad), 0.0)
    for s in ("2", "3"):
        d = _conv3x3_s2(x, W[f"fe2.dw{s}.w"], W[f"fe2.dw{s}.b"], time_pad)
        x = np.maximum(np.einsum("oc,ctf->otf", W[f"fe2.pw{s}.w"], d) + W[f"fe2.pw{s}.b"][:, None, None], 0.0)
    C, T8, F8 = x.shape
    flat = x.transpose(1, 0, 2).reshape(T8, C * F8)                    # channel-major per frame
    return flat @ W["fe2.lin.w"] + W["fe2.lin.b"]


def offline(W, mel):
    """The whole mel sequence [16 C, F] with the causal per-stage padding: [2 C, D]."""
    return stages(W, np.asarray(mel, np.float64), time_pad=2)


def stream(W, mel_tail, mel_new, pos):
    """One chunk: the first chunk of a stream (pos 0) is the offline computation of its 16
    frames; later chunks run valid in time over [mel_tail || mel_new] (30 -> 14 -> 6 -> 2)."""
    if pos == 0:
        return offline(W, mel_new)
    return stages(W, np.concatenate([mel_tail, mel_new], axis=0), time_pad=0)
