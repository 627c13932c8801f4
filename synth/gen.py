"""Seeded draws: weights, per-stream inputs and injected stream states.

Every tensor comes from its own generator,
``default_rng(SeedSequence([config_seed, crc32(name)]))``, so any single stream can be
regenerated on its own (the oracle checks sampled streams one by one while the GPU runs the
whole batch).

Distributions (the pages give none for synthetic runs, so these are stated choices):
matrices and biases ~ N(0, 1/fan_in) with fan_in the contraction length (depthwise: the
kernel width; front-end convs: 3 * input channels); LayerNorm gains 1 + 0.1 N(0,1), shifts
0.1 N(0,1); the positional biases u, v ~ N(0, 1/head_dim); the positional projection
~ N(0, 1/d_model); inputs and injected states ~ N(0,1).

For bf16 workloads every drawn value is rounded once to the nearest bf16 (ties to even) and
handed out as float32, so both sides start from exactly the same numbers.
"""
from __future__ import annotations

import zlib

import numpy as np

from .configs import DecConfig, EncConfig, MelConfig


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.array(x, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def _rng(cfg: EncConfig, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, zlib.crc32(name.encode())]))


def _draw(cfg: EncConfig, name: str, shape, std: float, mean: float = 0.0) -> np.ndarray:
    x = (mean + std * _rng(cfg, name).standard_normal(shape)).astype(np.float32)
    return bf16_round(x) if cfg.dtype == "bf16" else x


def _draw_unit(cfg: EncConfig, name: str, shape) -> np.ndarray:
    """N(0,1) drawn directly in float32 (inputs and injected states, the bulk of the data)."""
    x = _rng(cfg, name).standard_normal(shape, dtype=np.float32)
    return bf16_round(x) if cfg.dtype == "bf16" else x


def weight_names(cfg: EncConfig):
    """Ordered (name, shape, kind, fan_in) for every parameter of the workload."""
    D, F, H, hd, K = cfg.d_model, cfg.d_ff, cfg.n_heads, cfg.head_dim, cfg.dw_kernel
    specs = []

    def ln(prefix):
        specs.append((prefix + "ln_g", (D,), "gain", 0))
        specs.append((prefix + "ln_b", (D,), "shift", 0))

    for l in range(cfg.n_layers):
        p = f"l{l}."
        # FF1
        ln(p + "ff1.")
        specs += [(p + "ff1.w1", (D, F), "mat", D), (p + "ff1.b1", (F,), "mat", D),
                  (p + "ff1.w2", (F, D), "mat", F), (p + "ff1.b2", (D,), "mat", F)]
        # MHSA
        ln(p + "att.")
        for m in ("q", "k", "v"):
            specs += [(p + f"att.w{m}", (D, D), "mat", D), (p + f"att.b{m}", (D,), "mat", D)]
        specs += [(p + "att.wo", (D, D), "mat", D), (p + "att.bo", (D,), "mat", D),
                  (p + "att.pos_u", (H, hd), "mat", hd), (p + "att.pos_v", (H, hd), "mat", hd),
                  (p + "att.wpos", (D, D), "mat", D)]
        # conv module
        ln(p + "conv.")
        specs += [(p + "conv.pw1", (D, 2 * D), "mat", D), (p + "conv.pw1_b", (2 * D,), "mat", D),
                  (p + "conv.dw", (D, K), "mat", K), (p + "conv.dw_b", (D,), "mat", K),
                  (p + "conv.pw2", (D, D), "mat", D), (p + "conv.pw2_b", (D,), "mat", D)]
        # FF2
        ln(p + "ff2.")
        specs += [(p + "ff2.w1", (D, F), "mat", D), (p + "ff2.b1", (F,), "mat", D),
                  (p + "ff2.w2", (F, D), "mat", F), (p + "ff2.b2", (D,), "mat", F)]
        ln(p + "out.")
    if cfg.joint_dim:
        P = cfg.joint_dim
        specs += [("joint.w", (D, P), "mat", D), ("joint.b", (P,), "mat", D)]
    if cfg.frontend == 2:
        C, F8 = cfg.fe_channels, cfg.mel_bins // 8
        specs += [("fe2.c1.w", (C, 3, 3), "mat", 9), ("fe2.c1.b", (C,), "mat", 9),
                  ("fe2.dw2.w", (C, 3, 3), "mat", 9), ("fe2.dw2.b", (C,), "mat", 9),
                  ("fe2.pw2.w", (C, C), "mat", C), ("fe2.pw2.b", (C,), "mat", C),
                  ("fe2.dw3.w", (C, 3, 3), "mat", 9), ("fe2.dw3.b", (C,), "mat", 9),
                  ("fe2.pw3.w", (C, C), "mat", C), ("fe2.pw3.b", (C,), "mat", C),
                  ("fe2.lin.w", (C * F8, D), "mat", C * F8), ("fe2.lin.b", (D,), "mat", C * F8)]
    elif cfg.frontend:
        C, B = D, cfg.mel_bins
        specs += [("fe.c1.w", (C, B, 3), "mat", 3 * B), ("fe.c1.b", (C,), "mat", 3 * B),
                  ("fe.c2.w", (C, C, 3), "mat", 3 * C), ("fe.c2.b", (C,), "mat", 3 * C),
                  ("fe.c3.w", (D, C, 3), "mat", 3 * C), ("fe.c3.b", (D,), "mat", 3 * C)]
    return specs


def make_weights(cfg: EncConfig) -> dict:
    out = {}
    for name, shape, kind, fan in weight_names(cfg):
        if kind == "gain":
            out[name] = _draw(cfg, name, shape, 0.1, 1.0)
        elif kind == "shift":
            out[name] = _draw(cfg, name, shape, 0.1)
        else:
            out[name] = _draw(cfg, name, shape, 1.0 / np.sqrt(fan))
    return out


def make_token_head(cfg: EncConfig) -> dict:
    """Check-only greedy token head: ReLU(z + p0) @ wout + bout over ``token_classes``."""
    P, C = cfg.joint_dim, cfg.token_classes
    s = 1.0 / np.sqrt(640.0)
    r = lambda n, sh: (s * _rng(cfg, n).standard_normal(sh))  # noqa: E731
    return {"p0": r("head.p0", (P,)), "wout": r("head.wout", (P, C)), "bout": r("head.bout", (C,))}


def make_inputs(cfg: EncConfig, stream: int, chunks: int | None = None) -> np.ndarray:
    """Per-push inputs of one stream: [chunks, n_emit, d_model] subsampled frames, or
    [chunks, mel_per_chunk, mel_bins] log-mel frames when the front end is on."""
    n = cfg.chunks
    if cfg.frontend:
        x = _draw_unit(cfg, f"input.s{stream}", (n, cfg.mel_per_chunk, cfg.mel_bins))
    else:
        x = _draw_unit(cfg, f"input.s{stream}", (n, cfg.n_emit, cfg.d_model))
    return x if chunks is None else x[:chunks]


def state_position(cfg: EncConfig, stream: int) -> int:
    """Position of the injected state of one stream (see ``make_state``), drawn alone."""
    g = _rng(cfg, f"state.s{stream}.pos")
    c, Lc = cfg.att_chunk, cfg.att_left
    fill = c * int(g.integers(0, Lc // c + 1))
    return fill if fill < Lc else Lc + c * int(g.integers(0, 5001))


def make_state(cfg: EncConfig, stream: int) -> dict:
    """Injected mid-stream state of one stream (staggered workloads).

    Cache fill is uniform over {0, c, 2c, ..., Lc} (c = att_chunk). Below a full cache the
    stream has emitted exactly ``fill`` frames; at a full cache its position is
    Lc + c*U{0..5000}, so ring offsets vary. Layouts (float32):

    - ``pos``: frames already emitted (the stream position).
    - ``k``, ``v``: [L, Lc, D]; row r holds position pos - Lc + r; rows older than the
      fill (positions before 0) are zero.
    - ``conv``: [L, dw_kernel-1, D]; column j holds position pos - (dw_kernel-1) + j;
      positions before 0 are zero.
    - ``mel_tail``: [mel_tail, mel_bins] (front end only; zero for a stream at position 0).
    - ``x0_tail``: [n_lookahead, D] layer-0 inputs of the pending provisional frames
      pos .. pos+n_lookahead-1 (lookahead variant only).
    """
    L, Lc, D, Kc = cfg.n_layers, cfg.att_left, cfg.d_model, cfg.conv_cache
    pos = state_position(cfg, stream)
    fill = min(pos, Lc)
    k = _draw_unit(cfg, f"state.s{stream}.k", (L, Lc, D))
    v = _draw_unit(cfg, f"state.s{stream}.v", (L, Lc, D))
    k[:, : Lc - fill] = 0.0
    v[:, : Lc - fill] = 0.0
    conv = _draw_unit(cfg, f"state.s{stream}.conv", (L, Kc, D))
    nneg = max(0, Kc - pos)
    conv[:, :nneg] = 0.0
    st = {"pos": pos, "fill": fill, "k": k, "v": v, "conv": conv, "mel_tail": None, "x0_tail": None}
    if cfg.frontend:
        mt = _draw_unit(cfg, f"state.s{stream}.mel", (cfg.mel_tail, cfg.mel_bins))
        if pos == 0:
            mt[:] = 0.0
        st["mel_tail"] = mt
    if cfg.n_lookahead:
        st["x0_tail"] = _draw_unit(cfg, f"state.s{stream}.x0", (cfg.n_lookahead, D))
    return st


def dec_weight_names(cfg: DecConfig):
    """Ordered (name, shape, fan_in) of the decoder's parameters (matrices are [in][out])."""
    H, P, C = cfg.pred_hidden, cfg.joint_dim, cfg.classes
    specs = [("pred.embed", (C, H), 1)]
    for l in range(cfg.pred_layers):
        specs += [(f"pred.l{l}.w_ih", (H, 4 * H), H), (f"pred.l{l}.w_hh", (H, 4 * H), H),
                  (f"pred.l{l}.b_ih", (4 * H,), H), (f"pred.l{l}.b_hh", (4 * H,), H)]
    specs += [("pred.proj_w", (H, P), H), ("pred.proj_b", (P,), H),
              ("joint.out_w", (P, C), P), ("joint.out_b", (C,), P)]
    return specs


def make_dec_weights(cfg: DecConfig) -> dict:
    """Decoder weights, float32: every tensor ~ N(0, 1/fan_in) (the embedding N(0, 1)); the
    blank class's joint bias is raised by ``blank_bias`` so that most frames decode to blank,
    as a trained model's do."""
    out = {}
    for name, shape, fan in dec_weight_names(cfg):
        out[name] = (_rng(cfg, name).standard_normal(shape) / np.sqrt(fan)).astype(np.float32)
    out["joint.out_b"][cfg.vocab] += np.float32(cfg.blank_bias)
    return out


def make_dec_inputs(cfg: DecConfig, stream: int, calls: int | None = None) -> np.ndarray:
    """Projected encoder frames of one stream, [calls, frames, joint_dim] ~ N(0, 1) float32
    (the encoder's projected outputs have about unit scale)."""
    x = _rng(cfg, f"dec.input.s{stream}").standard_normal((cfg.calls, cfg.frames, cfg.joint_dim), dtype=np.float32)
    return x if calls is None else x[:calls]


def make_beam_inputs(cfg, stream: int, weights: dict) -> tuple:
    """Projected frames of one utterance for beam search: ([frames, joint_dim] float32, its
    length). Frames ~ N(0, 1); a random ``silence`` fraction of them also carries
    ``silence_gain`` * sqrt(P) / 4 times the unit vector along the positive part of the blank
    class's joint column, which raises the blank's score at those frames the way pauses do in
    speech (so transcripts grow at a speech-like rate instead of a label at every step). The
    length is uniform in [min_frames, frames]; frames past it are drawn but never read."""
    g = _rng(cfg, f"beam.input.s{stream}")
    P = cfg.joint_dim
    z = g.standard_normal((cfg.frames, P))
    quiet = g.random(cfg.frames) < cfg.silence
    u = np.maximum(np.asarray(weights["joint.out_w"], np.float64)[:, cfg.vocab], 0.0)
    u /= np.linalg.norm(u)
    z += (cfg.silence_gain * np.sqrt(P) / 4.0) * quiet[:, None] * u[None, :]
    length = int(g.integers(cfg.min_frames, cfg.frames + 1))
    return z.astype(np.float32), length


def make_audio(cfg: MelConfig, stream: int, chunks: int | None = None) -> np.ndarray:
    """Raw audio of one stream, [chunks, hops * hop] float32: white noise of amplitude 0.05 plus
    two tones (frequency uniform in 80 Hz - 7.5 kHz, amplitude uniform in 0.05 - 0.5) that hold
    for the whole stream (the pages' sample.wav is not available)."""
    g = _rng(cfg, f"audio.s{stream}")
    n = cfg.chunks * cfg.hops * cfg.hop
    t = np.arange(n) / cfg.sample_rate
    x = 0.05 * g.standard_normal(n)
    for _ in range(2):
        f, a, ph = g.uniform(80.0, 7500.0), g.uniform(0.05, 0.5), g.uniform(0.0, 2 * np.pi)
        x += a * np.sin(2 * np.pi * f * t + ph)
    x = x.astype(np.float32).reshape(cfg.chunks, cfg.hops * cfg.hop)
    return x if chunks is None else x[:chunks]
