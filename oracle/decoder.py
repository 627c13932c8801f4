"""Float64 oracle of greedy RNNT + EOU decoding over the projected encoder frames.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, per stream ("Parakeet-EOU-120M — Streaming ASR Model", "Decoder" and "Joint";
"Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon", §3.2 "NeMo's source already
shows the split"; "True streaming encode — implementation spec", "Decoder state carry"):
  - The prediction network is a token embedding followed by a stack of LSTM layers. It
    consumes the previous non-blank token; a fresh stream starts from the blank token.
  - Its top-layer output g is projected once per predictor update: p = g Wpred + bpred.
  - The joint after projection, for a projected encoder frame z (the encoder's hoisted joint
    projection): logits = ReLU(z + p) Wout + bout over vocab + blank + EOU classes.
  - Greedy decoding walks the frames in order. At each frame it takes the argmax class (ties
    to the lowest index). Blank moves to the next frame. Any other class (a vocabulary token or
    EOU) is emitted, the predictor advances on it, and the same frame is scored again; after
    max_symbols emissions at one frame the decoder moves on (a forced blank).
  - Across calls the stream carries its LSTM (h, c), its projected predictor output and the
    last emitted token; the predictor runs on that token only when the next joint needs it.

Readings where the pages leave a step open:
  D1 classes: vocabulary V tokens 0..V-1, blank = V, EOU = V+1 (the model card's class count
     vocab + 1 + 1 and its "eou_token_id is vocab_size + 1").
  D2 predictor: embedding width = LSTM width = H; 2 LSTM layers of 640 (the only predictor
     state shape the pages print is [2, K, 640]); torch LSTM gate order i, f, g, o with both
     biases b_ih and b_hh; the blank token's embedding row is whatever the weights hold.
  D3 the predictor is advanced on EOU like on any non-blank class (EOU debouncing is
     application policy, out of scope).
  D4 max_symbols caps emissions per frame (the pages give 10 for the beam decoder's default;
     the greedy workload states its own cap).

Parity status: pinned in ``tests/test_oracle_decoder_pins.py`` (LSTM steps against
torch.nn.LSTM, the joint against torch ops and the unsplit joint, the greedy state machine
against hand-made toy scorers, chunked decoding with state carry against one-call decoding).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


@dataclass
class DecState:
    """Per-stream decoder state: LSTM h, c [layers][H]; the projected predictor output p of
    the last predictor step (None before the first); the token the predictor still has to
    consume before the next joint (blank at stream start, None once consumed)."""
    h: np.ndarray
    c: np.ndarray
    p: np.ndarray | None
    pending: int | None

    def copy(self) -> "DecState":
        return DecState(self.h.copy(), self.c.copy(), None if self.p is None else self.p.copy(), self.pending)


def greedy_loop(n_frames: int, score, advance, blank: int, max_symbols: int):
    """The greedy RNNT state machine over ``n_frames`` frames. ``score(t)`` returns the class
    scores at frame t for the current predictor state; ``advance(k)`` moves the predictor on
    after emitting class k. Returns the emitted (frame, class) pairs in order."""
    out = []
    for t in range(n_frames):
        emitted = 0
        while emitted < max_symbols:
            s = np.asarray(score(t))
            k = int(np.argmax(s))          # first index of the maximum: ties to the lowest index
            if k == blank:
                break
            out.append((t, k))
            emitted += 1
            advance(k)
    return out


class GreedyDecoder:
    """Greedy RNNT + EOU decoding of one decoder configuration, in float64."""

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self.W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
        self.H, self.P, self.V = cfg.pred_hidden, cfg.joint_dim, cfg.vocab
        self.L = cfg.pred_layers
        self.blank, self.eou, self.C = self.V, self.V + 1, self.V + 2

    def new_state(self) -> DecState:
        return DecState(np.zeros((self.L, self.H)), np.zeros((self.L, self.H)), None, self.blank)

    # -- prediction network ---------------------------------------------------------------
    def lstm_step(self, token: int, h, c):
        """One step of the LSTM stack on ``token``; returns the new (h, c) [layers][H]."""
        W, H = self.W, self.H
        x = W["pred.embed"][token]
        h2, c2 = np.empty_like(h), np.empty_like(c)
        for l in range(self.L):
            g = x @ W[f"pred.l{l}.w_ih"] + W[f"pred.l{l}.b_ih"] + h[l] @ W[f"pred.l{l}.w_hh"] + W[f"pred.l{l}.b_hh"]
            i, f, gg, o = g[:H], g[H:2 * H], g[2 * H:3 * H], g[3 * H:]
            c2[l] = _sigmoid(f) * c[l] + _sigmoid(i) * np.tanh(gg)
            h2[l] = _sigmoid(o) * np.tanh(c2[l])
            x = h2[l]
        return h2, c2

    def pred_project(self, g):
        return g @ self.W["pred.proj_w"] + self.W["pred.proj_b"]

    def joint(self, z, p):
        """Joint after projection: ReLU(z + p) Wout + bout."""
        return np.maximum(np.asarray(z, np.float64) + p, 0.0) @ self.W["joint.out_w"] + self.W["joint.out_b"]

    def _consume_pending(self, st: DecState):
        if st.pending is not None:
            st.h, st.c = self.lstm_step(st.pending, st.h, st.c)
            st.p = self.pred_project(st.h[-1])
            st.pending = None

    # -- greedy decoding ------------------------------------------------------------------
    def decode(self, st: DecState, z):
        """Greedy decoding of one stream's projected encoder frames z [n, P], continuing from
        ``st`` (updated in place). Returns the emitted (frame, class) pairs."""
        z = np.asarray(z, np.float64)

        def score(t):
            self._consume_pending(st)
            return self.joint(z[t], st.p)

        def advance(k):
            st.pending = k

        return greedy_loop(z.shape[0], score, advance, self.blank, self.cfg.max_symbols)
