"""Float64 oracle of the encoder: offline masked encode (O1), cached chunk step (O2),
provisional-lookahead pass (O3) and the causal stride-2 conv front end.

TEST INFRASTRUCTURE ONLY (see the package docstring). Parity status: every function here is
pinned by a ``-m "not gpu"`` test against something other than itself (the offline/streaming
identity the streaming spec states, brute-force loops, closed forms and torch CPU library
routines); see ``tests/test_oracle_*.py``. The lookahead pass for right context R > 0 is an
approximation by design: it is pinned by its R = 0 reduction to exact streaming, by the
monotone shrinking of its error with the lookahead length, and by its bookkeeping invariants.

Readings taken where the pages are silent or ambiguous (ids as in the design notes):
  A1  FF1 and FF2 are Conformer macaron half steps: x + 1/2 FF(x).
  A2  FF activation: SiLU.  A3  LayerNorm over the last dim, biased variance, eps 1e-5,
      affine gain and shift.  A4  every dense and pointwise layer has a bias.
  A5  score = ((q + u).k + (q + v).p) / sqrt(head_dim), the scale applied to the sum.
  A6  MHSA output projection Wo + bo before the residual add.
  A7  PE[r, 2m] = sin(r 10000^(-2m/D)), PE[r, 2m+1] = cos(r 10000^(-2m/D)); the position
      projection is PE @ Wpos (no bias), split into heads like q; r = query pos - key pos.
  A9  chunked-causal mask on absolute positions: key q is visible from query p iff q >= 0 and
      cs(p) - Lc <= q <= cs(p) + c - 1, cs(p) = c floor(p / c) (c = 2, Lc = 70).
  A10 positions before 0 do not exist (masked).
  A11 a layer's new K/V rows enter its cache after all of that layer's reads; the cache keeps
      the newest Lc rows.
  A12 LN before pw1.  A13 GLU = a * sigmoid(b), a = first D channels of pw1.  A14 no separate
      batch norm (folded into the depthwise bias).  A15 SiLU after the depthwise conv.
  A16 depthwise: d_t = b + sum_{k=0}^{K-1} w_k * g_{t-(K-1)+k}, zeros before position 0.
  A17 no input scaling, no dropout.  A18 each block ends with its own ln_out; no extra final LN.
  A19 joint projection z = x Wj + bj on emitted frames only.
  A21 front end: 1-D causal convs over time with mel bins as channels, kernel 3, stride 2,
      output t reading inputs 2t-2 .. 2t; ReLU after conv1 and conv2, conv3 linear.
  A22 mel tail of 14 frames (2 + 4 + 8 receptive field).  A23 the first chunk of a stream
      uses per-layer zero left padding of 2 (equal to the offline front end).
  A25 lookahead variant: key q is visible from query p iff max(0, p - Lc) <= q <= p + R and q
      lies inside the current pass.  A26 a pass computes n_emit + n_lookahead frames (2 + 8)
      and emits n_emit.  A27 only emitted frames enter the K/V and conv caches; the pending
      layer-0 inputs are kept and recomputed on the next pass; a flush runs one pass over the
      pending frames and emits all of them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import subsample2d

EPS = 1e-5


# ----------------------------------------------------------------------------- primitives

def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = EPS) -> np.ndarray:
    """LayerNorm over the last axis (reading A3)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def sigmoid(x: np.ndarray) -> np.ndarray:
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis; -inf entries get probability exactly 0."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def sinusoid_rows(rel, d_model: int) -> np.ndarray:
    """Sinusoidal encodings of relative positions ``rel`` (reading A7): [len(rel), D]."""
    rel = np.asarray(rel, dtype=np.float64)
    m = np.arange(d_model // 2, dtype=np.float64)
    inv_freq = 10000.0 ** (-2.0 * m / d_model)
    ang = rel[:, None] * inv_freq[None, :]
    pe = np.empty((rel.shape[0], d_model))
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


def relshift(bd: np.ndarray) -> np.ndarray:
    """The square shift trick of the offline position term (streaming spec, "Per-chunk flow",
    step 3, attention bullet, which names it as the offline formulation).

    ``bd[..., i, k]`` holds query i against the position row of relative offset T-1-k
    (2T-1 columns, offsets T-1 down to -(T-1)). Prepending one zero column, viewing the
    [T, 2T] block as [2T, T], dropping the first row and viewing the rest as [T, 2T-1] moves
    every row i left by T-1-i, so the first T columns give ``out[..., i, j] =
    bd[..., i, T-1-i+j]``, i.e. relative offset i - j.
    """
    *lead, T, W = bd.shape
    assert W == 2 * T - 1
    padded = np.concatenate([np.zeros((*lead, T, 1)), bd], axis=-1)
    shifted = padded.reshape(*lead, 2 * T, T)[..., 1:, :]
    return shifted.reshape(*lead, T, 2 * T - 1)[..., :T]


# ----------------------------------------------------------------------------- state

@dataclass
class StreamState:
    """Per-stream carried state (streaming spec, "State"): K/V caches of at most Lc rows per
    layer, the conv cache of the last dw_kernel-1 GLU outputs per layer, the mel tail, the
    stream position ``pos`` (subT: frames emitted so far) and, for the lookahead variant, the
    pending layer-0 inputs ``x0`` of positions pos, pos+1, ..."""
    pos: int
    k: list
    v: list
    conv: list
    mel_tail: np.ndarray | None = None
    x0: np.ndarray | None = None
    finished: bool = False

    def copy(self) -> "StreamState":
        cp = lambda a: None if a is None else a.copy()  # noqa: E731
        return StreamState(self.pos, [a.copy() for a in self.k], [a.copy() for a in self.v],
                           [a.copy() for a in self.conv], cp(self.mel_tail), cp(self.x0),
                           self.finished)


# ----------------------------------------------------------------------------- model

class Oracle:
    """The encoder of one workload configuration, in float64."""

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self.W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
        self.D, self.H, self.hd = cfg.d_model, cfg.n_heads, cfg.d_model // cfg.n_heads
        self.L, self.K, self.Lc, self.c = cfg.n_layers, cfg.dw_kernel, cfg.att_left, cfg.att_chunk
        self.lookahead = cfg.n_lookahead > 0

    # -- masks --------------------------------------------------------------------------
    def visible(self, p, q):
        """Key visibility on absolute positions: A9 (chunked-causal) or A25 (sliding window
        with right context, lookahead variant). Whether q exists at all (inside the sequence
        or the pass) is decided by which keys are offered."""
        p = np.asarray(p)
        q = np.asarray(q)
        if self.lookahead:
            return (q >= 0) & (q >= p - self.Lc) & (q <= p + self.cfg.att_right)
        cs = self.c * (p // self.c)
        return (q >= 0) & (q >= cs - self.Lc) & (q <= cs + self.c - 1)

    # -- sub-blocks ---------------------------------------------------------------------
    def _ln(self, x, pre):
        return layer_norm(x, self.W[pre + "ln_g"], self.W[pre + "ln_b"])

    def feed_forward(self, x, pre):
        """FF(x) = W2 SiLU(W1 LN(x) + b1) + b2 (streaming spec step 3, FF1/FF2; A2, A4)."""
        W = self.W
        h = silu(self._ln(x, pre) @ W[pre + "w1"] + W[pre + "b1"])
        return h @ W[pre + "w2"] + W[pre + "b2"]

    def qkv(self, y, l):
        """q, k, v of LN'd rows y: [T, H, hd] each (step 3, "xln@Wk/Wv")."""
        W, p, T = self.W, f"l{l}.att.", y.shape[0]
        split = lambda a: a.reshape(T, self.H, self.hd)  # noqa: E731
        return (split(y @ W[p + "wq"] + W[p + "bq"]), split(y @ W[p + "wk"] + W[p + "bk"]),
                split(y @ W[p + "wv"] + W[p + "bv"]))

    def pos_proj(self, l, rel):
        """Projected position rows PE(rel) @ Wpos split into heads: [len(rel), H, hd]."""
        P = sinusoid_rows(rel, self.D) @ self.W[f"l{l}.att.wpos"]
        return P.reshape(len(rel), self.H, self.hd)

    def mhsa_offline(self, y, l):
        """O1 attention over a whole sequence: the content term as a [T, T] product and the
        position term via the relative shift trick over a [T, 2T-1] table."""
        W, p, T = self.W, f"l{l}.att.", y.shape[0]
        q, k, v = self.qkv(y, l)
        u, vb = W[p + "pos_u"], W[p + "pos_v"]
        P = self.pos_proj(l, np.arange(T - 1, -T, -1))             # offsets T-1 .. -(T-1)
        ac = np.einsum("ihd,jhd->hij", q + u, k)
        bd = relshift(np.einsum("ihd,khd->hik", q + vb, P))
        s = (ac + bd) / np.sqrt(self.hd)
        pos = np.arange(T)
        vis = self.visible(pos[:, None], pos[None, :])
        s = np.where(vis[None], s, -np.inf)
        o = np.einsum("hij,jhd->ihd", softmax_rows(s), v).reshape(T, self.D)
        return o @ W[p + "wo"] + W[p + "bo"]

    def mhsa_stream(self, y, l, pos0, k_cache, v_cache):
        """O2 attention of one stream's n new rows at positions pos0.. against its cache
        (rows at positions pos0-fill .. pos0-1) plus the new rows: the rectangular
        n x (fill+n) score with the position row picked directly by rel = p - q (step 3,
        attention bullet; mask on absolute positions). Returns (out, k_new, v_new)."""
        W, p, n = self.W, f"l{l}.att.", y.shape[0]
        q, kn, vn = self.qkv(y, l)
        fill = k_cache.shape[0]
        keys = np.concatenate([k_cache.reshape(fill, self.H, self.hd), kn], axis=0)
        vals = np.concatenate([v_cache.reshape(fill, self.H, self.hd), vn], axis=0)
        qpos = pos0 + np.arange(n)
        kpos = np.arange(pos0 - fill, pos0 + n)
        rel = qpos[:, None] - kpos[None, :]
        vis = self.visible(qpos[:, None], kpos[None, :])
        rlo, rhi = int(rel[vis].min()), int(rel[vis].max())
        P = self.pos_proj(l, np.arange(rlo, rhi + 1))               # rows for rel = rlo..rhi
        Pg = P[np.clip(rel - rlo, 0, rhi - rlo)]                   # [n, nk, H, hd]
        u, vb = W[p + "pos_u"], W[p + "pos_v"]
        ac = np.einsum("ihd,jhd->hij", q + u, keys)
        bd = np.einsum("ihd,ijhd->hij", q + vb, Pg)
        s = np.where(vis[None], (ac + bd) / np.sqrt(self.hd), -np.inf)
        o = np.einsum("hij,jhd->ihd", softmax_rows(s), vals).reshape(n, self.D)
        return o @ W[p + "wo"] + W[p + "bo"], kn.reshape(n, self.D), vn.reshape(n, self.D)

    def glu_in(self, x, l):
        """LN -> pw1 -> GLU: the depthwise conv's input g (A12, A13)."""
        W, p = self.W, f"l{l}.conv."
        g2 = self._ln(x, p) @ W[p + "pw1"] + W[p + "pw1_b"]
        return g2[:, : self.D] * sigmoid(g2[:, self.D:])

    def conv_tail(self, gseq, l, n_out):
        """Depthwise k-tap causal conv over gseq (the last n_out rows are the outputs' own
        positions; gseq carries K-1 earlier rows in front), then SiLU, pw2 (A15, A16)."""
        W, p, K = self.W, f"l{l}.conv.", self.K
        assert gseq.shape[0] == n_out + K - 1
        d = np.tile(W[p + "dw_b"], (n_out, 1))
        for kk in range(K):
            d = d + gseq[kk: kk + n_out] * W[p + "dw"][:, kk]
        return silu(d) @ W[p + "pw2"] + W[p + "pw2_b"]

    def conv_offline(self, x, l):
        g = self.glu_in(x, l)
        gseq = np.concatenate([np.zeros((self.K - 1, self.D)), g], axis=0)
        return self.conv_tail(gseq, l, x.shape[0])

    # -- O1: offline -------------------------------------------------------------------
    def layer_offline(self, x, l):
        pre = f"l{l}."
        x = x + 0.5 * self.feed_forward(x, pre + "ff1.")
        x = x + self.mhsa_offline(self._ln(x, pre + "att."), l)
        x = x + self.conv_offline(x, l)
        x = x + 0.5 * self.feed_forward(x, pre + "ff2.")
        return self._ln(x, pre + "out.")

    def joint(self, x):
        if not self.cfg.joint_dim:
            return x
        return x @ self.W["joint.w"] + self.W["joint.b"]

    def encode_offline(self, x, return_hidden=False):
        """O1: the whole sequence x [T, D] under the mask, all frames at once."""
        for l in range(self.L):
            x = self.layer_offline(x, l)
        return (self.joint(x), x) if return_hidden else self.joint(x)

    # -- front end -----------------------------------------------------------------------
    def _fe_layers(self):
        W = self.W
        return [(W["fe.c1.w"], W["fe.c1.b"], True), (W["fe.c2.w"], W["fe.c2.b"], True),
                (W["fe.c3.w"], W["fe.c3.b"], False)]

    @staticmethod
    def conv_s2(x, w, b, left_pad):
        """Stride-2, kernel-3 conv over time. With left_pad=2 this is the causal conv (output
        t reads inputs 2t-2..2t, zeros before the start); with left_pad=0 it is the valid
        conv (output j reads inputs 2j..2j+2). w: [C_out, C_in, 3]."""
        if left_pad:
            x = np.concatenate([np.zeros((left_pad, x.shape[1])), x], axis=0)
        n_out = (x.shape[0] - 3) // 2 + 1
        out = np.tile(b, (n_out, 1))
        for kk in range(3):
            out = out + x[kk: kk + 2 * n_out - 1: 2] @ w[:, :, kk].T
        return out

    def frontend_offline(self, mel):
        """Offline subsampling of a whole mel sequence [16C, B] -> [2C, D] (A21; the 2-D variant
        in ``subsample2d`` when cfg.frontend == 2)."""
        if self.cfg.frontend == 2:
            return subsample2d.offline(self.W, mel)
        x = mel
        for w, b, relu in self._fe_layers():
            x = self.conv_s2(x, w, b, left_pad=2)
            if relu:
                x = np.maximum(x, 0.0)
        return x

    def frontend_stream(self, st: StreamState, mel_new):
        """Streaming subsampling (step 2; "State", melTail): the first chunk of a stream uses
        the causal pads; later chunks run valid convs over [melTail || new] (14+16 -> 14 -> 6
        -> 2 frames). melTail becomes the last 14 mel frames seen."""
        if self.cfg.frontend == 2:
            x = subsample2d.stream(self.W, st.mel_tail, mel_new, st.pos)
        elif st.pos == 0:
            x = self.frontend_offline(mel_new)
        else:
            x = np.concatenate([st.mel_tail, mel_new], axis=0)
            for w, b, relu in self._fe_layers():
                x = self.conv_s2(x, w, b, left_pad=0)
                if relu:
                    x = np.maximum(x, 0.0)
        st.mel_tail = np.concatenate([st.mel_tail, mel_new], axis=0)[-self.cfg.mel_tail:]
        return x

    def frontend_stream_tails(self, tails: list, mel_new):
        """Alternative streaming subsampling with a 2-frame input tail per conv layer (zero at
        stream start), the equivalent form of A23. Updates ``tails`` in place."""
        x = mel_new
        for i, (w, b, relu) in enumerate(self._fe_layers()):
            win = np.concatenate([tails[i], x], axis=0)
            tails[i] = win[-2:].copy()
            x = self.conv_s2(win, w, b, left_pad=0)
            if relu:
                x = np.maximum(x, 0.0)
        return x

    # -- O2 / O3: streaming ----------------------------------------------------------------
    def new_state(self) -> StreamState:
        D, L = self.D, self.L
        return StreamState(
            pos=0, k=[np.zeros((0, D)) for _ in range(L)], v=[np.zeros((0, D)) for _ in range(L)],
            conv=[np.zeros((self.K - 1, D)) for _ in range(L)],
            mel_tail=np.zeros((self.cfg.mel_tail, self.cfg.mel_bins)) if self.cfg.frontend else None,
            x0=np.zeros((0, D)) if self.lookahead else None)

    def state_from(self, st: dict) -> StreamState:
        """Adopt an injected state in the layout of ``synth.make_state``."""
        fill, Lc = st["fill"], self.Lc
        f64 = lambda a: None if a is None else np.asarray(a, dtype=np.float64).copy()  # noqa: E731
        return StreamState(
            pos=int(st["pos"]),
            k=[f64(st["k"][l, Lc - fill:]) for l in range(self.L)],
            v=[f64(st["v"][l, Lc - fill:]) for l in range(self.L)],
            conv=[f64(st["conv"][l]) for l in range(self.L)],
            mel_tail=f64(st["mel_tail"]), x0=f64(st["x0_tail"]))

    def _layers_stream(self, states, xs, n_keep):
        """Run all layers over a batch of streams, each with the same number n of new rows
        (xs: [S, n, D]) at positions st.pos .. st.pos+n-1. Dense products run on the stacked
        rows of all streams; attention and the depthwise conv run per stream. Each layer's
        caches take the first n_keep rows after that layer's reads (A11, A27)."""
        S, n, D = xs.shape
        x = xs.reshape(S * n, D)
        for l in range(self.L):
            pre = f"l{l}."
            x = x + 0.5 * self.feed_forward(x, pre + "ff1.")
            y = self._ln(x, pre + "att.")
            att = np.empty_like(x)
            new_kv = []
            for s, st in enumerate(states):
                rows = slice(s * n, (s + 1) * n)
                att[rows], kn, vn = self.mhsa_stream(y[rows], l, st.pos, st.k[l], st.v[l])
                new_kv.append((kn, vn))
            x = x + att
            g = self.glu_in(x, l)
            conv = np.empty_like(x)
            for s, st in enumerate(states):
                rows = slice(s * n, (s + 1) * n)
                gseq = np.concatenate([st.conv[l], g[rows]], axis=0)
                conv[rows] = self.conv_tail(gseq, l, n)
                st.conv[l] = np.concatenate([st.conv[l], g[rows][:n_keep]], axis=0)[-(self.K - 1):]
                kn, vn = new_kv[s]
                st.k[l] = np.concatenate([st.k[l], kn[:n_keep]], axis=0)[-self.Lc:]
                st.v[l] = np.concatenate([st.v[l], vn[:n_keep]], axis=0)[-self.Lc:]
            x = x + conv
            x = x + 0.5 * self.feed_forward(x, pre + "ff2.")
            x = self._ln(x, pre + "out.")
        return x.reshape(S, n, D)

    def push(self, states, inputs):
        """O2 chunk step for a batch of streams (streaming spec "Per-chunk flow", steps 2-4).
        inputs: [S, n, D] subsampled frames, or [S, 16, B] mel frames with the front end.
        Returns z: [S, n, P] (or the hidden rows when there is no joint)."""
        if self.lookahead:
            return self.push_lookahead(states, inputs)
        inputs = np.asarray(inputs, dtype=np.float64)
        if self.cfg.frontend:
            xs = np.stack([self.frontend_stream(st, inputs[s]) for s, st in enumerate(states)])
        else:
            xs = inputs
        n = xs.shape[1]
        assert n % self.c == 0, "pushes must align to the attention chunk grid"
        for st in states:
            assert not st.finished
        out = self._layers_stream(states, xs, n_keep=n)
        for st in states:
            st.pos += n
        return self.joint(out)

    def push_lookahead(self, states, inputs):
        """O3 (streaming spec "Status", provisional tail): append the new frames to the pending
        layer-0 inputs; once n_emit + n_lookahead are pending, run one pass over them, emit
        the first n_emit, cache only those, and keep the rest pending. Returns z [S, m, P]
        where m is 0 (warm-up) or n_emit; all streams of one call are in the same phase."""
        inputs = np.asarray(inputs, dtype=np.float64)
        ne, nc = self.cfg.n_emit, self.cfg.n_compute
        for s, st in enumerate(states):
            assert not st.finished
            st.x0 = np.concatenate([st.x0, inputs[s]], axis=0)
        ready = [st.x0.shape[0] >= nc for st in states]
        assert all(ready) or not any(ready), "mixed warm-up phases in one oracle call"
        if not ready[0]:
            return np.zeros((len(states), 0, self.cfg.joint_dim or self.D))
        xs = np.stack([st.x0[:nc] for st in states])
        out = self._layers_stream(states, xs, n_keep=ne)
        for st in states:
            st.pos += ne
            st.x0 = st.x0[ne:]
        return self.joint(out[:, :ne])

    def flush(self, st: StreamState):
        """End of stream: the lookahead variant runs one pass over its pending frames and emits
        all of them; with whole chunks the other variants have nothing left to emit."""
        st.finished = True
        if not self.lookahead or st.x0.shape[0] == 0:
            return np.zeros((0, self.cfg.joint_dim or self.D))
        m = st.x0.shape[0]
        out = self._layers_stream([st], st.x0[None], n_keep=m)[0]
        st.pos += m
        st.x0 = st.x0[m:]
        return self.joint(out)
