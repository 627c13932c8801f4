"""Brute-force relative-position attention with plain Python loops (tiny shapes only).

TEST INFRASTRUCTURE ONLY. An independent restatement of one head-summed attention block from
the streaming spec ("Per-chunk flow", step 3: score[i,j] = (q_i + pbu).k_j + (q_i + pbv).p[rel]),
with readings A5-A7 and A9/A25 for the mask. Every dot product, sine, exponential and sum is a
scalar loop; nothing is shared with ``encoder.py``.
"""
from __future__ import annotations

import math


def _matvec(x, w, b):
    """x [n_in], w [n_in][n_out] (nested lists), b [n_out] -> x @ w + b."""
    return [b[j] + sum(x[i] * w[i][j] for i in range(len(x))) for j in range(len(b))]


def _pe(r, d_model):
    out = []
    for m in range(d_model // 2):
        ang = r * math.pow(10000.0, -2.0 * m / d_model)
        out += [math.sin(ang), math.cos(ang)]
    return out


def attention_brute(y, pos, W, prefix, n_heads, vis):
    """y: list of T LN'd rows (lists of D floats) at absolute positions ``pos``; W: dict of
    nested-list weights; vis(p, q) -> bool. Returns the attention block output (after Wo)
    for every row, as lists."""
    T, D = len(y), len(y[0])
    hd = D // n_heads
    g = lambda k: W[prefix + k]  # noqa: E731
    q = [_matvec(r, g("wq"), g("bq")) for r in y]
    k = [_matvec(r, g("wk"), g("bk")) for r in y]
    v = [_matvec(r, g("wv"), g("bv")) for r in y]
    zero = [0.0] * D
    out = []
    for i in range(T):
        o = [0.0] * D
        for h in range(n_heads):
            lo = h * hd
            scores = []
            for j in range(T):
                if not vis(pos[i], pos[j]):
                    scores.append(None)
                    continue
                p_row = _matvec(_pe(pos[i] - pos[j], D), g("wpos"), zero)
                s = 0.0
                for d in range(hd):
                    s += (q[i][lo + d] + g("pos_u")[h][d]) * k[j][lo + d]
                    s += (q[i][lo + d] + g("pos_v")[h][d]) * p_row[lo + d]
                scores.append(s / math.sqrt(hd))
            m = max(s for s in scores if s is not None)
            ex = [0.0 if s is None else math.exp(s - m) for s in scores]
            tot = sum(ex)
            for j in range(T):
                for d in range(hd):
                    o[lo + d] += ex[j] / tot * v[j][lo + d]
        out.append(_matvec(o, g("wo"), g("bo")))
    return out
