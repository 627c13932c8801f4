"""Pins of the oracle parts the encoder gate does not reach: the encoder-side joint projection,
the check-only greedy token head and its ambiguity bound, and the adoption of an injected
stream state (``Oracle.state_from``), each against something other than the oracle itself:
torch's linear layer, hand-built logit tables, an exhaustive search over perturbations, and
an uninterrupted run of the same stream."""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import Oracle
from oracle.tokens import ambiguous_frames, greedy_tokens, logits
from synth import C1, C2, make_weights
from synth.configs import EncConfig


def tiny(**kw):
    base = dict(name="tiny", seed=21, n_layers=2, d_model=8, n_heads=2, d_ff=16, joint_dim=6,
                dtype="f32", chunks=12, att_left=6)
    base.update(kw)
    return EncConfig(**base)


# ----------------------------------------------------------------------- joint projection

def test_joint_matches_torch_linear():
    """z = x Wj + bj ("Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon", "Delete
    Repeated Projection Work First": the encoder side of the joint is one linear map per
    frame; reading A19) against torch.nn.functional.linear in float64, on the workload's
    512 -> 640 weights."""
    orc = Oracle(C2, make_weights(C2))
    x = np.random.default_rng(3).standard_normal((37, 512)) * 2.0
    ref = F.linear(torch.from_numpy(x), torch.from_numpy(orc.W["joint.w"]).T.contiguous(),
                   torch.from_numpy(orc.W["joint.b"])).numpy()
    z = orc.joint(x)
    assert z.shape == (37, 640)
    assert np.abs(z - ref).max() < 1e-12
    # one frame at a time gives the same rows (the projection is per frame, no mixing)
    assert np.abs(np.stack([orc.joint(x[i:i + 1])[0] for i in range(37)]) - z).max() < 1e-12


def test_joint_absent_returns_hidden_rows():
    """A workload without a joint (joint_dim 0, the tiny encoder) hands out the hidden rows."""
    orc = Oracle(C1, make_weights(C1))
    x = np.random.default_rng(4).standard_normal((5, C1.d_model))
    assert orc.joint(x) is x


# ----------------------------------------------------------------------- greedy token head

def _head(p0, wout, bout):
    return {"p0": np.asarray(p0, np.float64), "wout": np.asarray(wout, np.float64),
            "bout": np.asarray(bout, np.float64)}


def test_greedy_tokens_hand_built_table():
    """Hand-computed logits ReLU(z + p0) Wout + bout, argmax with ties to the lowest index,
    and the top-1 minus top-2 margin (reading A20)."""
    wout = [[1, 0, 0, 1],
            [0, 1, 0, 0],
            [0, 0, 1, 0]]
    head = _head([10.0, 10.0, 10.0], wout, [0.0, 0.0, 0.0, 0.0])
    z = np.array([[1.0, 1.0, 0.0],    # logits 11 11 10 11: a three-way tie -> class 0
                  [0.0, 3.0, 1.0],    # 10 13 11 10 -> class 1, margin 2
                  [-1.0, 0.0, 4.5],   # 9 10 14.5 9 -> class 2, margin 4.5
                  [2.0, 2.0, 2.0]])   # 12 12 12 12 -> class 0, margin 0
    tok, margin = greedy_tokens(z, head)
    assert tok.tolist() == [0, 1, 2, 0]
    assert np.allclose(margin, [0.0, 2.0, 4.5, 0.0], atol=0, rtol=0)
    # the ReLU clips negative pre-activations: p0 = 0, z = (-5, 2, 0) -> (0, 2, 0)
    head2 = _head([0.0, 0.0, 0.0], wout, [0.5, 0.0, 0.0, 0.25])
    tok2, margin2 = greedy_tokens(np.array([[-5.0, 2.0, 0.0]]), head2)
    # logits 0.5, 2, 0, 0.25 -> class 1, margin 1.5
    assert tok2.tolist() == [1] and margin2[0] == 1.5


def test_greedy_tokens_tie_goes_to_lowest_index_among_equal_logits():
    """Ties at the top go to the lowest class index wherever they sit."""
    C = 7
    for top in itertools.combinations(range(C), 2):
        wout = np.zeros((1, C))
        bout = np.zeros(C)
        bout[list(top)] = 3.0
        tok, margin = greedy_tokens(np.zeros((1, 1)), _head([0.0], wout, bout))
        assert tok[0] == min(top) and margin[0] == 0.0


def test_logits_match_scalar_loops():
    rng = np.random.default_rng(5)
    P, C = 5, 9
    head = _head(rng.standard_normal(P), rng.standard_normal((P, C)), rng.standard_normal(C))
    z = rng.standard_normal((4, P))
    ref = np.zeros((4, C))
    for f in range(4):
        for c in range(C):
            s = float(head["bout"][c])
            for i in range(P):
                s += max(float(z[f, i] + head["p0"][i]), 0.0) * float(head["wout"][i, c])
            ref[f, c] = s
    assert np.abs(logits(z, head) - ref).max() < 1e-12


def test_ambiguity_bound_exhaustive_on_tiny_heads():
    """Frames the bound leaves unflagged keep their argmax under every perturbation dz with
    |dz|_inf no larger than the one measured. Each logit difference is a sum of monotone
    functions of single coordinates (ReLU per coordinate), so its extremes over the box sit at
    its corners: enumerating the 2^P sign patterns is an exhaustive search. The bound must also
    not be vacuous: some flagged frames really flip at a corner."""
    rng = np.random.default_rng(6)
    P, C, nf = 3, 5, 400
    flips_flagged = unflagged = 0
    corners = np.array(list(itertools.product([-1.0, 1.0], repeat=P)))
    for trial in range(6):
        head = _head(rng.standard_normal(P) * 0.3, rng.standard_normal((P, C)), rng.standard_normal(C) * 0.2)
        z = rng.standard_normal((nf, P))
        eps = [0.01, 0.03, 0.1][trial % 3]
        z_test = z + eps * corners[rng.integers(0, len(corners), nf)]
        amb = ambiguous_frames(z, z_test, head)
        tok, _ = greedy_tokens(z, head)
        for f in range(nf):
            moved = np.argmax(logits(z[f] + eps * corners, head), axis=-1)
            if amb[f]:
                flips_flagged += int(np.any(moved != tok[f]))
            else:
                unflagged += 1
                assert np.all(moved == tok[f]), (trial, f)
    assert unflagged > 1000
    assert flips_flagged > 0


def test_ambiguity_bound_flags_nothing_for_identical_outputs():
    rng = np.random.default_rng(7)
    head = _head(rng.standard_normal(4), rng.standard_normal((4, 6)), rng.standard_normal(6))
    z = rng.standard_normal((50, 4))
    assert not ambiguous_frames(z, z.copy(), head).any()


# ----------------------------------------------------------------------- injected states

def to_synth_layout(orc: Oracle, st, cfg) -> dict:
    """Write an oracle stream state in the layout ``synth.make_state`` documents, from the
    positions alone: K/V row r holds position pos - Lc + r, conv column j holds position
    pos - (K-1) + j, zeros for positions before 0."""
    L, Lc, D, Kc, pos = cfg.n_layers, cfg.att_left, cfg.d_model, cfg.dw_kernel - 1, st.pos
    k = np.zeros((L, Lc, D))
    v = np.zeros((L, Lc, D))
    for l in range(L):
        fill = st.k[l].shape[0]
        first = pos - fill                      # position of st.k[l][0]
        for r in range(Lc):
            p = pos - Lc + r
            if p >= 0 and p >= first:
                k[l, r] = st.k[l][p - first]
                v[l, r] = st.v[l][p - first]
    conv = np.zeros((L, Kc, D))
    for l in range(L):
        for j in range(Kc):
            if pos - Kc + j >= 0:
                conv[l, j] = st.conv[l][j]
    d = {"pos": pos, "fill": min(pos, Lc), "k": k, "v": v, "conv": conv,
         "mel_tail": None if st.mel_tail is None else st.mel_tail.copy(),
         "x0_tail": None if st.x0 is None else st.x0.copy()}
    return d


@pytest.mark.parametrize("cfg,cut", [
    (tiny(), 2),                                    # fill 4 < Lc 6
    (tiny(), 3),                                    # fill 6 = Lc, first wrap next chunk
    (tiny(), 9),                                    # ring wrapped several times
    (tiny(att_left=5, att_chunk=1, n_emit=1), 4),   # fill 4 < 5 with chunk 1
    (tiny(d_model=16, frontend=True, mel_bins=8), 4),
    (tiny(att_right=2, n_emit=2, n_lookahead=4), 6),
], ids=["partial-fill", "full", "wrapped", "chunk1", "frontend", "lookahead"])
def test_state_from_resumes_a_stream_exactly(cfg, cut):
    """Run a stream ``cut`` pushes, write its state in the injected-state layout, adopt that
    with ``state_from`` and continue: the outputs equal the uninterrupted run bit for bit."""
    orc = Oracle(cfg, make_weights(cfg))
    rng = np.random.default_rng(8)
    width = (cfg.mel_per_chunk, cfg.mel_bins) if cfg.frontend else (cfg.n_emit, cfg.d_model)
    xs = rng.standard_normal((cut + 6, *width))
    st = orc.new_state()
    for c in range(cut):
        orc.push([st], xs[c][None])
    st2 = orc.state_from(to_synth_layout(orc, st, cfg))
    assert st2.pos == st.pos
    for c in range(cut, cut + 6):
        a = orc.push([st], xs[c][None])
        b = orc.push([st2], xs[c][None])
        assert np.array_equal(a, b), c
    if cfg.n_lookahead:
        assert np.array_equal(orc.flush(st), orc.flush(st2))


def test_state_from_reads_rows_by_position():
    """A planted layout mistake (K/V rows in reverse order) changes the continuation, so the
    round trip above would catch a wrong row order in ``state_from``."""
    cfg = tiny()
    orc = Oracle(cfg, make_weights(cfg))
    xs = np.random.default_rng(9).standard_normal((8, cfg.n_emit, cfg.d_model))
    st = orc.new_state()
    for c in range(5):
        orc.push([st], xs[c][None])
    d = to_synth_layout(orc, st, cfg)
    bad = dict(d, k=d["k"][:, ::-1].copy())
    a = orc.push([orc.state_from(d)], xs[5][None])
    b = orc.push([orc.state_from(bad)], xs[5][None])
    assert not np.allclose(a, b)
