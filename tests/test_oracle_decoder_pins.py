"""Pins of the greedy RNNT + EOU decoding oracle (oracle/decoder.py) against things other than
itself: torch's LSTM and linear layers, the unsplit joint, hand-made toy scorers whose greedy
transcripts are worked out by hand, and one-call decoding against chunked decoding with the
state carried between calls."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.decoder import GreedyDecoder, greedy_loop
from synth import D1, make_dec_inputs, make_dec_weights


def small(**kw):
    base = dict(name="dec_small", seed=31, joint_dim=12, pred_hidden=10, pred_layers=2, vocab=5, max_symbols=3,
                blank_bias=0.0, frames=2, calls=20)
    base.update(kw)
    return D1.replace(**base)


def T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------------- prediction network

@pytest.mark.parametrize("layers", [1, 2, 3])
def test_lstm_steps_match_torch_lstm(layers):
    """A sequence of predictor steps equals torch.nn.LSTM (gate order i, f, g, o, both biases)
    over the embedded tokens, layer by layer (reading D2)."""
    cfg = small(pred_layers=layers)
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    W, H = dec.W, cfg.pred_hidden
    lstm = torch.nn.LSTM(H, H, num_layers=layers, dtype=torch.float64)
    with torch.no_grad():
        for l in range(layers):
            getattr(lstm, f"weight_ih_l{l}").copy_(T(W[f"pred.l{l}.w_ih"]).T)
            getattr(lstm, f"weight_hh_l{l}").copy_(T(W[f"pred.l{l}.w_hh"]).T)
            getattr(lstm, f"bias_ih_l{l}").copy_(T(W[f"pred.l{l}.b_ih"]))
            getattr(lstm, f"bias_hh_l{l}").copy_(T(W[f"pred.l{l}.b_hh"]))
    toks = [cfg.vocab, 3, 0, cfg.vocab + 1, 4, 4]            # blank start, tokens, EOU, a repeat
    st = dec.new_state()
    hs = []
    for k in toks:
        st.h, st.c = dec.lstm_step(k, st.h, st.c)
        hs.append(st.h[-1].copy())
    with torch.no_grad():
        ref, (hn, cn) = lstm(T(W["pred.embed"][toks])[:, None, :])
    assert np.abs(np.stack(hs) - ref[:, 0].numpy()).max() < 1e-13
    assert np.abs(st.h - hn[:, 0].numpy()).max() < 1e-13
    assert np.abs(st.c - cn[:, 0].numpy()).max() < 1e-13


def test_joint_after_projection_matches_torch_and_the_unsplit_joint():
    """ReLU(z + p) Wout + bout, with the encoder frame projected once and the predictor output
    projected once per update, equals the joint computed from the unprojected inputs inside one
    wrapper ("Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon", §3.1 and §3.2: the
    split is exact at the algorithm level)."""
    cfg = small()
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    rng = np.random.default_rng(2)
    enc = rng.standard_normal((7, 9))            # unprojected encoder rows (width 9)
    we, be = rng.standard_normal((9, cfg.joint_dim)), rng.standard_normal(cfg.joint_dim)
    g = rng.standard_normal((3, cfg.pred_hidden))   # predictor outputs
    W = dec.W
    # unsplit: project both inside the joint for every (frame, predictor output) pair
    x = (F.linear(T(enc), T(we).T, T(be))[:, None, :]
         + F.linear(T(g), T(W["pred.proj_w"]).T, T(W["pred.proj_b"]))[None, :, :])
    ref = F.linear(torch.relu(x), T(W["joint.out_w"]).T, T(W["joint.out_b"])).numpy()
    z = enc @ we + be
    p = np.stack([dec.pred_project(gi) for gi in g])
    got = np.stack([[dec.joint(z[t], p[j]) for j in range(3)] for t in range(7)])
    assert got.shape == (7, 3, cfg.vocab + 2)
    assert np.abs(got - ref).max() < 1e-12


# ----------------------------------------------------------------------- the state machine

def _toy(table, default_blank, C):
    """A toy scorer: scores(t, prefix) from a table, else a one-hot on blank."""
    prefix = []

    def score(t):
        s = np.zeros(C)
        s[table.get((t, tuple(prefix)), default_blank)] = 1.0
        return s

    def advance(k):
        prefix.append(k)

    return score, advance, prefix


def test_greedy_loop_on_toy_scorers():
    """Hand-worked transcripts: several labels at one frame, blank advancing time, an EOU
    emission, and the max-symbols cap moving on while the scorer would keep emitting."""
    V, blank, eou, C = 5, 5, 6, 7
    table = {(0, ()): 2, (0, (2,)): 4, (0, (2, 4)): blank,
             (1, (2, 4)): blank,
             (2, (2, 4)): eou, (2, (2, 4, eou)): 1, (2, (2, 4, eou, 1)): blank,
             (3, (2, 4, eou, 1)): 3}
    score, advance, prefix = _toy(table, blank, C)
    out = greedy_loop(5, score, advance, blank, max_symbols=3)
    assert out == [(0, 2), (0, 4), (2, eou), (2, 1), (3, 3)]
    assert prefix == [2, 4, eou, 1, 3]
    # a scorer that never gives blank at frame 0: three labels, then the cap moves on
    score, advance, prefix = _toy({(0, ()): 1, (0, (1,)): 1, (0, (1, 1)): 2, (0, (1, 1, 2)): 3}, blank, C)
    assert greedy_loop(2, score, advance, blank, max_symbols=3) == [(0, 1), (0, 1), (0, 2)]
    assert greedy_loop(0, score, advance, blank, max_symbols=3) == []


def test_greedy_ties_go_to_the_lowest_class():
    blank = 3
    calls = []

    def score(t):
        calls.append(t)
        return np.array([0.0, 2.0, 2.0, 2.0]) if len(calls) == 1 else np.array([0.0, 0.0, 0.0, 1.0])

    assert greedy_loop(1, score, lambda k: None, blank, max_symbols=4) == [(0, 1)]
    # a tie between a label and blank goes to the label when its index is lower
    assert greedy_loop(1, lambda t: np.array([1.0, 0.0, 0.0, 1.0]), lambda k: None, blank, max_symbols=2) == [(0, 0), (0, 0)]


def test_decoder_first_joint_uses_the_blank_prediction():
    """A fresh stream's first joint sees the predictor run once on the blank token from zero
    state; nothing runs on blank afterwards."""
    cfg = small()
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    z = make_dec_inputs(cfg, 0, 1)[0]
    st = dec.new_state()
    dec.decode(st, z[:0])            # no frames: nothing consumed
    assert st.pending == cfg.vocab and st.p is None
    h, c = dec.lstm_step(cfg.vocab, np.zeros((2, cfg.pred_hidden)), np.zeros((2, cfg.pred_hidden)))
    p0 = dec.pred_project(h[-1])
    st2 = dec.new_state()
    toks = dec.decode(st2, z[:1])
    first = dec.joint(z[0], p0)
    assert (int(np.argmax(first)) == cfg.vocab) == (len(toks) == 0 or toks[0][0] > 0)
    if not toks:
        assert np.array_equal(st2.p, p0) and st2.pending is None


@pytest.mark.parametrize("chunk", [1, 2, 5])
def test_chunked_decoding_with_state_carry_equals_one_call(chunk):
    """Decoding a stream in calls of ``chunk`` frames with the state carried between calls
    ("True streaming encode — implementation spec", "Decoder state carry": no reset and no
    re-prediction from blank between calls) gives the transcript of one call over all frames."""
    cfg = small(calls=30, frames=2)
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    z = make_dec_inputs(cfg, 0).reshape(-1, cfg.joint_dim)
    one = dec.decode(dec.new_state(), z)
    st = dec.new_state()
    parts = []
    for t0 in range(0, z.shape[0], chunk):
        parts += [(t0 + t, k) for t, k in dec.decode(st, z[t0:t0 + chunk])]
    assert parts == one
    assert len(one) > 5


def test_workload_decoder_emits_labels_and_blanks():
    """The 640-wide two-layer workload decoder emits both blanks and labels on its synthetic
    frames (the raised blank bias keeps most frames blank), and hits the per-frame cap."""
    cfg = D1.replace(calls=40)
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    st = dec.new_state()
    xs = make_dec_inputs(cfg, 0)
    toks = []
    for c in range(40):
        toks += [(2 * c + t, k) for t, k in dec.decode(st, xs[c])]
    frames_with = {t for t, _ in toks}
    assert 0 < len(frames_with) < 80
    assert max(sum(1 for t, _ in toks if t == f) for f in frames_with) <= cfg.max_symbols
