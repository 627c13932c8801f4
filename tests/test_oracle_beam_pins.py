"""Pins of the MALSD beam-search oracle (oracle/beam.py).

- With a beam wide enough that nothing is ever pruned and a label cap that never binds, the
  final beam holds every transcript with the log of its total probability over all of its
  alignments: checked against brute-force enumeration of the alignments.
- Beam 1 is greedy decoding with the same label cap: checked against the greedy state machine
  of oracle/decoder.py on a small model.
- Hand-built toy scorers for each fixture "Fast Accuracy-Preserving RNNT Beam Search on Apple
  Silicon" lists in §2.5 (blank/label ties, two alignments reaching one transcript,
  recombination after pruning, max-symbol blank forcing, an inactive final hypothesis kept in
  slot zero, normalisation changing the winner, transcripts a weak hash would confuse), each
  with its expected beam worked out by hand in the test.
"""
import itertools
import math

import numpy as np
import pytest

from oracle.beam import BeamTrace, ToyScorer, beam_decode, best, log_softmax, logsumexp, malsd, ranked
from oracle.decoder import GreedyDecoder
from synth.configs import DecConfig
from synth.gen import make_dec_weights

L = math.log


def live(slots):
    return {h.prefix: h.score for h in slots if h.live}


# -- brute force over alignments -------------------------------------------------------------
def all_alignments(scorer, T, blank, n_labels, max_symbols, max_len):
    """Every alignment of up to max_len labels over T frames (each frame: up to max_symbols
    labels, then blank), as (transcript, log-probability)."""
    out = []

    def walk(t, prefix, n_sym, lp):
        if t == T:
            out.append((prefix, lp))
            return
        row = scorer(t, prefix)
        walk(t + 1, prefix, 0, lp + row[blank])
        if n_sym < max_symbols and len(prefix) < max_len:
            for c in range(n_labels):
                if row[c] > -math.inf:
                    walk(t, prefix + (c,), n_sym + 1, lp + row[c])

    walk(0, (), 0, 0.0)
    return out


def random_toy(rng, T, n_labels, max_len):
    """Normalised random log-probabilities per (frame, prefix); labels impossible once the
    prefix holds max_len labels."""
    table = {}
    for t in range(T):
        for u in range(max_len + 1):
            for prefix in itertools.product(range(n_labels), repeat=u):
                x = rng.standard_normal(n_labels + 1)
                if u == max_len:
                    x[:n_labels] = -np.inf
                table[(t, prefix)] = log_softmax(x) if u < max_len else np.where(np.isinf(x), -np.inf, 0.0)
    return ToyScorer(table, np.zeros(n_labels + 1))


@pytest.mark.parametrize("T,n_labels,max_len,seed", [(3, 2, 2, 0), (4, 2, 2, 1), (2, 3, 3, 2), (5, 1, 4, 3)])
def test_wide_beam_equals_the_sum_over_all_alignments(T, n_labels, max_len, seed):
    scorer = random_toy(np.random.default_rng(seed), T, n_labels, max_len)
    blank = n_labels
    tr = BeamTrace()
    slots = malsd(scorer, T, beam=256, max_symbols=max_len + 1, blank=blank, trace=tr)
    assert tr.max_candidates <= 256                     # nothing was ever pruned
    totals = {}
    for prefix, lp in all_alignments(scorer, T, blank, n_labels, max_len + 1, max_len):
        totals.setdefault(prefix, []).append(lp)
    expect = {p: logsumexp(v) for p, v in totals.items()}
    got = live(slots)
    assert set(got) == set(expect)
    for p in expect:
        assert abs(got[p] - expect[p]) < 1e-12, p
    # the probabilities of all transcripts sum to one (every alignment ends in a final blank)
    assert abs(logsumexp(list(got.values()))) < 1e-12
    assert all(h.t == T for h in slots if h.live)


def test_a_planted_merge_before_prune_fails_the_fixture():
    """Merging equal transcripts before the pruning (the order the pages warn against) keeps a
    different beam on the recombination-after-pruning fixture."""
    scorer, T = _two_alignment_scorer()

    def merge_first(log_probs, n_frames, K, m, blank):
        beam = [(0.0, 0, (), 0)]
        while any(t < n_frames for _, t, _, _ in beam):
            cand = {}
            for s, t, p, n in beam:
                if t >= n_frames:
                    opts = [(s, t, p, n)]
                else:
                    lp = log_probs(t, p)
                    opts = [(s + lp[blank], t + 1, p, 0)]
                    if n < m:
                        opts += [(s + lp[c], t, p + (c,), n + 1) for c in range(len(lp)) if c != blank]
                for o in opts:
                    cand.setdefault(o[2], []).append(o)
            merged = []
            for p, os in cand.items():
                top = max(os, key=lambda o: o[0])
                merged.append((logsumexp([o[0] for o in os]), top[1], p, top[3]))
            beam = sorted(merged, key=lambda o: -o[0])[:K]
        return {p: s for s, _, p, _ in beam}

    other = merge_first(scorer, T, 2, 1, 1)
    ours = live(malsd(scorer, T, beam=2, max_symbols=1, blank=1))
    assert () in other and () not in ours


# -- beam 1 is greedy -------------------------------------------------------------------------
@pytest.mark.parametrize("blank_bias,seed", [(0.0, 1), (1.0, 2), (2.0, 3), (3.0, 4)])
def test_beam_one_is_greedy_with_the_same_label_cap(blank_bias, seed):
    cfg = DecConfig(name="tiny", seed=seed, joint_dim=64, pred_hidden=64, vocab=30, max_symbols=3,
                    blank_bias=blank_bias)
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    z = np.random.default_rng(seed).standard_normal((12, 64))
    greedy = [k for _, k in dec.decode(dec.new_state(), z)]
    slots = beam_decode(dec, z, 12, beam=1, max_symbols=3)
    assert list(slots[0].prefix) == greedy
    assert slots[0].t == 12


# -- toy fixtures -----------------------------------------------------------------------------
def test_blank_loses_a_tie_against_a_label():
    # classes: labels 0, 1, blank 2; label 1 and blank tie for the second place of a 2-beam
    s = ToyScorer({(0, ()): [L(.5), L(.25), L(.25)]}, [L(.2), L(.2), L(.6)])
    tr = BeamTrace()
    malsd(s, 1, beam=2, max_symbols=1, blank=2, trace=tr, keep_beams=True)
    first = tr.beams[0]
    assert [h.prefix for h in first] == [(0,), (1,)]
    assert [h.score for h in first] == [L(.5), L(.25)]
    assert tr.prune_gap == 0.0                              # the trace sees the tie at the boundary
    # beam 1: label 0 and blank tie at the first step: the label (lower class index) wins
    s1 = ToyScorer({(0, ()): [L(.5), L(.5)], (0, (0,)): [L(.2), L(.8)]}, [L(.5), L(.5)])
    out = malsd(s1, 1, beam=1, max_symbols=4, blank=1)
    assert out[0].prefix == (0,) and out[0].score == L(.5) + L(.8)


def test_equal_candidate_scores_go_to_the_lower_slot():
    # two hypotheses whose best extensions score the same: the lower slot's takes the beam
    s = ToyScorer({(0, ()): [L(.5), L(.5), -np.inf],
                   (0, (0,)): [L(.5), -np.inf, L(.5)], (0, (1,)): [-np.inf, L(.5), L(.5)]}, [0, 0, 0])
    tr = BeamTrace()
    malsd(s, 1, beam=2, max_symbols=3, blank=2, trace=tr, keep_beams=True)
    second = tr.beams[1]
    # candidates: slot 0 -> (0, 0) and (0,)+blank; slot 1 -> (1, 1) and (1,)+blank, all log .25
    assert [h.prefix for h in second] == [(0, 0), (0,)]
    assert tr.beams[0][0].prefix == (0,) and tr.beams[0][1].prefix == (1,)


def _two_alignment_scorer():
    # labels 0, blank 1; two frames; max_symbols 1
    table = {(0, ()): [L(.6), L(.4)], (0, (0,)): [L(.3), L(.7)],
             (1, ()): [L(.5), L(.5)], (1, (0,)): [L(.2), L(.8)], (1, (0, 0)): [L(.1), L(.9)]}
    return ToyScorer(table, [L(.5), L(.5)]), 2


def test_two_alignments_of_one_transcript_merge_by_log_sum_exp():
    scorer, T = _two_alignment_scorer()
    tr = BeamTrace()
    out = malsd(scorer, T, beam=4, max_symbols=1, blank=1, trace=tr, keep_beams=True)
    # iteration 2: (0,) reached by label-then-blank (.6 * .7) and by blank-then-label (.4 * .5)
    it2 = tr.beams[1]
    merged = [h for h in it2 if h.prefix == (0,) and h.live]
    assert len(merged) == 1 and abs(merged[0].score - L(.42 + .2)) < 1e-15
    # the kept member is the higher-scoring one (blank at frame 0: no label yet at frame 1)
    assert merged[0].n_sym == 0 and merged[0].t == 1
    assert sum(h.live for h in it2) == 2                    # (0,) and the final ()
    got = live(out)
    assert abs(got[(0,)] - L(.62 * .8)) < 1e-15           # = .6*.7*.8 + .4*.5*.8
    assert abs(got[()] - L(.4 * .5)) < 1e-15
    assert abs(got[(0, 0)] - L(.62 * .2 * .9)) < 1e-15
    assert best(out).prefix == (0,)


def test_recombination_after_pruning_leaves_the_slot_empty():
    scorer, T = _two_alignment_scorer()
    tr = BeamTrace()
    out = malsd(scorer, T, beam=2, max_symbols=1, blank=1, trace=tr, keep_beams=True)
    it2 = tr.beams[1]
    # pruned to A-blank (0,) and B-label (0,) (B-label beats B-blank on the class index), then
    # merged: one slot left empty, the dropped final () is not brought back
    assert it2[0].prefix == (0,) and abs(it2[0].score - L(.62)) < 1e-15
    assert not it2[1].live
    got = live(out)
    assert () not in got
    assert abs(got[(0,)] - L(.62 * .8)) < 1e-15 and abs(got[(0, 0)] - L(.62 * .2 * .9)) < 1e-15


@pytest.mark.parametrize("m,expect", [(2, (0, 0, 0, 0)), (1, (0, 0)), (3, (0,) * 6)])
def test_max_symbols_forces_blank(m, expect):
    s = ToyScorer({}, [L(.9), L(.1)])
    out = malsd(s, 2, beam=1, max_symbols=m, blank=1)
    assert out[0].prefix == expect
    assert abs(out[0].score - (2 * m * L(.9) + 2 * L(.1))) < 1e-12
    # the forced blank uses the blank's full log-probability even when blank is not in the top K
    s2 = ToyScorer({}, [L(.5), L(.45), L(.05)])
    out2 = malsd(s2, 1, beam=1, max_symbols=1, blank=2)
    assert out2[0].prefix == (0,) and abs(out2[0].score - (L(.5) + L(.05))) < 1e-15


def test_final_hypothesis_is_kept_in_slot_zero():
    table = {(0, ()): [L(.3), L(.7)], (0, (0,)): [L(.6), L(.4)], (0, (0, 0)): [L(.5), L(.5)]}
    s = ToyScorer(table, [L(.5), L(.5)])
    tr = BeamTrace()
    out = malsd(s, 1, beam=2, max_symbols=3, blank=1, trace=tr, keep_beams=True)
    for b in tr.beams:
        assert b[0].prefix == () and b[0].score == L(.7) and b[0].t == 1
    assert [h.prefix for h in out] == [(), (0, 0, 0)]
    assert abs(out[1].score - L(.3 * .6 * .5 * .5)) < 1e-15
    assert tr.iterations == 4


def test_normalisation_changes_the_winner():
    table = {(0, ()): [L(.7), L(.3)], (0, (0,)): [L(.8), L(.2)], (0, (0, 0)): [L(.9), L(.1)]}
    s = ToyScorer(table, [L(.6), L(.4)])
    out = malsd(s, 1, beam=2, max_symbols=3, blank=1)
    got = live(out)
    assert abs(got[()] - L(.3)) < 1e-15 and abs(got[(0, 0, 0)] - L(.7 * .8 * .9 * .4)) < 1e-15
    assert best(out, score_norm=False).prefix == ()
    assert best(out, score_norm=True).prefix == (0, 0, 0)     # -1.601 / 4 > -1.204 / 1
    assert [out[j].prefix for j in ranked(out)] == [(0, 0, 0), ()]


def test_transcripts_with_equal_length_and_last_label_stay_apart():
    # (0, 1) and (1, 1) share length and last label; a hash of those two alone would merge them
    table = {(0, ()): [L(.4), L(.4), L(.2)], (0, (0,)): [L(.1), L(.6), L(.3)],
             (0, (1,)): [L(.1), L(.6), L(.3)]}
    s = ToyScorer(table, [L(.3), L(.3), L(.4)])
    out = malsd(s, 1, beam=4, max_symbols=2, blank=2)
    got = live(out)
    assert abs(got[(0, 1)] - L(.4 * .6 * .4)) < 1e-15
    assert abs(got[(1, 1)] - L(.4 * .6 * .4)) < 1e-15
    assert abs(got[()] - L(.2)) < 1e-15
    assert abs(got[(0,)] - L(.4 * .3)) < 1e-15
    assert len(got) == 4


def test_zero_frames_and_model_scorer_normalisation():
    out = malsd(ToyScorer({}, [0.0]), 0, beam=3, max_symbols=2, blank=0)
    assert out[0].prefix == () and out[0].score == 0.0 and not out[1].live
    cfg = DecConfig(name="tiny", seed=9, joint_dim=64, pred_hidden=64, vocab=20, max_symbols=2)
    dec = GreedyDecoder(cfg, make_dec_weights(cfg))
    from oracle.beam import ModelScorer
    sc = ModelScorer(dec, np.random.default_rng(1).standard_normal((3, 64)))
    for prefix in ((), (3,), (3, 7)):
        lp = sc(1, prefix)
        assert abs(np.exp(lp).sum() - 1.0) < 1e-12
        # the predictor output after a prefix is the LSTM stepped over blank then the prefix
        h = np.zeros((dec.L, dec.H)); c = h.copy()
        for tok in (dec.blank,) + prefix:
            h, c = dec.lstm_step(tok, h, c)
        assert np.array_equal(sc.pred(prefix), dec.pred_project(h[-1]))
