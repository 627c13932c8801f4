"""Float64 oracle of batched MALSD beam search (modified alignment-length synchronous decoding)
over the projected encoder frames of one utterance per stream.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ("Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon", §2.2 "One
pinned iteration", §2.3 "Equality and recombination", §2.4 "Configuration fields that can change
output"; §4.1 "Fixed storage" for the per-hypothesis state). A beam of K slots; slot 0 starts
with score 0 at frame 0 with an empty transcript, the other slots start empty. Each iteration
moves every live hypothesis by exactly one alignment step:
  1. each live hypothesis that still has frames scores the classes with the joint at its frame
     and its predictor output: log_softmax over all classes;
  2. its candidates are its K best classes (score + log-probability), unless it has already
     emitted max_symbols labels at its frame: then its only candidate is blank (score + the
     blank log-probability, blank forced); a hypothesis past its last frame (final) offers
     itself, unchanged, as its only candidate;
  3. the K best of all candidates survive into the K slots (pruning);
  4. blank moves a survivor to the next frame; a label appends to its transcript and keeps the
     frame;
  5. survivors with the same transcript are merged after the pruning: the one with the highest
     score keeps its slot and takes the log-sum-exp of the group's scores, the others leave the
     beam, and their slots stay empty for this iteration;
  6. the predictor advances on each new label; blank keeps the parent's predictor state.
The loop ends when no live hypothesis has frames left. The answer is the hypothesis with the
best normalised score.

Readings where the pages leave a step open:
  B1 order and ties: candidates are ranked by score, then by slot, then by class index (the
     order a sorted top-K per hypothesis followed by a global top-K over the K x K candidates
     in slot-major order gives, with ties to the lower index in both).
  B2 the per-hypothesis top-K followed by the global top-K is the same as the global top-K over
     every (hypothesis, class) pair, so the oracle takes the latter directly.
  B3 equality for recombination is equality of the whole non-blank transcript (which implies
     equal last label and length; no hash, so no collision can merge two transcripts). Among
     equal hypotheses the kept one is the highest-scoring, ties to the lower slot.
  B4 empty slots (score -inf) offer no candidates and take no part in recombination; the loop
     runs while a live hypothesis has frames left (the slots that are empty never change a
     live hypothesis's result).
  B5 score normalisation divides the score by the transcript length + 1 (the predictor's input
     sequence, with its start symbol); with normalisation off, the raw score decides. Ties go
     to the lower slot.
  B6 the start symbol is blank (the predictor starts on the blank token with zero state), as in
     the greedy decoder.
  B7 frames per stream: a stream's utterance has its own length; frames past it are never read.

Parity status: pinned in ``tests/test_oracle_beam_pins.py`` (exact sums over every alignment
by brute force when the beam is wide enough to prune nothing, beam 1 against the greedy state
machine, and hand-built toy scorers for each fixture the pages list: blank/label ties, two
alignments of one transcript, recombination after pruning, max-symbol blank forcing, a final
hypothesis kept in the beam, normalisation changing the winner, and transcripts a weak hash
would confuse).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NEG_INF = -math.inf


@dataclass
class Hyp:
    """One beam slot: score (log-probability), frame index t, non-blank transcript and the
    number of labels emitted at frame t."""
    score: float
    t: int
    prefix: tuple
    n_sym: int

    @property
    def live(self) -> bool:
        return self.score > NEG_INF


@dataclass
class BeamTrace:
    """What the decisions of one run depended on (for comparisons with a decoder that computes
    in lower precision): the smallest score gap at any pruning boundary (the K-th kept
    candidate against the best dropped one), the smallest gap between the best and second-best
    score inside a merged group whose members differ in labels at their frame, and the number
    of iterations; per iteration, the smaller of the two gaps (inf when no decision was close
    to a boundary) and the largest |score| kept. Beams after every iteration are kept when
    asked."""
    prune_gap: float = math.inf
    merge_gap: float = math.inf
    iterations: int = 0
    max_candidates: int = 0
    gaps: list = field(default_factory=list)
    scale: list = field(default_factory=list)
    beams: list = field(default_factory=list)


def log_softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - m - math.log(np.exp(x - m).sum())


def logsumexp(vals):
    vals = [v for v in vals if v > NEG_INF]
    if not vals:
        return NEG_INF
    m = max(vals)
    return m + math.log(sum(math.exp(v - m) for v in vals))


def malsd(log_probs, n_frames: int, beam: int, max_symbols: int, blank: int, trace: BeamTrace | None = None,
          keep_beams: bool = False):
    """MALSD beam search over ``n_frames`` frames with ``beam`` slots. ``log_probs(t, prefix)``
    returns the log-probabilities of every class at frame t after the non-blank transcript
    ``prefix``. Returns the final beam: a list of ``beam`` Hyp (empty slots have score -inf)."""
    K = beam
    slots = [Hyp(0.0, 0, (), 0)] + [Hyp(NEG_INF, 0, (), 0) for _ in range(K - 1)]
    while any(h.live and h.t < n_frames for h in slots):
        # candidates: (score, slot, class or None for a final hypothesis)
        cands = []
        for k, h in enumerate(slots):
            if not h.live:
                continue
            if h.t >= n_frames:
                cands.append((h.score, k, None))
                continue
            lp = np.asarray(log_probs(h.t, h.prefix), dtype=np.float64)
            if h.n_sym >= max_symbols:
                cands.append((h.score + float(lp[blank]), k, blank))
                continue
            # B2: only this hypothesis's K + 1 best classes can be kept or be the best dropped
            # candidate; ranked by log-probability, then class index
            order = np.lexsort((np.arange(lp.size), -lp))[:K + 1]
            for c in order:
                s = h.score + float(lp[c])
                if s > NEG_INF:
                    cands.append((s, k, int(c)))
        # B1/B2: score descending, then slot, then class (a final hypothesis has one candidate)
        cands.sort(key=lambda x: (-x[0], x[1], -1 if x[2] is None else x[2]))
        kept = cands[:K]
        gap = math.inf
        if trace is not None:
            trace.iterations += 1
            trace.max_candidates = max(trace.max_candidates, len(cands))
            if len(cands) > K:
                gap = kept[-1][0] - cands[K][0]
                trace.prune_gap = min(trace.prune_gap, gap)
        new = []
        for s, k, c in kept:
            h = slots[k]
            if c is None:
                new.append(Hyp(s, h.t, h.prefix, h.n_sym))
            elif c == blank:
                new.append(Hyp(s, h.t + 1, h.prefix, 0))
            else:
                new.append(Hyp(s, h.t, h.prefix + (c,), h.n_sym + 1))
        new += [Hyp(NEG_INF, 0, (), 0) for _ in range(K - len(new))]
        # recombination after pruning (B3)
        groups: dict = {}
        for j, h in enumerate(new):
            if h.live:
                groups.setdefault(h.prefix, []).append(j)
        for members in groups.values():
            if len(members) < 2:
                continue
            best = max(members, key=lambda j: (new[j].score, -j))
            if trace is not None and len({new[j].n_sym for j in members}) > 1:
                sc = sorted((new[j].score for j in members), reverse=True)
                trace.merge_gap = min(trace.merge_gap, sc[0] - sc[1])
                gap = min(gap, sc[0] - sc[1])
            total = logsumexp([new[j].score for j in members])
            for j in members:
                if j != best:
                    new[j] = Hyp(NEG_INF, new[j].t, new[j].prefix, new[j].n_sym)
            new[best] = Hyp(total, new[best].t, new[best].prefix, new[best].n_sym)
        slots = new
        if trace is not None:
            trace.gaps.append(gap)
            trace.scale.append(max((abs(h.score) for h in slots if h.live), default=0.0))
        if trace is not None and keep_beams:
            trace.beams.append([Hyp(h.score, h.t, h.prefix, h.n_sym) for h in slots])
    return slots


def normalised(h: Hyp, score_norm: bool = True) -> float:
    """B5: score / (length + 1) with normalisation, the raw score without."""
    return h.score / (len(h.prefix) + 1) if score_norm else h.score


def ranked(slots, score_norm: bool = True):
    """Indices of the live slots, best first (normalised score descending, ties to the lower
    slot)."""
    live = [j for j, h in enumerate(slots) if h.live]
    return sorted(live, key=lambda j: (-normalised(slots[j], score_norm), j))


def best(slots, score_norm: bool = True) -> Hyp:
    return slots[ranked(slots, score_norm)[0]]


class ToyScorer:
    """A table of log-probabilities per (frame, transcript prefix), for testing the state
    machine without a model ("Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon",
    §2.5). Entries missing from the table fall back to ``default``."""

    def __init__(self, table: dict, default):
        self.table = {k: np.asarray(v, dtype=np.float64) for k, v in table.items()}
        self.default = np.asarray(default, dtype=np.float64)

    def __call__(self, t, prefix):
        return self.table.get((t, tuple(prefix)), self.default)


class ModelScorer:
    """Log-probabilities of the joint after projection for one stream: frame t of the projected
    encoder frames z [T, P] against the predictor output after the transcript prefix (the
    prediction network's state depends only on the non-blank prefix; the start symbol is blank,
    B6). Predictor states are kept per prefix."""

    def __init__(self, dec, z):
        self.dec = dec
        self.z = np.asarray(z, dtype=np.float64)
        h0 = np.zeros((dec.L, dec.H))
        h, c = dec.lstm_step(dec.blank, h0, h0.copy())
        self.state = {(): (h, c, dec.pred_project(h[-1]))}

    def _state(self, prefix):
        if prefix not in self.state:
            h, c, _ = self._state(prefix[:-1])
            h2, c2 = self.dec.lstm_step(prefix[-1], h, c)
            self.state[prefix] = (h2, c2, self.dec.pred_project(h2[-1]))
        return self.state[prefix]

    def pred(self, prefix):
        return self._state(tuple(prefix))[2]

    def __call__(self, t, prefix):
        return log_softmax(self.dec.joint(self.z[t], self.pred(prefix)))


def beam_decode(dec, z, n_frames: int, beam: int, max_symbols: int, trace: BeamTrace | None = None):
    """Beam search of one stream with a decoder's weights (an ``oracle.decoder.GreedyDecoder``):
    returns the final beam."""
    return malsd(ModelScorer(dec, z), n_frames, beam, max_symbols, dec.blank, trace)
