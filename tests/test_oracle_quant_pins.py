"""Pins of the int8 weight compression (oracle/quant.py): scalar loops, the half-step error
bound, ties to even, zero columns, which tensors it touches, and the compressed encoder's
distance from the full-precision one (the approximation row of this path)."""
import numpy as np
import pytest

from oracle import Oracle
from oracle.quant import compress_weights, compressed_name, dequantize, quantize_columns
from synth import C1, C2, make_inputs, make_weights

# Bar of the approximation: ||z_int8 - z||_inf / ||z||_inf of the 17-layer encoder on its seeded
# inputs (measured 4.1e-2 over 40 chunks with N(0, 1/fan_in) weights; the bar leaves 2x).
INT8_REL_BAR = 8e-2


def test_quantize_columns_matches_scalar_loops():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((37, 11)) * np.exp(rng.standard_normal(11))).astype(np.float32)
    q, s = quantize_columns(w)
    for n in range(11):
        m = np.float32(0.0)
        for k in range(37):
            m = max(m, abs(w[k, n]))
        sn = np.float32(m / np.float32(127.0))
        assert s[n] == sn
        for k in range(37):
            v = float(np.float32(w[k, n] / sn))
            lo = np.floor(v)
            code = lo + 1 if v - lo > 0.5 or (v - lo == 0.5 and lo % 2 == 1) else lo
            assert q[k, n] == int(max(-127, min(127, code))), (k, n)


def test_quantization_error_is_at_most_half_a_step():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((512, 64)).astype(np.float32) / 20
    q, s = quantize_columns(w)
    err = np.abs(dequantize(q, s) - w.astype(np.float64))
    assert np.all(err <= s.astype(np.float64) * (0.5 + 1e-6))
    assert np.array_equal(np.abs(q).max(axis=0), np.full(64, 127))  # every column's largest weight maps to 127


def test_ties_to_even_and_zero_columns():
    w = np.zeros((4, 3), np.float32)
    w[:, 0] = [127.0, 2.5, -2.5, 3.5]      # scale 1: codes 127, 2, -2, 4
    w[:, 2] = [0.0, 254.0, 1.0, -3.0]      # scale 2: 0.5 -> 0, -1.5 -> -2
    q, s = quantize_columns(w)
    assert s.tolist() == [1.0, 0.0, 2.0]
    assert q[:, 0].tolist() == [127, 2, -2, 4]
    assert q[:, 1].tolist() == [0, 0, 0, 0]
    assert q[:, 2].tolist() == [0, 127, 0, -2]


def test_representable_weights_are_left_exactly():
    """Weights that already are codes times their column scale reconstruct exactly, so the
    compressed encoder equals the plain one on them."""
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, (64, 16)).astype(np.float32)
    q[0] = 127.0
    s = np.float32(2.0) ** rng.integers(-8, -2, 16).astype(np.float32)
    w = q * s
    q2, s2 = quantize_columns(w)
    assert np.array_equal(s2, s) and np.array_equal(q2.astype(np.float32), q)


def test_compress_weights_touches_only_dense_matrices():
    W = make_weights(C1)
    Wq = compress_weights(W)
    touched = [n for n in W if not np.array_equal(np.asarray(Wq[n], np.float64), np.asarray(W[n], np.float64))]
    assert touched and all(compressed_name(n) for n in touched)
    assert {n.split(".", 1)[1] for n in touched} == {"ff1.w1", "ff1.w2", "att.wq", "att.wk", "att.wv", "att.wo",
                                                      "conv.pw1", "conv.pw2", "ff2.w1", "ff2.w2"}
    assert not compressed_name("l0.att.wpos") and not compressed_name("l0.conv.dw") and compressed_name("joint.w")


@pytest.mark.slow
def test_int8_encoder_stays_within_its_approximation_bar():
    """The 17-layer encoder on int8 weights against full precision over 20 chunks."""
    W = make_weights(C2)
    a, b = Oracle(C2, W), Oracle(C2, compress_weights(W))
    sa, sb = a.new_state(), b.new_state()
    xs = make_inputs(C2, 0, 20)
    worst = 0.0
    for c in range(20):
        za = a.push([sa], xs[c][None].astype(np.float64))
        zb = b.push([sb], xs[c][None].astype(np.float64))
        worst = max(worst, float(np.abs(za - zb).max() / np.abs(za).max()))
    assert 1e-3 < worst <= INT8_REL_BAR, worst
