"""Pins of the streaming log-mel oracle (oracle/mel.py): the Slaney mel scale's closed forms,
the filters' shape and unit area, the power spectrum against a scalar DFT and Parseval's
identity, a pure tone landing in its own mel band, and chunked streaming equal to the offline
computation."""
import math

import numpy as np
import pytest

from oracle.mel import (HOP, LOG_GUARD, N_FFT, N_MELS, SR, WIN, MelStream, hann, hz_to_mel, logmel_offline,
                        mel_filters, mel_to_hz, power_spectrum)


def test_slaney_mel_scale_closed_forms():
    assert hz_to_mel(0.0) == 0.0
    assert abs(hz_to_mel(1000.0) - 15.0) < 1e-12
    assert abs(hz_to_mel(6400.0) - 42.0) < 1e-12          # 15 + 27 ln(6.4) / ln(6.4)
    assert abs(hz_to_mel(500.0) - 7.5) < 1e-12
    f = np.array([0.0, 120.0, 999.0, 1000.0, 3210.0, 8000.0])
    assert np.abs(mel_to_hz(hz_to_mel(f)) - f).max() < 1e-9


def test_filters_are_unit_area_triangles_on_mel_spaced_edges():
    fb = mel_filters()
    assert fb.shape == (N_MELS, N_FFT // 2 + 1)
    edges = mel_to_hz(np.linspace(0.0, hz_to_mel(8000.0), N_MELS + 2))
    freqs = np.arange(N_FFT // 2 + 1) * SR / N_FFT
    for m in range(N_MELS):
        lo, mid, hi = edges[m], edges[m + 1], edges[m + 2]
        inside = (freqs > lo) & (freqs < hi)
        assert np.all(fb[m][~inside] == 0.0)
        # the continuous triangle of height 2 / (hi - lo) has unit area; sample it at a bin
        for k in np.nonzero(inside)[0][:3]:
            tri = (freqs[k] - lo) / (mid - lo) if freqs[k] <= mid else (hi - freqs[k]) / (hi - mid)
            assert abs(fb[m, k] - tri * 2.0 / (hi - lo)) < 1e-15


def test_power_spectrum_matches_a_scalar_dft_and_parseval():
    rng = np.random.default_rng(1)
    frame = rng.standard_normal(WIN)
    p = power_spectrum(frame[None])[0]
    w = frame * hann()
    for k in (0, 1, 37, 128, 256):
        re = sum(w[n] * math.cos(2 * math.pi * k * n / N_FFT) for n in range(WIN))
        im = -sum(w[n] * math.sin(2 * math.pi * k * n / N_FFT) for n in range(WIN))
        assert abs(p[k] - (re * re + im * im)) < 1e-9 * max(1.0, p[k])
    # Parseval over the two-sided spectrum: interior bins count twice
    two_sided = p[0] + p[-1] + 2.0 * p[1:-1].sum()
    assert abs(two_sided - N_FFT * (w ** 2).sum()) < 1e-9 * two_sided
    assert np.allclose(hann()[[0, WIN // 2]], [0.0, 1.0])


@pytest.mark.parametrize("f0", [300.0, 1250.0, 4321.0])
def test_a_tone_lands_in_its_own_mel_band(f0):
    t = np.arange(HOP * 20) / SR
    lm = logmel_offline(np.sin(2 * np.pi * f0 * t))
    m = int(np.argmax(lm[10]))
    edges = mel_to_hz(np.linspace(0.0, hz_to_mel(8000.0), N_MELS + 2))
    assert edges[m] <= f0 <= edges[m + 2]


def test_silence_is_the_log_guard_and_the_first_frames_see_zeros():
    lm = logmel_offline(np.zeros(HOP * 4))
    assert np.all(lm == math.log(LOG_GUARD))
    x = np.zeros(HOP * 6)
    x[HOP * 3 + 5] = 1.0                              # an impulse in hop 3
    lm = logmel_offline(x)
    assert np.all(lm[:3] == math.log(LOG_GUARD))      # causal frames: nothing before hop 3
    assert np.all(lm[3] > math.log(LOG_GUARD))


@pytest.mark.parametrize("chunks", [[16] * 5, [1, 7, 16, 2, 30], [3] * 9])
def test_streaming_chunks_equal_the_offline_frames(chunks):
    """The streaming mel (a tail of raw samples carried between pushes) equals the offline mel
    frame for frame ("True streaming encode — implementation spec", "Status": StreamingMel
    exact)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal(HOP * sum(chunks)) * 0.3
    off = logmel_offline(x)
    ms, out, s = MelStream(), [], 0
    for c in chunks:
        out.append(ms.push(x[s * HOP:(s + c) * HOP]))
        s += c
    assert np.abs(np.concatenate(out) - off).max() < 1e-12


def test_streaming_equals_offline_for_other_frame_shapes():
    rng = np.random.default_rng(4)
    for n_fft, win, hop in ((256, 200, 80), (1024, 800, 320)):
        x = rng.standard_normal(hop * 12)
        off = logmel_offline(x, n_fft, win, hop)
        ms = MelStream(n_fft, win, hop)
        got = np.concatenate([ms.push(x[i * hop * 3:(i + 1) * hop * 3]) for i in range(4)])
        assert np.abs(got - off).max() < 1e-12
