"""Float64 oracle of the streaming log-mel front of the encoder (audio -> log-mel frames).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages compute the mel frames of each chunk on the CPU from [melTail || chunk] and report
the streaming mel as exact against the offline one ("True streaming encode — implementation
spec", "Per-chunk flow" step 1 and "Status": StreamingMel exact); the model card gives a
10 ms hop at 16 kHz ("Config": hopLength 160) and the workloads 128 mel bins. Everything else is
a reading (M1-M6), taken as the usual speech front end:
  M1 preemphasis y[n] = x[n] - 0.97 x[n-1], x[-1] = 0.
  M2 frame g covers the 400 preemphasised samples that end at the hop boundary 160 (g + 1)
     (samples before the stream start are 0): frames are causal, so a chunk of whole hops
     yields exactly its own frames and the stream carries the last 241 raw samples.
  M3 periodic Hann window of 400 samples, zero-padded to a 512-point DFT; power spectrum
     |X[k]|^2 for k = 0 .. 256.
  M4 128 triangular mel filters between 0 Hz and 8 kHz on the Slaney mel scale (linear below
     1 kHz: mel = 3 f / 200; logarithmic above: mel = 15 + 27 ln(f / 1000) / ln 6.4), each
     scaled to unit area (2 / (f_right - f_left)).
  M5 log(mel + 2^-24).
  M6 no dither, no per-feature normalisation (a streaming front end has no utterance stats).

Parity status: pinned in ``tests/test_oracle_mel_pins.py`` (the mel scale's closed forms, the
filters' shape and area, the DFT power against a scalar DFT and Parseval, a tone landing in its
mel band, and chunked streaming against the offline computation).
"""
from __future__ import annotations

import numpy as np

SR, N_FFT, WIN, HOP, N_MELS, FMIN, FMAX, PREEMPH = 16000, 512, 400, 160, 128, 0.0, 8000.0, 0.97
LOG_GUARD = 2.0 ** -24


def hz_to_mel(f):
    f = np.asarray(f, dtype=np.float64)
    lin = 3.0 * f / 200.0
    logpart = 15.0 + 27.0 * np.log(np.maximum(f, 1e-300) / 1000.0) / np.log(6.4)
    return np.where(f < 1000.0, lin, logpart)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    lin = 200.0 * m / 3.0
    logpart = 1000.0 * np.exp((m - 15.0) * np.log(6.4) / 27.0)
    return np.where(m < 15.0, lin, logpart)


def mel_filters(n_mels=N_MELS, n_fft=N_FFT, sr=SR, fmin=FMIN, fmax=FMAX):
    """[n_mels, n_fft // 2 + 1] triangular filters on the DFT bin frequencies (M4)."""
    edges = mel_to_hz(np.linspace(hz_to_mel(fmin), hz_to_mel(fmax), n_mels + 2))
    freqs = np.arange(n_fft // 2 + 1) * sr / n_fft
    fb = np.zeros((n_mels, freqs.size))
    for m in range(n_mels):
        lo, mid, hi = edges[m], edges[m + 1], edges[m + 2]
        up = (freqs - lo) / (mid - lo)
        down = (hi - freqs) / (hi - mid)
        fb[m] = np.maximum(0.0, np.minimum(up, down)) * (2.0 / (hi - lo))
    return fb


def hann(n=WIN):
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * np.arange(n) / n)


def power_spectrum(frames, n_fft=N_FFT):
    """|rfft(frame * hann, n_fft)|^2 of frames [G, win] (M3)."""
    frames = np.asarray(frames, np.float64)
    return np.abs(np.fft.rfft(frames * hann(frames.shape[-1]), n=n_fft, axis=-1)) ** 2


def logmel_offline(x, n_fft=N_FFT, win=WIN, hop=HOP):
    """Log-mel frames [len(x) // hop, N_MELS] of a whole signal (M1-M6)."""
    x = np.asarray(x, dtype=np.float64)
    y = x - PREEMPH * np.concatenate([[0.0], x[:-1]])
    G = x.size // hop
    ypad = np.concatenate([np.zeros(win - hop), y])
    frames = np.stack([ypad[g * hop: g * hop + win] for g in range(G)]) if G else np.zeros((0, win))
    return np.log(power_spectrum(frames, n_fft) @ mel_filters(n_fft=n_fft).T + LOG_GUARD)


class MelStream:
    """Streaming log-mel of one stream: each push of whole hops returns its own frames; the
    stream carries the last win - hop + 1 raw samples."""

    def __init__(self, n_fft=N_FFT, win=WIN, hop=HOP):
        self.n_fft, self.win, self.hop = n_fft, win, hop
        self.tail = np.zeros(win - hop + 1)

    def push(self, chunk):
        chunk = np.asarray(chunk, dtype=np.float64)
        win, hop = self.win, self.hop
        assert chunk.size % hop == 0
        xx = np.concatenate([self.tail, chunk])               # raw samples, one before the window
        y = xx[1:] - PREEMPH * xx[:-1]                        # preemphasis of tail[1:] || chunk
        G = chunk.size // hop
        frames = np.stack([y[g * hop: g * hop + win] for g in range(G)]) if G else np.zeros((0, win))
        self.tail = xx[-(win - hop + 1):]
        return np.log(power_spectrum(frames, self.n_fft) @ mel_filters(n_fft=self.n_fft).T + LOG_GUARD)
