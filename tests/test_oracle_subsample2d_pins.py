"""Pins of the 2-D time x frequency subsampling oracle (oracle/subsample2d.py): each stage and
the whole stack against torch's conv2d / linear, and chunked streaming (mel tail) against the
offline computation of the whole sequence, alone and in front of the encoder."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import Oracle
from oracle import subsample2d as s2
from synth import make_weights
from synth.configs import EncConfig


def tiny2d(**kw):
    base = dict(name="tiny2d", seed=41, n_layers=1, d_model=16, n_heads=2, d_ff=32, joint_dim=0, dtype="f32",
                chunks=8, frontend=2, fe_channels=6, mel_bins=16)
    base.update(kw)
    return EncConfig(**base)


def T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def torch_stack(W, mel):
    """The same stack assembled from torch CPU routines (causal time pad 2, frequency pad 1)."""
    C = W["fe2.c1.w"].shape[0]
    x = T(mel)[None, None]                                                   # [1, 1, T, F]
    pad = lambda t: F.pad(t, (1, 1, 2, 0))  # noqa: E731  (freq left, right, time top, bottom)
    x = F.relu(F.conv2d(pad(x), T(W["fe2.c1.w"])[:, None], T(W["fe2.c1.b"]), stride=2))
    for s in ("2", "3"):
        x = F.conv2d(pad(x), T(W[f"fe2.dw{s}.w"])[:, None], T(W[f"fe2.dw{s}.b"]), stride=2, groups=C)
        x = F.relu(F.conv2d(x, T(W[f"fe2.pw{s}.w"])[:, :, None, None], T(W[f"fe2.pw{s}.b"])))
    b, c, t, f = x.shape
    flat = x.permute(0, 2, 1, 3).reshape(t, c * f)
    return F.linear(flat, T(W["fe2.lin.w"]).T, T(W["fe2.lin.b"])).numpy()


@pytest.mark.parametrize("frames", [16, 48])
def test_offline_stack_matches_torch(frames):
    cfg = tiny2d()
    W = {k: np.asarray(v, np.float64) for k, v in make_weights(cfg).items()}
    mel = np.random.default_rng(frames).standard_normal((frames, cfg.mel_bins))
    got = s2.offline(W, mel)
    assert got.shape == (frames // 8, cfg.d_model)
    assert np.abs(got - torch_stack(W, mel)).max() < 1e-12


def test_streaming_chunks_equal_offline():
    cfg = tiny2d()
    W = {k: np.asarray(v, np.float64) for k, v in make_weights(cfg).items()}
    mel = np.random.default_rng(3).standard_normal((16 * 7, cfg.mel_bins))
    off = s2.offline(W, mel)
    tail = np.zeros((14, cfg.mel_bins))
    out = []
    for c in range(7):
        new = mel[16 * c: 16 * (c + 1)]
        out.append(s2.stream(W, tail, new, pos=2 * c))
        tail = np.concatenate([tail, new])[-14:]
    assert np.abs(np.concatenate(out) - off).max() < 1e-12


def test_encoder_with_2d_front_end_streams_like_offline():
    """The whole encoder behind the 2-D stack: cached chunk steps equal the offline encode."""
    cfg = tiny2d(n_layers=2, att_left=6)
    orc = Oracle(cfg, make_weights(cfg))
    mel = np.random.default_rng(4).standard_normal((16 * 6, cfg.mel_bins))
    off = orc.encode_offline(orc.frontend_offline(mel))
    st = orc.new_state()
    got = np.concatenate([orc.push([st], mel[None, 16 * c: 16 * (c + 1)])[0] for c in range(6)])
    assert np.abs(got - off).max() < 1e-12
