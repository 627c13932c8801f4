"""GPU streaming log-mel (include/cac_mel.h, through the C ABI) against the float64 oracle
(oracle/mel.py): every stream of the 1024-stream workload over several chunks, other pushes
sizes and window shapes, reset, and the mel frames feeding the encoder's front end.

Bar: max-abs 1e-5 on the log-mel values in float32 output: the GPU transform runs in float64
from the same float32 samples, so the output's own float32 rounding (|log-mel| < 20, 1e-6) is
what remains. bf16 output: within one bf16 rounding (2^-8 relative) of the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import log
from synth import A4, make_audio

pytestmark = pytest.mark.gpu

MEL_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_conformer_amd  # noqa: F401
    yield


def _oracle_frames(cfg, ids, chunks):
    from oracle.mel import MelStream
    out = []
    for s in ids:
        ms = MelStream()
        x = make_audio(cfg, s, chunks)
        out.append(np.stack([ms.push(x[c]) for c in range(chunks)]))
    return np.stack(out)  # [n, chunks, hops, n_mels]


def test_logmel_1024_streams_match_the_oracle():
    from cache_aware_conformer_amd import StreamingMel
    cfg = A4.replace(out_dtype="f32")
    S, chunks = cfg.streams, 3
    mel = StreamingMel(cfg)
    x = np.stack([make_audio(cfg, s, chunks) for s in range(S)])            # [S, chunks, samples]
    xd = torch.from_numpy(np.ascontiguousarray(x.swapaxes(0, 1))).to("cuda:0")
    got = np.stack([mel.push(list(range(S)), xd[c]).cpu().numpy() for c in range(chunks)], axis=1)
    sample = list(range(0, S, 4))
    ref = _oracle_frames(cfg, sample, chunks)
    err = np.abs(got[sample] - ref).max()
    log(f"log-mel, {len(sample)} of {S} streams x {chunks} chunks: max-abs {err:.3e}")
    assert err <= MEL_TOL


@pytest.mark.parametrize("n_fft,win,hop,pushes", [(512, 400, 160, [1, 7, 16, 3]), (256, 200, 80, [5, 2, 9]),
                                                  (1024, 800, 320, [2, 4])])
def test_logmel_shapes_and_push_sizes(n_fft, win, hop, pushes):
    """Other transform sizes and pushes of any whole number of hops, against the oracle's offline
    definition on the same samples."""
    import oracle.mel as om
    from cache_aware_conformer_amd import StreamingMel
    cfg = A4.replace(n_fft=n_fft, win_length=win, hop=hop, streams=3, hops=max(pushes), out_dtype="f32")
    mel = StreamingMel(cfg)
    rng = np.random.default_rng(n_fft)
    total = sum(pushes) * hop
    x = (rng.standard_normal((3, total)) * 0.1 + np.sin(np.arange(total) * 0.3)).astype(np.float32)
    xd = torch.from_numpy(x).to("cuda:0")
    got, t0 = [], 0
    for p in pushes:
        got.append(mel.push([0, 1, 2], xd[:, t0:t0 + p * hop].contiguous()).cpu().numpy())
        t0 += p * hop
    got = np.concatenate(got, axis=1)
    ref = np.stack([om.logmel_offline(x[s].astype(np.float64), n_fft, win, hop) for s in range(3)])
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= MEL_TOL


def test_logmel_bf16_output_and_reset():
    from cache_aware_conformer_amd import StreamingMel
    from synth import bf16_round
    cfg = A4.replace(streams=4)
    mel = StreamingMel(cfg)
    x = np.stack([make_audio(cfg, s, 2) for s in range(4)])
    junk = torch.randn((4, 2560), device="cuda:0")
    mel.push([0, 1, 2, 3], junk)
    mel.reset([0, 1, 2, 3])
    got = [mel.push([0, 1, 2, 3], torch.from_numpy(np.ascontiguousarray(x[:, c])).to("cuda:0")) for c in range(2)]
    got = np.stack([g.float().cpu().numpy() for g in got], axis=1)
    ref = _oracle_frames(cfg, range(4), 2)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + MEL_TOL)
    assert np.array_equal(got, bf16_round(got))


def test_audio_to_encoder_pipeline_matches_the_oracle_pipeline():
    """Raw audio -> GPU log-mel (bf16) -> GPU front end + 2-layer encoder, against the oracle
    log-mel (rounded once to bf16, as every bf16 input is) -> oracle front end + encoder, for 6
    fresh streams over 5 chunks: within the bf16 bar."""
    from cache_aware_conformer_amd import StreamingEncoder, StreamingMel
    from oracle import Oracle
    from oracle.mel import MelStream
    from synth import C4, bf16_round, make_weights
    cfg = C4.replace(n_layers=2, streams=6, staggered=False)
    W = make_weights(cfg)
    mel = StreamingMel(A4.replace(streams=6))
    enc = StreamingEncoder(cfg, W, max_streams=6)
    orc = Oracle(cfg, W)
    sts, mss = [orc.new_state() for _ in range(6)], [MelStream() for _ in range(6)]
    x = np.stack([make_audio(A4, s, 5) for s in range(6)])
    worst = 0.0
    for c in range(5):
        m = mel.push(list(range(6)), torch.from_numpy(np.ascontiguousarray(x[:, c])).to("cuda:0"))
        out, _ = enc.push_chunk(list(range(6)), m)
        mref = np.stack([bf16_round(np.float32(ms.push(x[s, c]))) for s, ms in enumerate(mss)])
        ref = orc.push(sts, mref.astype(np.float64))
        r = float(np.abs(out.cpu().numpy() - ref).max() / np.abs(ref).max())
        worst = max(worst, r)
        assert r <= 2e-2, (c, r)
    log(f"audio -> log-mel -> encoder: worst rel {worst:.3e}")
