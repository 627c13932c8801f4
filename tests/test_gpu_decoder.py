"""GPU greedy RNNT + EOU decoding (include/cac_decode.h, through the C ABI) against the float64
oracle (oracle/decoder.py): identical emitted classes and frames, call by call, with the
decoder state carried across calls; and the whole path, encoder chunk step then decoding on
the GPU, against the oracle encoder then the oracle decoder."""
import numpy as np
import pytest
import torch

import oracle_pool
from gpu_util import log, to_dev
from synth import C2, D1, D2, make_dec_inputs, make_dec_weights, make_inputs, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_conformer_amd  # noqa: F401  (fails loudly when libcac.so is missing)
    yield


def _dec(cfg, **kw):
    from cache_aware_conformer_amd import StreamingDecoder
    return StreamingDecoder(cfg, make_dec_weights(cfg), **kw)


def _pairs(tok, frm, cnt):
    """GPU outputs of one stream -> [(frame, class), ...]."""
    n = int(cnt)
    assert np.all(tok[n:] == -1) and np.all(frm[n:] == -1)
    return [(int(f), int(k)) for f, k in zip(frm[:n], tok[:n])]


def _run(cfg, ids, calls, dec=None):
    """GPU decoding of streams ``ids`` (their seeded frames) over ``calls`` calls."""
    dec = dec or _dec(cfg, max_streams=max(ids) + 1)
    xs = np.stack([make_dec_inputs(cfg, s, calls) for s in ids])      # [n, calls, nf, P]
    z = torch.from_numpy(np.ascontiguousarray(xs.swapaxes(0, 1))).to("cuda:0")  # [calls, n, nf, P]
    out = {s: [] for s in ids}
    for c in range(calls):
        tok, frm, cnt = dec.decode(ids, z[c])
        tok, frm, cnt = tok.cpu().numpy(), frm.cpu().numpy(), cnt.cpu().numpy()
        for i, s in enumerate(ids):
            out[s].append(_pairs(tok[i], frm[i], cnt[i]))
    return out


def _compare(got, ref, tag):
    emitted = sum(len(x) for calls in ref.values() for x in calls)
    frames_with = sum(1 for calls in ref.values() for x in calls for f in {t for t, _ in x})
    log(f"{tag}: {len(ref)} streams, {emitted} emitted classes on {frames_with} frames")
    for s in ref:
        for c, (g, r) in enumerate(zip(got[s], ref[s])):
            assert g == r, (tag, s, c, g, r)
    assert emitted > 0


def test_d1_one_stream_300_calls():
    """One stream, 300 calls of 2 frames: the state carried across every call."""
    h = oracle_pool.submit_decode(D1, [0], 300)
    got = _run(D1, [0], 300)
    _compare(got, oracle_pool.collect_decode(h), "D1")


@pytest.mark.slow
def test_d2_1024_streams_4_calls():
    """Every stream of the 1024-stream decode workload over 4 calls."""
    ids = list(range(D2.streams))
    h = oracle_pool.submit_decode(D2, ids, 4)
    got = _run(D2, ids, 4)
    _compare(got, oracle_pool.collect_decode(h), "D2")


@pytest.mark.parametrize("cfg", [D1.replace(name="D_m1", max_symbols=1, streams=6),
                                 D1.replace(name="D_f5", frames=5, streams=5, max_symbols=3),
                                 D1.replace(name="D_small", joint_dim=128, pred_hidden=64, pred_layers=3, vocab=70,
                                            streams=70, blank_bias=1.0)],
                         ids=["max-symbols-1", "5-frames", "small-3-layers"])
def test_decoder_shapes(cfg):
    ids = list(range(cfg.streams))
    h = oracle_pool.submit_decode(cfg, ids, 12)
    got = _run(cfg, ids, 12)
    _compare(got, oracle_pool.collect_decode(h), cfg.name)


def test_decoder_reset_and_stream_independence():
    """A reset stream decodes like a fresh one; a stream's classes do not depend on the other
    streams of the call or their order."""
    cfg = D1.replace(streams=8)
    ids = list(range(8))
    a = _run(cfg, ids, 6)
    dec = _dec(cfg, max_streams=8)
    perm = [5, 2, 7, 0, 3, 6, 1, 4]
    xs = np.stack([make_dec_inputs(cfg, s, 6) for s in perm])
    junk = torch.randn((8, cfg.frames, cfg.joint_dim), device="cuda:0")
    dec.decode(ids, junk)
    dec.reset(ids)
    for c in range(6):
        tok, frm, cnt = dec.decode(perm, torch.from_numpy(np.ascontiguousarray(xs[:, c])).to("cuda:0"))
        tok, frm, cnt = tok.cpu().numpy(), frm.cpu().numpy(), cnt.cpu().numpy()
        for i, s in enumerate(perm):
            assert _pairs(tok[i], frm[i], cnt[i]) == a[s][c], (s, c)


def test_encoder_then_decoder_tokens_match_the_oracle_pipeline():
    """The one-stream float32 encoder (17 layers) on the GPU feeding the GPU decoder, against the
    oracle encoder feeding the oracle decoder: identical classes over 120 chunks. The two
    pipelines share only the seeded weights and inputs."""
    from cache_aware_conformer_amd import StreamingEncoder
    from oracle import Oracle
    from oracle.decoder import GreedyDecoder
    chunks = 120
    W = make_weights(C2)
    enc = StreamingEncoder(C2, W, max_streams=1)
    dec = _dec(D1, max_streams=1)
    xs = make_inputs(C2, 0, chunks)
    orc, odec = Oracle(C2, W), GreedyDecoder(D1, make_dec_weights(D1))
    ost, dst = orc.new_state(), odec.new_state()
    emitted = 0
    for c in range(chunks):
        z, _ = enc.push_chunk([0], to_dev(xs[c][None], C2))
        tok, frm, cnt = dec.decode([0], z)
        got = _pairs(tok.cpu().numpy()[0], frm.cpu().numpy()[0], cnt.cpu().numpy()[0])
        zr = orc.push([ost], xs[c][None].astype(np.float64))[0]
        ref = odec.decode(dst, zr)
        assert got == ref, (c, got, ref)
        emitted += len(ref)
    log(f"encoder + decoder, {chunks} chunks: {emitted} classes, identical")


def test_decoder_graph_replay_and_profiling_match_direct_launches():
    """Graph replays (re-pointed to other buffers every call, with eager work and host syncs in
    between) and profiled direct launches give the classes of direct launches; the profile
    times every kernel and gives the joint its flops."""
    cfg = D1.replace(streams=40)
    ids = list(range(40))
    xs = np.stack([make_dec_inputs(cfg, s, 8) for s in ids])
    z = torch.from_numpy(np.ascontiguousarray(xs.swapaxes(0, 1))).to("cuda:0")
    g, d, p = _dec(cfg, max_streams=40), _dec(cfg, max_streams=40), _dec(cfg, max_streams=40)
    d.set_graph(False)
    p.profile(True)
    bufs = [[torch.empty((40, cfg.frames * cfg.max_symbols), dtype=torch.int32, device="cuda:0") for _ in range(2)]
            + [torch.empty(40, dtype=torch.int32, device="cuda:0")] for _ in range(3)]
    scratch = torch.randn(1 << 16, device="cuda:0")
    for c in range(8):
        zc = z[c].clone()
        tg, fg, cg = g.decode(ids, zc, *bufs[c % 3])
        scratch.mul_(1.0001).add_(0.5)
        td, fd, cd = d.decode(ids, zc)
        tp, fp, cp = p.decode(ids, zc)
        torch.cuda.synchronize()
        for a, b in ((tg, td), (fg, fd), (cg, cd), (tp, td), (fp, fd), (cp, cd)):
            assert torch.equal(a, b), c
    prof = p.profile_read()
    p.profile(False)
    rounds = 1 + cfg.frames * cfg.max_symbols
    launches = sum(v[0] for v in prof.values())
    assert launches == 8 * (3 + rounds * (cfg.pred_layers + 3)), prof.keys()
    assert prof["dec_joint"][3] > 0 and prof["dec_lstm"][3] > 0
