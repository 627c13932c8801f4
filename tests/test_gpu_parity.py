"""GPU parity of the HIP chunk step (through the C ABI) against the float64 oracle.

Bars: float32 workloads max-abs <= 1e-4 on every output and identical greedy tokens on every
frame (frames the token head's bound would call ambiguous are only counted and logged); bf16
workloads ||z_gpu - z_ref||_inf / ||z_ref||_inf <= 2e-2 on every step over every checked
stream. The GPU always runs the whole batch of a workload; the oracle checks every stream of
the 256- and 1024-stream workloads and a fixed 64-stream subset of the lookahead workload,
computed in worker processes while the GPU runs (streams are independent)."""
import numpy as np
import pytest
import torch

import oracle_pool
from gpu_util import dev_dtype, import_staggered, log, rel_inf, to_dev
from synth import C1, C2, C3, C4, C5, make_inputs, make_state, make_token_head, make_weights, state_position

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_conformer_amd  # noqa: F401  (fails loudly when libcac.so is missing)
    yield


def _enc(cfg, W, **kw):
    from cache_aware_conformer_amd import StreamingEncoder
    return StreamingEncoder(cfg, W, **kw)


def _oracle(cfg, W):
    from oracle import Oracle
    return Oracle(cfg, W)


# ----------------------------------------------------------------------------- dense kernels

GEMM_SHAPES = [(2048, 512), (512, 2048), (1536, 512), (640, 512), (1024, 512), (512, 384)]


@pytest.mark.parametrize("dtype,path,M", [("f32", 1, 1), ("f32", 1, 2), ("f32", 1, 5), ("f32", 1, 8), ("f32", 1, 19),
                                          ("bf16", 1, 2), ("bf16", 1, 7), ("bf16", 2, 64), ("bf16", 2, 100),
                                          ("bf16", 2, 512), ("bf16", 2, 2048), ("bf16", 3, 300), ("bf16", 4, 300),
                                          ("bf16", 5, 300), ("bf16", 6, 300), ("bf16", 7, 300), ("bf16", 8, 300),
                                          ("bf16", 8, 24), ("bf16", 9, 300), ("bf16", 10, 300), ("bf16", 10, 40),
                                          ("bf16", 3, 7), ("bf16", 11, 300), ("bf16", 12, 300), ("bf16", 12, 2048)])
def test_gemm_kernels(dtype, path, M):
    """Paths 7 and 8 (split-K partials summed by the residual row kernel) take N a multiple of
    256 up to 1024 and K a multiple of 128 / 256; paths 9 to 12 (k-steps over 2 or 4 groups of
    waves) K a multiple of 128 (256 for path 10); the other shapes are skipped for them."""
    from cache_aware_conformer_amd.binding import CAC_BF16, CAC_F32, test_gemm
    rng = np.random.default_rng(M * 7 + path)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for N, K in GEMM_SHAPES:
        if path in (7, 8) and (N % 256 or N > 1024 or K % (128 if path == 7 else 256)):
            continue
        if path in (9, 10, 11, 12) and K % (256 if path == 10 else 128):
            continue
        log(f"gemm {dtype} path={path} M={M} N={N} K={K}")
        A = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to("cuda:0").to(tdt)
        W = torch.from_numpy((rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K)).astype(np.float32)).to("cuda:0").to(tdt)
        b = torch.from_numpy(rng.standard_normal(N, dtype=np.float32)).to("cuda:0")
        C = test_gemm(CAC_BF16 if dtype == "bf16" else CAC_F32, path, A, W, b)
        torch.cuda.synchronize()
        ref = A.double().cpu().numpy() @ W.double().cpu().numpy().T + b.double().cpu().numpy()
        err = rel_inf(C.cpu().numpy(), ref)
        assert err < 1e-5, (N, K, err)


# ----------------------------------------------------------------------------- float32 workloads

def _run_single_stream(cfg, chunks, **kw):
    W = make_weights(cfg)
    enc = _enc(cfg, W, max_streams=1, **kw)
    orc = _oracle(cfg, W)
    st = orc.new_state()
    xs = make_inputs(cfg, 0, chunks)
    got, ref = [], []
    for c in range(chunks):
        out, em = enc.push_chunk([0], to_dev(xs[c][None], cfg))
        got.append(out.cpu().numpy()[0])
        ref.append(orc.push([st], xs[c][None].astype(np.float64))[0])
    return np.stack(got), np.stack(ref)


def test_c1_tiny_f32_all_chunks():
    log("C1 tiny f32, 1 stream x 100 chunks")
    got, ref = _run_single_stream(C1, C1.chunks)
    err = np.abs(got - ref).max(axis=(1, 2))
    log(f"C1 max-abs per chunk: max {err.max():.3e}")
    assert err.max() <= F32_TOL
    # error does not grow with the number of chunks (bounded dependency depth)
    assert err[-20:].max() <= 10 * max(err[:20].max(), 1e-7)


def _check_tokens(got, ref, tag):
    """Greedy tokens of both paths identical on every frame; the frames whose oracle margin
    the token head's perturbation bound would not cover are counted as a diagnostic."""
    from oracle.tokens import ambiguous_frames, greedy_tokens
    head = make_token_head(C2)
    zg, zr = got.reshape(-1, C2.joint_dim), ref.reshape(-1, C2.joint_dim)
    tg, _ = greedy_tokens(zg, head)
    tr, margin = greedy_tokens(zr, head)
    amb = ambiguous_frames(zr, zg, head)
    log(f"{tag} tokens: {int((tg != tr).sum())} differ of {len(tr)}; {int(amb.sum())} frames inside the "
        f"ambiguity bound; smallest oracle margin {float(margin.min()):.3e}")
    assert np.array_equal(tg, tr), np.nonzero(tg != tr)[0][:20]


def test_c2_eou_f32_one_stream_tokens():
    chunks = 80  # the 70-row cache fills at chunk 35 and wraps after
    log(f"C2 f32 17 layers, 1 stream x {chunks} chunks")
    got, ref = _run_single_stream(C2, chunks)
    err = np.abs(got - ref).max()
    log(f"C2 max-abs {err:.3e}")
    assert err <= F32_TOL
    _check_tokens(got, ref, "C2/80")


@pytest.mark.slow
def test_c2_eou_f32_all_1000_chunks():
    """The whole workload: max-abs on every output and identical tokens on all 2000 frames.
    The oracle runs in a worker process while the GPU pushes."""
    log("C2 f32 all 1000 chunks")
    h = oracle_pool.submit_streams(C2, [0], C2.chunks, staggered=False)
    W = make_weights(C2)
    enc = _enc(C2, W, max_streams=1)
    xs = make_inputs(C2, 0, C2.chunks)
    got = []
    for c in range(C2.chunks):
        out, _ = enc.push_chunk([0], to_dev(xs[c][None], C2))
        got.append(out.cpu().numpy()[0])
    got = np.stack(got)
    refs, _ = oracle_pool.collect(h)
    ref = np.stack([r[0] for r in refs])
    err = np.abs(got - ref).max(axis=(1, 2))
    log(f"C2/1000 max-abs {err.max():.3e} (chunk {int(err.argmax())})")
    assert err.max() <= F32_TOL
    _check_tokens(got, ref, "C2/1000")


def test_c2q_int8_weights_one_stream():
    """The one-stream encoder with int8 dense weights over 300 chunks: max-abs <= 1e-4 and
    identical tokens against the oracle on the reconstructed weights, and within the int8
    approximation bar of the full-precision oracle."""
    from synth import C2Q
    from test_oracle_quant_pins import INT8_REL_BAR
    chunks = 300
    hq = oracle_pool.submit_streams(C2Q, [0], chunks, staggered=False)
    hf = oracle_pool.submit_streams(C2, [0], chunks, staggered=False)
    enc = _enc(C2Q, make_weights(C2Q), max_streams=1)
    xs = make_inputs(C2Q, 0, chunks)
    got = np.stack([enc.push_chunk([0], to_dev(xs[c][None], C2Q))[0].cpu().numpy()[0] for c in range(chunks)])
    ref = np.stack([r[0] for r in oracle_pool.collect(hq)[0]])
    full = np.stack([r[0] for r in oracle_pool.collect(hf)[0]])
    err = np.abs(got - ref).max()
    approx = float(np.abs(got - full).max() / np.abs(full).max())
    log(f"C2 int8: max-abs {err:.3e} against the reconstructed-weight oracle; {approx:.3e} relative to full precision")
    assert err <= F32_TOL
    assert approx <= INT8_REL_BAR
    _check_tokens(got, ref, "C2 int8/300")


# ----------------------------------------------------------------------------- bf16 workloads

def _check_workload(cfg, chunks, check, flush=False, extra=None):
    """The GPU pushes ``chunks`` chunks for every stream of the workload (from their injected
    states); the oracle runs the streams ``check`` over those chunks, and optionally the
    streams of ``extra = (ids, more_chunks)`` over a longer run, in worker processes started
    before the GPU work. Every step must meet the bf16 bar over all checked streams."""
    W = make_weights(cfg)
    S = cfg.streams
    check = sorted(check)
    run = chunks
    handles = [(check, chunks, oracle_pool.submit_streams(cfg, check, chunks, staggered=cfg.staggered, flush=flush))]
    if extra:
        ex_ids, ex_chunks = sorted(extra[0]), extra[1]
        handles.append((ex_ids, ex_chunks, oracle_pool.submit_streams(cfg, ex_ids, ex_chunks, staggered=cfg.staggered)))
        run = max(run, ex_chunks)
    enc = _enc(cfg, W, max_streams=S)
    log(f"{cfg.name}: importing {S} staggered states")
    positions = import_staggered(enc, cfg, S) if cfg.staggered else [0] * S
    inputs = np.stack([make_inputs(cfg, s, run) for s in range(S)])  # [S, chunks, ...]
    ids = list(range(S))
    got, em = [], []
    for c in range(run):
        out, e = enc.push_chunk(ids, to_dev(inputs[:, c], cfg))
        got.append(out.cpu().numpy())
        em.append(e)
    fl_got = enc.flush(check) if flush else None
    worst = 0.0
    for sel, nch, h in handles:
        refs, fl_ref = oracle_pool.collect(h)
        sel = np.asarray(sel)
        per_stream = np.zeros(len(sel))
        for c in range(nch):
            ref = refs[c]
            m = ref.shape[1]
            assert np.all(em[c][sel] == m), c
            if m == 0:
                continue
            g = got[c][sel, :m]
            r = rel_inf(g, ref)
            rms = float(np.sqrt(np.mean((g - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
            per_stream = np.maximum(per_stream, np.abs(g - ref).max(axis=(1, 2)) / np.abs(ref).max())
            worst = max(worst, r)
            log(f"{cfg.name} chunk {c}, {len(sel)} streams: rel {r:.3e}, rms-rel {rms:.3e}")
            assert r <= BF16_TOL, (c, r)
        log(f"{cfg.name}: {len(sel)} streams x {nch} chunks, worst stream {int(sel[per_stream.argmax()])} "
            f"at {float(per_stream.max()):.3e}")
        if fl_ref is not None:
            out, frames = fl_got
            out = out.cpu().numpy()
            for j, ref in enumerate(fl_ref):
                assert frames[j] == ref.shape[0], (sel[j], frames[j], ref.shape)
                r = rel_inf(out[j, : ref.shape[0]], ref)
                worst = max(worst, r)
                assert r <= BF16_TOL, (sel[j], r)
            log(f"{cfg.name}: flush of {len(fl_ref)} streams within the bar")
    return enc, positions, worst


def _wrapping(cfg, positions, frames, R, k):
    """Up to k streams whose K/V ring slot (position mod R) passes the end of the ring within
    ``frames`` frames, spread over the batch."""
    wrap = [s for s, p in enumerate(positions) if p % R + frames >= R]
    return [wrap[i] for i in np.linspace(0, len(wrap) - 1, min(k, len(wrap))).astype(int)] if wrap else []


@pytest.mark.slow
def test_c3_bf16_256_staggered_streams():
    """Every stream of the 256-stream workload over 8 chunks."""
    _check_workload(C3, 8, range(C3.streams))


@pytest.mark.slow
def test_c4_bf16_1024_streams_frontend():
    """Every stream of the 1024-stream front-end workload over 4 chunks, plus 64 streams over
    12 chunks, most of them chosen so that their K/V ring (att_left + 8 slots, the binding's
    default push limit) wraps during the run."""
    R = C4.att_left + 8
    pos = [state_position(C4, s) for s in range(C4.streams)]
    wrap = _wrapping(C4, pos, 24, R, 48)
    rest = [s for s in np.linspace(0, C4.streams - 1, 64).astype(int) if s not in wrap][: 64 - len(wrap)]
    fresh = [s for s, p in enumerate(pos) if p == 0][:2]
    extra = sorted(set(wrap) | set(rest[: 64 - len(wrap) - len(fresh)]) | set(fresh))
    log(f"C4: {len(wrap)} of the 12-chunk streams wrap their ring; fresh streams {fresh}")
    _check_workload(C4, 4, range(C4.streams), extra=(extra, 12))


@pytest.mark.slow
def test_c4s_bf16_1024_streams_2d_front_end():
    """Every stream of the 1024-stream workload on the 2-D time x frequency front end over 4
    chunks."""
    from synth import C4S
    _check_workload(C4S, 4, range(C4S.streams))


def test_2d_front_end_fresh_streams():
    """Fresh streams through the 2-D front end (the rows before the stream start are zero at
    every stage) over 6 chunks, 2 layers, one stream and five."""
    from synth import C4S
    for S in (1, 5):
        _check_workload(C4S.replace(n_layers=2, streams=S, staggered=False, chunks=6), 6, range(S))


@pytest.mark.parametrize("bins,channels", [(64, 64), (256, 64)], ids=["bins64-fused", "bins256-separate"])
def test_2d_front_end_other_widths(bins, channels):
    """The 2-D front end with 64 mel bins and 64 channels (stage 1 and the first depthwise stage
    in one launch, half its threads idle) and with 256 bins (a stage-1 map too wide for that
    launch's LDS: the separate stage kernels), 2 layers, fresh and staggered streams."""
    from synth import C4S
    cfg = C4S.replace(name=f"C4S_b{bins}_c{channels}", n_layers=2, streams=6, mel_bins=bins, fe_channels=channels,
                      chunks=4)
    _check_workload(cfg, 4, range(cfg.streams))
    _check_workload(cfg.replace(staggered=False), 4, range(cfg.streams))


@pytest.mark.parametrize("d_model,heads", [(256, 4), (1024, 16)], ids=["d256", "d1024"])
def test_bf16_layernorm_carried_at_other_widths(d_model, heads):
    """2048 rows (1024 streams x 2 frames), where the LayerNorms before qkv, pw1 and FF2 up ride
    on the products, at 4 and 16 tiles of 64 columns per row; 64 staggered streams checked over
    4 chunks."""
    cfg = C3.replace(name=f"C3_d{d_model}_1024", n_layers=2, d_model=d_model, n_heads=heads, d_ff=4 * d_model,
                     joint_dim=0, streams=1024, chunks=4)
    _check_workload(cfg, 4, range(0, cfg.streams, 16))


@pytest.mark.slow
def test_c5_bf16_lookahead_512_streams_and_flush():
    """A fixed 64-stream subset (every 8th stream) over 8 passes, then the flush of all 64."""
    _check_workload(C5, 8, range(0, C5.streams, 8), flush=True)


@pytest.mark.parametrize("cfg", [
    # head size 16: the general attention kernel in bf16, LayerNorm launches (D not a multiple of 256)
    C1.replace(name="C1_bf16_staggered", dtype="bf16", streams=6, staggered=True, chunks=6),
    # MFMA attention with 1, 4 and 5 query rows per stream (chunk 1, chunk 4, lookahead 2 + 3)
    C3.replace(name="C3_chunk1", n_layers=2, streams=12, att_chunk=1, n_emit=1, chunks=6),
    C3.replace(name="C3_chunk4", n_layers=2, streams=12, att_chunk=4, n_emit=4, chunks=6),
    C5.replace(name="C5_la3", n_layers=2, streams=12, n_lookahead=3, chunks=6),
    # wide rings: 8 slot tiles with 2 query rows, and with 10 (register budget above 128)
    C3.replace(name="C3_left110", n_layers=2, streams=12, att_left=110, chunks=6),
    C5.replace(name="C5_left100", n_layers=2, streams=8, att_left=100, chunks=5),
], ids=["bf16-hd16", "mfma-att-1row", "mfma-att-4rows", "mfma-att-5rows-lookahead", "mfma-att-8tiles",
        "mfma-att-8tiles-10rows"])
def test_bf16_attention_shapes(cfg):
    _check_workload(cfg, cfg.chunks, range(cfg.streams))


@pytest.mark.parametrize("cfg", [
    # the depthwise conv in pw1's epilogue: kernel sizes 5 and 3 (fewer taps than the 8 older rows
    # it loads), 3 taps over 4 frames per stream (frames whose taps start inside the call), fresh
    # streams (taps reaching before the stream start)
    C3.replace(name="C3_dw5", n_layers=2, streams=40, dw_kernel=5, chunks=6),
    C3.replace(name="C3_dw3_chunk4", n_layers=2, streams=40, dw_kernel=3, att_chunk=4, n_emit=4, chunks=6),
    C3.replace(name="C3_dw9_fresh", n_layers=2, streams=40, staggered=False, chunks=6),
    # kernel size 15 (14 older rows): the separate depthwise kernel
    C3.replace(name="C3_dw15", n_layers=2, streams=40, dw_kernel=15, chunks=6),
    # 5 and 10 frames per pass (lookahead): streams whose rows cross a multiple of 64 rows get
    # their conv from the small kernel after pw1, the others in its epilogue
    C5.replace(name="C5_la3_dw", n_layers=2, streams=40, n_lookahead=3, chunks=6),
    C5.replace(name="C5_dw_40", n_layers=2, streams=40, chunks=6),
], ids=["dw5", "dw3-4rows", "dw9-fresh", "dw15-separate", "dw-5rows-crossing", "dw-10rows-crossing"])
def test_bf16_depthwise_conv_shapes(cfg):
    _check_workload(cfg, cfg.chunks, range(cfg.streams))


def test_bf16_depthwise_conv_in_128_row_tiles():
    """5120 rows (2560 streams x 2 frames): pw1 with the conv in its epilogue on 128x64 tiles
    (the tile rule would pick 128x128, which has no LDS room for the conv's rows), LayerNorm
    carried; 64 staggered streams checked over 2 chunks."""
    cfg = C3.replace(name="C3_dw_2560", n_layers=2, streams=2560, chunks=2)
    _check_workload(cfg, 2, range(0, cfg.streams, 40))


def test_bf16_single_stream_small_m_path():
    """1 stream in bf16 runs every dense product through the small-M kernel."""
    cfg = C3.replace(streams=1, staggered=False, chunks=40)
    log("bf16 1 stream x 40 chunks")
    got, ref = _run_single_stream(cfg, 40)
    for c in range(40):
        assert rel_inf(got[c], ref[c]) <= BF16_TOL, c


def test_fresh_lookahead_stream_warmup_and_flush():
    cfg = C5.replace(n_layers=3, streams=2, staggered=False)
    W = make_weights(cfg)
    enc = _enc(cfg, W, max_streams=2)
    orc = _oracle(cfg, W)
    st = orc.new_state()
    xs = make_inputs(cfg, 0, 9)
    for c in range(9):
        out, em = enc.push_chunk([0], to_dev(xs[c][None], cfg))
        ref = orc.push([st], xs[c][None].astype(np.float64))[0]
        assert em[0] == ref.shape[0]
        if ref.shape[0]:
            assert rel_inf(out.cpu().numpy()[0], ref) <= BF16_TOL
    out, frames = enc.flush([0])
    ref = orc.flush(st)
    assert frames[0] == ref.shape[0] == 8
    assert rel_inf(out.cpu().numpy()[0], ref) <= BF16_TOL


# ----------------------------------------------------------------------------- invariants

def test_batch_order_invariance_and_isolation():
    """A stream's outputs do not depend on the other streams of the call or their order, and
    a NaN in one stream's input stays in that stream."""
    cfg = C3.replace(n_layers=2, streams=24, staggered=False)
    W = make_weights(cfg)
    xs = np.stack([make_inputs(cfg, s, 6) for s in range(24)])
    perm = np.random.default_rng(0).permutation(24)
    encA = _enc(cfg, W, max_streams=24)
    encB = _enc(cfg, W, max_streams=24)
    for c in range(6):
        a, _ = encA.push_chunk(list(range(24)), to_dev(xs[:, c], cfg))
        b, _ = encB.push_chunk(perm.tolist(), to_dev(xs[perm, c], cfg))
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(a[perm], b), c
    bad = xs[:, 0].copy()
    bad[5, 0, 3] = np.nan
    encC = _enc(cfg, W, max_streams=24)
    out, _ = encC.push_chunk(list(range(24)), to_dev(bad, cfg))
    out = out.cpu().numpy()
    assert np.isnan(out[5]).any()
    assert np.isfinite(np.delete(out, 5, axis=0)).all()


def test_reset_equals_fresh_stream():
    cfg = C1
    W = make_weights(cfg)
    enc = _enc(cfg, W, max_streams=2)
    xs = make_inputs(cfg, 0, 10)
    junk = make_inputs(cfg, 1, 7)
    for c in range(7):
        enc.push_chunk([0], to_dev(junk[c][None], cfg))
    enc.reset_stream([0])
    for c in range(10):
        a, _ = enc.push_chunk([0], to_dev(xs[c][None], cfg))
        b, _ = enc.push_chunk([1], to_dev(xs[c][None], cfg))
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), c


@pytest.mark.parametrize("cfg", [C1, C3.replace(n_layers=3, streams=4, staggered=False),
                                 C5.replace(n_layers=2, streams=4, staggered=False)], ids=["f32", "bf16", "lookahead"])
def test_export_import_resume(cfg):
    W = make_weights(cfg)
    n = 30
    xs = make_inputs(cfg, 0, n)
    enc = _enc(cfg, W, max_streams=4)
    outs = []
    for c in range(n):
        o, em = enc.push_chunk([2], to_dev(xs[c][None], cfg))
        outs.append(o.cpu().numpy()[0, : em[0]])
        if c == 14:
            pos, pend, blob = enc.export_state([2])
    enc2 = _enc(cfg, W, max_streams=4)
    enc2.import_state([1], pos, pend, blob)
    for c in range(15, n):
        o, em = enc2.push_chunk([1], to_dev(xs[c][None], cfg))
        assert np.array_equal(o.cpu().numpy()[0, : em[0]], outs[c]), c


def test_import_rejects_state_of_another_config():
    """A state exported from one context imports into a context of the same config (whatever
    its capacity) and is rejected with CAC_ESTATE, changing nothing, by a context of another
    config: the header is read back from device memory."""
    from cache_aware_conformer_amd.binding import CAC_ESTATE, CacError
    cfg = C1
    W = make_weights(cfg)
    enc = _enc(cfg, W, max_streams=2)
    xs = make_inputs(cfg, 0, 3)
    for c in range(3):
        enc.push_chunk([0], to_dev(xs[c][None], cfg))
    pos, pend, blob = enc.export_state([0])
    other = cfg.replace(d_ff=128)
    enc2 = _enc(other, make_weights(other), max_streams=2)
    with pytest.raises(CacError) as ei:
        enc2.import_state([1], pos, pend, blob)
    assert ei.value.code == CAC_ESTATE
    assert enc2.stream_info(1).pos == 0
    enc3 = _enc(cfg, W, max_streams=3, max_push_frames=4)
    enc3.import_state([2], pos, pend, blob)
    assert enc3.stream_info(2).pos == pos[0] == 6


def test_poisoned_cache_slots_never_reach_outputs():
    """With NaN in every unwritten cache slot, outputs are finite and identical to the zero
    reset: nothing read from a slot that does not hold a valid row reaches an output (attention
    stages whole rings and must discard such slots exactly, never as 0 * NaN)."""
    from cache_aware_conformer_amd import CAC_FLAG_POISON
    from synth import C4S
    for cfg in (C1, C4.replace(n_layers=2, streams=3, staggered=False), C4S.replace(n_layers=2, streams=3, staggered=False)):
        W = make_weights(cfg)
        a = _enc(cfg, W, max_streams=3)
        b = _enc(cfg, W, max_streams=3, flags=CAC_FLAG_POISON)
        xs = np.stack([make_inputs(cfg, s, 40) for s in range(3)])
        for c in range(40):
            oa, _ = a.push_chunk([0, 1, 2], to_dev(xs[:, c], cfg))
            ob, _ = b.push_chunk([0, 1, 2], to_dev(xs[:, c], cfg))
            ob = ob.cpu().numpy()
            assert np.isfinite(ob).all(), c
            assert np.array_equal(oa.cpu().numpy(), ob), c


@pytest.mark.parametrize("cfg", [C1, C3.replace(n_layers=2, streams=12, staggered=False),
                                 C5.replace(n_layers=2, streams=3, staggered=False)], ids=["f32", "bf16-mfma", "lookahead"])
def test_graph_replay_matches_direct_launches(cfg):
    """Pushes replayed from a recorded graph (re-pointed to a different input slice and output
    buffer every call) equal direct launches bit for bit, with unrelated eager work and host
    synchronisations between replays."""
    W = make_weights(cfg)
    S = cfg.streams
    g = _enc(cfg, W, max_streams=S)
    d = _enc(cfg, W, max_streams=S)
    d.set_graph(False)
    xs = to_dev(np.stack([make_inputs(cfg, s, 14) for s in range(S)]).swapaxes(0, 1).copy(), cfg)
    outs_g = [torch.zeros((S, cfg.n_emit, cfg.joint_dim or cfg.d_model), dtype=torch.float32, device="cuda:0")
              for _ in range(3)]
    scratch = torch.randn(1 << 16, device="cuda:0")
    for c in range(14):
        og, eg = g.push_chunk(list(range(S)), xs[c], outs_g[c % 3])
        scratch.mul_(1.0001).add_(0.5)              # unrelated eager work between replays
        od, ed = d.push_chunk(list(range(S)), xs[c])
        torch.cuda.synchronize()
        assert np.array_equal(eg, ed)
        a, b = og.cpu().numpy()[:, : int(eg.max())], od.cpu().numpy()[:, : int(ed.max())]
        if not np.array_equal(a, b):
            torch.cuda.synchronize()
            a2 = og.cpu().numpy()[:, : int(eg.max())]
            raise AssertionError(f"chunk {c}: graph/direct differ; nan graph {int(np.isnan(a).sum())} direct "
                                 f"{int(np.isnan(b).sum())}; max|diff| {float(np.nanmax(np.abs(a - b)))}; zeros in "
                                 f"graph rows {[(int((r == 0).sum())) for r in a.reshape(-1, a.shape[-1])]}; "
                                 f"graph output changed on a second read: {not np.array_equal(a, a2)}")


def test_profiled_launches_time_every_kernel_and_match_graph_replay():
    """Profiled pushes (direct launches, each kernel timed by events bound to its own dispatch)
    give the same outputs as graph replays, and every kernel of every push is timed."""
    cfg = C2.replace(n_layers=3)
    W = make_weights(cfg)
    g = _enc(cfg, W, max_streams=1)
    p = _enc(cfg, W, max_streams=1)
    xs = make_inputs(cfg, 0, 4)
    p.profile(True)
    for c in range(4):
        og, _ = g.push_chunk([0], to_dev(xs[c][None], cfg))
        op, _ = p.push_chunk([0], to_dev(xs[c][None], cfg))
        torch.cuda.synchronize()
        assert np.array_equal(og.cpu().numpy(), op.cpu().numpy()), c
    prof = p.profile_read()
    p.profile(False)
    # per push: 8 dense products per layer + attention per layer, the joint, and the input
    # kernel (which also advances the positions)
    assert sum(v[0] for v in prof.values()) == 4 * (9 * cfg.n_layers + 2)
    for n, (launches, ms, _, _) in prof.items():
        assert launches % 4 == 0 and ms > 0.0, n


def test_profile_replay_times_one_kernel_family():
    """The family replay chains exactly the family's launches of the last replayed push."""
    from cache_aware_conformer_amd.binding import CacError
    cfg = C2.replace(n_layers=3)
    enc = _enc(cfg, make_weights(cfg), max_streams=1)
    xs = make_inputs(cfg, 0, 3)
    for c in range(2):
        enc.push_chunk([0], to_dev(xs[c][None], cfg))
    torch.cuda.synchronize()
    rep = enc.profile_replay("gemm_tworow_f32", reps=5)
    assert rep["launches"] == 8 * cfg.n_layers + 1   # 8 dense products per layer + the joint
    assert rep["us_per_launch"] > 0.0 and rep["bytes_per_launch"] > 0.0
    att = enc.profile_replay("attention", reps=5)
    assert att["launches"] == cfg.n_layers
    # the replayed attention work is that of the last push's cache fill, not of the push that
    # recorded the graph: one more push of 2 frames reads 2 more K/V rows of D float32 values
    # each (K and V), and 6 flops per query row, key row and dimension
    enc.push_chunk([0], to_dev(xs[2][None], cfg))
    torch.cuda.synchronize()
    att3 = enc.profile_replay("attention", reps=5)
    assert att3["bytes_per_launch"] - att["bytes_per_launch"] == pytest.approx(2 * 2 * cfg.d_model * 4)
    assert att3["flops_per_launch"] - att["flops_per_launch"] == pytest.approx(6 * 2 * 2 * cfg.d_model)
    with pytest.raises(CacError):
        enc.profile_replay("no_such_kernel", reps=5)
