"""Host-side tests of the C ABI: the library loads and exports every declared symbol, the
parameter/state layouts agree with the binding, and argument validation and stream
bookkeeping behave as the header states. No device work: dry-run contexts only."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import cache_aware_conformer_amd as cac
from cache_aware_conformer_amd.binding import CAC_EINVAL, CAC_ENODEV, CAC_ENOMEM, CAC_ESTATE, CacError, cac_config
from synth import C1, C2, C3, C4, C4S, C5, make_weights, weight_names

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h")]


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(cac_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = cac.load()
    names = header_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", cac.binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (cac_[a-z_]+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(names) == set(cac.binding.SIGNATURES)


def test_int8_weights_config_and_push_limits():
    """int8 dense weights: no front end or lookahead; a push carries at most two rows."""
    from synth import C2Q
    lib = cac.load()
    for field, value in [("frontend", 1), ("n_lookahead", 8), ("d_ff", 2112)]:
        c = cac.make_config(C2Q, max_streams=2)
        setattr(c, field, value)
        if field == "n_lookahead":
            c.att_right = 3
        assert lib.cac_workspace_bytes(C.byref(c)) == 0, field
    c16 = cac.make_config(C2, max_streams=2)
    c8 = cac.make_config(C2Q, max_streams=2)
    assert 0 < lib.cac_workspace_bytes(C.byref(c8)) < lib.cac_workspace_bytes(C.byref(c16))
    enc = dry(C2Q, streams=2)
    assert push(enc, [0], 2)[0] == CAC_ENODEV
    assert push(enc, [0, 1], 2)[0] == CAC_EINVAL
    assert push(enc, [1], 4)[0] == CAC_EINVAL


@pytest.mark.parametrize("cfg", [C1, C2, C3, C4, C5, C4S], ids=lambda c: c.name)
def test_param_and_state_layouts(cfg):
    lib = cac.load()
    c = cac.make_config(cfg)
    n = lib.cac_param_count(C.byref(c))
    assert n == sum(int(np.prod(s)) for _, s in cac.param_order(cfg))
    # the generator and the binding name the same tensors in the same order
    assert [nm for nm, _ in cac.param_order(cfg)] == [nm for nm, *_ in weight_names(cfg)]
    L, Lc, D = cfg.n_layers, cfg.att_left, cfg.d_model
    expect = 2 * L * Lc * D + L * (cfg.dw_kernel - 1) * D
    expect += cfg.mel_tail * cfg.mel_bins if cfg.frontend else 0
    expect += cfg.n_lookahead * D
    assert lib.cac_state_floats(C.byref(c)) == 4 + expect  # 4-word header in front
    assert lib.cac_workspace_bytes(C.byref(c)) > 0


@pytest.mark.parametrize("field,value", [("d_model", 100), ("n_heads", 3), ("d_ff", 100), ("dtype", 7),
                                         ("max_streams", 0), ("att_chunk", 0), ("max_push_frames", 3),
                                         ("att_right", 2), ("dw_kernel", 0), ("n_layers", 0)])
def test_bad_config_rejected(field, value):
    lib = cac.load()
    c = cac.make_config(C1)
    setattr(c, field, value)
    assert lib.cac_param_count(C.byref(c)) == 0
    assert lib.cac_workspace_bytes(C.byref(c)) == 0
    ctx = C.c_void_p()
    rc = lib.cac_create_streams(C.byref(c), None, 0, None, 0, None, C.byref(ctx))
    assert rc == CAC_EINVAL and not ctx.value
    assert lib.cac_last_error(None)


def test_create_rejects_small_workspace_and_wrong_param_count():
    lib = cac.load()
    c = cac.make_config(C1)
    flat = cac.pack_params(C1, make_weights(C1))
    ctx = C.c_void_p()
    fp = flat.ctypes.data_as(C.POINTER(C.c_float))
    need = lib.cac_workspace_bytes(C.byref(c))
    # fake (never touched) aligned address: the size check comes before any device call
    assert lib.cac_create_streams(C.byref(c), fp, flat.size, C.c_void_p(1 << 20), need - 1, None, C.byref(ctx)) == CAC_ENOMEM
    assert b"too small" in lib.cac_last_error(None)
    assert lib.cac_create_streams(C.byref(c), fp, flat.size - 1, C.c_void_p(1 << 20), need, None, C.byref(ctx)) == CAC_EINVAL
    assert lib.cac_create_streams(C.byref(c), fp, flat.size, C.c_void_p((1 << 20) + 4), need, None, C.byref(ctx)) == CAC_EINVAL


def dry(cfg, streams=4):
    return cac.StreamingEncoder(cfg, make_weights(cfg), max_streams=streams, flags=cac.CAC_FLAG_DRY_RUN)


def push(enc, ids, n_frames):
    ids_a = np.asarray(ids, dtype=np.int32)
    em = np.zeros(len(ids_a), dtype=np.int32)
    rc = enc.lib.cac_push_chunk(enc.ctx, len(ids_a), ids_a.ctypes.data_as(C.POINTER(C.c_int32)), n_frames,
                                C.c_void_p(16), C.c_void_p(32), em.ctypes.data_as(C.POINTER(C.c_int32)))
    return rc, em


def test_push_validation_and_positions():
    enc = dry(C1)
    assert push(enc, [0, 1], 2)[0] == CAC_ENODEV          # validated, bookkept, no device
    assert enc.stream_info(0).pos == 2 and enc.stream_info(2).pos == 0
    assert push(enc, [0], 3)[0] == CAC_EINVAL             # off the chunk grid
    assert push(enc, [0], 10)[0] == CAC_EINVAL            # beyond max_push_frames
    assert push(enc, [4], 2)[0] == CAC_EINVAL             # unknown id
    assert push(enc, [-1], 2)[0] == CAC_EINVAL
    assert push(enc, [1, 1], 2)[0] == CAC_EINVAL          # duplicate id
    assert b"twice" in enc.lib.cac_last_error(enc.ctx)
    assert push(enc, [], 2)[0] == CAC_EINVAL              # empty call
    assert push(enc, [0, 1, 2, 3, 0], 2)[0] == CAC_EINVAL  # more ids than max_streams
    assert b"count" in enc.lib.cac_last_error(enc.ctx)
    assert enc.stream_info(1).pos == 2                     # failed calls change nothing
    assert push(enc, [3, 0], 4)[0] == CAC_ENODEV
    assert enc.stream_info(0).pos == 6 and enc.stream_info(3).pos == 4
    rc = enc.lib.cac_push_chunk(enc.ctx, 1, np.zeros(1, np.int32).ctypes.data_as(C.POINTER(C.c_int32)), 2, None, None, None)
    assert rc == CAC_EINVAL
    rc = enc.lib.cac_push_chunk(enc.ctx, 1, np.zeros(1, np.int32).ctypes.data_as(C.POINTER(C.c_int32)), 2,
                                C.c_void_p(16), C.c_void_p(16), None)
    assert rc == CAC_EINVAL and b"different" in enc.lib.cac_last_error(enc.ctx)


def test_flush_then_push_needs_reset():
    enc = dry(C1)
    push(enc, [2], 2)
    with pytest.raises(CacError) as e:
        enc.flush([2])
    assert e.value.code == CAC_ENODEV
    assert enc.stream_info(2).flushed
    assert push(enc, [2], 2)[0] == CAC_ESTATE
    assert push(enc, [1, 2], 2)[0] == CAC_ESTATE
    assert enc.stream_info(1).pos == 0
    with pytest.raises(CacError):
        enc.reset_stream([2])
    info = enc.stream_info(2)
    assert info.pos == 0 and not info.flushed
    assert push(enc, [2], 2)[0] == CAC_ENODEV


def test_lookahead_bookkeeping():
    """Streams warm up until n_emit + n_lookahead frames are pending, then emit n_emit per
    push; a flush emits what is pending."""
    cfg = C5.replace(n_layers=1, streams=3)
    enc = dry(cfg, streams=3)
    seen = []
    for k in range(6):
        rc, em = push(enc, [0, 1] if k < 3 else [0, 1, 2], 2)
        assert rc == CAC_ENODEV
        seen.append(em.tolist())
    assert [s[0] for s in seen] == [0, 0, 0, 0, 2, 2]
    assert seen[5][2] == 0
    assert push(enc, [0], 4)[0] == CAC_EINVAL   # the lookahead variant takes n_emit frames
    i0, i2 = enc.stream_info(0), enc.stream_info(2)
    assert (i0.pos, i0.pending) == (4, 8) and (i2.pos, i2.pending) == (0, 6)
    frames = np.zeros(2, np.int32)
    ids = np.array([0, 2], np.int32)
    rc = enc.lib.cac_flush(enc.ctx, 2, ids.ctypes.data_as(C.POINTER(C.c_int32)), C.c_void_p(16),
                           frames.ctypes.data_as(C.POINTER(C.c_int32)))
    assert rc == CAC_ENODEV and frames.tolist() == [8, 6]
    assert enc.stream_info(0).pos == 12 and enc.stream_info(2).pos == 6


def test_frontend_push_is_one_mel_chunk():
    enc = dry(C4.replace(n_layers=1, streams=2), streams=2)
    assert push(enc, [0], 4)[0] == CAC_EINVAL
    assert push(enc, [0], 2)[0] == CAC_ENODEV


def _blob(enc, n, header=None):
    """Zero state blobs of n streams with a header (the context's own by default)."""
    b = np.zeros((n, enc.sfloats), np.float32)
    b[:, :4] = enc.state_header() if header is None else header
    return b


def test_import_validation():
    enc = dry(C5.replace(n_layers=1, streams=2), streams=2)
    ids = np.array([0], np.int32)
    ip = lambda a: np.asarray(a, np.int32).ctypes.data_as(C.POINTER(C.c_int32))  # noqa: E731
    lib = enc.lib
    blob = _blob(enc, 1)
    bp = blob.ctypes.data_as(C.c_void_p)
    assert lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), ip([9]), bp) == CAC_ESTATE
    assert lib.cac_import_state(enc.ctx, 1, ip(ids), ip([-2]), ip([8]), bp) == CAC_ESTATE
    assert lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), ip([8]), None) == CAC_EINVAL
    assert lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), ip([8]), bp) == CAC_ENODEV
    enc2 = dry(C1)
    b2 = _blob(enc2, 1)
    assert lib.cac_import_state(enc2.ctx, 1, ip(ids), ip([3]), None, b2.ctypes.data_as(C.c_void_p)) == CAC_ESTATE


@pytest.mark.parametrize("field,value", [("d_ff", 128), ("att_left", 69), ("n_heads", 2), ("dtype", 1),
                                         ("joint_dim", 640), ("n_layers", 3)])
def test_import_rejects_a_blob_of_another_config(field, value):
    """The state blob carries the config it was made with: a blob whose header names any other
    model config is rejected with CAC_ESTATE, and the stream keeps its state."""
    enc = dry(C1, streams=2)
    other = cac.make_config(C1, max_streams=2, flags=cac.binding.CAC_FLAG_DRY_RUN)
    setattr(other, field, value)
    h = np.zeros(4, np.uint32)
    assert enc.lib.cac_state_header(C.byref(other), h.ctypes.data_as(C.POINTER(C.c_uint32))) == 0
    assert not np.array_equal(h.view(np.float32), enc.state_header())
    ids = np.array([1], np.int32)
    ip = lambda a: np.asarray(a, np.int32).ctypes.data_as(C.POINTER(C.c_int32))  # noqa: E731
    bad = _blob(enc, 1, h.view(np.float32))
    assert enc.lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), None, bad.ctypes.data_as(C.c_void_p)) == CAC_ESTATE
    assert b"different config" in enc.lib.cac_last_error(enc.ctx)
    assert enc.stream_info(1).pos == 0
    # a blob without any header (old layout, or not a state blob) is rejected too
    raw = _blob(enc, 1, np.zeros(4, np.float32))
    assert enc.lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), None, raw.ctypes.data_as(C.c_void_p)) == CAC_ESTATE
    # the context's own header passes validation (a dry-run context then stops before device work)
    good = _blob(enc, 1)
    assert enc.lib.cac_import_state(enc.ctx, 1, ip(ids), ip([4]), None, good.ctypes.data_as(C.c_void_p)) == CAC_ENODEV


def test_state_header_ignores_capacity_and_flags():
    """Contexts that differ only in capacity (max_streams, max_push_frames) or flags share a
    header: a stream's state moves between them."""
    lib = cac.load()
    a = cac.make_config(C3, max_streams=4)
    b = cac.make_config(C3, max_streams=1024, max_push_frames=16, flags=cac.binding.CAC_FLAG_POISON)
    ha, hb = np.zeros(4, np.uint32), np.zeros(4, np.uint32)
    assert lib.cac_state_header(C.byref(a), ha.ctypes.data_as(C.POINTER(C.c_uint32))) == 0
    assert lib.cac_state_header(C.byref(b), hb.ctypes.data_as(C.POINTER(C.c_uint32))) == 0
    assert np.array_equal(ha, hb) and ha[0] == 0x53434143 and ha[1] == 1
    bad = cac.make_config(C3)
    bad.d_model = 100
    assert lib.cac_state_header(C.byref(bad), ha.ctypes.data_as(C.POINTER(C.c_uint32))) == CAC_EINVAL


def test_profile_replay_needs_a_replayed_push_graph():
    enc = dry(C1)
    us, n = C.c_double(), C.c_int32()
    assert enc.lib.cac_profile_replay(enc.ctx, b"gemm", 5, C.byref(us), C.byref(n), None, None) == CAC_EINVAL
    assert b"no push graph" in enc.lib.cac_last_error(enc.ctx)
    assert enc.lib.cac_profile_replay(enc.ctx, None, 5, None, None, None, None) == CAC_EINVAL
    assert enc.lib.cac_profile_replay(enc.ctx, b"gemm", 0, None, None, None, None) == CAC_EINVAL


# ----------------------------------------------------------------------- greedy decoding ABI

def test_decoder_param_layout_and_validation():
    from synth import D1, dec_weight_names, make_dec_weights
    lib = cac.load()
    c = cac.binding.make_dec_config(D1, max_streams=4)
    n = lib.cac_dec_param_count(C.byref(c))
    assert n == sum(int(np.prod(s)) for _, s in cac.binding.dec_param_order(D1))
    assert [nm for nm, _ in cac.binding.dec_param_order(D1)] == [nm for nm, *_ in dec_weight_names(D1)]
    assert lib.cac_dec_workspace_bytes(C.byref(c)) > 0
    for field, value in [("joint_dim", 100), ("pred_hidden", 96), ("pred_layers", 0), ("vocab", 0),
                         ("max_symbols", 0), ("max_streams", 0), ("max_frames", 17)]:
        bad = cac.binding.make_dec_config(D1, max_streams=4)
        setattr(bad, field, value)
        assert lib.cac_dec_param_count(C.byref(bad)) == 0, field
        assert lib.cac_dec_workspace_bytes(C.byref(bad)) == 0, field
    dec = cac.StreamingDecoder(D1, make_dec_weights(D1), max_streams=4, flags=cac.CAC_FLAG_DRY_RUN)
    ip = lambda a: np.asarray(a, np.int32).ctypes.data_as(C.POINTER(C.c_int32))  # noqa: E731
    z = C.c_void_p(256)
    assert lib.cac_dec_greedy(dec.ctx, 1, ip([0]), 2, z, z, None, z) == CAC_ENODEV
    assert lib.cac_dec_greedy(dec.ctx, 2, ip([1, 1]), 2, z, z, None, z) == CAC_EINVAL
    assert b"twice" in lib.cac_dec_last_error(dec.ctx)
    assert lib.cac_dec_greedy(dec.ctx, 1, ip([4]), 2, z, z, None, z) == CAC_EINVAL
    assert lib.cac_dec_greedy(dec.ctx, 1, ip([0]), 3, z, z, None, z) == CAC_EINVAL   # max_frames is 2
    assert lib.cac_dec_greedy(dec.ctx, 1, ip([0]), 0, z, z, None, z) == CAC_EINVAL
    assert lib.cac_dec_greedy(dec.ctx, 1, ip([0]), 2, None, z, None, z) == CAC_EINVAL
    assert lib.cac_dec_greedy(dec.ctx, 0, ip([0]), 2, z, z, None, z) == CAC_EINVAL
    assert lib.cac_dec_reset(dec.ctx, 1, ip([3])) == CAC_ENODEV
    assert lib.cac_dec_reset(dec.ctx, 1, ip([-1])) == CAC_EINVAL
    with pytest.raises(CacError):
        cac.StreamingDecoder(D1, {k: v[:1] for k, v in make_dec_weights(D1).items()}, max_streams=4,
                             flags=cac.CAC_FLAG_DRY_RUN)


# ----------------------------------------------------------------------- streaming log-mel ABI

def test_mel_config_and_push_validation():
    from synth import A4
    lib = cac.load()
    c = cac.binding.make_mel_config(A4, max_streams=4)
    assert lib.cac_mel_workspace_bytes(C.byref(c)) > 0
    for field, value in [("n_fft", 500), ("win_length", 600), ("win_length", 160), ("win_length", 401), ("n_mels", 0),
                         ("fmax", 9000.0), ("preemph", 1.5), ("max_hops", 0), ("max_streams", 0), ("out_dtype", 5)]:
        bad = cac.binding.make_mel_config(A4, max_streams=4)
        setattr(bad, field, value)
        assert lib.cac_mel_workspace_bytes(C.byref(bad)) == 0, field
    mel = cac.StreamingMel(A4, max_streams=4, flags=cac.CAC_FLAG_DRY_RUN)
    ip = lambda a: np.asarray(a, np.int32).ctypes.data_as(C.POINTER(C.c_int32))  # noqa: E731
    p = C.c_void_p(256)
    assert lib.cac_mel_push(mel.ctx, 1, ip([0]), 2560, p, p) == CAC_ENODEV
    assert lib.cac_mel_push(mel.ctx, 1, ip([0]), 2561, p, p) == CAC_EINVAL
    assert lib.cac_mel_push(mel.ctx, 1, ip([0]), 160 * 17, p, p) == CAC_EINVAL
    assert lib.cac_mel_push(mel.ctx, 2, ip([3, 3]), 160, p, p) == CAC_EINVAL
    assert lib.cac_mel_push(mel.ctx, 1, ip([0]), 160, None, p) == CAC_EINVAL
    assert lib.cac_mel_reset(mel.ctx, 1, ip([9])) == CAC_EINVAL


def _beam_cfg(**kw):
    from cache_aware_conformer_amd.binding import make_beam_config
    from synth import B8
    c = make_beam_config(B8, max_streams=4, max_frames=32)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_beam_config_validation_and_sizes():
    """Beam search: the greedy decoder's parameter count, a workspace that grows with the
    beam, the utterance count and the frames, and invalid sizes refused."""
    from synth import B8
    lib = cac.load()
    dc = cac.binding.make_dec_config(B8.replace(streams=4, frames=8), max_streams=4, max_frames=8)
    assert lib.cac_beam_param_count(C.byref(_beam_cfg())) == lib.cac_dec_param_count(C.byref(dc)) > 0
    base = lib.cac_beam_workspace_bytes(C.byref(_beam_cfg()))
    assert base > 0
    for kw in ({"beam": 8}, {"max_streams": 8}, {"max_frames": 64}):
        small = lib.cac_beam_workspace_bytes(C.byref(_beam_cfg(**{**kw, list(kw)[0]: list(kw.values())[0] // 2})))
        assert small < lib.cac_beam_workspace_bytes(C.byref(_beam_cfg(**kw)))
    for kw in ({"beam": 0}, {"beam": 9}, {"vocab": 2047}, {"max_symbols": 0}, {"max_symbols": 17}, {"max_streams": 0},
               {"max_streams": 4097}, {"max_frames": 0}, {"max_frames": 4097}, {"score_norm": 2},
               {"joint_dim": 100}, {"pred_hidden": 32}, {"pred_layers": 0}, {"flags": 0x40}):
        assert lib.cac_beam_workspace_bytes(C.byref(_beam_cfg(**kw))) == 0, kw
        assert lib.cac_beam_param_count(C.byref(_beam_cfg(**kw))) == 0, kw


def test_beam_decode_argument_checks_on_a_dry_context():
    from cache_aware_conformer_amd import BeamSearch
    from cache_aware_conformer_amd.binding import CAC_FLAG_DRY_RUN
    from synth import B8
    cfg = B8.replace(streams=4, frames=16)
    W = {nm: np.zeros(shape, np.float32) for nm, shape in cac.binding.dec_param_order(cfg)}
    bs = BeamSearch(cfg, W, flags=CAC_FLAG_DRY_RUN)
    lib, ctx = bs.lib, bs.ctx
    lens = np.array([16, 3, 0, 1], np.int32)
    lp = lens.ctypes.data_as(C.POINTER(C.c_int32))
    fake = 1 << 20
    assert lib.cac_beam_decode(ctx, 4, lp, 16, fake, 0, fake, fake, fake, None) == CAC_ENODEV
    assert lib.cac_beam_decode(ctx, 5, lp, 16, fake, 0, fake, fake, fake, None) == CAC_EINVAL   # too many
    assert lib.cac_beam_decode(ctx, 4, lp, 17, fake, 0, fake, fake, fake, None) == CAC_EINVAL   # frames
    assert lib.cac_beam_decode(ctx, 4, lp, 15, fake, 0, fake, fake, fake, None) == CAC_EINVAL   # 16 > 15
    assert lib.cac_beam_decode(ctx, 4, lp, 16, fake, -1, fake, fake, fake, None) == CAC_EINVAL  # max_steps
    assert lib.cac_beam_decode(ctx, 4, lp, 16, fake + 4, 0, fake, fake, fake, None) == CAC_EINVAL  # alignment
    assert lib.cac_beam_decode(ctx, 4, None, 16, fake, 0, fake, fake, fake, None) == CAC_EINVAL
    assert lib.cac_beam_decode(ctx, 4, lp, 16, fake, 0, None, fake, fake, None) == CAC_EINVAL
    assert b"max_steps" in lib.cac_beam_last_error(ctx) or True


@pytest.mark.parametrize("dtype,path,M,N,K", [
    ("bf16", 13, 64, 64, 128),    # no such path
    ("f32", 3, 64, 64, 128),      # MFMA paths take bf16 only
    ("bf16", 3, 64, 64, 96),      # K not a multiple of 64
    ("bf16", 4, 64, 12, 128),     # N not a multiple of 8
    ("bf16", 11, 64, 64, 192),    # two wave groups: K a multiple of 128
    ("bf16", 10, 64, 64, 384),    # four wave groups: K a multiple of 256
    ("bf16", 7, 64, 200, 256),    # split-K partials: N a multiple of 256
])
def test_test_gemm_rejects_shapes_a_path_does_not_take(dtype, path, M, N, K):
    """The test GEMM entry points validate path and shape on the host before any device work
    (the device pointers are stand-ins that are never touched)."""
    lib = cac.load()
    dt = cac.binding.CAC_BF16 if dtype == "bf16" else cac.binding.CAC_F32
    fake = C.c_void_p(0x1000)
    for fn in (lib.cac_test_gemm, lib.cac_test_gemm_noalloc):
        rc = fn(dt, path, M, N, K, fake, fake, None, fake, None)
        assert rc == CAC_EINVAL, (fn, rc)
        assert lib.cac_last_error(None).decode()
