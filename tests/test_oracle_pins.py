"""Pins of the float64 oracle against things other than itself: torch CPU library routines,
brute-force Python loops, closed forms, and the streaming spec's own gate (a chunk-by-chunk
cached encode equals the offline masked encode)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import Oracle, layer_norm, relshift, silu, sinusoid_rows
from oracle.brute import attention_brute
from synth import C1, C2, make_inputs, make_weights
from synth.configs import EncConfig



@pytest.fixture(autouse=True)
def _float64_default():
    """torch reference ops of this module run in float64; the default is restored afterwards
    so that tests collected later (the GPU parity tests) allocate float32 as they expect."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def tiny(**kw):
    base = dict(name="tiny", seed=11, n_layers=2, d_model=8, n_heads=2, d_ff=16, joint_dim=6,
                dtype="f32", chunks=12)
    base.update(kw)
    return EncConfig(**base)


def T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------------- library routines

def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    x, g, b = rng.standard_normal((7, 64)) * 3 + 1, rng.standard_normal(64), rng.standard_normal(64)
    ref = F.layer_norm(T(x), (64,), T(g), T(b), eps=1e-5).numpy()
    assert np.abs(layer_norm(x, g, b) - ref).max() < 1e-12


def test_silu_matches_torch_including_large_inputs():
    x = np.linspace(-800, 800, 2001)
    assert np.abs(silu(x) - F.silu(T(x)).numpy()).max() < 1e-12


def test_feed_forward_matches_torch_modules():
    cfg = tiny(d_model=16, d_ff=64)
    orc = Oracle(cfg, make_weights(cfg))
    W = orc.W
    x = np.random.default_rng(1).standard_normal((5, 16))
    ln = torch.nn.LayerNorm(16, eps=1e-5)
    l1, l2 = torch.nn.Linear(16, 64), torch.nn.Linear(64, 16)
    with torch.no_grad():
        ln.weight.copy_(T(W["l0.ff1.ln_g"])); ln.bias.copy_(T(W["l0.ff1.ln_b"]))
        l1.weight.copy_(T(W["l0.ff1.w1"]).T); l1.bias.copy_(T(W["l0.ff1.b1"]))
        l2.weight.copy_(T(W["l0.ff1.w2"]).T); l2.bias.copy_(T(W["l0.ff1.b2"]))
        ref = l2(F.silu(l1(ln(T(x))))).numpy()
    assert np.abs(orc.feed_forward(x, "l0.ff1.") - ref).max() < 1e-12


def test_conv_module_matches_torch_conv1d():
    """LN -> pw1 -> GLU -> causal depthwise (left pad 8, groups=D) -> SiLU -> pw2, built from
    torch.nn.functional routines (readings A12-A16)."""
    cfg = tiny(d_model=16)
    orc = Oracle(cfg, make_weights(cfg))
    W, D, K = orc.W, 16, cfg.dw_kernel
    x = np.random.default_rng(2).standard_normal((13, D))
    y = F.layer_norm(T(x), (D,), T(W["l1.conv.ln_g"]), T(W["l1.conv.ln_b"]), eps=1e-5)
    g = F.glu(F.linear(y, T(W["l1.conv.pw1"]).T, T(W["l1.conv.pw1_b"])), dim=-1)
    gt = F.pad(g.T.unsqueeze(0), (K - 1, 0))
    d = F.conv1d(gt, T(W["l1.conv.dw"]).unsqueeze(1), T(W["l1.conv.dw_b"]), groups=D)[0].T
    ref = F.linear(F.silu(d), T(W["l1.conv.pw2"]).T, T(W["l1.conv.pw2_b"])).numpy()
    assert np.abs(orc.conv_offline(x, 1) - ref).max() < 1e-12


def test_frontend_matches_torch_strided_conv1d():
    """Offline subsampling = three torch conv1d(stride 2, kernel 3) with left zero pad 2,
    ReLU after the first two (reading A21)."""
    cfg = tiny(d_model=16, frontend=True, mel_bins=8)
    orc = Oracle(cfg, make_weights(cfg))
    mel = np.random.default_rng(3).standard_normal((48, 8))
    x = T(mel).T.unsqueeze(0)
    for i in (1, 2, 3):
        x = F.conv1d(F.pad(x, (2, 0)), T(orc.W[f"fe.c{i}.w"]), T(orc.W[f"fe.c{i}.b"]), stride=2)
        if i < 3:
            x = F.relu(x)
    ref = x[0].T.numpy()
    out = orc.frontend_offline(mel)
    assert out.shape == (6, 16)
    assert np.abs(out - ref).max() < 1e-12


def test_attention_special_case_is_textbook_sdpa():
    """u = v = 0 and Wpos = 0 remove the position term: the block reduces to masked scaled
    dot-product attention (torch CPU), with Wo = I, bo = 0 exposing o itself."""
    cfg = tiny(d_model=16, n_heads=4, att_left=3)
    W = make_weights(cfg)
    for l in range(cfg.n_layers):
        W[f"l{l}.att.pos_u"][:] = 0; W[f"l{l}.att.pos_v"][:] = 0; W[f"l{l}.att.wpos"][:] = 0
        W[f"l{l}.att.wo"] = np.eye(16, dtype=np.float32); W[f"l{l}.att.bo"][:] = 0
    orc = Oracle(cfg, W)
    y = np.random.default_rng(4).standard_normal((11, 16))
    q, k, v = (T(a).permute(1, 0, 2) for a in orc.qkv(y, 0))
    pos = np.arange(11)
    mask = T(orc.visible(pos[:, None], pos[None, :]).astype(np.float64)).bool()
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask).permute(1, 0, 2).reshape(11, 16)
    assert np.abs(orc.mhsa_offline(y, 0) - ref.numpy()).max() < 1e-12


def test_attention_single_visible_key_returns_its_value():
    """With Lc = 0 and a chunk of 1, each frame sees only itself: o = v (closed form)."""
    cfg = tiny(d_model=8, att_left=0, att_chunk=1)
    W = make_weights(cfg)
    W["l0.att.wo"] = np.eye(8, dtype=np.float32); W["l0.att.bo"][:] = 0
    orc = Oracle(cfg, W)
    y = np.random.default_rng(5).standard_normal((6, 8))
    _, _, v = orc.qkv(y, 0)
    assert np.abs(orc.mhsa_offline(y, 0) - v.reshape(6, 8)).max() < 1e-12


# ----------------------------------------------------------------------- closed forms

def test_sinusoid_closed_form():
    D = 16
    pe = sinusoid_rows(np.array([0, 1, 5, -3]), D)
    assert np.allclose(pe[0, 0::2], 0.0) and np.allclose(pe[0, 1::2], 1.0)
    assert math.isclose(pe[2, 0], math.sin(5.0)) and math.isclose(pe[2, 1], math.cos(5.0))
    assert math.isclose(pe[3, 14], math.sin(-3 * 10000 ** (-14 / 16)))
    assert np.allclose(pe[:, 0::2] ** 2 + pe[:, 1::2] ** 2, 1.0)


def test_relshift_picks_relative_offset():
    rng = np.random.default_rng(6)
    for Tn in (1, 2, 5, 9):
        bd = rng.standard_normal((3, Tn, 2 * Tn - 1))
        out = relshift(bd)
        for h in range(3):
            for i in range(Tn):
                for j in range(Tn):
                    assert out[h, i, j] == bd[h, i, Tn - 1 - i + j]


def test_mask_window_is_chunk_start_minus_lc_to_chunk_start_plus_one():
    """Streaming spec, "Why this is provably correct": with chunks of 2 and a left context of
    70, a frame sees the 70 frames before its chunk's first frame plus its own chunk."""
    orc = Oracle(C2, {})
    for p in (0, 1, 2, 3, 70, 71, 140, 141, 1001):
        cs = p - p % 2
        keys = [q for q in range(-5, p + 10) if orc.visible(p, q)]
        assert keys == list(range(max(0, cs - 70), cs + 2))
        assert len(keys) <= 72


# ----------------------------------------------------------------------- brute force

@pytest.mark.parametrize("d_model,n_heads,att_left,att_chunk", [(8, 2, 3, 2), (4, 2, 70, 2), (8, 4, 0, 2),
                                                                (8, 2, 2, 1)])
def test_attention_offline_and_streaming_match_brute_force(d_model, n_heads, att_left, att_chunk):
    cfg = tiny(d_model=d_model, n_heads=n_heads, att_left=att_left, att_chunk=att_chunk)
    orc = Oracle(cfg, make_weights(cfg))
    Tn = 8
    y = np.random.default_rng(7).standard_normal((Tn, d_model))
    Wl = {k: v.tolist() for k, v in orc.W.items() if k.startswith("l0.att.")}
    ref = np.array(attention_brute(y.tolist(), list(range(Tn)), Wl, "l0.att.", n_heads,
                                   lambda p, q: bool(orc.visible(p, q))))
    assert np.abs(orc.mhsa_offline(y, 0) - ref).max() < 1e-11
    # streaming: rows 0..3 as cache (K/V from the same projection), rows 4..7 new
    _, k, v = orc.qkv(y, 0)
    cut = 4
    kc = k[:cut].reshape(cut, d_model)[max(0, cut - att_left):]
    vc = v[:cut].reshape(cut, d_model)[max(0, cut - att_left):]
    out, _, _ = orc.mhsa_stream(y[cut:], 0, cut, kc, vc)
    assert np.abs(out - ref[cut:]).max() < 1e-11


def test_sliding_mask_attention_matches_brute_force():
    cfg = tiny(att_left=3, att_right=2, n_emit=2, n_lookahead=2)
    orc = Oracle(cfg, make_weights(cfg))
    y = np.random.default_rng(8).standard_normal((9, 8))
    Wl = {k: v.tolist() for k, v in orc.W.items() if k.startswith("l0.att.")}
    ref = np.array(attention_brute(y.tolist(), list(range(9)), Wl, "l0.att.", 2,
                                   lambda p, q: q >= 0 and p - 3 <= q <= p + 2))
    assert np.abs(orc.mhsa_offline(y, 0) - ref).max() < 1e-11


# ----------------------------------------------------------------------- the gate

def _stream(orc, cfg, xs, sizes):
    st = orc.new_state()
    outs, t = [], 0
    for n in sizes:
        outs.append(orc.push([st], xs[None, t:t + n])[0])
        t += n
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("att_left,sizes", [(70, [2] * 12), (4, [2] * 12), (4, [4, 2, 8, 2, 6, 2]),
                                            (1, [2, 2, 4, 2, 2, 8, 4]), (0, [2] * 10)])
def test_offline_equals_cached_streaming_tiny(att_left, sizes):
    """Streaming spec gate: chunk-by-chunk cached encode == offline masked encode."""
    cfg = tiny(att_left=att_left)
    orc = Oracle(cfg, make_weights(cfg))
    Tn = sum(sizes)
    xs = np.random.default_rng(9).standard_normal((Tn, cfg.d_model))
    err = np.abs(_stream(orc, cfg, xs, sizes) - orc.encode_offline(xs)).max()
    assert err < 1e-12, err


def test_offline_equals_cached_streaming_c1_full():
    """The tiny workload: 2 layers, d 64, 100 chunks of 2 frames (cache wraps many times)."""
    orc = Oracle(C1, make_weights(C1))
    xs = make_inputs(C1, 0).reshape(-1, C1.d_model).astype(np.float64)
    err = np.abs(_stream(orc, C1, xs, [2] * C1.chunks) - orc.encode_offline(xs)).max()
    assert err < 1e-10, err


@pytest.mark.slow
def test_offline_equals_cached_streaming_c2_shape():
    """The 17-layer d 512 encoder over 40 chunks (80 frames: the 70-row cache fills and
    rolls over)."""
    cfg = C2.replace(chunks=40)
    orc = Oracle(cfg, make_weights(C2))
    xs = make_inputs(C2, 0, 40).reshape(-1, 512).astype(np.float64)
    err = np.abs(_stream(orc, cfg, xs, [2] * 40) - orc.encode_offline(xs)).max()
    assert err < 1e-9, err


def test_frontend_streaming_equals_offline():
    """Mel-tail continuation (and the per-layer 2-frame tail form of A23) equal the offline
    padded convs, chunk by chunk, and the whole front end + encoder equals offline."""
    cfg = tiny(d_model=16, frontend=True, mel_bins=8)
    orc = Oracle(cfg, make_weights(cfg))
    C = 7
    mel = np.random.default_rng(10).standard_normal((16 * C, 8))
    ref_x = orc.frontend_offline(mel)
    st = orc.new_state()
    tails = [np.zeros((2, 8)), np.zeros((2, 16)), np.zeros((2, 16))]
    zs = []
    for c in range(C):
        chunk = mel[16 * c:16 * (c + 1)]
        probe = st.copy()
        x_tail = orc.frontend_stream(probe, chunk)
        x_alt = orc.frontend_stream_tails(tails, chunk)
        assert np.abs(x_tail - ref_x[2 * c:2 * c + 2]).max() < 1e-12
        assert np.abs(x_alt - ref_x[2 * c:2 * c + 2]).max() < 1e-12
        zs.append(orc.push([st], chunk[None])[0])
    ref_z = orc.encode_offline(ref_x)
    assert np.abs(np.concatenate(zs) - ref_z).max() < 1e-12


def test_frontend_receptive_field_is_14_past_mel_frames():
    """Streaming spec, "State", melTail: three causal stride-2 k=3 convs need 2 + 4 + 8 = 14
    past mel frames. Perturbing mel frame 16c-14 changes chunk c's frames; 16c-15 does not."""
    cfg = tiny(d_model=16, frontend=True, mel_bins=8)
    orc = Oracle(cfg, make_weights(cfg))
    mel = np.random.default_rng(12).standard_normal((16 * 4, 8))
    c = 3
    base = orc.frontend_offline(mel)[2 * c:2 * c + 2]
    for frame, changes in ((16 * c - 14, True), (16 * c - 15, False)):
        m2 = mel.copy()
        m2[frame] += 10.0
        diff = np.abs(orc.frontend_offline(m2)[2 * c:2 * c + 2] - base).max()
        assert (diff > 1e-9) == changes


# ----------------------------------------------------------------------- lookahead (O3)

def _lookahead_vs_offline(cfg, n_push):
    orc = Oracle(cfg, make_weights(cfg))
    xs = np.random.default_rng(13).standard_normal((2 * n_push, cfg.d_model))
    st = orc.new_state()
    outs = [orc.push([st], xs[None, 2 * i:2 * i + 2])[0] for i in range(n_push)]
    outs.append(orc.flush(st))
    got = np.concatenate(outs)
    assert got.shape[0] == 2 * n_push and st.pos == 2 * n_push
    return np.abs(got - orc.encode_offline(xs)).max()


def test_lookahead_with_zero_right_context_is_exact():
    cfg = tiny(att_left=5, att_right=0, n_emit=2, n_lookahead=8)
    assert _lookahead_vs_offline(cfg, 15) < 1e-12


def test_lookahead_covering_the_cascade_is_exact():
    """Right context cascades through layers (streaming spec, "Status", Nemotron bullet): with
    L layers of right context R the exact value needs L*R future frames. When the lookahead
    covers that (2 * 3 <= 8), the provisional pass is exact."""
    cfg = tiny(n_layers=2, att_left=5, att_right=3, n_emit=2, n_lookahead=8)
    assert _lookahead_vs_offline(cfg, 15) < 1e-12


def test_lookahead_error_shrinks_with_longer_lookahead():
    """When L*R exceeds the lookahead the pass is approximate; its error against offline
    under the same mask shrinks as the lookahead grows (qualitative, as the page reports for
    B = 2, 3, 4)."""
    errs = []
    for la in (2, 4, 6, 8):
        cfg = tiny(n_layers=6, d_model=16, n_heads=2, att_left=6, att_right=3, n_emit=2, n_lookahead=la)
        errs.append(_lookahead_vs_offline(cfg, 14))
    assert errs[0] > 1e-6
    assert all(b < a for a, b in zip(errs, errs[1:])), errs


def test_lookahead_warmup_emits_nothing_until_a_full_pass():
    cfg = tiny(att_left=5, att_right=3, n_emit=2, n_lookahead=8)
    orc = Oracle(cfg, make_weights(cfg))
    st = orc.new_state()
    xs = np.random.default_rng(14).standard_normal((12, 8))
    sizes = [orc.push([st], xs[None, 2 * i:2 * i + 2])[0].shape[0] for i in range(6)]
    assert sizes == [0, 0, 0, 0, 2, 2]
    assert st.pos == 4 and st.x0.shape[0] == 8 and st.k[0].shape[0] == 4


# ----------------------------------------------------------------------- batching

def test_batch_of_streams_equals_streams_alone():
    cfg = tiny()
    orc = Oracle(cfg, make_weights(cfg))
    rng = np.random.default_rng(15)
    xs = rng.standard_normal((3, 10, 2, 8))
    alone = []
    for s in range(3):
        st = orc.new_state()
        alone.append(np.stack([orc.push([st], xs[s, c][None])[0] for c in range(10)]))
    sts = [orc.new_state() for _ in range(3)]
    batched = np.stack([orc.push(sts, xs[:, c]) for c in range(10)], axis=1)
    assert np.abs(batched - np.stack(alone)).max() < 1e-12


# ----------------------------------------------------------------------- one whole layer

def test_one_layer_matches_torch_modules():
    """One Conformer block assembled from torch modules in the order the streaming spec lists
    (FF1, MHSA, conv module, FF2, ln_out; readings A1, A6, A12-A18). The attention uses
    torch's scaled_dot_product_attention with the query shifted by u and the position term
    (q + v).p[rel] / sqrt(hd) passed as an additive mask."""
    cfg = tiny(d_model=16, n_heads=4, d_ff=32, att_left=3)
    orc = Oracle(cfg, make_weights(cfg))
    W = {k: T(v) for k, v in orc.W.items()}
    D, H, hd, K, Tn = 16, 4, 4, cfg.dw_kernel, 10
    x = T(np.random.default_rng(16).standard_normal((Tn, D)))
    ln = lambda t, p: F.layer_norm(t, (D,), W[p + "ln_g"], W[p + "ln_b"], eps=1e-5)  # noqa: E731
    lin = lambda t, w, b: F.linear(t, w.T, b)  # noqa: E731

    def ff(t, p):
        return lin(F.silu(lin(ln(t, p), W[p + "w1"], W[p + "b1"])), W[p + "w2"], W[p + "b2"])

    h = x + 0.5 * ff(x, "l0.ff1.")
    y = ln(h, "l0.att.")
    heads = lambda t: t.reshape(Tn, H, hd).permute(1, 0, 2)  # noqa: E731
    q = heads(lin(y, W["l0.att.wq"], W["l0.att.bq"]))
    k = heads(lin(y, W["l0.att.wk"], W["l0.att.bk"]))
    v = heads(lin(y, W["l0.att.wv"], W["l0.att.bv"]))
    pos = np.arange(Tn)
    rel = pos[:, None] - pos[None, :]
    pe = np.zeros((Tn, Tn, D))
    for i in range(Tn):
        for j in range(Tn):
            for m in range(D // 2):
                a = rel[i, j] * 10000.0 ** (-2 * m / D)
                pe[i, j, 2 * m], pe[i, j, 2 * m + 1] = math.sin(a), math.cos(a)
    P = (T(pe) @ W["l0.att.wpos"]).reshape(Tn, Tn, H, hd)
    bd = torch.einsum("hid,ijhd->hij", q + W["l0.att.pos_v"][:, None, :], P) / math.sqrt(hd)
    vis = T(orc.visible(pos[:, None], pos[None, :]).astype(np.float64)).bool()
    bias = torch.where(vis, bd, torch.tensor(float("-inf")))
    o = F.scaled_dot_product_attention(q + W["l0.att.pos_u"][:, None, :], k, v, attn_mask=bias)
    h = h + lin(o.permute(1, 0, 2).reshape(Tn, D), W["l0.att.wo"], W["l0.att.bo"])
    g = F.glu(lin(ln(h, "l0.conv."), W["l0.conv.pw1"], W["l0.conv.pw1_b"]), dim=-1)
    d = F.conv1d(F.pad(g.T[None], (K - 1, 0)), W["l0.conv.dw"][:, None, :], W["l0.conv.dw_b"], groups=D)[0].T
    h = h + lin(F.silu(d), W["l0.conv.pw2"], W["l0.conv.pw2_b"])
    h = h + 0.5 * ff(h, "l0.ff2.")
    ref = ln(h, "l0.out.").numpy()
    assert np.abs(orc.layer_offline(x.numpy(), 0) - ref).max() < 1e-11


# ----------------------------------------------------------------------- page facts

def test_page_facts_golden():
    """Structural numbers the pages print (tests/golden/page_facts.json, each cited)."""
    import json, os
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
    f = {e["key"]: e["value"] for e in facts["facts"]}
    assert (C2.n_layers, C2.d_model, C2.att_left) == (f["encoder_layers"], f["encoder_hidden"], f["attention_context"])
    assert (C2.att_chunk, C2.mel_tail, C2.conv_cache) == (f["att_chunk"], f["mel_tail_frames"], f["conv_cache_cols"])
    assert f["mel_tail_frames"] == 2 + 2 * 2 + 4 * 2
    orc = Oracle(C2, {})
    for n in (2, 4, 6, 8):
        for pos0 in (0, 2, 70, 1000):
            qs = pos0 + np.arange(n)
            keys = set(range(max(0, pos0 - 70), pos0 + n))
            cols = [sum(bool(orc.visible(p, q)) for q in keys) for p in qs]
            assert len(keys) <= f["att_left"] + n and max(cols) <= f["softmax_cols_max"]
    assert C2.token_classes == 1024 + f["joint_extra_classes"]
    la = C2.replace(att_right=3, n_lookahead=8)
    assert la.att_right == f["lookahead_right_context"]
