"""ctypes binding of libcac.so (include/cac.h). Argument marshalling only: every step of the
chunk step runs in the library's HIP kernels; torch provides device memory and the stream.

The library must have been built (``__graft_entry__.build()`` or
``python cache_aware_conformer_amd/build.py``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcac.so")

CAC_OK, CAC_EINVAL, CAC_ESTATE, CAC_ENOMEM, CAC_EHIP, CAC_ENODEV = 0, -1, -2, -3, -4, -5
CAC_F32, CAC_BF16, CAC_F32_I8 = 0, 1, 2
CAC_FLAG_DRY_RUN, CAC_FLAG_POISON = 1, 2
ERROR_NAMES = {CAC_EINVAL: "CAC_EINVAL", CAC_ESTATE: "CAC_ESTATE", CAC_ENOMEM: "CAC_ENOMEM",
               CAC_EHIP: "CAC_EHIP", CAC_ENODEV: "CAC_ENODEV"}

# every function the header declares, with (restype, argtypes)
_i32, _sz, _vp, _ip, _fp = C.c_int32, C.c_size_t, C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_float)


class cac_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "d_ff", "dw_kernel", "att_left", "att_chunk", "att_right",
        "n_emit", "n_lookahead", "joint_dim", "frontend", "mel_bins", "mel_per_chunk", "mel_tail",
        "dtype", "max_streams", "max_push_frames", "flags", "fe_channels")]


class cac_dec_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "joint_dim", "pred_hidden", "pred_layers", "vocab", "max_symbols", "max_streams", "max_frames", "flags")]


class cac_mel_config(C.Structure):
    _fields_ = [("sample_rate", C.c_int32), ("n_fft", C.c_int32), ("win_length", C.c_int32), ("hop", C.c_int32),
                ("n_mels", C.c_int32), ("fmin", C.c_double), ("fmax", C.c_double), ("preemph", C.c_double),
                ("out_dtype", C.c_int32), ("max_streams", C.c_int32), ("max_hops", C.c_int32), ("flags", C.c_int32)]


class cac_beam_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "joint_dim", "pred_hidden", "pred_layers", "vocab", "beam", "max_symbols", "max_streams", "max_frames",
        "score_norm", "flags")]


CAC_BEAM_FLAG_WEAK_HASH = 0x100

_CFGP = C.POINTER(cac_config)
_DCFGP = C.POINTER(cac_dec_config)
_MCFGP = C.POINTER(cac_mel_config)
_BCFGP = C.POINTER(cac_beam_config)
_PROFILE_READ = [_vp, _i32, C.c_char_p, _i32, C.POINTER(C.c_int64), C.POINTER(C.c_double),
                 C.POINTER(C.c_double), C.POINTER(C.c_double)]
SIGNATURES = {
    # include/cac_beam.h
    "cac_beam_param_count": (_sz, [_BCFGP]),
    "cac_beam_workspace_bytes": (_sz, [_BCFGP]),
    "cac_beam_create": (_i32, [_BCFGP, _fp, _sz, _vp, _sz, _vp, C.POINTER(_vp)]),
    "cac_beam_decode": (_i32, [_vp, _i32, _ip, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
    "cac_beam_set_graph": (_i32, [_vp, _i32]),
    "cac_beam_profile": (_i32, [_vp, _i32]),
    "cac_beam_profile_read": (_i32, _PROFILE_READ),
    "cac_beam_destroy": (_i32, [_vp]),
    "cac_beam_last_error": (C.c_char_p, [_vp]),
    # include/cac_mel.h
    "cac_mel_workspace_bytes": (_sz, [_MCFGP]),
    "cac_mel_create": (_i32, [_MCFGP, _vp, _sz, _vp, C.POINTER(_vp)]),
    "cac_mel_push": (_i32, [_vp, _i32, _ip, _i32, _vp, _vp]),
    "cac_mel_reset": (_i32, [_vp, _i32, _ip]),
    "cac_mel_destroy": (_i32, [_vp]),
    "cac_mel_last_error": (C.c_char_p, [_vp]),
    # include/cac_decode.h
    "cac_dec_param_count": (_sz, [_DCFGP]),
    "cac_dec_workspace_bytes": (_sz, [_DCFGP]),
    "cac_dec_create": (_i32, [_DCFGP, _fp, _sz, _vp, _sz, _vp, C.POINTER(_vp)]),
    "cac_dec_greedy": (_i32, [_vp, _i32, _ip, _i32, _vp, _vp, _vp, _vp]),
    "cac_dec_reset": (_i32, [_vp, _i32, _ip]),
    "cac_dec_destroy": (_i32, [_vp]),
    "cac_dec_last_error": (C.c_char_p, [_vp]),
    "cac_dec_set_graph": (_i32, [_vp, _i32]),
    "cac_dec_profile": (_i32, [_vp, _i32]),
    "cac_dec_profile_read": (_i32, [_vp, _i32, C.c_char_p, _i32, C.POINTER(C.c_int64), C.POINTER(C.c_double),
                                    C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    # include/cac.h
    "cac_param_count": (_sz, [_CFGP]),
    "cac_workspace_bytes": (_sz, [_CFGP]),
    "cac_state_floats": (_sz, [_CFGP]),
    "cac_create_streams": (_i32, [_CFGP, _fp, _sz, _vp, _sz, _vp, C.POINTER(_vp)]),
    "cac_push_chunk": (_i32, [_vp, _i32, _ip, _i32, _vp, _vp, _ip]),
    "cac_reset_stream": (_i32, [_vp, _i32, _ip]),
    "cac_flush": (_i32, [_vp, _i32, _ip, _vp, _ip]),
    "cac_export_state": (_i32, [_vp, _i32, _ip, _ip, _ip, _vp]),
    "cac_import_state": (_i32, [_vp, _i32, _ip, _ip, _ip, _vp]),
    "cac_stream_info": (_i32, [_vp, _i32, _ip, _ip, _ip]),
    "cac_set_stream": (_i32, [_vp, _vp]),
    "cac_set_graph": (_i32, [_vp, _i32]),
    "cac_synchronize": (_i32, [_vp]),
    "cac_destroy": (_i32, [_vp]),
    "cac_last_error": (C.c_char_p, [_vp]),
    "cac_test_gemm": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "cac_profile": (_i32, [_vp, _i32]),
    "cac_profile_read": (_i32, [_vp, _i32, C.c_char_p, _i32, C.POINTER(C.c_int64), C.POINTER(C.c_double),
                                C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "cac_state_header": (_i32, [_CFGP, C.POINTER(C.c_uint32)]),
    "cac_test_gemm_noalloc": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "cac_profile_replay": (_i32, [_vp, C.c_char_p, _i32, C.POINTER(C.c_double), C.POINTER(C.c_int32),
                                  C.POINTER(C.c_double), C.POINTER(C.c_double)]),
}

_lib = None


def load() -> C.CDLL:
    """Load libcac.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


class CacError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def param_order(cfg):
    """(name, shape) of the parameters in the order cac_create_streams reads them (the
    order the header documents)."""
    D, F, H, K, P = cfg.d_model, cfg.d_ff, cfg.n_heads, cfg.dw_kernel, cfg.joint_dim
    hd = D // H
    out = []
    for l in range(cfg.n_layers):
        p = f"l{l}."
        ff = lambda pre: [(pre + "ln_g", (D,)), (pre + "ln_b", (D,)), (pre + "w1", (D, F)), (pre + "b1", (F,)),  # noqa: E731
                          (pre + "w2", (F, D)), (pre + "b2", (D,))]
        out += ff(p + "ff1.")
        out += [(p + "att.ln_g", (D,)), (p + "att.ln_b", (D,))]
        for m in "qkv":
            out += [(p + f"att.w{m}", (D, D)), (p + f"att.b{m}", (D,))]
        out += [(p + "att.wo", (D, D)), (p + "att.bo", (D,)), (p + "att.pos_u", (H, hd)),
                (p + "att.pos_v", (H, hd)), (p + "att.wpos", (D, D))]
        out += [(p + "conv.ln_g", (D,)), (p + "conv.ln_b", (D,)), (p + "conv.pw1", (D, 2 * D)),
                (p + "conv.pw1_b", (2 * D,)), (p + "conv.dw", (D, K)), (p + "conv.dw_b", (D,)),
                (p + "conv.pw2", (D, D)), (p + "conv.pw2_b", (D,))]
        out += ff(p + "ff2.")
        out += [(p + "out.ln_g", (D,)), (p + "out.ln_b", (D,))]
    if P:
        out += [("joint.w", (D, P)), ("joint.b", (P,))]
    if cfg.frontend == 2:
        Cc, F8 = cfg.fe_channels, cfg.mel_bins // 8
        out += [("fe2.c1.w", (Cc, 3, 3)), ("fe2.c1.b", (Cc,)), ("fe2.dw2.w", (Cc, 3, 3)), ("fe2.dw2.b", (Cc,)),
                ("fe2.pw2.w", (Cc, Cc)), ("fe2.pw2.b", (Cc,)), ("fe2.dw3.w", (Cc, 3, 3)), ("fe2.dw3.b", (Cc,)),
                ("fe2.pw3.w", (Cc, Cc)), ("fe2.pw3.b", (Cc,)), ("fe2.lin.w", (Cc * F8, D)), ("fe2.lin.b", (D,))]
    elif cfg.frontend:
        B = cfg.mel_bins
        out += [("fe.c1.w", (D, B, 3)), ("fe.c1.b", (D,)), ("fe.c2.w", (D, D, 3)), ("fe.c2.b", (D,)),
                ("fe.c3.w", (D, D, 3)), ("fe.c3.b", (D,))]
    return out


def make_config(cfg, max_streams=None, max_push_frames=8, flags=0) -> cac_config:
    """cac_config from any object with the workload attribute names (dtype 'f32'/'bf16')."""
    c = cac_config()
    for name in ("n_layers", "d_model", "n_heads", "d_ff", "dw_kernel", "att_left", "att_chunk",
                 "att_right", "n_emit", "n_lookahead", "joint_dim", "mel_bins", "mel_per_chunk", "mel_tail"):
        setattr(c, name, int(getattr(cfg, name)))
    c.frontend = int(cfg.frontend)
    c.fe_channels = int(getattr(cfg, "fe_channels", 0)) if c.frontend == 2 else 0
    dt = str(cfg.dtype)
    c.dtype = CAC_BF16 if dt in ("bf16", "bfloat16", str(CAC_BF16)) else CAC_F32_I8 if dt in ("i8w", str(CAC_F32_I8)) else CAC_F32
    c.max_streams = int(max_streams if max_streams is not None else cfg.streams)
    c.max_push_frames = int(max_push_frames)
    c.flags = int(flags)
    return c


def pack_params(cfg, params: dict) -> np.ndarray:
    order = param_order(cfg)
    flat = np.empty(sum(int(np.prod(s)) for _, s in order), dtype=np.float32)
    o = 0
    for name, shape in order:
        a = np.asarray(params[name], dtype=np.float32)
        if a.shape != tuple(shape):
            raise ValueError(f"{name}: expected shape {shape}, got {a.shape}")
        n = a.size
        flat[o:o + n] = a.reshape(-1)
        o += n
    return flat


def _ids(ids) -> tuple:
    arr = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
    return arr, arr.ctypes.data_as(_ip)


@dataclass
class StreamInfo:
    pos: int
    pending: int
    flushed: bool


class StreamingEncoder:
    """One library context: repacked weights and the state of ``max_streams`` streams in one
    device workspace (a torch uint8 tensor), work enqueued on the current torch stream."""

    def __init__(self, cfg, params: dict, max_streams=None, max_push_frames=8, flags=0, device="cuda:0"):
        self.lib = load()
        self.cfg = cfg
        self.c = make_config(cfg, max_streams, max_push_frames, flags)
        self.dry = bool(flags & CAC_FLAG_DRY_RUN)
        self.P = cfg.joint_dim or cfg.d_model
        n = self.lib.cac_param_count(C.byref(self.c))
        if n == 0:
            self.lib.cac_create_streams(C.byref(self.c), None, 0, None, 0, None, C.byref(C.c_void_p()))
            raise CacError(CAC_EINVAL, self.lib.cac_last_error(None).decode())
        flat = pack_params(cfg, params)
        assert flat.size == n, (flat.size, n)
        self.ws_bytes = self.lib.cac_workspace_bytes(C.byref(self.c))
        self.sfloats = self.lib.cac_state_floats(C.byref(self.c))
        ctx = C.c_void_p()
        if self.dry:
            ws_ptr, stream = None, None
            self.ws = None
        else:
            import torch
            self.torch = torch
            self.device = torch.device(device)
            self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
            base = self.ws.data_ptr()
            ws_ptr = (base + 255) // 256 * 256
            stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.cac_create_streams(C.byref(self.c), flat.ctypes.data_as(_fp), n, ws_ptr,
                                         self.ws_bytes, stream, C.byref(ctx))
        if rc != CAC_OK:
            raise CacError(rc, self.lib.cac_last_error(None).decode())
        self.ctx = ctx

    # -- helpers -----------------------------------------------------------------------
    def _check(self, rc):
        if rc < 0:
            raise CacError(rc, self.lib.cac_last_error(self.ctx).decode())
        return rc

    def out_frames(self):
        return self.cfg.n_lookahead if self.cfg.n_lookahead else None

    # -- calls -------------------------------------------------------------------------
    def push_chunk(self, stream_ids, x, out=None, n_frames=None):
        """x: device tensor [n, n_frames, D] (or [n, 16, mel_bins]) in the compute dtype.
        Returns (out [n, n_frames_out, P] float32, emitted per stream as np.int32)."""
        ids, idp = _ids(stream_ids)
        n = ids.size
        if hasattr(x, "is_contiguous"):
            want = self.torch.bfloat16 if self.c.dtype == CAC_BF16 else self.torch.float32
            if not x.is_contiguous() or x.dtype != want or x.shape[0] != n:
                raise ValueError(f"input must be a contiguous {want} tensor with {n} rows, got "
                                 f"{x.dtype} {tuple(x.shape)} contiguous={x.is_contiguous()}")
        if n_frames is None:
            if self.cfg.n_lookahead:
                n_frames = self.cfg.n_emit
            elif self.cfg.frontend:
                n_frames = 2
            else:
                n_frames = x.shape[1]
        if out is None and not self.dry:
            out = self.torch.empty((n, n_frames, self.P), dtype=self.torch.float32, device=self.device)
        elif hasattr(out, "is_contiguous"):
            if not out.is_contiguous() or out.dtype != self.torch.float32 or out.numel() < n * n_frames * self.P:
                raise ValueError(f"out must be a contiguous float32 tensor of at least {n}x{n_frames}x{self.P} "
                                 f"elements, got {out.dtype} {tuple(out.shape)} contiguous={out.is_contiguous()}")
        emitted = np.zeros(n, dtype=np.int32)
        xp = None if x is None else (x.data_ptr() if hasattr(x, "data_ptr") else int(x))
        op = None if out is None else (out.data_ptr() if hasattr(out, "data_ptr") else int(out))
        self._check(self.lib.cac_push_chunk(self.ctx, n, idp, int(n_frames), xp, op, emitted.ctypes.data_as(_ip)))
        return out, emitted

    def reset_stream(self, stream_ids):
        ids, idp = _ids(stream_ids)
        return self._check(self.lib.cac_reset_stream(self.ctx, ids.size, idp))

    def flush(self, stream_ids, out=None):
        ids, idp = _ids(stream_ids)
        n = ids.size
        if out is None and not self.dry and self.cfg.n_lookahead:
            out = self.torch.empty((n, self.cfg.n_lookahead, self.P), dtype=self.torch.float32, device=self.device)
        elif out is not None and (not out.is_contiguous() or out.dtype != self.torch.float32
                                  or out.numel() < n * self.cfg.n_lookahead * self.P):
            raise ValueError(f"out must be a contiguous float32 tensor of at least {n}x{self.cfg.n_lookahead}x{self.P} "
                             f"elements, got {out.dtype} {tuple(out.shape)}")
        frames = np.zeros(n, dtype=np.int32)
        op = None if out is None else out.data_ptr()
        self._check(self.lib.cac_flush(self.ctx, n, idp, op, frames.ctypes.data_as(_ip)))
        return out, frames

    def export_state(self, stream_ids):
        ids, idp = _ids(stream_ids)
        n = ids.size
        blob = self.torch.empty((n, self.sfloats), dtype=self.torch.float32, device=self.device)
        pos = np.zeros(n, dtype=np.int32)
        pend = np.zeros(n, dtype=np.int32)
        self._check(self.lib.cac_export_state(self.ctx, n, idp, pos.ctypes.data_as(_ip),
                                              pend.ctypes.data_as(_ip), blob.data_ptr()))
        return pos, pend, blob

    def import_state(self, stream_ids, pos, pending, blob):
        ids, idp = _ids(stream_ids)
        pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int32))
        pend = np.ascontiguousarray(np.asarray(pending if pending is not None else np.zeros_like(pos), dtype=np.int32))
        bp = blob.data_ptr() if blob is not None else None
        return self._check(self.lib.cac_import_state(self.ctx, ids.size, idp, pos.ctypes.data_as(_ip),
                                                     pend.ctypes.data_as(_ip), bp))

    def state_header(self) -> np.ndarray:
        """The 4-word state-blob header of this context's config, as 4 float32 slots."""
        h = np.zeros(4, dtype=np.uint32)
        self._check(self.lib.cac_state_header(C.byref(self.c), h.ctypes.data_as(C.POINTER(C.c_uint32))))
        return h.view(np.float32)

    def state_blob(self, st: dict) -> np.ndarray:
        """Canonical float32 state blob (header layout) of one stream from a dict with keys
        k, v [L][Lc][D], conv [L][K-1][D], mel_tail (front end), x0_tail (lookahead)."""
        parts = [self.state_header(), np.asarray(st["k"], np.float32).reshape(-1),
                 np.asarray(st["v"], np.float32).reshape(-1), np.asarray(st["conv"], np.float32).reshape(-1)]
        if self.cfg.frontend:
            parts.append(np.asarray(st["mel_tail"], np.float32).reshape(-1))
        if self.cfg.n_lookahead:
            parts.append(np.asarray(st["x0_tail"], np.float32).reshape(-1))
        blob = np.concatenate(parts)
        assert blob.size == self.sfloats, (blob.size, self.sfloats)
        return blob

    def import_state_dicts(self, stream_ids, states, pending=None):
        """Import per-stream state dicts (see state_blob; positions from st['pos'])."""
        blob = self.torch.from_numpy(np.stack([self.state_blob(st) for st in states])).to(self.device)
        pos = [int(st["pos"]) for st in states]
        if pending is None and self.cfg.n_lookahead:
            pending = [len(st["x0_tail"]) for st in states]
        return self.import_state(stream_ids, pos, pending, blob)

    def stream_info(self, stream_id) -> StreamInfo:
        p, q, f = C.c_int32(), C.c_int32(), C.c_int32()
        self._check(self.lib.cac_stream_info(self.ctx, int(stream_id), C.byref(p), C.byref(q), C.byref(f)))
        return StreamInfo(p.value, q.value, bool(f.value))

    def set_graph(self, enable: bool):
        return self._check(self.lib.cac_set_graph(self.ctx, int(bool(enable))))

    def set_stream(self, stream):
        return self._check(self.lib.cac_set_stream(self.ctx, stream))

    def synchronize(self):
        return self._check(self.lib.cac_synchronize(self.ctx))

    def profile(self, enable: bool):
        return self._check(self.lib.cac_profile(self.ctx, int(bool(enable))))

    def profile_read(self) -> dict:
        """{kernel name: (launches, total_ms, bytes, flops)} of the launches since profile(True)."""
        n = self._check(self.lib.cac_profile_read(self.ctx, 0, None, 64, None, None, None, None))
        names = C.create_string_buffer(64 * max(n, 1))
        launches = (C.c_int64 * max(n, 1))()
        ms, by, fl = (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))()
        n = self._check(self.lib.cac_profile_read(self.ctx, n, names, 64, launches, ms, by, fl))
        out = {}
        for i in range(n):
            nm = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
            out[nm] = (int(launches[i]), float(ms[i]), float(by[i]), float(fl[i]))
        return out

    def profile_replay(self, prefix: str, reps: int = 20) -> dict:
        """Back-to-back duration of the kernel family `prefix` from the last replayed push graph
        (leaves the streams of that push in an unspecified state)."""
        us, nb, by, fl = C.c_double(), C.c_int32(), C.c_double(), C.c_double()
        self._check(self.lib.cac_profile_replay(self.ctx, prefix.encode(), int(reps), C.byref(us), C.byref(nb),
                                                C.byref(by), C.byref(fl)))
        return {"us_per_launch": us.value, "launches": nb.value, "bytes_per_launch": by.value,
                "flops_per_launch": fl.value}

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.cac_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def test_gemm(dtype: int, path: int, A, W, bias=None, out=None, stream=None, noalloc=False):
    """C = A W^T + bias through the library's dense kernels (test-only export; noalloc: the
    variant that allocates nothing and keeps split-K partials in the library's scratch)."""
    import torch
    lib = load()
    M, K = A.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    s = stream if stream is not None else torch.cuda.current_stream(A.device).cuda_stream
    fn = lib.cac_test_gemm_noalloc if noalloc else lib.cac_test_gemm
    rc = fn(dtype, path, M, N, K, A.data_ptr(), W.data_ptr(), None if bias is None else bias.data_ptr(),
            out.data_ptr(), s)
    if rc != CAC_OK:
        raise CacError(rc, lib.cac_last_error(None).decode() or "test GEMM failed")
    return out


# ----------------------------------------------------------------------------- greedy decoding

def dec_param_order(cfg):
    """(name, shape) of the decoder parameters in the order cac_dec_create takes them."""
    H, P, C_ = cfg.pred_hidden, cfg.joint_dim, cfg.vocab + 2
    out = [("pred.embed", (C_, H))]
    for l in range(cfg.pred_layers):
        out += [(f"pred.l{l}.w_ih", (H, 4 * H)), (f"pred.l{l}.w_hh", (H, 4 * H)),
                (f"pred.l{l}.b_ih", (4 * H,)), (f"pred.l{l}.b_hh", (4 * H,))]
    out += [("pred.proj_w", (H, P)), ("pred.proj_b", (P,)), ("joint.out_w", (P, C_)), ("joint.out_b", (C_,))]
    return out


def make_dec_config(cfg, max_streams=None, max_frames=None, flags=0) -> cac_dec_config:
    c = cac_dec_config()
    for name in ("joint_dim", "pred_hidden", "pred_layers", "vocab", "max_symbols"):
        setattr(c, name, int(getattr(cfg, name)))
    c.max_streams = int(max_streams if max_streams is not None else cfg.streams)
    c.max_frames = int(max_frames if max_frames is not None else cfg.frames)
    c.flags = int(flags)
    return c


class StreamingDecoder:
    """One greedy-decoding context (include/cac_decode.h): repacked float32 decoder weights and
    the predictor state of ``max_streams`` streams in one device workspace, work enqueued on the
    current torch stream."""

    def __init__(self, cfg, params: dict, max_streams=None, max_frames=None, flags=0, device="cuda:0"):
        self.lib = load()
        self.cfg = cfg
        self.c = make_dec_config(cfg, max_streams, max_frames, flags)
        self.dry = bool(flags & CAC_FLAG_DRY_RUN)
        self.m = cfg.max_symbols
        n = self.lib.cac_dec_param_count(C.byref(self.c))
        if n == 0:
            self.lib.cac_dec_create(C.byref(self.c), None, 0, None, 0, None, C.byref(C.c_void_p()))
            raise CacError(CAC_EINVAL, self.lib.cac_dec_last_error(None).decode())
        flat = np.ascontiguousarray(np.concatenate([np.asarray(params[nm], np.float32).reshape(-1)
                                                    for nm, shape in dec_param_order(cfg)]))
        self.ws_bytes = self.lib.cac_dec_workspace_bytes(C.byref(self.c))
        ctx = C.c_void_p()
        if self.dry:
            ws_ptr, stream, self.ws = None, None, None
        else:
            import torch
            self.torch = torch
            self.device = torch.device(device)
            self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
            ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
            stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.cac_dec_create(C.byref(self.c), flat.ctypes.data_as(_fp), flat.size, ws_ptr, self.ws_bytes,
                                     stream, C.byref(ctx))
        if rc != CAC_OK:
            raise CacError(rc, self.lib.cac_dec_last_error(None).decode())
        self.ctx = ctx

    def _check(self, rc):
        if rc < 0:
            raise CacError(rc, self.lib.cac_dec_last_error(self.ctx).decode())
        return rc

    def decode(self, stream_ids, z, tokens=None, frames=None, counts=None):
        """z: device float32 [n, n_frames, P]. Returns device int32 (tokens [n, n_frames *
        max_symbols], token frames (same shape), counts [n])."""
        ids, idp = _ids(stream_ids)
        n = ids.size
        nf = int(z.shape[1]) if hasattr(z, "shape") else int(self.c.max_frames)
        if hasattr(z, "is_contiguous") and (not z.is_contiguous() or z.dtype != self.torch.float32 or z.shape[0] != n):
            raise ValueError(f"z must be a contiguous float32 tensor with {n} rows, got {z.dtype} {tuple(z.shape)}")
        if not self.dry:
            t = self.torch
            if tokens is None:
                tokens = t.empty((n, nf * self.m), dtype=t.int32, device=self.device)
            if frames is None:
                frames = t.empty((n, nf * self.m), dtype=t.int32, device=self.device)
            if counts is None:
                counts = t.empty(n, dtype=t.int32, device=self.device)
        ptr = lambda x: None if x is None else (x.data_ptr() if hasattr(x, "data_ptr") else int(x))  # noqa: E731
        self._check(self.lib.cac_dec_greedy(self.ctx, n, idp, nf, ptr(z), ptr(tokens), ptr(frames), ptr(counts)))
        return tokens, frames, counts

    def reset(self, stream_ids):
        ids, idp = _ids(stream_ids)
        return self._check(self.lib.cac_dec_reset(self.ctx, ids.size, idp))

    def set_graph(self, enable: bool):
        return self._check(self.lib.cac_dec_set_graph(self.ctx, int(bool(enable))))

    def profile(self, enable: bool):
        return self._check(self.lib.cac_dec_profile(self.ctx, int(bool(enable))))

    def profile_read(self) -> dict:
        """{kernel name: (launches, total_ms, bytes, flops)} of the launches since profile(True)."""
        n = self._check(self.lib.cac_dec_profile_read(self.ctx, 0, None, 64, None, None, None, None))
        names = C.create_string_buffer(64 * max(n, 1))
        launches = (C.c_int64 * max(n, 1))()
        ms, by, fl = (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))()
        n = self._check(self.lib.cac_dec_profile_read(self.ctx, n, names, 64, launches, ms, by, fl))
        out = {}
        for i in range(n):
            nm = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
            out[nm] = (int(launches[i]), float(ms[i]), float(by[i]), float(fl[i]))
        return out

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.cac_dec_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- beam search

def make_beam_config(cfg, max_streams=None, max_frames=None, flags=0) -> cac_beam_config:
    c = cac_beam_config()
    for name in ("joint_dim", "pred_hidden", "pred_layers", "vocab", "beam", "max_symbols"):
        setattr(c, name, int(getattr(cfg, name)))
    c.max_streams = int(max_streams if max_streams is not None else cfg.streams)
    c.max_frames = int(max_frames if max_frames is not None else cfg.frames)
    c.score_norm = int(bool(cfg.score_norm))
    c.flags = int(flags)
    return c


class BeamSearch:
    """One beam-search context (include/cac_beam.h): repacked float32 decoder weights (the
    greedy decoder's parameters) and the beams of ``max_streams`` utterances in one device
    workspace, work enqueued on the current torch stream."""

    def __init__(self, cfg, params: dict, max_streams=None, max_frames=None, flags=0, device="cuda:0"):
        self.lib = load()
        self.cfg = cfg
        self.c = make_beam_config(cfg, max_streams, max_frames, flags)
        self.dry = bool(flags & CAC_FLAG_DRY_RUN)
        self.K, self.m = int(cfg.beam), int(cfg.max_symbols)
        n = self.lib.cac_beam_param_count(C.byref(self.c))
        if n == 0:
            self.lib.cac_beam_create(C.byref(self.c), None, 0, None, 0, None, C.byref(C.c_void_p()))
            raise CacError(CAC_EINVAL, self.lib.cac_beam_last_error(None).decode())
        flat = np.ascontiguousarray(np.concatenate([np.asarray(params[nm], np.float32).reshape(-1)
                                                    for nm, shape in dec_param_order(cfg)]))
        self.ws_bytes = self.lib.cac_beam_workspace_bytes(C.byref(self.c))
        ctx = C.c_void_p()
        if self.dry:
            ws_ptr, stream, self.ws = None, None, None
        else:
            import torch
            self.torch = torch
            self.device = torch.device(device)
            self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
            ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
            stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.cac_beam_create(C.byref(self.c), flat.ctypes.data_as(_fp), flat.size, ws_ptr, self.ws_bytes,
                                      stream, C.byref(ctx))
        if rc != CAC_OK:
            raise CacError(rc, self.lib.cac_beam_last_error(None).decode())
        self.ctx = ctx

    def _check(self, rc):
        if rc < 0:
            raise CacError(rc, self.lib.cac_beam_last_error(self.ctx).decode())
        return rc

    def decode(self, z, lengths, max_steps=0, out=None):
        """z: device float32 [n, n_frames, P]; lengths: n frame counts. Returns (tokens [n, K,
        n_frames * max_symbols], lengths [n, K], scores [n, K], frames [n, K], iterations): the
        K slots of each utterance best first (device tensors) and the iteration count."""
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32).reshape(-1))
        n = lens.size
        nf = int(z.shape[1]) if hasattr(z, "shape") else int(self.c.max_frames)
        if hasattr(z, "is_contiguous") and (not z.is_contiguous() or z.dtype != self.torch.float32 or z.shape[0] != n):
            raise ValueError(f"z must be a contiguous float32 tensor with {n} rows, got {z.dtype} {tuple(z.shape)}")
        tokens = tl = sc = fr = None
        if out is not None:
            tokens, tl, sc, fr = out
        elif not self.dry:
            t = self.torch
            tokens = t.empty((n, self.K, nf * self.m), dtype=t.int32, device=self.device)
            tl = t.empty((n, self.K), dtype=t.int32, device=self.device)
            sc = t.empty((n, self.K), dtype=t.float32, device=self.device)
            fr = t.empty((n, self.K), dtype=t.int32, device=self.device)
        ptr = lambda x: None if x is None else (x.data_ptr() if hasattr(x, "data_ptr") else int(x))  # noqa: E731
        it = self._check(self.lib.cac_beam_decode(self.ctx, n, lens.ctypes.data_as(_ip), nf, ptr(z), int(max_steps),
                                                  ptr(tokens), ptr(tl), ptr(sc), ptr(fr)))
        return tokens, tl, sc, fr, it

    def set_graph(self, enable: bool):
        return self._check(self.lib.cac_beam_set_graph(self.ctx, int(bool(enable))))

    def profile(self, enable: bool):
        return self._check(self.lib.cac_beam_profile(self.ctx, int(bool(enable))))

    def profile_read(self) -> dict:
        """{kernel name: (launches, total_ms, bytes, flops)} of the launches since profile(True)."""
        n = self._check(self.lib.cac_beam_profile_read(self.ctx, 0, None, 64, None, None, None, None))
        names = C.create_string_buffer(64 * max(n, 1))
        launches = (C.c_int64 * max(n, 1))()
        ms, by, fl = (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))(), (C.c_double * max(n, 1))()
        n = self._check(self.lib.cac_beam_profile_read(self.ctx, n, names, 64, launches, ms, by, fl))
        out = {}
        for i in range(n):
            nm = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
            out[nm] = (int(launches[i]), float(ms[i]), float(by[i]), float(fl[i]))
        return out

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.cac_beam_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- streaming log-mel

def make_mel_config(cfg, max_streams=None, max_hops=None, flags=0) -> cac_mel_config:
    c = cac_mel_config()
    for name in ("sample_rate", "n_fft", "win_length", "hop", "n_mels"):
        setattr(c, name, int(getattr(cfg, name)))
    c.fmin, c.fmax, c.preemph = float(cfg.fmin), float(cfg.fmax), float(cfg.preemph)
    c.out_dtype = CAC_BF16 if str(cfg.out_dtype) in ("bf16", str(CAC_BF16)) else CAC_F32
    c.max_streams = int(max_streams if max_streams is not None else cfg.streams)
    c.max_hops = int(max_hops if max_hops is not None else cfg.hops)
    c.flags = int(flags)
    return c


class StreamingMel:
    """One log-mel context (include/cac_mel.h): tables and every stream's sample tail in one
    device workspace, work on the current torch stream."""

    def __init__(self, cfg, max_streams=None, max_hops=None, flags=0, device="cuda:0"):
        self.lib = load()
        self.cfg = cfg
        self.c = make_mel_config(cfg, max_streams, max_hops, flags)
        self.dry = bool(flags & CAC_FLAG_DRY_RUN)
        self.ws_bytes = self.lib.cac_mel_workspace_bytes(C.byref(self.c))
        ctx = C.c_void_p()
        if self.dry:
            ws_ptr, stream, self.ws = None, None, None
        else:
            import torch
            self.torch = torch
            self.device = torch.device(device)
            self.ws = torch.empty(max(self.ws_bytes, 1) + 256, dtype=torch.uint8, device=self.device)
            ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
            stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.cac_mel_create(C.byref(self.c), ws_ptr, self.ws_bytes, stream, C.byref(ctx))
        if rc != CAC_OK:
            raise CacError(rc, self.lib.cac_mel_last_error(None).decode())
        self.ctx = ctx

    def _check(self, rc):
        if rc < 0:
            raise CacError(rc, self.lib.cac_mel_last_error(self.ctx).decode())
        return rc

    def push(self, stream_ids, audio, out=None):
        """audio: device float32 [n, n_samples]. Returns device [n, n_samples // hop, n_mels]."""
        ids, idp = _ids(stream_ids)
        n, ns = ids.size, int(audio.shape[1])
        if not self.dry:
            t = self.torch
            if audio.dtype != t.float32 or not audio.is_contiguous() or audio.shape[0] != n:
                raise ValueError(f"audio must be a contiguous float32 tensor with {n} rows")
            if out is None:
                dt = t.bfloat16 if self.c.out_dtype == CAC_BF16 else t.float32
                out = t.empty((n, ns // self.c.hop, self.c.n_mels), dtype=dt, device=self.device)
        ptr = lambda x: None if x is None else (x.data_ptr() if hasattr(x, "data_ptr") else int(x))  # noqa: E731
        self._check(self.lib.cac_mel_push(self.ctx, n, idp, ns, ptr(audio), ptr(out)))
        return out

    def reset(self, stream_ids):
        ids, idp = _ids(stream_ids)
        return self._check(self.lib.cac_mel_reset(self.ctx, ids.size, idp))

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.cac_mel_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
