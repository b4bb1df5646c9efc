"""Python binding of libiskv (include/iskv.h): argument marshalling only.

Every step of the compressed-cache path runs in the HIP kernels of
libiskv.so; this module checks tensor shapes, dtypes and devices, passes raw
device pointers and the current HIP stream through ctypes, and turns status
codes into exceptions. PyTorch provides device memory and streams.

There is no fallback: if libiskv.so is missing, loading fails loudly.
"""

import ctypes
import os

import torch  # imported first so the HIP runtime libiskv binds to is torch's

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiskv.so")

ISKV_OK = 0
ISKV_ERR_ARG = -1
ISKV_ERR_WORKSPACE = -2
ISKV_ERR_CAPACITY = -3
ISKV_ERR_HIP = -4
ISKV_ERR_NUMERIC = -5
ISKV_ERR_POISONED = -6
ISKV_ERR_STATE = -7
ISKV_ERR_SCRATCH = -8

ISKV_F32 = 0
ISKV_BF16 = 1
ISKV_I8 = 2  # coordinates only: int8 codes of U with one fp32 scale per row
MODE_JOINT, MODE_FIXED_COORDS, MODE_FIXED_BASIS = 0, 1, 2  # ISKV_MODE_* in iskv.h
FLAG_SWEEP_CAP = 0x1
FLAG_NONFINITE = 0x2

EXPORTED = [
    "iskv_workspace_bytes", "iskv_init", "iskv_reset", "iskv_set_mode", "iskv_append_block", "iskv_prefill_block",
    "iskv_prefill_oneshot",
    "iskv_decode_attn", "iskv_append_decode", "iskv_reconstruct", "iskv_counts", "iskv_export_state", "iskv_set_counts",
    "iskv_import_state", "iskv_fold_stats", "iskv_status", "iskv_destroy", "iskv_strerror",
    "iskv_set_fold_events", "iskv_decode_attn_static", "iskv_export_scales", "iskv_import_scales",
]


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "layers", "kv_heads", "q_heads", "head_dim", "block", "rank_k", "rank_v",
        "window", "max_tokens", "coord_dtype", "kv_dtype")]


class ISKVError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s (%d)" % (what, _strerror(code), code))


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


def load(path: str = None):
    """Load libiskv.so (built by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libiskv.so not found at %s: build it with __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    lib.iskv_workspace_bytes.argtypes = [ctypes.POINTER(Config)]
    lib.iskv_workspace_bytes.restype = ctypes.c_size_t
    lib.iskv_init.argtypes = [ctypes.POINTER(Config), _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]
    lib.iskv_reset.argtypes = [_vp, _vp]
    lib.iskv_set_mode.argtypes = [_vp, _i32]
    lib.iskv_set_fold_events.argtypes = [_vp, ctypes.POINTER(_vp)]
    lib.iskv_append_block.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _vp]
    lib.iskv_prefill_block.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
    lib.iskv_decode_attn.argtypes = [_vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp]
    lib.iskv_decode_attn_static.argtypes = [_vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp]
    lib.iskv_append_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp]
    lib.iskv_reconstruct.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp]
    P32 = ctypes.POINTER(_i32)
    lib.iskv_counts.argtypes = [_vp, _i32, P32, P32, P32, P32]
    lib.iskv_export_state.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.iskv_set_counts.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32]
    lib.iskv_import_state.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.iskv_fold_stats.argtypes = [_vp, _i32, _vp, _vp, _vp]
    lib.iskv_export_scales.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp]
    lib.iskv_import_scales.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp]
    lib.iskv_status.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.iskv_destroy.argtypes = [_vp]
    lib.iskv_strerror.argtypes = [ctypes.c_int]
    lib.iskv_strerror.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name != "iskv_workspace_bytes" and name != "iskv_strerror":
            getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _strerror(code):
    try:
        return load().iskv_strerror(code).decode()
    except Exception:  # library not loadable: describe the code generically
        return "status"


def _check(code, what):
    if code != ISKV_OK:
        raise ISKVError(code, what)


def make_config(batch, layers, kv_heads, q_heads, block, rank_k, rank_v, window, max_tokens,
                coord_dtype="bf16", kv_dtype="bf16", head_dim=128) -> Config:
    dt = {"f32": ISKV_F32, "bf16": ISKV_BF16, "i8": ISKV_I8}
    return Config(batch, layers, kv_heads, q_heads, head_dim, block, rank_k, rank_v, window,
                  max_tokens, dt[coord_dtype], dt[kv_dtype])


def config_from_workload(w, coord_dtype=None, max_tokens=None) -> Config:
    return make_config(w.batch, w.layers, w.kv_heads, w.q_heads, w.block, w.rank_k, w.rank_v,
                       w.window, max_tokens or w.max_tokens, coord_dtype or w.coord_dtype,
                       w.kv_dtype, w.head_dim)


def workspace_bytes(cfg: Config) -> int:
    return int(load().iskv_workspace_bytes(ctypes.byref(cfg)))


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(stream)


_TDT = {ISKV_F32: torch.float32, ISKV_BF16: torch.bfloat16, ISKV_I8: torch.int8}


class Cache:
    """A compressed KV cache over a caller-owned torch workspace (C-ABI handle)."""

    def __init__(self, cfg: Config, device="cuda", stream=None):
        self.lib = load()
        self.cfg = cfg
        n = workspace_bytes(cfg)
        if n == 0:
            raise ISKVError(ISKV_ERR_ARG, "iskv_workspace_bytes")
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        h = _vp()
        _check(self.lib.iskv_init(ctypes.byref(cfg), _vp(self.workspace.data_ptr()), n,
                                  _stream(stream), ctypes.byref(h)), "iskv_init")
        self.h = h
        self.kv_dtype = _TDT[cfg.kv_dtype]
        self.coord_dtype = _TDT[cfg.coord_dtype]

    # -- helpers ---------------------------------------------------------
    def _t(self, x, shape, dtype, name):
        if not isinstance(x, torch.Tensor) or x.device != self.device:
            raise ValueError("%s must be a tensor on %s" % (name, self.device))
        if x.dtype != dtype or tuple(x.shape) != tuple(shape) or not x.is_contiguous():
            raise ValueError("%s: expected contiguous %s %s, got %s %s" % (
                name, dtype, tuple(shape), x.dtype, tuple(x.shape)))
        return _vp(x.data_ptr())

    # -- API -------------------------------------------------------------
    def reset(self, stream=None):
        _check(self.lib.iskv_reset(self.h, _stream(stream)), "iskv_reset")

    def set_mode(self, mode):
        """Update mode of later folds: MODE_JOINT (the method), MODE_FIXED_COORDS
        or MODE_FIXED_BASIS (ablations)."""
        _check(self.lib.iskv_set_mode(self.h, int(mode)), "iskv_set_mode")

    def append_block(self, k_rows, v_rows, layer0=0, stream=None):
        """k_rows, v_rows: [batch, nlayers, kv_heads, nrows, 128] in kv dtype."""
        c = self.cfg
        if k_rows.dim() != 5:
            raise ValueError("rows must be 5-D [batch, nlayers, kv_heads, nrows, d]")
        nl, nrows = k_rows.shape[1], k_rows.shape[3]
        shape = (c.batch, nl, c.kv_heads, nrows, c.head_dim)
        kp = self._t(k_rows, shape, self.kv_dtype, "k_rows")
        vp = self._t(v_rows, shape, self.kv_dtype, "v_rows")
        _check(self.lib.iskv_append_block(self.h, kp, vp, nrows, layer0, nl, _stream(stream)),
               "iskv_append_block")

    def prefill_block(self, k_rows, v_rows, layer0=0, stream=None):
        c = self.cfg
        nl = k_rows.shape[1]
        shape = (c.batch, nl, c.kv_heads, c.block, c.head_dim)
        kp = self._t(k_rows, shape, self.kv_dtype, "k_rows")
        vp = self._t(v_rows, shape, self.kv_dtype, "v_rows")
        _check(self.lib.iskv_prefill_block(self.h, kp, vp, layer0, nl, _stream(stream)),
               "iskv_prefill_block")

    def prefill_oneshot(self, k_rows, v_rows, layer0=0, stream=None):
        """All prompt rows [batch, nlayers, kv_heads, nrows, 128] factorised at
        once into the (empty) history of those layers."""
        c = self.cfg
        nl, nrows = k_rows.shape[1], k_rows.shape[3]
        shape = (c.batch, nl, c.kv_heads, nrows, c.head_dim)
        kp = self._t(k_rows, shape, self.kv_dtype, "k_rows")
        vp = self._t(v_rows, shape, self.kv_dtype, "v_rows")
        _check(self.lib.iskv_prefill_oneshot(self.h, kp, vp, nrows, layer0, nl, _stream(stream)),
               "iskv_prefill_oneshot")

    def decode_attn(self, q, out=None, layer0=0, scale=None, stream=None):
        """q: [batch, nlayers, q_heads, 128] in kv dtype; returns fp32 out of the same shape."""
        c = self.cfg
        nl = q.shape[1]
        shape = (c.batch, nl, c.q_heads, c.head_dim)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        qp = self._t(q, shape, self.kv_dtype, "q")
        op = self._t(out, shape, torch.float32, "out")
        s = float(c.head_dim ** -0.5) if scale is None else float(scale)
        _check(self.lib.iskv_decode_attn(self.h, qp, op, layer0, nl, ctypes.c_float(s), _stream(stream)),
               "iskv_decode_attn")
        return out

    def decode_attn_static(self, q, out=None, layer0=0, scale=None, stream=None):
        """iskv_decode_attn_static: decode attention with its partials in the
        library's static device array (no allocation by the library)."""
        c = self.cfg
        nl = q.shape[1]
        shape = (c.batch, nl, c.q_heads, c.head_dim)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        qp = self._t(q, shape, self.kv_dtype, "q")
        op = self._t(out, shape, torch.float32, "out")
        s = float(c.head_dim ** -0.5) if scale is None else float(scale)
        _check(self.lib.iskv_decode_attn_static(self.h, qp, op, layer0, nl, ctypes.c_float(s), _stream(stream)),
               "iskv_decode_attn_static")
        return out

    def append_decode(self, k_rows, v_rows, q, out=None, layer0=0, scale=None, stream=None):
        """One decode step: k_rows, v_rows [batch, nlayers, kv_heads, 1, 128] and
        q [batch, nlayers, q_heads, 128] in kv dtype; returns fp32 out like q."""
        c = self.cfg
        nl = q.shape[1]
        rshape = (c.batch, nl, c.kv_heads, 1, c.head_dim)
        qshape = (c.batch, nl, c.q_heads, c.head_dim)
        if out is None:
            out = torch.empty(qshape, dtype=torch.float32, device=self.device)
        kp = self._t(k_rows, rshape, self.kv_dtype, "k_rows")
        vp = self._t(v_rows, rshape, self.kv_dtype, "v_rows")
        qp = self._t(q, qshape, self.kv_dtype, "q")
        op = self._t(out, qshape, torch.float32, "out")
        s = float(c.head_dim ** -0.5) if scale is None else float(scale)
        _check(self.lib.iskv_append_decode(self.h, kp, vp, qp, op, layer0, nl, ctypes.c_float(s),
                                           _stream(stream)), "iskv_append_decode")
        return out

    def counts(self, layer=0):
        v = [_i32() for _ in range(4)]
        _check(self.lib.iskv_counts(self.h, layer, *[ctypes.byref(x) for x in v]), "iskv_counts")
        return tuple(int(x.value) for x in v)  # n, e, k_k, k_v

    def reconstruct(self, which, batch, layer, head, stream=None):
        n, e, _, _ = self.counts(layer)
        out = torch.empty((n + e, self.cfg.head_dim), dtype=torch.float32, device=self.device)
        _check(self.lib.iskv_reconstruct(self.h, which, batch, layer, head, _vp(out.data_ptr()),
                                         _stream(stream)), "iskv_reconstruct")
        return out

    def rank(self, which):
        return self.cfg.rank_k if which == 0 else self.cfg.rank_v

    def export_state(self, which, batch, layer, head, stream=None):
        """Returns (C [n, r], sigma [r], Bt [r, 128], window [e, 128]) as device tensors."""
        n, e, _, _ = self.counts(layer)
        r = self.rank(which)
        C = torch.empty((n, r), dtype=self.coord_dtype, device=self.device)
        sig = torch.empty(r, dtype=torch.float32, device=self.device)
        Bt = torch.empty((r, self.cfg.head_dim), dtype=torch.float32, device=self.device)
        W = torch.empty((e, self.cfg.head_dim), dtype=self.kv_dtype, device=self.device)
        _check(self.lib.iskv_export_state(self.h, which, batch, layer, head, _vp(C.data_ptr()),
                                          _vp(sig.data_ptr()), _vp(Bt.data_ptr()), _vp(W.data_ptr()),
                                          _stream(stream)), "iskv_export_state")
        return C, sig, Bt, W

    def export_scales(self, which, batch, layer, head, stream=None):
        """int8 coordinates only: the per-row scales of U [n] fp32 (history row i is
        (C[i] * scale[i]) * sigma B^T)."""
        n, _, _, _ = self.counts(layer)
        sc = torch.empty(n, dtype=torch.float32, device=self.device)
        _check(self.lib.iskv_export_scales(self.h, which, batch, layer, head, _vp(sc.data_ptr()),
                                           _stream(stream)), "iskv_export_scales")
        return sc

    def import_scales(self, which, batch, layer, head, scales, stream=None):
        n, _, _, _ = self.counts(layer)
        sp = self._t(scales, (n,), torch.float32, "scales")
        _check(self.lib.iskv_import_scales(self.h, which, batch, layer, head, sp, _stream(stream)),
               "iskv_import_scales")

    def set_counts(self, layer, n, e, k_k, k_v):
        _check(self.lib.iskv_set_counts(self.h, layer, n, e, k_k, k_v), "iskv_set_counts")

    def import_state(self, which, batch, layer, head, C=None, sigma=None, Bt=None, window=None,
                     stream=None):
        n, e, _, _ = self.counts(layer)
        r = self.rank(which)
        d = self.cfg.head_dim
        cp = self._t(C, (n, r), self.coord_dtype, "C") if C is not None else None
        sp = self._t(sigma, (r,), torch.float32, "sigma") if sigma is not None else None
        bp = self._t(Bt, (r, d), torch.float32, "Bt") if Bt is not None else None
        wp = self._t(window, (e, d), self.kv_dtype, "window") if window is not None else None
        _check(self.lib.iskv_import_state(self.h, which, batch, layer, head, cp, sp, bp, wp,
                                          _stream(stream)), "iskv_import_state")

    def fold_stats(self, which, stream=None):
        """(sweeps [units] int32, discarded [units] fp32) of each unit's last fold."""
        U = self.cfg.batch * self.cfg.layers * self.cfg.kv_heads
        sw = torch.empty(U, dtype=torch.int32, device=self.device)
        dc = torch.empty(U, dtype=torch.float32, device=self.device)
        _check(self.lib.iskv_fold_stats(self.h, which, _vp(sw.data_ptr()), _vp(dc.data_ptr()),
                                        _stream(stream)), "iskv_fold_stats")
        return sw, dc

    def status(self, stream=None):
        f = ctypes.c_uint32(0)
        rc = self.lib.iskv_status(self.h, _stream(stream), ctypes.byref(f))
        if rc not in (ISKV_OK, ISKV_ERR_NUMERIC):
            raise ISKVError(rc, "iskv_status")
        return int(f.value)

    def close(self):
        if getattr(self, "h", None):
            self.lib.iskv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # unit index order used by fold_stats: [layer][batch][kv_head]
    def unit(self, batch, layer, head):
        return (layer * self.cfg.batch + batch) * self.cfg.kv_heads + head
