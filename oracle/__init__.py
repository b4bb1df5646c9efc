"""fp64 CPU oracle of the iS-KV compressed KV cache -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package. The GPU library never links, loads or calls it, and
the two share no code.

The arithmetic lives in ``iskv_oracle.c`` (plain C, fp64, built with gcc);
this module only marshals numpy arrays through ctypes, plus two plain
drivers: ``run_unit`` (one K or V stream through prefill and decode appends)
and ``attend`` (dense attention over the reconstructed rows).
Source page: "iS-KV: Online Low-Rank KV Cache Compression via
Block-Incremental SVD", sections "Theoretical Foundation",
"Block-Incremental Decoding Updates" and "Reconstruction and Storage".
"""

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iskv_oracle.c")
_LIB = os.path.join(_HERE, "libiskv_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True, extra_flags=()) -> str:
    """Compile the oracle with gcc into oracle/libiskv_oracle.so."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", *extra_flags, _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def build_variant(out_path: str, defines=()) -> str:
    """Compile a copy of the oracle with extra -D flags (used by mutation tests)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", *["-D" + x for x in defines],
           _SRC, "-o", out_path, "-lm"]
    subprocess.check_call(cmd)
    return out_path


class _FoldInfo(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int), ("p", ctypes.c_int), ("kplus", ctypes.c_int),
                ("sweeps", ctypes.c_int), ("discarded", ctypes.c_double)]


def _bind(lib):
    lib.ora_jacobi.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, _D, ctypes.c_int]
    lib.ora_jacobi.restype = ctypes.c_int
    lib.ora_singular_values.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, ctypes.c_int]
    lib.ora_singular_values.restype = ctypes.c_int
    lib.ora_fold.argtypes = [ctypes.c_int] * 5 + [_D, ctypes.c_int, _D, _D, _D, ctypes.c_int,
                                                  ctypes.c_int, ctypes.POINTER(_FoldInfo)]
    lib.ora_fold.restype = ctypes.c_int
    lib.ora_run.argtypes = [ctypes.c_int] * 6 + [_D, ctypes.c_int, ctypes.c_int, _D, _D, _D, _I, _D,
                                                 ctypes.c_int]
    lib.ora_run.restype = ctypes.c_int
    lib.ora_reconstruct.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _D,
                                    ctypes.c_int, _D, _D]
    lib.ora_reconstruct.restype = None
    lib.ora_attend.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _D, _D,
                               ctypes.c_double, _D]
    lib.ora_attend.restype = None
    lib.ora_prefill_oneshot.argtypes = [ctypes.c_int] * 3 + [_D, _D, ctypes.c_int, _D, _D,
                                                              ctypes.POINTER(_FoldInfo)]
    lib.ora_prefill_oneshot.restype = ctypes.c_int
    lib.ora_store_i8.argtypes = [ctypes.c_int] * 3 + [_D, ctypes.POINTER(ctypes.c_int8), ctypes.c_int, _D]
    lib.ora_store_i8.restype = None
    lib.ora_store_u_i8.argtypes = [ctypes.c_int] * 3 + [_D, _D, ctypes.POINTER(ctypes.c_int8), ctypes.c_int, _D]
    lib.ora_store_u_i8.restype = None
    lib.ora_fold_i8.argtypes = [ctypes.c_int] * 5 + [_D, ctypes.c_int, _D, _D, _D, ctypes.c_int,
                                                     ctypes.POINTER(_FoldInfo)]
    lib.ora_fold_i8.restype = ctypes.c_int
    lib.ora_storage_bytes.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_double]
    lib.ora_storage_bytes.restype = ctypes.c_double
    return lib


def load(path: str = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        alt = os.environ.get("ISKV_ORACLE_LIB")  # a planted-mistake variant under test
        if alt:
            _lib = _bind(ctypes.CDLL(alt))
            return _lib
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _p(a):
    return a.ctypes.data_as(_D)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


class OracleError(RuntimeError):
    pass


# --------------------------------------------------------------------------
# Thin wrappers
# --------------------------------------------------------------------------

def jacobi(Z, maxsweeps=60, lib=None):
    """One-sided Jacobi on Z (m x c). Returns (Z H, H, column norms, sweeps)."""
    lib = lib or load()
    Z = _f64(Z)
    m, c = Z.shape
    zbuf = np.ascontiguousarray(Z.T)  # column-major storage of Z = rows of Z^T
    H = np.zeros((c, c))
    sv = np.zeros(c)
    sweeps = lib.ora_jacobi(m, c, _p(zbuf), _p(H), _p(sv), maxsweeps)
    if sweeps == -1:
        raise ValueError("one-sided Jacobi needs rows >= columns")
    if sweeps < 0:
        raise OracleError("Jacobi did not converge")
    # H is column-major: H[j*c + i] = H(i, j) -> buffer row j is column j
    return zbuf.T.copy(), H.T.copy(), sv, sweeps


def singular_values(X, lib=None):
    lib = lib or load()
    X = _f64(X)
    m, c = X.shape
    out = np.zeros(c)
    rc = lib.ora_singular_values(m, c, _p(X), _p(out), 200)
    if rc < 0:
        raise OracleError("Jacobi did not converge")
    return out


@dataclass
class UnitState:
    """State of one K or V stream: history C (n x k), sigma (k), basis Bt (k x d), window rows."""
    d: int
    b: int
    r: int
    C: np.ndarray          # (capacity, d); rows 0..n-1 valid, columns 0..k-1
    sigma: np.ndarray      # (d,)
    Bt: np.ndarray         # (d, d); rows 0..k-1 valid
    n: int = 0
    k: int = 0
    window: list = field(default_factory=list)
    log: list = field(default_factory=list)  # per fold: (k, p, kplus, sweeps, discarded)
    store: str = "f64"     # "f64", or "i8": C holds int8-stored rows (ora_store_i8)

    @classmethod
    def empty(cls, d, b, r, capacity):
        return cls(d=d, b=b, r=r, C=np.zeros((capacity + b, d)), sigma=np.zeros(d), Bt=np.zeros((d, d)))

    @property
    def e(self):
        return len(self.window)

    def fold(self, F, mode=0, porder=0, lib=None):
        lib = lib or load()
        F = _f64(F)
        assert F.shape == (self.b, self.d)
        if self.n + self.b > self.C.shape[0]:
            grow = np.zeros((self.n + self.b + self.b, self.d))
            grow[: self.C.shape[0]] = self.C
            self.C = grow
        info = _FoldInfo()
        if self.store == "i8":
            if mode != 0:
                raise ValueError("int8 coordinate storage is defined for the joint update only")
            rc = lib.ora_fold_i8(self.d, self.b, self.r, self.n, self.k, _p(self.C), self.d,
                                 _p(self.sigma), _p(self.Bt), _p(F), porder, ctypes.byref(info))
        else:
            rc = lib.ora_fold(self.d, self.b, self.r, self.n, self.k, _p(self.C), self.d,
                              _p(self.sigma), _p(self.Bt), _p(F), mode, porder, ctypes.byref(info))
        if rc != 0:
            raise OracleError("ora_fold failed: %d" % rc)
        self.log.append((info.k, info.p, info.kplus, info.sweeps, info.discarded))
        self.n += self.b
        self.k = info.kplus
        return info

    def append(self, rows, w, mode=0, lib=None):
        """Rows enter the exact window; once it holds >= w + b rows the oldest b fold."""
        folds = 0
        for row in _f64(rows).reshape(-1, self.d):
            self.window.append(row.copy())
            if len(self.window) >= w + self.b:
                F = np.stack(self.window[: self.b])
                del self.window[: self.b]
                self.fold(F, mode=mode, lib=lib)
                folds += 1
        return folds

    def prefill(self, rows, mode=0, lib=None):
        """Fold whole blocks straight into history (window must be empty)."""
        assert not self.window
        rows = _f64(rows).reshape(-1, self.d)
        assert rows.shape[0] % self.b == 0
        for s in range(0, rows.shape[0], self.b):
            self.fold(rows[s: s + self.b], mode=mode, lib=lib)

    def prefill_oneshot(self, rows, lib=None):
        """Factorise all prompt rows at once into the history (the cache must
        be empty): truncated SVD, k = min(r, rows, d)."""
        assert self.n == 0 and not self.window
        lib = lib or load()
        rows = _f64(rows).reshape(-1, self.d)
        N = rows.shape[0]
        if self.C.shape[0] < N + self.b:
            self.C = np.zeros((N + self.b, self.d))
        info = _FoldInfo()
        kp = lib.ora_prefill_oneshot(self.d, self.r, N, _p(rows), _p(self.C), self.d, _p(self.sigma),
                                     _p(self.Bt), ctypes.byref(info))
        if kp < 0:
            raise OracleError("ora_prefill_oneshot failed: %d" % kp)
        if self.store == "i8":
            lib.ora_store_u_i8(N, kp, self.d, _p(self.C), _p(self.sigma), None, 0, None)
        self.log.append((info.k, info.p, info.kplus, info.sweeps, info.discarded))
        self.n = N
        self.k = kp
        return info

    def history(self):
        """History coordinates and basis: (C[:n, :k], sigma[:k], Bt[:k])."""
        return self.C[: self.n, : self.k], self.sigma[: self.k], self.Bt[: self.k]

    def window_rows(self):
        return np.stack(self.window) if self.window else np.zeros((0, self.d))

    def reconstruct(self, lib=None):
        return reconstruct(self.C[: self.n, : self.d], self.Bt[: self.k], self.window_rows(),
                           k=self.k, lib=lib)


def reconstruct(C, Bt, W, k=None, lib=None):
    """X~ = [C B^T ; W] (history rows then exact window rows)."""
    lib = lib or load()
    C = _f64(C)
    Bt = _f64(Bt)
    W = _f64(W).reshape(-1, Bt.shape[1] if Bt.size else W.shape[-1])
    n = C.shape[0]
    d = W.shape[1] if W.size else Bt.shape[1]
    k = Bt.shape[0] if k is None else k
    ldc = C.shape[1] if C.ndim == 2 and C.shape[1] > 0 else 1
    if ldc < k:
        raise ValueError("C narrower than k")
    Bt_full = np.zeros((max(k, 1), d))
    Bt_full[:k] = Bt[:k]
    Cc = np.ascontiguousarray(C) if n else np.zeros((0, max(ldc, 1)))
    out = np.zeros((n + W.shape[0], d))
    lib.ora_reconstruct(d, n, k, max(ldc, 1), _p(Cc), _p(Bt_full), W.shape[0], _p(_f64(W)), _p(out))
    return out


def attend(Kt, Vt, q, scale, lib=None):
    """Dense attention of g query rows over T reconstructed rows, fp64."""
    lib = lib or load()
    Kt, Vt, q = _f64(Kt), _f64(Vt), _f64(np.atleast_2d(q))
    T, d = Kt.shape
    g = q.shape[0]
    out = np.zeros((g, d))
    lib.ora_attend(d, T, g, _p(Kt), _p(Vt), _p(q), float(scale), _p(out))
    return out


def store_i8(C, k, lib=None):
    """Per-row int8 storage of C's first k columns (ora_store_i8).
    Returns (stored values, int8 codes, per-row scales)."""
    lib = lib or load()
    S = _f64(C).copy()
    rows, ldc = S.shape
    Q = np.zeros((rows, ldc), dtype=np.int8)
    sc = np.zeros(rows)
    lib.ora_store_i8(rows, k, ldc, _p(S), Q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), ldc, _p(sc))
    return S, Q, sc


def store_u_i8(C, sigma, k, lib=None):
    """int8 storage of a history C = U Sigma (ora_store_u_i8): U = C Sigma^-1
    stored per row. Returns (stored C, int8 codes of U, per-row scales of U)."""
    lib = lib or load()
    S = _f64(C).copy()
    rows, ldc = S.shape
    sg = np.zeros(max(ldc, k))
    sg[:k] = _f64(sigma)[:k]
    Q = np.zeros((rows, ldc), dtype=np.int8)
    sc = np.zeros(rows)
    lib.ora_store_u_i8(rows, k, ldc, _p(S), _p(sg), Q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), ldc,
                       _p(sc))
    return S, Q, sc


def run_unit(X, d, b, r, w, prefill=0, mode=0, store="f64", lib=None):
    """Drive one stream through the C driver: prefill rows fold directly, the
    rest arrive one at a time through the window. store="i8" keeps the
    coordinates as int8 rows with per-row scales. Returns a UnitState."""
    lib = lib or load()
    X = _f64(X)
    N = X.shape[0]
    C = np.zeros((max(N, 1), d))
    sigma = np.zeros(d)
    Bt = np.zeros((d, d))
    counts = np.zeros(3, dtype=np.int32)
    cap = N // b + 1
    log = np.zeros((cap, 5))
    folds = lib.ora_run(d, b, r, w, N, prefill, _p(X), mode, 1 if store == "i8" else 0, _p(C),
                        _p(sigma), _p(Bt), counts.ctypes.data_as(_I), _p(log), cap)
    if folds < 0:
        raise OracleError("ora_run failed: %d" % folds)
    n, e, k = (int(x) for x in counts)
    st = UnitState(d=d, b=b, r=r, C=C, sigma=sigma, Bt=Bt, n=n, k=k, store=store)
    st.window = [row.copy() for row in X[N - e:]]
    st.log = [(int(a), int(p_), int(kp), int(sw), float(ds)) for a, p_, kp, sw, ds in log[:folds]]
    return st


def storage_bytes(d, kk, nk, ek, kv, nv, ev, beta_f, beta_e, lib=None):
    lib = lib or load()
    return lib.ora_storage_bytes(d, kk, nk, ek, kv, nv, ev, float(beta_f), float(beta_e))
