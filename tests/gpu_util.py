"""Shared helpers of the GPU parity tests (run the HIP path, run the oracle,
compare). Tolerances follow the numbers stated for the path:
  singular values  max |s_gpu - s_ora| / s_1 <= 1e-4, and per value relative
                   <= 1e-4 for s >= 0.05 s_1 (fp32 coordinates)
  reconstruction   ||X~_gpu - X~_ora||_F / ||X~_ora||_F <= 1e-4 (fp32 coordinates)
  decode           max |o_gpu - o_ora| / max |o_ora| <= 2e-3 with the oracle run
                   on the GPU's own stored factors and window
  ranks            the (k, p, k+) sequence of every fold identical
"""

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth
from incremental_rank_svd_amd import iskv

D = 128
SIG_TOL = 1e-4
REC_TOL = 1e-4
DEC_TOL = 2e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def host_rows(w, which, b, l, h, n, seed=0):
    return synth.kv_rows(w, which, b, l, h, n, seed=seed)


def to_dev(x, dtype, dev):
    return torch.tensor(np.asarray(x), dtype=torch.float32, device=dev).to(dtype)


def oracle_units(jobs):
    """Run oracle.run_unit for several (X, d, b, r, w, prefill) jobs in parallel threads."""
    def one(j):
        X, b, r, w, prefill = j
        return oracle.run_unit(X, D, b, r, w, prefill=prefill)
    with ThreadPoolExecutor(max_workers=8) as ex:
        return list(ex.map(one, jobs))


def compare_sigma(sig_gpu, sig_ora):
    s1 = sig_ora[0]
    err = np.abs(sig_gpu - sig_ora).max() / s1 if len(sig_ora) else 0.0
    big = sig_ora >= 0.05 * s1
    rel = (np.abs(sig_gpu - sig_ora)[big] / sig_ora[big]).max() if big.any() else 0.0
    return float(err), float(rel)


def unit_state(cache, which, b, l, h):
    C, sig, Bt, W = cache.export_state(which, b, l, h)
    n, e, kk, kv = cache.counts(l)
    k = kk if which == 0 else kv
    return (C.float().cpu().double().numpy(), sig.cpu().double().numpy(), Bt.cpu().double().numpy(),
            W.float().cpu().double().numpy(), n, e, k)


def check_unit(cache, which, b, l, h, st, rec_tol=REC_TOL, sig_tol=SIG_TOL, label=""):
    C, sig, Bt, W, n, e, k = unit_state(cache, which, b, l, h)
    assert (n, e, k) == (st.n, st.e, st.k), (label, (n, e, k), (st.n, st.e, st.k))
    err, rel = compare_sigma(sig[:k], st.sigma[:k])
    assert err <= sig_tol and rel <= sig_tol, (label, "sigma", err, rel)
    assert np.all(sig[k:] == 0) and np.all(C[:, k:] == 0) and np.all(Bt[k:] == 0)
    rec = cache.reconstruct(which, b, l, h).cpu().double().numpy()
    ref = st.reconstruct()
    rerr = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
    assert rerr <= rec_tol, (label, "reconstruction", rerr)
    # the window part is exact
    assert np.array_equal(rec[n:], ref[n:]), (label, "window rows")
    return err, rel, rerr


def decode_reference_on_gpu_factors(cache, b, l, h, q_group, scale):
    """Dense fp64 attention over the reconstruction of the GPU's own stored state."""
    recs = []
    for which in (0, 1):
        C, sig, Bt, W, n, e, k = unit_state(cache, which, b, l, h)
        recs.append(oracle.reconstruct(C, Bt[:k], W, k=k))
    return oracle.attend(recs[0], recs[1], q_group, scale)


def decode_err(o_gpu, o_ref):
    return float(np.abs(o_gpu - o_ref).max() / np.abs(o_ref).max())
