"""Ablation modes of the update on the GPU against the oracle in the same mode.

[iS-KV] "The Basis Drift Problem": updating the basis while stored rows keep
their coordinates makes the history drift; [iS-KV] "Ablation Study": keeping
the basis fixed. Each mode is the oracle's mode run on the same rows (fp32
rows and coordinates, so sigma and reconstruction are gated at 1e-4 like the
method itself); the drift ||X_hist - C B^T|| / ||X_hist|| of the three modes
is then compared on the GPU's own results.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import D, compare_sigma, note, to_dev, unit_state

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def iskv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv as m
    return m


def _stream(w, kind, changing):
    """Rows of one unit: the workload's recipe, or (changing) the same
    power-law spectrum whose directions switch to a new random basis after
    the first quarter."""
    X = synth.kv_rows(w, kind, 0, 0, 0, w.total_tokens, dtype="f32")
    if not changing:
        return X
    rng = np.random.default_rng(5 if kind == "K" else 6)
    W2, _ = np.linalg.qr(rng.standard_normal((D, D)))
    q = w.total_tokens // 4
    X = X.copy()
    X[q:] = X[q:] @ W2  # same spectrum, new right singular vectors
    return synth.round_to(X, "f32")


def _drift(rec, X, n):
    return float(np.linalg.norm(rec[:n] - X[:n]) / np.linalg.norm(X[:n]))


@pytest.mark.parametrize("changing", [False, True])
def test_modes_match_oracle_and_order_drift(iskv, changing):
    w = replace(synth.get_config(0), kv_dtype="f32", coord_dtype="f32", decode_tokens=1024, cfg_id=40)
    note("case: ablation modes, %s stream" % ("changing" if changing else "stationary"))
    X = {x: _stream(w, x, changing) for x in "KV"}
    Kd = to_dev(X["K"][None, None, None], torch.float32, DEV)
    Vd = to_dev(X["V"][None, None, None], torch.float32, DEV)
    drift = {}
    for mode, name in ((iskv.MODE_JOINT, "joint"), (iskv.MODE_FIXED_COORDS, "fixed coordinates"),
                       (iskv.MODE_FIXED_BASIS, "fixed basis")):
        cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype="f32"), device=DEV)
        cache.set_mode(mode)
        for t in range(0, w.total_tokens, 16):
            cache.append_block(Kd[:, :, :, t:t + 16].contiguous(), Vd[:, :, :, t:t + 16].contiguous())
        assert cache.status() == 0
        worst = [0.0, 0.0, 0.0]
        for which, x in ((0, "K"), (1, "V")):
            r = w.rank_k if x == "K" else w.rank_v
            st = oracle.UnitState.empty(D, w.block, r, w.total_tokens)
            st.append(X[x], w.window, mode=mode)
            C, sig, Bt, Wn, n, e, k = unit_state(cache, which, 0, 0, 0)
            assert (n, e, k) == (st.n, st.e, st.k), (name, x)
            err, rel = compare_sigma(sig[:k], st.sigma[:k])
            rec = cache.reconstruct(which, 0, 0, 0).cpu().double().numpy()
            ref = st.reconstruct()
            rerr = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
            assert err <= 1e-4 and rel <= 1e-4 and rerr <= 1e-4, (name, x, err, rel, rerr)
            worst = [max(a, b_) for a, b_ in zip(worst, (err, rel, rerr))]
            drift[(name, x)] = (_drift(rec, X[x], n), _drift(ref, X[x], n))
        note("  %-17s sigma %.1e/%.1e recon %.1e | drift K %.3f V %.3f (oracle %.3f %.3f)" % (
            name, worst[0], worst[1], worst[2], drift[(name, "K")][0], drift[(name, "V")][0],
            drift[(name, "K")][1], drift[(name, "V")][1]))
        cache.close()
    for x in "KV":
        j, fc, fb = drift[("joint", x)][0], drift[("fixed coordinates", x)][0], drift[("fixed basis", x)][0]
        assert fc > 2 * j, (x, j, fc)
        if changing:
            assert fb > 2 * j, (x, j, fb)
        else:
            assert fb >= 0.99 * j, (x, j, fb)


def test_mode_and_step_arguments_checked_on_host(iskv):
    """Invalid modes and missing buffers are rejected before any device work;
    a rejected call leaves the counters unchanged."""
    w = replace(synth.get_config(1), layers=1, kv_heads=2, q_heads=8, decode_tokens=200, cfg_id=41)
    cache = iskv.Cache(iskv.config_from_workload(w), device=DEV)
    for bad in (-1, 3, 99):
        assert cache.lib.iskv_set_mode(cache.h, bad) == iskv.ISKV_ERR_ARG
    k = torch.zeros((1, 1, 2, 1, D), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((1, 1, 8, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, 1, 8, D), dtype=torch.float32, device=DEV)
    vp = iskv._vp
    f = torch.float32
    rc = cache.lib.iskv_append_decode(cache.h, vp(k.data_ptr()), None, vp(q.data_ptr()), vp(out.data_ptr()),
                                      0, 1, iskv.ctypes.c_float(0.1), None)
    assert rc == iskv.ISKV_ERR_ARG and cache.counts(0) == (0, 0, 0, 0)
    rc = cache.lib.iskv_append_decode(cache.h, vp(k.data_ptr()), vp(k.data_ptr()), vp(q.data_ptr()),
                                      vp(out.data_ptr()), 0, 2, iskv.ctypes.c_float(0.1), None)
    assert rc == iskv.ISKV_ERR_ARG and cache.counts(0) == (0, 0, 0, 0)  # layer range beyond the cache
    o = cache.append_decode(k, k, q)
    assert cache.counts(0) == (0, 1, 0, 0) and o.dtype == f and torch.isfinite(o).all()
    cache.close()
