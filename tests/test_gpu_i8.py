"""GPU parity of int8 coordinate storage (ISKV_I8) against the fp64 oracle.

Storage reading (oracle ``ora_store_u_i8``): the history keeps U = C Sigma^-1
as int8 codes with one fp32 scale per row (scale = max|u| / 127, codes rounded
half to even); sigma and the basis stay fp32; every fold stores the rotated
old rows and the new rows again. A code is an integer decided by floating
point: both sides take it from the row's own product, the GPU in fp32 and the
oracle in fp64, so codes are compared exactly except where the fp64 value
lies within 2e-3 of a rounding boundary (one code apart there), and at most
1e-3 of them may differ. Decode is compared with fp64 attention over the
GPU's own stored factors (2e-3), sigma of one fold from the GPU's own stored
state with the oracle's fold of that state (1e-4).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import D, DEC_TOL, SIG_TOL, compare_sigma, decode_err, note, tdtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TIE = 2e-3        # codes may differ by one within this distance of a rounding boundary
FLIP_FRAC = 1e-3  # ... and at most this fraction of them


@pytest.fixture(scope="module")
def iskv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv
    return iskv


def _workload(rank_k, rank_v, block, window, layers=2, kv_heads=4, group=4, tokens=1024, cfg_id=60):
    return replace(synth.get_config(1), layers=layers, kv_heads=kv_heads, q_heads=kv_heads * group,
                   rank_k=rank_k, rank_v=rank_v, block=block, window=window, decode_tokens=tokens,
                   cfg_id=cfg_id)


def _cache(iskv, w, max_tokens=None):
    return iskv.Cache(iskv.config_from_workload(w, coord_dtype="i8", max_tokens=max_tokens), device=DEV)


def _rows_all(w, ntok):
    out = {}
    for x in "KV":
        a = np.zeros((w.batch, w.layers, w.kv_heads, ntok, D))
        for b in range(w.batch):
            for l in range(w.layers):
                for h in range(w.kv_heads):
                    a[b, l, h] = synth.kv_rows(w, x, b, l, h, ntok)
        out[x] = a
    return out


def _feed(cache, rows, t0, t1, step):
    K = to_dev(rows["K"][:, :, :, t0:t1], torch.bfloat16, DEV)
    V = to_dev(rows["V"][:, :, :, t0:t1], torch.bfloat16, DEV)
    for t in range(0, t1 - t0, step):
        s = min(step, t1 - t0 - t)
        cache.append_block(K[:, :, :, t:t + s].contiguous(), V[:, :, :, t:t + s].contiguous())


def _state(cache, which, b, l, h):
    """(codes [n, r] int, scales [n], sigma [r], Bt [r, D], window [e, D], n, e, k) on the host."""
    C, sig, Bt, W = cache.export_state(which, b, l, h)
    sc = cache.export_scales(which, b, l, h)
    n, e, kk, kv = cache.counts(l)
    k = kk if which == 0 else kv
    return (C.cpu().numpy().astype(np.int64), sc.cpu().double().numpy(), sig.cpu().double().numpy(),
            Bt.cpu().double().numpy(), W.float().cpu().double().numpy(), n, e, k)


def _stored_C(codes, scales, sigma, k):
    """History coordinates C = U Sigma of what is stored."""
    return codes[:, :k] * scales[:, None] * sigma[:k]


def _check_codes(codes, U_exact, label):
    """codes of each row of U against round(127 u / max|u|) of the exact fp64 row."""
    m = np.abs(U_exact).max(axis=1, keepdims=True)
    x = np.where(m > 0, 127.0 * U_exact / np.where(m > 0, m, 1.0), 0.0)
    want = np.rint(x)
    diff = np.abs(codes - want)
    near = np.abs(np.abs(x - np.floor(x)) - 0.5) < TIE
    bad = (diff > 1) | ((diff == 1) & ~near)
    frac = float((diff > 0).mean())
    assert not bad.any(), (label, "codes off beyond the rounding boundaries", int(bad.sum()))
    assert frac <= FLIP_FRAC, (label, frac)
    assert np.all(np.abs(codes) <= 127)
    return frac


@pytest.mark.parametrize("shape", [
    dict(rank_k=32, rank_v=32, block=64, window=128),     # the 8B-GQA shape
    dict(rank_k=24, rank_v=48, block=64, window=128),     # ragged K step, 24-byte rows
    dict(rank_k=64, rank_v=96, block=128, window=256),    # the 13B-MHA shape (k + b > d)
    dict(rank_k=128, rank_v=16, block=64, window=64),     # k reaches d; one column tile
])
def test_i8_fold_matches_oracle_fold_of_stored_state(iskv, shape):
    """Three folds, each checked from the GPU's own stored state before it:
    sigma against the oracle's fold of that state, every stored code (old rows
    rotated, new rows) against the exact fp64 rows of U, every scale."""
    b, wnd = shape["block"], shape["window"]
    w = _workload(tokens=wnd + 5 * b, cfg_id=61 + shape["rank_k"], **shape)
    note("case: int8 fold %s" % shape)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, rows, 0, wnd + 2 * b, b)  # two folds
    t = wnd + 2 * b
    worst_flip = 0.0
    for fold in range(3):
        _feed(cache, rows, t, t + b - 1, b)
        t += b - 1
        before = {(x, l, h): _state(cache, x, 0, l, h) for x in (0, 1) for l in range(2) for h in range(4)}
        _feed(cache, rows, t, t + 1, 1)  # triggers exactly one fold
        t += 1
        for (x, l, h), (q0, s0, sg0, B0, W0, n, e, k0) in before.items():
            r = w.rank_k if x == 0 else w.rank_v
            # the oracle's fp64 fold of the GPU's stored history (the int8 fold stores its result)
            st = oracle.UnitState.empty(D, b, r, n + b)
            st.C[:n, :k0] = _stored_C(q0, s0, sg0, k0)
            st.sigma[:k0] = sg0[:k0]
            st.Bt[:k0] = B0[:k0]
            st.n, st.k = n, k0
            F = np.vstack([W0, rows["KV"[x]][0, l, h, t - 1:t]])[:b]
            info = st.fold(F)
            q1, s1, sg1, B1, _, n1, _, k1 = _state(cache, x, 0, l, h)
            assert (n1, k1) == (n + b, info.kplus)
            err, rel = compare_sigma(sg1[:k1], st.sigma[:k1])
            assert err <= SIG_TOL and rel <= SIG_TOL, ("sigma", err, rel)
            # exact rows of U: C_old B_old^T B_new for the old rows, F B_new for
            # the new ones, over the new sigma (the GPU's own bases)
            Cx = np.vstack([_stored_C(q0, s0, sg0, k0)[:n] @ B0[:k0] @ B1[:k1].T, F @ B1[:k1].T])
            U = Cx / sg1[:k1]
            worst_flip = max(worst_flip, _check_codes(q1[:, :k1], U, (x, l, h, fold)))
            assert np.all(q1[:, k1:] == 0)
            m = np.abs(U).max(axis=1)
            np.testing.assert_allclose(s1, m / 127.0, rtol=2e-5, atol=0)
    assert cache.status() == 0
    note("  largest fraction of codes one apart: %.2e" % worst_flip)


def _decode_ref(cache, b, l, h, qg, scale):
    recs = []
    for which in (0, 1):
        q, sc, sg, Bt, W, n, e, k = _state(cache, which, b, l, h)
        recs.append(oracle.reconstruct(_stored_C(q, sc, sg, k), Bt[:k], W, k=k))
    return oracle.attend(recs[0], recs[1], qg, scale)


@pytest.mark.parametrize("shape", [
    dict(rank_k=32, rank_v=32, block=64, window=128, group=4),
    dict(rank_k=64, rank_v=96, block=128, window=256, group=1),
    dict(rank_k=24, rank_v=48, block=64, window=128, group=4),
    dict(rank_k=8, rank_v=128, block=64, window=64, group=2),
])
def test_i8_decode_on_stored_factors(iskv, shape):
    """Decode over int8 history + window: whole-unit launches, the split
    history of a one-layer call, the fused append, and the static-scratch
    entry point; each against fp64 attention over the stored factors."""
    w = _workload(tokens=3000, cfg_id=70 + shape["rank_v"], **shape)
    note("case: int8 decode %s" % shape)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, rows, 0, w.total_tokens - 3, w.block)
    scale = D ** -0.5
    g = w.group

    def qs(step, nl):
        return np.stack([np.stack([synth.queries(w, step, 0, l) for l in range(nl)])])

    def check(out, q, layers):
        o = out.float().cpu().double().numpy()
        errs = [decode_err(o[0, i, h * g:(h + 1) * g], _decode_ref(cache, 0, l, h, q[0, i, h * g:(h + 1) * g], scale))
                for i, l in enumerate(layers) for h in range(w.kv_heads)]
        assert max(errs) <= DEC_TOL, errs
        return max(errs)

    q = qs(0, w.layers)
    e1 = check(cache.decode_attn(to_dev(q, torch.bfloat16, DEV)), q, range(w.layers))
    q1 = q[:, 1:2].copy()
    e2 = check(cache.decode_attn(to_dev(q1, torch.bfloat16, DEV), layer0=1), q1, [1])     # split history
    e3 = check(cache.decode_attn_static(to_dev(q, torch.bfloat16, DEV)), q, range(w.layers))
    t = w.total_tokens - 3
    K = to_dev(rows["K"][:, :, :, t:t + 1], torch.bfloat16, DEV)
    V = to_dev(rows["V"][:, :, :, t:t + 1], torch.bfloat16, DEV)
    q2 = qs(1, w.layers)
    e4 = check(cache.append_decode(K, V, to_dev(q2, torch.bfloat16, DEV)), q2, range(w.layers))
    assert cache.status() == 0
    note("  decode errors: %.2e %.2e %.2e %.2e" % (e1, e2, e3, e4))


def test_i8_run_stays_with_the_oracle_i8_run(iskv):
    """A whole stream of the 8B-GQA shape (1024 tokens, 14 folds) in int8 on
    both sides: ranks identical; sigma within 1e-3 and the reconstruction
    within 5e-3 of the oracle's int8 run (the two trajectories part only
    where a code sits on a rounding boundary); the GPU's error against the
    true rows within 1% of the oracle's; reconstruction = stored factors."""
    w = _workload(32, 32, 64, 128, layers=1, kv_heads=2, tokens=1024, cfg_id=80)
    note("case: int8 run")
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, rows, 0, w.total_tokens, 1)
    assert cache.status() == 0
    for x in (0, 1):
        for h in range(2):
            X = rows["KV"[x]][0, 0, h]
            Xb = synth.bf16_round(X).astype(np.float64)
            st = oracle.run_unit(Xb, D, w.block, 32, w.window, store="i8")
            q, sc, sg, Bt, W, n, e, k = _state(cache, x, 0, 0, h)
            assert (n, e, k) == (st.n, st.e, st.k)
            err, rel = compare_sigma(sg[:k], st.sigma[:k])
            assert err <= 1e-3, ("sigma", err)
            rec = cache.reconstruct(x, 0, 0, h).cpu().double().numpy()
            mine = oracle.reconstruct(_stored_C(q, sc, sg, k), Bt[:k], W, k=k)
            assert np.linalg.norm(rec - mine) <= 1e-5 * np.linalg.norm(mine)
            ref = st.reconstruct()
            d = np.linalg.norm(rec - ref) / np.linalg.norm(ref)
            assert d <= 5e-3, ("reconstruction", d)
            eg = np.linalg.norm(rec - Xb) / np.linalg.norm(Xb)
            eo = np.linalg.norm(ref - Xb) / np.linalg.norm(Xb)
            assert eg <= 1.01 * eo, (eg, eo)
            note("  %s head %d: sigma %.1e, reconstruction %.1e, error %.4f vs oracle %.4f" % ("KV"[x], h, err, d, eg, eo))


@pytest.mark.parametrize("nrows,rk,rv", [(1000, 32, 48), (8192, 64, 96)])
def test_i8_prefill_oneshot(iskv, nrows, rk, rv):
    """One-shot prompt factorisation stored in int8: sigma against the
    oracle's truncated SVD, codes against the exact rows of U = X B^T Sigma^-1
    (the GPU's basis), scales; then 200 appends fold into that history."""
    w = _workload(rk, rv, 64, 128, layers=1, kv_heads=2, tokens=nrows + 200, cfg_id=90 + rk)
    note("case: int8 one-shot %d rows" % nrows)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    cache.prefill_oneshot(to_dev(rows["K"][:, :, :, :nrows], torch.bfloat16, DEV),
                          to_dev(rows["V"][:, :, :, :nrows], torch.bfloat16, DEV))
    for x in (0, 1):
        for h in range(2):
            r = rk if x == 0 else rv
            X = synth.bf16_round(rows["KV"[x]][0, 0, h, :nrows]).astype(np.float64)
            st = oracle.UnitState.empty(D, 64, r, nrows + 64)
            st.prefill_oneshot(X)
            q, sc, sg, Bt, W, n, e, k = _state(cache, x, 0, 0, h)
            assert (n, e, k) == (nrows, 0, st.k)
            err, rel = compare_sigma(sg[:k], st.sigma[:k])
            assert err <= SIG_TOL and rel <= SIG_TOL, ("sigma", err, rel)
            U = (X @ Bt[:k].T) / sg[:k]
            _check_codes(q[:, :k], U, (x, h))
            np.testing.assert_allclose(sc, np.abs(U).max(axis=1) / 127.0, rtol=2e-5, atol=0)
    _feed(cache, rows, nrows, nrows + 200, 1)
    assert cache.counts(0)[:2] == (nrows + 64, 136)
    assert cache.status() == 0


def test_i8_arguments_checked(iskv):
    w = _workload(32, 32, 64, 128, layers=1, kv_heads=1, tokens=256, cfg_id=99)
    cache = _cache(iskv, w)
    with pytest.raises(iskv.ISKVError):
        cache.set_mode(iskv.MODE_FIXED_COORDS)
    with pytest.raises(iskv.ISKVError):
        cache.set_mode(iskv.MODE_FIXED_BASIS)
    bf = iskv.Cache(iskv.config_from_workload(w, coord_dtype="bf16"), device=DEV)
    with pytest.raises(iskv.ISKVError):
        bf.export_scales(0, 0, 0, 0)
