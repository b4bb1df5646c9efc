"""One-shot prefill ([iS-KV] Prefill Compression; protection not modelled)
against the oracle's one-shot truncated SVD of the same rows, then ordinary
appends folding into that history on both sides."""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (D, DEC_TOL, check_unit, decode_err, decode_reference_on_gpu_factors, note, tdtype,
                      to_dev, unit_state)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def iskv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv as m
    return m


def _rows(w, ntok):
    out = {}
    for x in "KV":
        a = np.zeros((w.batch, w.layers, w.kv_heads, ntok, D))
        for b in range(w.batch):
            for l in range(w.layers):
                for h in range(w.kv_heads):
                    a[b, l, h] = synth.kv_rows(w, x, b, l, h, ntok)
        out[x] = a
    return out


@pytest.mark.parametrize("nrows,rk,rv,coord", [
    (1000, 32, 48, "f32"),   # several 128-row QR blocks and a ragged tail (blockwise QR)
    (40, 64, 64, "f32"),     # fewer rows than d: k = nrows, exact
    (128, 128, 128, "f32"),  # untruncated, one full block
    (700, 32, 32, "bf16"),   # bf16 coordinates
    (8192, 32, 48, "f32"),   # Cholesky-QR of the Gram matrix
    (4096, 32, 48, "bf16"),  # Cholesky-QR, bf16 coordinates
])
def test_prefill_oneshot_matches_oracle(iskv, nrows, rk, rv, coord):
    extra = 300
    w = replace(synth.get_config(3), layers=2, kv_heads=2, q_heads=8, rank_k=rk, rank_v=rv,
                prefill_blocks=0, decode_tokens=nrows + extra, cfg_id=60 + rk + nrows % 97)
    note("case: one-shot prefill nrows=%d rk=%d rv=%d coords %s" % (nrows, rk, rv, coord))
    rows = _rows(w, nrows + extra)
    cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype=coord), device=DEV)
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"], dt, DEV)
    V = to_dev(rows["V"], dt, DEV)
    cache.prefill_oneshot(K[:, :, :, :nrows].contiguous(), V[:, :, :, :nrows].contiguous())
    assert cache.status() == 0
    assert cache.counts(0) == (nrows, 0, min(rk, nrows, D), min(rv, nrows, D))
    assert cache.counts(1) == cache.counts(0)
    units = [(0, 0, 0), (0, 1, 1)]
    keys = [(which, b, l, h) for (b, l, h) in units for which in (0, 1)]

    def one(key):
        which, b, l, h = key
        st = oracle.UnitState.empty(D, w.block, (rk, rv)[which], nrows + extra)
        st.prefill_oneshot(rows["KV"[which]][b, l, h, :nrows])
        return st

    with ThreadPoolExecutor(max_workers=4) as ex:
        states = dict(zip(keys, ex.map(one, keys)))
    for (b, l, h) in units:
        for which, (x, r) in enumerate((("K", rk), ("V", rv))):
            st = states[(which, b, l, h)]
            if coord == "f32":
                e1, e2, e3 = check_unit(cache, which, b, l, h, st, label=(nrows, x))
                note("  %s sigma %.2e/%.2e recon %.2e" % (x, e1, e2, e3))
            else:
                C, sig, Bt, W, n, e, k = unit_state(cache, which, b, l, h)
                assert (n, e, k) == (st.n, st.e, st.k)
                rec = cache.reconstruct(which, b, l, h).cpu().double().numpy()
                ref = st.reconstruct()
                rel = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
                assert rel <= 2.0 ** -7, (x, rel)
                note("  %s bf16 recon vs fp64 oracle %.2e" % (x, rel))
            if nrows <= D and r >= nrows:  # nothing truncated: the history is exact
                rec = cache.reconstruct(which, b, l, h).cpu().double().numpy()
                X = rows[x][b, l, h, :nrows]
                assert np.linalg.norm(rec - X) <= (1e-5 if coord == "f32" else 1e-2) * np.linalg.norm(X)
    # decode straight on the one-shot factors (empty window)
    g = w.group
    q = np.stack([synth.queries(w, 3, 0, l) for l in range(w.layers)])[None]
    out = cache.decode_attn(to_dev(q, dt, DEV)).cpu().double().numpy()
    for (b, l, h) in units:
        ref = decode_reference_on_gpu_factors(cache, b, l, h, q[b, l, h * g:(h + 1) * g], D ** -0.5)
        assert decode_err(out[b, l, h * g:(h + 1) * g], ref) <= DEC_TOL
    # later tokens go through the window and fold into the one-shot history
    for t in range(nrows, nrows + extra):
        cache.append_block(K[:, :, :, t:t + 1].contiguous(), V[:, :, :, t:t + 1].contiguous())
    assert cache.status() == 0
    if coord == "f32":
        for (which, b, l, h), st in states.items():
            x = "KV"[which]
            st.append(rows[x][b, l, h, nrows:nrows + extra], w.window)
            check_unit(cache, which, b, l, h, st, label=(nrows, x, "after appends"))


def test_prefill_oneshot_argument_and_state_checks(iskv):
    w = replace(synth.get_config(3), layers=2, kv_heads=2, q_heads=8, prefill_blocks=0, decode_tokens=400,
                cfg_id=59)
    rows = _rows(w, 400)
    cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype="f32"), device=DEV)
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"], dt, DEV)
    V = to_dev(rows["V"], dt, DEV)
    with pytest.raises(iskv.ISKVError) as ei:  # more rows than the cache holds
        cache.prefill_oneshot(K.repeat(1, 1, 1, 2, 1).contiguous(), V.repeat(1, 1, 1, 2, 1).contiguous())
    assert ei.value.code == iskv.ISKV_ERR_CAPACITY
    assert cache.counts(0) == (0, 0, 0, 0)
    cache.append_block(K[:, :, :, :1].contiguous(), V[:, :, :, :1].contiguous())
    with pytest.raises(iskv.ISKVError) as ei:  # not empty any more
        cache.prefill_oneshot(K[:, :, :, :100].contiguous(), V[:, :, :, :100].contiguous())
    assert ei.value.code == iskv.ISKV_ERR_STATE
    assert cache.status() == 0


@pytest.mark.parametrize("nrows,max_tokens", [
    (200, 300),    # blockwise QR
    (2048, 8192),  # Cholesky-QR of the Gram matrix (pivots of rounding give zero rows)
])
def test_prefill_oneshot_rank_deficient_rows(iskv, nrows, max_tokens):
    """Rows of rank 3 under a rank budget of 8: the five extra basis vectors
    are completed orthonormally; the history equals the rows."""
    # fp32 rows: in bf16 the rounding itself would lift the rank to d
    w = replace(synth.get_config(3), layers=1, kv_heads=1, q_heads=4, rank_k=8, rank_v=8, prefill_blocks=0,
                decode_tokens=max_tokens, kv_dtype="f32", coord_dtype="f32", cfg_id=58)
    note("case: rank-3 one-shot prefill nrows=%d" % nrows)
    rows = _rows(w, nrows)
    rng = np.random.default_rng(5)
    rows["K"][0, 0, 0] = rng.standard_normal((nrows, 3)) @ rng.standard_normal((3, D))
    cache = iskv.Cache(iskv.config_from_workload(w, max_tokens=max_tokens), device=DEV)
    K = to_dev(rows["K"], torch.float32, DEV)
    V = to_dev(rows["V"], torch.float32, DEV)
    cache.prefill_oneshot(K.contiguous(), V.contiguous())
    assert cache.status() == 0
    C, sig, Bt, W, n, e, k = unit_state(cache, 0, 0, 0, 0)
    assert (n, e, k) == (nrows, 0, 8)
    assert np.abs(Bt[:k] @ Bt[:k].T - np.eye(k)).max() < 1e-5
    X = cache.reconstruct(0, 0, 0, 0).cpu().double().numpy()
    ref = K[0, 0, 0].double().cpu().numpy()
    assert np.linalg.norm(X - ref) <= 1e-5 * np.linalg.norm(ref)
    assert sig[3:k].max() <= 1e-5 * sig[0]
    # the values (full rank) against the oracle
    st = oracle.UnitState.empty(D, w.block, 8, max_tokens)
    st.prefill_oneshot(rows["V"][0, 0, 0])
    check_unit(cache, 1, 0, 0, 0, st, label=("rank-deficient keys, values", nrows))


def test_prefill_oneshot_layer_subset(iskv):
    """One-shot prompt of layer 1 only (layer0 = 1 of 3, the input holding that
    layer alone): layers 0 and 2 stay empty and then take block prefills."""
    w = replace(synth.get_config(3), layers=3, kv_heads=2, q_heads=8, prefill_blocks=0, decode_tokens=600,
                cfg_id=57)
    rows = _rows(w, 512)
    cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype="f32"), device=DEV)
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"], dt, DEV)
    V = to_dev(rows["V"], dt, DEV)
    cache.prefill_oneshot(K[:, 1:2].contiguous(), V[:, 1:2].contiguous(), layer0=1)
    assert cache.counts(0) == (0, 0, 0, 0) and cache.counts(2) == (0, 0, 0, 0)
    assert cache.counts(1) == (512, 0, w.rank_k, w.rank_v)
    for which, (x, r) in enumerate((("K", w.rank_k), ("V", w.rank_v))):
        for h in range(w.kv_heads):
            st = oracle.UnitState.empty(D, w.block, r, 600)
            st.prefill_oneshot(rows[x][0, 1, h])
            check_unit(cache, which, 0, 1, h, st, label=("layer subset", x, h))
    cache.prefill_block(K[:, 0:1, :, :w.block].contiguous(), V[:, 0:1, :, :w.block].contiguous(), layer0=0)
    assert cache.counts(0)[:2] == (w.block, 0) and cache.counts(1)[0] == 512 and cache.counts(2) == (0, 0, 0, 0)
    assert cache.status() == 0


def test_prefill_oneshot_long_input_full_size(iskv):
    """The long-input workload's prompt at full size: 65536 rows for each of
    its 256 units (K and V), one iskv_prefill_oneshot call (the launch the
    prefill benchmark times); sampled units against the oracle's one-shot
    truncated SVD of the same rows (fp32 coordinates), the rest checked for
    orthonormal bases."""
    w = replace(synth.get_config(3), decode_tokens=0)
    P = w.prefill_blocks * w.block
    note("case: one-shot prefill of %d rows x %d units" % (P, w.units))
    dev_rows = {x: synth.kv_rows_torch(w, x, P, DEV) for x in "KV"}
    samples = [(0, 0, 0), (0, 31, 5)]
    host = {}
    for (b, l, h) in samples:
        for x in "KV":
            host[(x, b, l, h)] = synth.kv_rows(w, x, b, l, h, P)
            dev_rows[x][b, l, h] = to_dev(host[(x, b, l, h)], torch.bfloat16, DEV)
    cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype="f32"), device=DEV)
    cache.prefill_oneshot(dev_rows["K"], dev_rows["V"])
    del dev_rows
    assert cache.status() == 0
    assert cache.counts(0) == (P, 0, w.rank_k, w.rank_v)
    keys = [(which, b, l, h) for (b, l, h) in samples for which in (0, 1)]

    def one(key):
        which, b, l, h = key
        st = oracle.UnitState.empty(D, w.block, (w.rank_k, w.rank_v)[which], P)
        st.prefill_oneshot(host[("KV"[which], b, l, h)])
        return st

    with ThreadPoolExecutor(max_workers=4) as ex:
        states = dict(zip(keys, ex.map(one, keys)))
    for (which, b, l, h), st in states.items():
        e1, e2, e3 = check_unit(cache, which, b, l, h, st, label=("long input", which, b, l, h))
        note("  %s %s sigma %.2e/%.2e recon %.2e" % ("KV"[which], (b, l, h), e1, e2, e3))
    for (b, l, h) in [(0, 7, 3), (0, 20, 7)]:
        for which in (0, 1):
            C, sig, Bt, W, n, e, k = unit_state(cache, which, b, l, h)
            assert np.abs(Bt[:k] @ Bt[:k].T - np.eye(k)).max() < 1e-5
            assert np.all(np.diff(sig[:k]) <= 1e-6 * sig[0])
