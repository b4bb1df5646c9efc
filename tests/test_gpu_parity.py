"""GPU parity of the HIP path against the fp64 oracle on identical seeded inputs.

Every call goes through the C ABI (libiskv.so) via its ctypes binding.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (D, DEC_TOL, check_unit, decode_err, decode_reference_on_gpu_factors,
                      note, oracle_units, tdtype, to_dev, unit_state)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv
    return iskv


@pytest.fixture(scope="module")
def iskv():
    return _need_gpu()


def _cache(iskv, w, coord=None, max_tokens=None):
    return iskv.Cache(iskv.config_from_workload(w, coord_dtype=coord, max_tokens=max_tokens), device=DEV)


def _rows_all(w, ntok, seed=0):
    """Host rows of every unit: dict which -> array [batch, layers, kvh, ntok, D]."""
    out = {}
    for x in "KV":
        a = np.zeros((w.batch, w.layers, w.kv_heads, ntok, D))
        for b in range(w.batch):
            for l in range(w.layers):
                for h in range(w.kv_heads):
                    a[b, l, h] = synth.kv_rows(w, x, b, l, h, ntok, seed=seed)
        out[x] = a
    return out


def _feed(cache, w, rows, t0, t1, step):
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"][:, :, :, t0:t1], dt, DEV)
    V = to_dev(rows["V"][:, :, :, t0:t1], dt, DEV)
    for t in range(0, t1 - t0, step):
        s = min(step, t1 - t0 - t)
        cache.append_block(K[:, :, :, t:t + s].contiguous(), V[:, :, :, t:t + s].contiguous())


def _queries(w, step, nl=None):
    nl = w.layers if nl is None else nl
    q = np.stack([np.stack([synth.queries(w, step, b, l) for l in range(nl)]) for b in range(w.batch)])
    return q  # [batch, layers, qh, D]


def _check_decode(cache, w, q, out, units, scale=D ** -0.5, tol=DEC_TOL):
    errs = []
    o = out.float().cpu().double().numpy()
    g = w.group
    for (b, l, h) in units:
        ref = decode_reference_on_gpu_factors(cache, b, l, h, q[b, l, h * g:(h + 1) * g], scale)
        errs.append(decode_err(o[b, l, h * g:(h + 1) * g], ref))
    assert max(errs) <= tol, errs
    return max(errs)


# ---------------------------------------------------------------------------


def test_single_head_fp32_workload_end_to_end(iskv):
    """Single-head fp32 workload: 1024 rows one at a time, 15 folds, decode."""
    w = synth.get_config(0)
    note("case: single_head_fp32 full run")
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    ks = []
    for t in range(w.total_tokens):
        _feed(cache, w, rows, t, t + 1, 1)
        n, e, kk, kv = cache.counts(0)
        if not ks or ks[-1][0] != n:
            ks.append((n, kk, kv))
    q = _queries(w, 0)
    out = cache.decode_attn(to_dev(q, torch.float32, DEV))
    assert cache.status() == 0
    st = oracle_units([(rows[x][0, 0, 0], w.block, w.rank_k, w.window, 0) for x in "KV"])
    # rank sequence: (k before, p, k+) of every fold
    gpu_seq = [(ks[i][1], min(w.block, D - ks[i][1]), ks[i + 1][1]) for i in range(len(ks) - 1)]
    ora_seq = [(a, p, kp) for (a, p, kp, _, _) in st[0].log]
    assert gpu_seq == ora_seq
    for x, s in zip((0, 1), st):
        e1, e2, e3 = check_unit(cache, x, 0, 0, 0, s, label="K" if x == 0 else "V")
        note("  %s sigma %.2e/%.2e recon %.2e" % ("KV"[x], e1, e2, e3))
    # decode: on the GPU's own factors (gate) and against the oracle's own state
    derr = _check_decode(cache, w, q, out, [(0, 0, 0)])
    o_ora = oracle.attend(st[0].reconstruct(), st[1].reconstruct(), q[0, 0], D ** -0.5)
    o = out.float().cpu().double().numpy()[0, 0]
    assert decode_err(o, o_ora) <= DEC_TOL
    sw, dc = cache.fold_stats(0)
    assert int(sw[0]) >= 1
    assert abs(float(dc[0]) - st[0].log[-1][4]) <= 1e-3 * max(st[0].log[-1][4], 1e-30) + 1e-6
    note("  decode err %.2e" % derr)


@pytest.mark.parametrize("coord", ["f32", "bf16"])
def test_gqa_multi_unit(iskv, coord):
    """batch 2 x 2 layers x 2 kv heads, GQA group 4, bf16 rows: every unit
    against the oracle (fp32 coordinates gate sigma/reconstruction; bf16
    coordinates gate decode on the stored factors)."""
    from dataclasses import replace

    w = replace(synth.get_config(1), batch=2, layers=2, kv_heads=2, q_heads=8, rank_v=24,
                decode_tokens=1000, cfg_id=11)
    note("case: gqa_multi_unit coord=%s" % coord)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w, coord=coord)
    _feed(cache, w, rows, 0, 400, 1)      # one row at a time
    _feed(cache, w, rows, 400, 1000, 37)  # ragged multi-row appends
    q = _queries(w, 3)
    out = cache.decode_attn(to_dev(q, torch.bfloat16, DEV))
    assert cache.status() == 0
    units = [(b, l, h) for b in range(2) for l in range(2) for h in range(2)]
    if coord == "f32":
        jobs = []
        for (b, l, h) in units:
            for x, r in (("K", w.rank_k), ("V", w.rank_v)):
                jobs.append((rows[x][b, l, h], w.block, r, w.window, 0))
        st = oracle_units(jobs)
        for i, (b, l, h) in enumerate(units):
            for x in (0, 1):
                check_unit(cache, x, b, l, h, st[2 * i + x], label=str((b, l, h, x)))
    derr = _check_decode(cache, w, q, out, units)
    note("  decode err %.2e" % derr)


def _rotation_check(C0, B0, k0, n, C1, B1, k1):
    """Old rows after a fold against C_old (B_old B_new^T) in fp64, which is
    C_old H_top for any correct fold (B_new = [B_old P] H, B_old P = 0):
    every value within one bf16 ulp of the rounded product, plus the fp32
    floor of a k-term product (16 fp32 ulps of the row's norm: H_top and
    the basis are fp32 and re-orthonormalised to first order, so values far
    below their row's norm carry that absolute error), for all but 1e-3 of
    them; returns the max deviation relative to the largest value."""
    Ht = B0[:k0] @ B1[:k1].T  # k0 x k1
    ref = C0[:n, :k0] @ Ht
    ref_bf = synth.bf16_round(ref).astype(np.float64)
    got = C1[:n, :k1]
    _, ex = np.frexp(ref_bf)
    ulp = np.ldexp(1.0, ex - 8)  # one bf16 ulp at each value
    floor32 = 16 * 2.0 ** -24 * np.linalg.norm(C0[:n, :k0], axis=1, keepdims=True)
    over = np.abs(got - ref_bf) > ulp * 1.0001 + floor32
    note("  beyond 1 ulp: %.2e, beyond 1 ulp + fp32 floor: %.2e"
         % ((np.abs(got - ref_bf) > ulp * 1.0001).mean(), over.mean()))
    assert over.mean() <= 1e-3, over.mean()
    assert np.all(C1[:n, k1:] == 0)
    return float(np.abs(got - ref).max() / np.abs(ref).max())


@pytest.mark.parametrize("shape", [
    dict(rank_k=32, rank_v=32, block=64, window=128),    # K steps S = 1, column tiles T = 2
    dict(rank_k=24, rank_v=48, block=64, window=128),    # ragged K step, T = 2 and 3
    dict(rank_k=96, rank_v=64, block=64, window=64),     # the rank grows 64 -> 96 at the second fold
    dict(rank_k=64, rank_v=96, block=128, window=256),   # the 13B-MHA shape: S = 2 and 3, T = 4 and 6
    dict(rank_k=128, rank_v=16, block=64, window=64),    # T = 8 (S up to 4, three row groups) and T = 1
    dict(rank_k=80, rank_v=112, block=64, window=64),    # T = 5 and 7, ragged last K step
])
def test_rewrite_is_rotation_of_stored_rows(iskv, shape):
    """Each of the second to fourth folds rewrites every old row as
    C_old H_top (bf16 coordinates, matrix-core rewrite), including folds
    where the rank grows (k+ > k)."""
    from dataclasses import replace

    b, wnd = shape["block"], shape["window"]
    w = replace(synth.get_config(1), layers=2, kv_heads=4, q_heads=16, decode_tokens=wnd + 4 * b,
                cfg_id=12 + shape["rank_k"], **shape)
    note("case: rewrite rotation %s" % shape)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, wnd + b, b)  # first fold (empty history)
    t = wnd + b
    worst = 0.0
    for fold in range(3):
        _feed(cache, w, rows, t, t + b - 1, b)
        t += b - 1
        n0 = cache.counts(0)[0]
        before = {(x, l, h): unit_state(cache, x, 0, l, h) for x in (0, 1) for l in range(2) for h in range(4)}
        _feed(cache, w, rows, t, t + 1, 1)  # this row triggers exactly one fold
        t += 1
        assert cache.counts(0)[0] == n0 + b
        for (x, l, h), (C0, s0, B0, _, n, _, k0) in before.items():
            C1, s1, B1, _, n_, _, k1 = unit_state(cache, x, 0, l, h)
            worst = max(worst, _rotation_check(C0, B0, k0, n, C1, B1, k1))
    assert cache.status() == 0
    note("  max rel dev from fp64 rotation %.2e" % worst)


def test_rewrite_long_history_all_rows(iskv):
    """One fold over 40000 stored rows (more rows than one launch gives each
    unit workgroups for, so the workgroups stride over the rows), ranks 24 and
    48; then decode over the long history (matrix-core decode, r_K = 24,
    r_V = 48)."""
    from dataclasses import replace

    n0 = 40000
    w = replace(synth.get_config(1), layers=1, kv_heads=2, q_heads=8, rank_k=24, rank_v=48,
                decode_tokens=n0 + 192, cfg_id=40)
    note("case: rewrite over %d rows" % n0)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    dt = tdtype(w.kv_dtype)
    cache.prefill_oneshot(to_dev(rows["K"][:, :, :, :n0], dt, DEV), to_dev(rows["V"][:, :, :, :n0], dt, DEV))
    before = {(x, h): unit_state(cache, x, 0, 0, h) for x in (0, 1) for h in range(2)}
    _feed(cache, w, rows, n0, n0 + w.window + w.block, w.block)
    assert cache.counts(0)[:2] == (n0 + w.block, w.window)
    worst = 0.0
    for (x, h), (C0, s0, B0, _, n, _, k0) in before.items():
        C1, s1, B1, _, n_, _, k1 = unit_state(cache, x, 0, 0, h)
        worst = max(worst, _rotation_check(C0, B0, k0, n, C1, B1, k1))
    q = _queries(w, 2)
    out = cache.decode_attn(to_dev(q, dt, DEV))
    derr = _check_decode(cache, w, q, out, [(0, 0, 0), (0, 0, 1)])
    assert cache.status() == 0
    note("  max rel dev from fp64 rotation %.2e, decode err %.2e" % (worst, derr))


@pytest.mark.parametrize("shape", [
    dict(block=64, rank_k=128, rank_v=128, window=64, decode_tokens=700),    # untruncated; k reaches d
    dict(block=128, rank_k=64, rank_v=96, window=256, decode_tokens=1200),   # k + b > d: QR first
    dict(block=63, rank_k=20, rank_v=33, window=10, decode_tokens=700),      # odd core sizes
    dict(block=5, rank_k=3, rank_v=7, window=2, decode_tokens=160),          # tiny blocks
])
def test_core_shapes_fp32(iskv, shape):
    from dataclasses import replace

    w = replace(synth.get_config(0), kv_dtype="f32", coord_dtype="f32", cfg_id=20 + shape["block"], **shape)
    note("case: core shape %s" % shape)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, w.total_tokens, 1 if w.block < 8 else 17)
    assert cache.status() == 0
    st = oracle_units([(rows["K"][0, 0, 0], w.block, w.rank_k, w.window, 0),
                       (rows["V"][0, 0, 0], w.block, w.rank_v, w.window, 0)])
    for x in (0, 1):
        e1, e2, e3 = check_unit(cache, x, 0, 0, 0, st[x], label=str(shape))
        note("  %s sigma %.2e/%.2e recon %.2e" % ("KV"[x], e1, e2, e3))
    q = _queries(w, 1)
    out = cache.decode_attn(to_dev(q, torch.float32, DEV))
    _check_decode(cache, w, q, out, [(0, 0, 0)])


def test_prefill_then_decode(iskv):
    """Prompt blocks fold straight into history (window empty), then decode rows
    go through the window; decode with an empty window right after prefill."""
    from dataclasses import replace

    w = replace(synth.get_config(3), layers=2, kv_heads=2, q_heads=8, prefill_blocks=10,
                decode_tokens=300, cfg_id=13)
    note("case: prefill then decode")
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w, coord="f32")
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"], dt, DEV)
    V = to_dev(rows["V"], dt, DEV)
    pre = w.prefill_blocks * w.block
    for s in range(0, pre, w.block):
        cache.prefill_block(K[:, :, :, s:s + w.block].contiguous(), V[:, :, :, s:s + w.block].contiguous())
    assert cache.counts(0)[:2] == (pre, 0)
    q = _queries(w, 5)
    out = cache.decode_attn(to_dev(q, dt, DEV))
    _check_decode(cache, w, q, out, [(0, 0, 1), (0, 1, 0)])
    for t in range(pre, w.total_tokens):
        cache.append_block(K[:, :, :, t:t + 1].contiguous(), V[:, :, :, t:t + 1].contiguous())
    assert cache.status() == 0
    st = oracle_units([(rows[x][0, l, h], w.block, r, w.window, pre)
                       for (l, h) in ((0, 0), (1, 1)) for x, r in (("K", w.rank_k), ("V", w.rank_v))])
    check_unit(cache, 0, 0, 0, 0, st[0])
    check_unit(cache, 1, 0, 0, 0, st[1])
    check_unit(cache, 0, 0, 1, 1, st[2])
    check_unit(cache, 1, 0, 1, 1, st[3])


def test_window_only_decode_and_peaked_query(iskv):
    """Decode before any fold (history empty), and a query aligned with one
    stored key (softmax nearly one-hot on it)."""
    from dataclasses import replace

    w = replace(synth.get_config(1), layers=1, kv_heads=1, q_heads=4, decode_tokens=300, cfg_id=14)
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, 50, 1)
    assert cache.counts(0)[0] == 0
    q = _queries(w, 0)
    out = cache.decode_attn(to_dev(q, torch.bfloat16, DEV))
    _check_decode(cache, w, q, out, [(0, 0, 0)])
    _feed(cache, w, rows, 50, 300, 1)
    assert cache.counts(0)[0] > 0
    kvec = rows["K"][0, 0, 0, 17]
    qp = np.zeros((1, 1, 4, D))
    qp[0, 0, :] = synth.bf16_round(8.0 * kvec / np.linalg.norm(kvec) * np.sqrt(D))
    out = cache.decode_attn(to_dev(qp, torch.bfloat16, DEV))
    _check_decode(cache, w, qp, out, [(0, 0, 0)])


def test_zero_rows_and_nan_flag(iskv):
    """An all-zero block folds without flags; a NaN row raises the numeric flag."""
    from dataclasses import replace

    w = replace(synth.get_config(0), decode_tokens=400, cfg_id=15)
    rows = _rows_all(w, w.total_tokens)
    rows["K"][0, 0, 0, :200] = 0.0
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, 400, 16)
    assert cache.status() == 0
    st = oracle_units([(rows["K"][0, 0, 0], w.block, w.rank_k, w.window, 0)])
    C, sig, Bt, W, n, e, k = unit_state(cache, 0, 0, 0, 0)
    assert np.all(np.isfinite(C)) and np.all(np.isfinite(Bt))
    assert np.abs(Bt[:k] @ Bt[:k].T - np.eye(k)).max() < 1e-4
    rec = cache.reconstruct(0, 0, 0, 0).cpu().double().numpy()
    ref = st[0].reconstruct()
    assert np.linalg.norm(rec - ref) <= 1e-4 * np.linalg.norm(ref)
    bad = np.array(rows["V"][0, 0, 0, :64])
    bad[3, 5] = np.nan
    t = to_dev(bad.reshape(1, 1, 1, 64, D), torch.float32, DEV)
    cache2 = _cache(iskv, w)
    cache2.prefill_block(t, t)
    assert cache2.status() & iskv.FLAG_NONFINITE


def test_rank_deficient_rows(iskv):
    """Rows of rank 3 under a rank budget of 8: five kept singular values are
    at the rounding level, so the core takes its rotation-accumulating route;
    the basis stays orthonormal and the history matches the oracle."""
    from dataclasses import replace

    w = replace(synth.get_config(0), decode_tokens=400, rank_k=8, cfg_id=16)
    rows = _rows_all(w, w.total_tokens)
    rng = np.random.default_rng(77)
    rows["K"][0, 0, 0] = rng.standard_normal((w.total_tokens, 3)) @ rng.standard_normal((3, D))
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, 400, 16)
    assert cache.status() == 0
    st = oracle_units([(rows["K"][0, 0, 0], w.block, w.rank_k, w.window, 0)])
    C, sig, Bt, W, n, e, k = unit_state(cache, 0, 0, 0, 0)
    assert k == 8
    assert np.abs(Bt[:k] @ Bt[:k].T - np.eye(k)).max() < 1e-4
    np.testing.assert_allclose(sig[:3], st[0].sigma[:3], rtol=1e-4)
    assert sig[3:k].max() <= 1e-4 * sig[0]
    rec = cache.reconstruct(0, 0, 0, 0).cpu().double().numpy()
    ref = st[0].reconstruct()
    assert np.linalg.norm(rec - ref) <= 1e-4 * np.linalg.norm(ref)


def test_deterministic_and_checkpoint_resume(iskv):
    """Two identical runs are bitwise equal; exporting every unit's state into a
    fresh cache and continuing gives the same bits as an uninterrupted run."""
    from dataclasses import replace

    w = replace(synth.get_config(1), layers=2, kv_heads=2, q_heads=8, decode_tokens=900, cfg_id=16)
    rows = _rows_all(w, w.total_tokens)
    a = _cache(iskv, w)
    b = _cache(iskv, w)
    _feed(a, w, rows, 0, 500, 7)
    _feed(b, w, rows, 0, 500, 7)
    c = _cache(iskv, w)
    for l in range(2):
        n, e, kk, kv = a.counts(l)
        c.set_counts(l, n, e, kk, kv)
        for h in range(2):
            for x in (0, 1):
                C, sig, Bt, W = a.export_state(x, 0, l, h)
                c.import_state(x, 0, l, h, C=C, sigma=sig, Bt=Bt, window=W)
    _feed(a, w, rows, 500, 900, 7)
    _feed(b, w, rows, 500, 900, 7)
    _feed(c, w, rows, 500, 900, 7)
    q = to_dev(_queries(w, 9), torch.bfloat16, DEV)
    oa, ob, oc = a.decode_attn(q), b.decode_attn(q), c.decode_attn(q)
    assert torch.equal(oa, ob) and torch.equal(oa, oc)
    for l in range(2):
        for h in range(2):
            for x in (0, 1):
                sa, sb, sc = (z.export_state(x, 0, l, h) for z in (a, b, c))
                for ta, tb, tc in zip(sa, sb, sc):
                    assert torch.equal(ta, tb) and torch.equal(ta, tc)


def test_error_paths_leave_state_unchanged(iskv):
    from dataclasses import replace

    w = replace(synth.get_config(1), layers=2, kv_heads=1, q_heads=4, decode_tokens=300, cfg_id=17)
    cache = _cache(iskv, w, max_tokens=300)
    rows = _rows_all(w, 300)
    dt = tdtype(w.kv_dtype)
    q = to_dev(_queries(w, 0), dt, DEV)
    with pytest.raises(iskv.ISKVError) as ei:
        cache.decode_attn(q)
    assert ei.value.code == iskv.ISKV_ERR_STATE
    _feed(cache, w, rows, 0, 300, 64)
    before = cache.counts(0)
    K = to_dev(rows["K"][:, :, :, :65], dt, DEV)
    with pytest.raises(iskv.ISKVError) as ei:
        cache.append_block(K, K)  # 65 rows > b
    assert ei.value.code == iskv.ISKV_ERR_ARG
    with pytest.raises(iskv.ISKVError) as ei:
        cache.append_block(K[:, :, :, :1].contiguous(), K[:, :, :, :1].contiguous())
    assert ei.value.code == iskv.ISKV_ERR_CAPACITY
    with pytest.raises(iskv.ISKVError) as ei:
        cache.prefill_block(K[:, :, :, :64].contiguous(), K[:, :, :, :64].contiguous())
    assert ei.value.code in (iskv.ISKV_ERR_STATE, iskv.ISKV_ERR_CAPACITY)
    with pytest.raises(iskv.ISKVError):
        cache.append_block(K[:, :1, :, :1].contiguous(), K[:, :1, :, :1].contiguous(), layer0=2)
    assert cache.counts(0) == before
    assert cache.status() == 0


@pytest.mark.parametrize("rk,rv,g,b", [(64, 96, 1, 128), (128, 8, 8, 64), (8, 128, 2, 64), (48, 24, 4, 64),
                                      (32, 48, 4, 64)])
def test_bf16_decode_rank_and_group_shapes(iskv, rk, rv, g, b):
    """Matrix-core decode over several rank / GQA-group shapes, history long
    enough for several 1024-row blocks plus a ragged tail."""
    from dataclasses import replace

    w = replace(synth.get_config(1), layers=1, kv_heads=2, q_heads=2 * g, block=b, rank_k=rk,
                rank_v=rv, window=3 * b // 2, decode_tokens=2600, cfg_id=30 + rk + rv + g)
    note("case: bf16 decode rk=%d rv=%d g=%d b=%d" % (rk, rv, g, b))
    rows = _rows_all(w, w.total_tokens)
    cache = _cache(iskv, w)
    _feed(cache, w, rows, 0, w.total_tokens, b)
    n, e, kk, kv = cache.counts(0)
    assert n > 2048 and e > 0
    for step in range(3):
        q = _queries(w, step)
        out = cache.decode_attn(to_dev(q, torch.bfloat16, DEV))
        derr = _check_decode(cache, w, q, out, [(0, 0, 0), (0, 0, 1)])
    assert cache.status() == 0
    note("  decode err %.2e" % derr)


@pytest.mark.parametrize("shape", [
    dict(),                                                            # fused launch (bf16, window in LDS)
    dict(block=128, rank_k=64, rank_v=96, window=256, decode_tokens=700),  # window too big for LDS: two calls
    dict(coord_dtype="f32", decode_tokens=400),                        # fp32 coordinates: two calls
])
def test_append_decode_equals_append_then_decode(iskv, shape):
    """iskv_append_decode gives bit-identical outputs and state to
    iskv_append_block(nrows = 1) followed by iskv_decode_attn, across folds."""
    from dataclasses import replace

    base = dict(layers=2, kv_heads=4, q_heads=16, decode_tokens=450, cfg_id=31)
    base.update(shape)
    w = replace(synth.get_config(1), **base)
    note("case: append_decode %s" % shape)
    T = w.total_tokens
    rows = _rows_all(w, T)
    dt = tdtype(w.kv_dtype)
    K = to_dev(rows["K"], dt, DEV)
    V = to_dev(rows["V"], dt, DEV)
    A = _cache(iskv, w, coord=w.coord_dtype)
    B = _cache(iskv, w, coord=w.coord_dtype)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    worst = 0
    for t in range(T):
        q = torch.randn((w.batch, w.layers, w.q_heads, D), generator=gen, device=DEV).to(dt)
        kt = K[:, :, :, t:t + 1].contiguous()
        vt = V[:, :, :, t:t + 1].contiguous()
        oa = A.append_decode(kt, vt, q)
        B.append_block(kt, vt)
        ob = B.decode_attn(q)
        if t % 37 == 0 or t == T - 1:
            assert A.counts(0) == B.counts(0)
            d = (oa - ob).abs().max().item()
            worst = max(worst, d)
            assert d == 0.0, (t, d)
    assert A.status() == 0 and B.status() == 0
    for x in (0, 1):
        for (l, h) in ((0, 0), (1, 3)):
            sa = A.export_state(x, 0, l, h)
            sb = B.export_state(x, 0, l, h)
            for ta, tb in zip(sa, sb):
                assert torch.equal(ta, tb)
    note("  %d steps, max |out difference| %.1e, final counts %s" % (T, worst, A.counts(0)))
