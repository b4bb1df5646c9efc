"""Pins of the oracle's int8 coordinate storage (CPU).

Reading of the pages (low-bit storage is named as the next step in the iS-KV
page's "Conclusion" and in the JoLT abstract on the "Tensor Decomposition of
Transformer Key-Value Caches" page, without a format): the history keeps
U = C Sigma^-1 (the factor the page's equation for U+ updates) as int8 codes
with one scale per row, s = max|u| / 127 and q = round-half-even(127 u / max|u|);
sigma and the basis stay fp32. A fold runs the method on the stored history
and stores every row again with the new sigma. The pins below check that definition
through properties a mistake would break (grid, error bound, ties, the
rotation identity C_old B_old^T B_new of the update equations, the run driver
against explicit folds), not by retyping the formula.
"""

import numpy as np
import pytest

import oracle
import synth

D = 128


def _rows(n, seed=0, kind="K"):
    w = synth.get_config(0)
    X = synth.kv_rows(w, kind, 0, 0, 0, max(n, 1024))
    return X[:n]


def _grid_ok(S, k, sigma=None):
    """Rows of S (of U = S Sigma^-1 when sigma is given) lie on their own int8
    grid: S_i = q_i s_i, |q| <= 127, max |q| = 127."""
    if sigma is not None:
        S = np.hstack([S[:, :k] / sigma[:k], S[:, k:]])
    m = np.abs(S[:, :k]).max(axis=1)
    nz = m > 0
    s = m[nz] / 127.0
    q = S[nz, :k] / s[:, None]
    return bool(np.all(np.abs(q - np.rint(q)) < 1e-6) and np.all(np.abs(np.rint(q)) <= 127)
                and np.all(S[:, k:] == 0) and np.all(S[~nz] == 0))


def test_store_i8_codes_scales_and_error_bound():
    rng = np.random.default_rng(3)
    C = rng.standard_normal((200, 40)) * np.exp(rng.uniform(-8, 8, size=(200, 1)))
    C[5] = 0.0                      # zero row
    C[6] = 0.0
    C[6, 17] = -3.0                 # one nonzero entry
    k = 33
    S, Q, sc = oracle.store_i8(C, k)
    assert np.all(S[:, k:] == 0) and np.all(Q[:, k:] == 0)
    assert Q.dtype == np.int8
    assert np.all(np.abs(Q.astype(int)) <= 127)
    for i in range(C.shape[0]):
        m = np.abs(C[i, :k]).max()
        if m == 0:
            assert sc[i] == 0 and np.all(Q[i] == 0) and np.all(S[i] == 0)
            continue
        j = int(np.argmax(np.abs(C[i, :k])))
        assert abs(int(Q[i, j])) == 127 and np.sign(Q[i, j]) == np.sign(C[i, j])
        assert sc[i] == pytest.approx(m / 127.0, rel=1e-15)
        np.testing.assert_array_equal(S[i, :k], Q[i, :k].astype(np.float64) * sc[i])
        assert np.all(np.abs(C[i, :k] - S[i, :k]) <= 0.5 * sc[i] * (1 + 1e-12))
    assert S[6, 17] == -3.0 and np.count_nonzero(S[6]) == 1


def test_store_i8_ties_round_to_even():
    # max 127 gives scale 1: the codes are the entries rounded, ties to even
    C = np.array([[127.0, 2.5, -3.5, 0.5, 1.5, -0.5, -126.5, 4.4999]])
    S, Q, sc = oracle.store_i8(C, 8)
    assert sc[0] == 1.0
    assert Q[0].tolist() == [127, 2, -4, 0, 2, 0, -126, 4]


def test_store_i8_is_idempotent_and_exact_on_grid():
    rng = np.random.default_rng(4)
    q = rng.integers(-127, 128, size=(50, 24)).astype(np.float64)
    q[:, 3] = 127.0 * np.where(rng.random(50) < 0.5, 1, -1)   # each row reaches +-127
    s = np.ldexp(1.0, rng.integers(-20, 20, size=50))
    C = q * s[:, None]
    S, Q, sc = oracle.store_i8(C, 24)
    np.testing.assert_array_equal(S, C)
    np.testing.assert_array_equal(Q.astype(np.float64), q)
    S2, Q2, _ = oracle.store_i8(S, 24)
    np.testing.assert_array_equal(S2, S)


def _state_after(X, b, r, w, store):
    st = oracle.UnitState.empty(D, b, r, X.shape[0])
    st.store = store
    st.append(X, w)
    return st


@pytest.mark.parametrize("n,b,r", [(640, 64, 32), (704, 128, 96), (300, 64, 128)])
def test_fold_i8_rows_are_rotated_old_rows_and_projected_new_rows(n, b, r):
    X = _rows(n + b)
    st = oracle.UnitState.empty(D, b, r, n + 2 * b)
    st.store = "i8"
    for s0 in range(0, n - n % b, b):
        st.fold(X[s0:s0 + b])
    assert _grid_ok(st.C[:st.n], st.k, st.sigma)
    n0, k0 = st.n, st.k
    C_old = st.C[:n0, :k0].copy()
    B_old = st.Bt[:k0].copy()
    F = X[n0:n0 + b]
    info = st.fold(F)
    kp = info.kplus
    B_new = st.Bt[:kp]
    # update equations: old rows C_old H_top with H_top = B_old^T B_new (B_old^T P = 0),
    # new rows [FB FP] H_r = F B_new; each then stored in int8
    # rows of U = C Sigma^-1 with the new sigma
    sg = st.sigma[:kp]
    expect = np.vstack([C_old @ B_old @ B_new.T, F @ B_new.T]) / sg
    got = st.C[:n0 + b, :kp] / sg
    s = np.abs(expect).max(axis=1) / 127.0
    err = np.abs(got - expect)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-12 * np.abs(expect).max()), err.max()
    assert _grid_ok(st.C[:n0 + b], kp, st.sigma)
    assert np.all(st.C[:n0 + b, kp:] == 0)


def test_fold_i8_sigma_and_basis_are_the_folds_on_the_stored_history():
    X = _rows(704)
    a = oracle.UnitState.empty(D, 64, 32, 800)
    a.store = "i8"
    for s0 in range(0, 640, 64):
        a.fold(X[s0:s0 + 64])
    b_ = oracle.UnitState(d=D, b=64, r=32, C=a.C.copy(), sigma=a.sigma.copy(), Bt=a.Bt.copy(),
                          n=a.n, k=a.k)
    F = X[640:704]
    a.fold(F)
    b_.fold(F)  # fp64 fold of the same stored history
    np.testing.assert_array_equal(a.sigma, b_.sigma)
    np.testing.assert_array_equal(a.Bt, b_.Bt)
    # and the int8 rows are the fp64 fold's rows stored again
    S, _, _ = oracle.store_u_i8(b_.C[:a.n], b_.sigma, a.k)
    np.testing.assert_array_equal(a.C[:a.n], S)


@pytest.mark.parametrize("prefill,w", [(0, 64), (256, 64), (128, 0)])
def test_run_i8_equals_explicit_i8_folds(prefill, w):
    X = _rows(700)
    st = oracle.run_unit(X, D, 64, 32, w, prefill=prefill, store="i8")
    ref = oracle.UnitState.empty(D, 64, 32, 700)
    ref.store = "i8"
    ref.prefill(X[:prefill])
    ref.append(X[prefill:], w)
    assert (st.n, st.e, st.k) == (ref.n, ref.e, ref.k)
    np.testing.assert_allclose(st.C[:st.n], ref.C[:ref.n], rtol=0, atol=1e-12)
    np.testing.assert_allclose(st.sigma, ref.sigma, rtol=0, atol=1e-12)
    assert _grid_ok(st.C[:st.n], st.k, st.sigma)


def _u_step_bound(st):
    """Largest per-fold perturbation of the stored history, relative to the
    rows' norm: half a step (max|u_i| / 254) on each of k entries of a row of
    U, times sigma."""
    C, sg = st.C[:st.n, :st.k], st.sigma[:st.k]
    U = C / sg
    step = np.abs(U).max(axis=1, keepdims=True) / 254.0
    return np.linalg.norm(step * sg) / np.linalg.norm(C)


@pytest.mark.parametrize("cfg,kind", [(0, "K"), (0, "V"), (4, "V")])
def test_run_i8_stays_near_the_fp64_run(cfg, kind):
    """Storing U in int8 perturbs each fold's history by at most half a step
    per entry; the run's history must stay within the sum of those bounds of
    the fp64 method, and its error against the true rows near the fp64
    truncation error."""
    w = synth.get_config(cfg)
    N = w.window + 24 * w.block if cfg else w.total_tokens
    X = synth.kv_rows(w, kind, 0, 0, 0, N)
    r = w.rank_k if kind == "K" else w.rank_v
    a = oracle.run_unit(X, D, w.block, r, w.window, store="i8")
    f = oracle.run_unit(X, D, w.block, r, w.window)
    Ra, Rf = a.reconstruct(), f.reconstruct()
    nrm = np.linalg.norm(X)
    dev = np.linalg.norm(Ra - Rf) / nrm
    folds = len(f.log)
    bound = folds * _u_step_bound(a)
    assert 0 < dev <= bound, (dev, bound)
    ea = np.linalg.norm(Ra - X) / nrm
    ef = np.linalg.norm(Rf - X) / nrm
    assert ef * (1 - 1e-3) <= ea <= ef + bound
    np.testing.assert_allclose(a.sigma[:a.k], f.sigma[:f.k], rtol=0, atol=1e-2 * f.sigma[0])
    assert [x[:3] for x in a.log] == [x[:3] for x in f.log]


def test_oneshot_then_store_i8():
    X = _rows(900)
    st = oracle.UnitState.empty(D, 64, 48, 1000)
    st.store = "i8"
    st.prefill_oneshot(X)
    ref = oracle.UnitState.empty(D, 64, 48, 1000)
    ref.prefill_oneshot(X)
    S, _, _ = oracle.store_u_i8(ref.C[:900], ref.sigma, ref.k)
    np.testing.assert_array_equal(st.C[:900], S)
    assert _grid_ok(st.C[:900], st.k, st.sigma)
    np.testing.assert_array_equal(st.sigma, ref.sigma)
