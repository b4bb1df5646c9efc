"""Pins of the fp64 oracle against facts fixed outside it.

The pages print no worked example with numbers, so every pin here is a
closed form, an invariant of the update equations, brute force on tiny
inputs, or LAPACK (numpy.linalg.svd) as an independent opinion. Source page:
"iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD".
"""

import numpy as np
import pytest

import oracle
import synth

D = 128


def _rows(cfg_id=0, kind="K", n=1024, h=0):
    cfg = synth.get_config(cfg_id)
    return synth.kv_rows(cfg, kind, 0, 0, h, n)


def _best_rank_r(M, r):
    u, s, vt = np.linalg.svd(M, full_matrices=False)
    return (u[:, :r] * s[:r]) @ vt[:r], s


# --------------------------------------------------------------------------
# Core SVD (section "Theoretical Foundation": SVD_r with orthonormal factors)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("a,b,c,d", [(3.0, 1.0, -2.0, 0.5), (1.0, 0.0, 0.0, 1.0),
                                     (2.0, 2.0, 2.0, 2.0), (1e-3, 5.0, -7.0, 1e3),
                                     (0.0, 1.0, 1.0, 0.0), (-4.0, 3.0, 2.0, -1.0)])
def test_jacobi_2x2_closed_form(a, b, c, d):
    M = np.array([[a, b], [c, d]])
    _, H, sv, _ = oracle.jacobi(M)
    s1 = (np.hypot(a + d, b - c) + np.hypot(a - d, b + c)) / 2
    s2 = abs(np.hypot(a + d, b - c) - np.hypot(a - d, b + c)) / 2
    got = np.sort(sv)[::-1]
    assert abs(got[0] - s1) <= 1e-15 * max(s1, 1) * 4
    assert abs(got[1] - s2) <= 1e-15 * max(s1, 1) * 4
    assert np.abs(H.T @ H - np.eye(2)).max() < 1e-15 * 4


@pytest.mark.parametrize("m,c", [(96, 96), (88, 88), (192, 128), (40, 12), (9, 6)])
def test_jacobi_matches_lapack_and_rotates(m, c):
    rng = np.random.default_rng(m * 1000 + c)
    Z = rng.standard_normal((m, c)) * (np.arange(1, c + 1) ** -1.5)
    ZH, H, sv, sweeps = oracle.jacobi(Z)
    ref = np.linalg.svd(Z, compute_uv=False)
    got = np.sort(sv)[::-1][: len(ref)]
    assert np.abs(got - ref).max() <= 1e-12 * ref[0]
    assert np.abs(H.T @ H - np.eye(c)).max() < 1e-13
    assert np.abs(Z @ H - ZH).max() < 1e-13 * ref[0]
    G = ZH.T @ ZH
    off = G - np.diag(np.diag(G))
    assert np.abs(off).max() < 1e-12 * ref[0] ** 2
    assert 1 <= sweeps < 60


def test_singular_values_sorted_vs_lapack():
    X = _rows(0, "K", 300)
    sv = oracle.singular_values(X)
    ref = np.linalg.svd(X, compute_uv=False)
    assert np.all(np.diff(sv) <= 0)
    assert np.abs(sv - ref).max() <= 1e-11 * ref[0]


# --------------------------------------------------------------------------
# Update identities (section "Block-Incremental Decoding Updates")
# --------------------------------------------------------------------------

def test_untruncated_incremental_equals_exact_svd():
    """With r = d nothing is truncated: the incremental factors are an exact
    SVD of the stacked history (singular values to 1e-10 relative)."""
    X = _rows(0, "K", 1024)
    st = oracle.run_unit(X, D, 64, 128, 64)
    assert (st.n, st.e, st.k) == (960, 64, 128)
    hist = X[: st.n]
    ref = np.linalg.svd(hist, compute_uv=False)
    ora_sv = oracle.singular_values(hist)
    assert np.abs(st.sigma[: st.k] - ref).max() <= 1e-10 * ref[0]
    assert np.abs(st.sigma[: st.k] - ora_sv).max() <= 1e-10 * ref[0]
    Xt = st.reconstruct()
    assert np.linalg.norm(Xt[: st.n] - hist) <= 1e-10 * np.linalg.norm(hist)
    assert np.array_equal(Xt[st.n:], X[st.n:])


def test_fold_is_eckart_young_of_stacked_matrix():
    """Each fold returns the best rank-r approximation of M = [A; F]
    (A = current history reconstruction), with error sqrt(discarded)."""
    X = _rows(0, "V", 64 * 8, h=0)
    b, r = 64, 32
    st = oracle.UnitState.empty(D, b, r, 64 * 8)
    for t in range(8):
        F = X[t * b:(t + 1) * b]
        C, s, Bt = st.history()
        A = C @ Bt
        M = np.vstack([A, F])
        info = st.fold(F)
        C2, s2, Bt2 = st.history()
        approx = C2 @ Bt2
        best, sv = _best_rank_r(M, r)
        tail = float(np.sum(sv[r:] ** 2))
        err2 = float(np.linalg.norm(M - approx) ** 2)
        assert abs(err2 - info.discarded) <= 1e-10 * np.sum(sv ** 2)
        assert abs(info.discarded - tail) <= 1e-10 * np.sum(sv ** 2)
        assert np.linalg.norm(approx - best) <= 1e-9 * np.linalg.norm(M)
        assert np.abs(s2 - sv[: len(s2)]).max() <= 1e-10 * sv[0]


def test_cumulative_error_is_sum_of_discarded():
    X = _rows(0, "K", 1024)
    st = oracle.run_unit(X, D, 64, 32, 64)
    hist = X[: st.n]
    err2 = np.linalg.norm(st.reconstruct()[: st.n] - hist) ** 2
    total = sum(l[4] for l in st.log)
    assert abs(err2 - total) <= 1e-10 * np.linalg.norm(hist) ** 2
    # the one-shot SVD_r of all history rows is optimal, so never worse
    best, sv = _best_rank_r(hist, 32)
    assert np.linalg.norm(hist - best) ** 2 <= err2 * (1 + 1e-12)


def test_factors_orthonormal_after_many_folds():
    X = _rows(1, "V", 64 * 40)
    st = oracle.run_unit(X, D, 64, 32, 0)
    C, s, Bt = st.history()
    assert np.abs(Bt @ Bt.T - np.eye(st.k)).max() < 1e-12
    G = C.T @ C
    assert np.abs(G - np.diag(s ** 2)).max() < 1e-12 * s[0] ** 2
    assert np.all(np.diff(s) <= 0)


def test_first_fold_is_truncated_svd_of_block():
    F = _rows(1, "K", 64)
    st = oracle.UnitState.empty(D, 64, 24, 64)
    st.fold(F)
    C, s, Bt = st.history()
    best, sv = _best_rank_r(F, 24)
    assert np.linalg.norm(C @ Bt - best) <= 1e-10 * np.linalg.norm(F)
    assert np.abs(s - sv[:24]).max() <= 1e-12 * sv[0]


def test_residual_basis_choice_does_not_change_result():
    """Any orthonormal P spanning the residual gives the same singular values
    and the same reconstruction (the core changes by a right rotation)."""
    X = _rows(0, "K", 64 * 6)
    a = oracle.UnitState.empty(D, 64, 32, 64 * 6)
    b = oracle.UnitState.empty(D, 64, 32, 64 * 6)
    for t in range(6):
        F = X[t * 64:(t + 1) * 64]
        a.fold(F, porder=0)
        b.fold(F, porder=1)
    assert np.abs(a.sigma - b.sigma).max() <= 1e-12 * a.sigma[0]
    ra, rb = a.reconstruct(), b.reconstruct()
    assert np.linalg.norm(ra - rb) <= 1e-12 * np.linalg.norm(ra)


def test_rank_sequence_closed_form():
    """k_t = min(r, n_t, d) and p_t = min(b, d - k_t), including k = d, p = 0."""
    d, b = 8, 3
    rng = np.random.default_rng(5)
    for r in (2, 5, 8):
        st = oracle.UnitState.empty(d, b, r, 40)
        n = 0
        for t in range(6):
            info = st.fold(rng.standard_normal((b, d)))
            k_before = min(r, n, d)
            assert info.k == k_before
            assert info.p == min(b, d - k_before)
            n += b
            assert info.kplus == min(r, n, d)
        if r == d:
            assert st.log[-1][1] == 0  # p = 0 once the basis spans R^d


def test_brute_force_tiny_d4_b2():
    """d = 4, b = 2: every fold against the SVD of the explicitly stacked matrix."""
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((12, 4)) @ np.diag([3.0, 1.0, 0.3, 0.1])
    for r in (1, 2, 3, 4):
        st = oracle.UnitState.empty(4, 2, r, 12)
        approx_hist = np.zeros((0, 4))
        for t in range(6):
            F = rows[2 * t: 2 * t + 2]
            M = np.vstack([approx_hist, F])
            st.fold(F)
            C, s, Bt = st.history()
            best, sv = _best_rank_r(M, r)
            assert np.allclose(C @ Bt, best, atol=1e-12, rtol=0)
            assert np.allclose(s, sv[: len(s)], atol=1e-12, rtol=0)
            approx_hist = C @ Bt


def test_zero_and_repeated_blocks():
    """Degenerate blocks (all zero; rows already in span of B) fold without NaN."""
    st = oracle.UnitState.empty(D, 64, 32, 64 * 4)
    st.fold(np.zeros((64, D)))
    assert st.k == 32 and np.all(st.sigma == 0) and np.all(np.isfinite(st.Bt))
    assert np.abs(st.Bt[:32] @ st.Bt[:32].T - np.eye(32)).max() < 1e-12
    X = _rows(0, "K", 64)
    st.fold(X)
    C, s, Bt = st.history()
    st.fold(C[-64:] @ Bt)  # rows already inside span(B)
    assert np.all(np.isfinite(st.C)) and np.abs(st.Bt[:32] @ st.Bt[:32].T - np.eye(32)).max() < 1e-12


# --------------------------------------------------------------------------
# Basis drift (section "The Basis Drift Problem")
# --------------------------------------------------------------------------

def _drift(X, st):
    hist = X[: st.n]
    return np.linalg.norm(st.reconstruct()[: st.n] - hist) / np.linalg.norm(hist)


def test_joint_update_has_no_drift_naive_does():
    X = _rows(0, "K", 1024)
    joint = oracle.run_unit(X, D, 64, 128, 64, mode=0)
    naive = oracle.run_unit(X, D, 64, 128, 64, mode=1)
    assert _drift(X, joint) < 1e-12
    assert _drift(X, naive) > 0.1
    joint32 = oracle.run_unit(X, D, 64, 32, 64, mode=0)
    naive32 = oracle.run_unit(X, D, 64, 32, 64, mode=1)
    assert _drift(X, naive32) > 2 * _drift(X, joint32)
    assert _drift(X, naive32) - _drift(X, joint32) > 0.1


def test_fixed_basis_stores_projection_onto_first_basis():
    """Ablation "keeping bases fixed" ([iS-KV] Ablation Study): after the first
    fold, every block is stored as its orthogonal projection onto the basis of
    that first fold (computed here with numpy from the exported basis), the
    old rows, sigma and the rank stay, and the lost energy is ||F - F B B^T||^2."""
    X = _rows(0, "V", 640)
    b, r = 64, 32
    st = oracle.UnitState.empty(D, b, r, 640)
    st.fold(X[:b], mode=0)
    B0 = st.Bt[:st.k].copy()
    C0 = st.C[:b, :st.k].copy()
    s0 = st.sigma[:st.k].copy()
    lost = 0.0
    for s in range(b, 640, b):
        F = X[s:s + b]
        info = st.fold(F, mode=2)
        ref = F @ B0.T @ B0
        assert info.kplus == st.k == B0.shape[0] and info.p == 0
        assert np.allclose(st.C[s:s + b, :st.k] @ B0, ref, atol=1e-12)
        assert np.all(st.C[s:s + b, st.k:] == 0)
        assert abs(info.discarded - np.linalg.norm(F - ref) ** 2) <= 1e-10 * np.linalg.norm(F) ** 2
        lost += info.discarded
    assert np.array_equal(st.Bt[:st.k], B0) and np.array_equal(st.sigma[:st.k], s0)
    assert np.array_equal(st.C[:b, :st.k], C0)
    # the stored history misses exactly the energy outside span(B0) of the later
    # blocks, plus the first fold's truncation
    err2 = np.linalg.norm(X[:640] - st.C[:640, :st.k] @ B0) ** 2
    assert abs(err2 - (lost + st.log[0][4])) <= 1e-9 * np.linalg.norm(X[:640]) ** 2


def test_fixed_basis_loses_more_than_joint_update():
    """On a stream whose dominant directions change, a frozen first-block basis
    keeps much more error than the joint update (the pages' ablation claim,
    qualitatively; their accuracy numbers need the model and are not used)."""
    rng = np.random.default_rng(11)
    W1, _ = np.linalg.qr(rng.standard_normal((D, D)))
    W2, _ = np.linalg.qr(rng.standard_normal((D, D)))
    s = np.arange(1, D + 1) ** -1.0
    X = np.vstack([(rng.standard_normal((256, D)) * s) @ W1.T, (rng.standard_normal((512, D)) * s) @ W2.T])
    joint = oracle.run_unit(X, D, 64, 32, 0, mode=0)
    fixed = oracle.UnitState.empty(D, 64, 32, X.shape[0])
    fixed.fold(X[:64], mode=0)
    for t in range(64, X.shape[0], 64):
        fixed.fold(X[t:t + 64], mode=2)
    ej, ef = _drift(X, joint), _drift(X, fixed)
    assert ef > 2 * ej and ef - ej > 0.2, (ej, ef)


# --------------------------------------------------------------------------
# Reconstruction, attention, storage (section "Reconstruction and Storage")
# --------------------------------------------------------------------------

def test_reconstruct_history_then_window():
    rng = np.random.default_rng(3)
    C = rng.standard_normal((5, 4))
    Bt = np.eye(4)
    W = rng.standard_normal((2, 4))
    out = oracle.reconstruct(C, Bt, W)
    assert np.array_equal(out[:5], C) and np.array_equal(out[5:], W)
    out2 = oracle.reconstruct(C[:, :2], Bt[:2] * 2.0, W, k=2)
    assert np.allclose(out2[:5, :2], 2 * C[:, :2]) and np.all(out2[:5, 2:] == 0)


def test_attend_closed_forms():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((7, 16))
    V = rng.standard_normal((7, 16))
    # zero query: uniform weights, the mean of the values
    out = oracle.attend(K, V, np.zeros((1, 16)), 0.25)
    assert np.allclose(out[0], V.mean(axis=0), atol=1e-14)
    # one row: the row itself
    out = oracle.attend(K[:1], V[:1], rng.standard_normal((1, 16)), 0.25)
    assert np.allclose(out[0], V[0], atol=1e-15)
    # two rows: weight of the first is the logistic of the score gap
    q = rng.standard_normal((1, 16))
    s = 0.3 * (K[:2] @ q[0])
    w0 = 1.0 / (1.0 + np.exp(s[1] - s[0]))
    out = oracle.attend(K[:2], V[:2], q, 0.3)
    assert np.allclose(out[0], w0 * V[0] + (1 - w0) * V[1], atol=1e-14)
    # huge scores: no overflow, one-hot on the winner
    Kp = np.eye(16)[:3] * 1e4
    out = oracle.attend(Kp, V[:3], np.eye(16)[1:2], 1.0)
    assert np.allclose(out[0], V[1], atol=1e-14)
    # permutation invariance over rows
    perm = rng.permutation(7)
    q = rng.standard_normal((3, 16))
    assert np.allclose(oracle.attend(K, V, q, 0.2), oracle.attend(K[perm], V[perm], q, 0.2), atol=1e-14)


def test_storage_formula_counts_state():
    """Storage (per layer) = beta_f sum_X k_X (n_X + d + 1) + beta_e d sum_X e_X,
    checked against an element count of an actual oracle state."""
    X = _rows(0, "K", 700)
    Y = _rows(0, "V", 700, h=0)
    sk = oracle.run_unit(X, D, 64, 32, 64)
    sv = oracle.run_unit(Y, D, 64, 24, 64)
    def elems(st):
        C, s, Bt = st.history()
        return C.size + s.size + Bt.size, st.e * D
    fk, ek = elems(sk)
    fv, ev = elems(sv)
    for bf, be in ((2, 2), (4, 4), (2, 4)):
        formula = oracle.storage_bytes(D, sk.k, sk.n, sk.e, sv.k, sv.n, sv.e, bf, be)
        assert formula == bf * (fk + fv) + be * (ek + ev)


def test_window_policy_counts_match_workloads():
    """Fold trigger (window holds w + b rows) gives the expected final counts."""
    X = _rows(0, "K", 1024)
    st = oracle.run_unit(X, D, 64, 32, 64)
    assert (st.n, st.e, len(st.log)) == synth.get_config(0).final_counts()
    assert synth.get_config(1).final_counts() == (8064, 128, 126)
    assert synth.get_config(3).final_counts() == (66432, 128, 1038)
    assert synth.get_config(4).final_counts() == (16128, 256, 126)


# --------------------------------------------------------------------------
# One-shot prefill (page "iS-KV ...", section "Prefill Compression": a
# truncated SVD of the prompt rows; k = min(r, n, d) per "Theoretical
# Foundation")
# --------------------------------------------------------------------------

def test_oneshot_prefill_is_the_truncated_svd():
    rng = np.random.default_rng(11)
    d, N, r = 128, 300, 32
    X = rng.standard_normal((N, d)) * np.geomspace(1.0, 1e-3, d)
    st = oracle.UnitState.empty(d, 64, r, N)
    info = st.prefill_oneshot(X)
    assert (st.n, st.e, st.k) == (N, 0, r)
    C, sig, Bt = st.history()
    S = np.linalg.svd(X, compute_uv=False)           # LAPACK, independent of the oracle's Jacobi
    assert np.abs(sig - S[:r]).max() <= 1e-12 * S[0]
    np.testing.assert_allclose(Bt @ Bt.T, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(C, X @ Bt.T, atol=1e-10 * S[0])   # C = X V_r = U_r Sigma_r
    np.testing.assert_allclose(C.T @ C, np.diag(sig ** 2), atol=1e-9 * S[0] ** 2)
    # Eckart-Young: the error is exactly the discarded energy
    err2 = np.linalg.norm(X - C @ Bt) ** 2
    assert abs(err2 - (S[r:] ** 2).sum()) <= 1e-9 * (S ** 2).sum()
    assert abs(info.discarded - (S[r:] ** 2).sum()) <= 1e-9 * (S ** 2).sum()
    # sign rule: each basis vector's entry of largest magnitude is positive
    for j in range(r):
        assert Bt[j, np.argmax(np.abs(Bt[j]))] > 0


def test_oneshot_prefill_short_prompt_is_exact():
    rng = np.random.default_rng(12)
    d, N, r = 128, 40, 64
    X = rng.standard_normal((N, d))
    st = oracle.UnitState.empty(d, 64, r, N)
    st.prefill_oneshot(X)
    assert st.k == N                                  # k = min(r, n, d)
    C, sig, Bt = st.history()
    np.testing.assert_allclose(C @ Bt, X, atol=1e-11)
    np.testing.assert_allclose(sig, np.linalg.svd(X, compute_uv=False), rtol=1e-12)


def test_oneshot_prefill_then_folds_match_folding_everything():
    """When nothing is truncated (r = d), a one-shot history followed by folds
    reconstructs the same rows as folding every block: both are exact."""
    rng = np.random.default_rng(13)
    d, b, w, N, M = 128, 16, 8, 64, 100
    X = rng.standard_normal((N + M, d))
    a = oracle.UnitState.empty(d, b, d, N + M)
    a.prefill_oneshot(X[:N])
    a.append(X[N:], w)
    np.testing.assert_allclose(a.reconstruct(), X, atol=1e-9)


# --------------------------------------------------------------------------
# Fixed-coordinate update (section "The Basis Drift Problem": the basis moves,
# the stored rows keep the coordinates they were written with)
# --------------------------------------------------------------------------

def _copy_state(st):
    return oracle.UnitState(d=st.d, b=st.b, r=st.r, C=st.C.copy(), sigma=st.sigma.copy(),
                            Bt=st.Bt.copy(), n=st.n, k=st.k)


def test_fixed_coordinates_is_joint_fold_without_rewrite():
    """From any state, a fold with fixed coordinates must equal a joint fold
    from the same state in everything but the old rows, which keep their
    previous values exactly (the rank never shrinks, so "cut or zero-padded
    to k+" is the old columns followed by zeros). The chain continues in the
    fixed-coordinate mode, so later states are ones the joint update never
    reaches; the rank grows during the first folds (k+ > k) and then stays."""
    X = _rows(0, "V", 64 * 9)
    b, r = 64, 96
    st = oracle.UnitState.empty(D, b, r, X.shape[0])
    for t in range(9):
        F = X[t * b:(t + 1) * b]
        n, k = st.n, st.k
        old = st.C[:n].copy()
        ref = _copy_state(st)
        ir = ref.fold(F, mode=0)
        info = st.fold(F, mode=1)
        assert (info.k, info.p, info.kplus) == (ir.k, ir.p, ir.kplus)
        assert info.kplus >= k
        assert abs(info.discarded - ir.discarded) <= 1e-12 * max(ir.discarded, 1e-300)
        assert np.array_equal(st.Bt, ref.Bt) and np.array_equal(st.sigma, ref.sigma)
        assert np.array_equal(st.C[n:n + b], ref.C[n:n + b])
        assert np.array_equal(st.C[:n, :k], old[:, :k])
        assert np.all(st.C[:n, k:] == 0)
        if t >= 2:
            # the joint fold rewrote the old rows; the fixed one did not
            assert np.linalg.norm(ref.C[:n, :ir.kplus] - old[:, :ir.kplus]) > 1e-3 * np.linalg.norm(old)


def test_fixed_coordinates_history_is_old_rows_in_new_basis():
    """Plain definition of the drifting history: after a fixed-coordinate
    fold, the reconstruction of an old row is its unchanged coordinates times
    the NEW basis, so its error against the true row is measurable by hand."""
    X = _rows(0, "K", 64 * 4)
    b, r = 64, 128
    st = oracle.UnitState.empty(D, b, r, X.shape[0])
    st.fold(X[:b], mode=1)
    C0 = st.C[:b, :st.k].copy()
    st.fold(X[b:2 * b], mode=1)
    rec = st.reconstruct()
    np.testing.assert_allclose(rec[:b], C0 @ st.Bt[:C0.shape[1]], atol=1e-12)
    # the first fold (untruncated) stored the rows exactly; the basis change moved them
    assert np.linalg.norm(rec[:b] - X[:b]) > 1e-2 * np.linalg.norm(X[:b])
    # the new block itself is exact (r = d: nothing truncated)
    np.testing.assert_allclose(rec[b:2 * b], X[b:2 * b], atol=1e-10)


# --------------------------------------------------------------------------
# Whole-stream driver with a prefill (section "Architecture Overview": the
# exact window; prompt blocks fold straight into history)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("prefill,N,w", [(128, 500, 64), (256, 256, 32), (64, 300, 0)])
def test_run_with_prefill_untruncated_is_exact(prefill, N, w):
    """With r = d nothing is truncated, so whatever the driver folds, history
    plus window must reproduce every input row in order; the counts must
    follow the window policy's closed form (synth.Workload.final_counts)."""
    rng = np.random.default_rng(prefill + N)
    X = rng.standard_normal((N, D)) * np.geomspace(1.0, 1e-2, D)
    b = 64
    st = oracle.run_unit(X, D, b, D, w, prefill=prefill)
    from dataclasses import replace
    wl = replace(synth.get_config(0), window=w, block=b, prefill_blocks=prefill // b,
                 decode_tokens=N - prefill)
    n, e, folds = wl.final_counts()
    assert (st.n, st.e, len(st.log)) == (n, e, folds)
    np.testing.assert_allclose(st.reconstruct(), X, atol=1e-10 * np.abs(X).max())
    # rank sequence of the prefill folds: k = min(r, n, d) before each
    for t in range(prefill // b):
        assert st.log[t][0] == min(D, t * b)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_run_with_prefill_equals_explicit_folds(mode):
    """The driver with a prefill equals the prompt folded block by block in
    order, then the remaining rows through the window (truncating rank, every
    update mode): same rank log, same stored history and window."""
    X = _rows(0, "K", 700)
    b, r, w, P = 64, 32, 64, 192
    st = oracle.run_unit(X, D, b, r, w, prefill=P, mode=mode)
    ref = oracle.UnitState.empty(D, b, r, X.shape[0])
    for s in range(0, P, b):
        ref.fold(X[s:s + b], mode=mode)
    for t in range(P, X.shape[0]):
        ref.window.append(X[t].copy())
        if len(ref.window) >= w + b:
            F = np.stack(ref.window[:b])
            del ref.window[:b]
            ref.fold(F, mode=mode)
    assert (st.n, st.e, st.k) == (ref.n, ref.e, ref.k)
    assert [l[:3] for l in st.log] == [l[:3] for l in ref.log]
    np.testing.assert_allclose(st.reconstruct(), ref.reconstruct(), atol=1e-12 * np.abs(X).max())
    np.testing.assert_allclose(st.sigma, ref.sigma, atol=1e-12 * ref.sigma[0])
