"""Pins of the fp64 oracle against facts that do not come from the oracle.

Every check here uses an independent route to the answer: exact rational
arithmetic, a direct factorisation, a least-squares solve of the objective
itself, a closed form, or the characterisation of the CG iterate as a Krylov
projection.  The passages are from the MesaNet summary page (gist.science,
paper 2506.05233), section "A Camada Mesa": the displayed objective, the
output Delta_t = Phi_t q_t with q*_t = (H_t + Lambda)^-1 q_t solved by CG, and
the bullet on dynamic computation (per-token iteration counts).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from test_regression_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def zeta(gamma, t):
    """zeta_{t t'} for t' = 0..t (0-based) as explicit products of gammas."""
    return np.array([np.prod(gamma[tp + 1:t + 1]) for tp in range(t + 1)])


def brute_states(k, v, gamma, t):
    """H_t, G_t straight from their definition as zeta-weighted sums."""
    z = zeta(gamma, t)
    Hm = sum(z[i] * np.outer(k[i], k[i]) for i in range(t + 1))
    Gm = sum(z[i] * np.outer(v[i], k[i]) for i in range(t + 1))
    return Hm, Gm


def rand_problem(rng, T, dk, dv, glo=0.6, lam=None):
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((1, 1, T, dv))
    g = rng.uniform(glo, 1.0, (1, 1, T))
    lam = rng.uniform(0.3, 2.0, (1, dk)) if lam is None else lam
    return q, k, v, g, lam


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# golden hand-worked examples
# --------------------------------------------------------------------------
def test_hand_worked_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    assert cases
    for c in cases:
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        g = np.array(c["gamma"])[None, None]
        lam = np.array(c["lam"])[None]
        res = oracle.forward(q, k, v, g, lam, c["max_iters"], 0.0)
        exact = np.array([[float(Fraction(n, d)) for n, d in row] for row in c["out_num_den"]])
        np.testing.assert_allclose(res["out"][0, 0], exact, rtol=1e-12, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(exact, np.array(c["out"]), rtol=1e-15)


# --------------------------------------------------------------------------
# P1: converged CG equals a Cholesky solve of (H_t + Lambda)
# --------------------------------------------------------------------------
def test_converged_matches_cholesky():
    rng = np.random.default_rng(1)
    T, dk, dv = 24, 6, 4
    q, k, v, g, lam = rand_problem(rng, T, dk, dv)
    res = oracle.forward(q, k, v, g, lam, max_iters=4 * dk, tol=1e-13)
    for t in range(T):
        Hm, Gm = brute_states(k[0, 0], v[0, 0], g[0, 0], t)
        c = scipy.linalg.cho_factor(Hm + np.diag(lam[0]))
        x = scipy.linalg.cho_solve(c, q[0, 0, t])
        assert rel(res["out"][0, 0, t], Gm @ x) < 1e-10, t


# --------------------------------------------------------------------------
# P2: the objective itself, solved as weighted least squares
# --------------------------------------------------------------------------
def test_objective_least_squares_and_normal_equations():
    rng = np.random.default_rng(2)
    T, dk, dv = 15, 5, 3   # dk != dv: a transposed G cannot pass
    q, k, v, g, lam = rand_problem(rng, T, dk, dv)
    res = oracle.forward(q, k, v, g, lam, max_iters=6 * dk, tol=1e-14, final_state=True)
    K, V, gam = k[0, 0], v[0, 0], g[0, 0]
    for t in [0, 3, 7, T - 1]:
        sz = np.sqrt(zeta(gam, t))
        # minimise sum zeta |v - Phi k|^2 + Tr(Phi Lambda Phi^T) = |A Phi^T - Y|_F^2
        A = np.vstack([sz[:, None] * K[:t + 1], np.diag(np.sqrt(lam[0]))])
        Y = np.vstack([sz[:, None] * V[:t + 1], np.zeros((dk, dv))])
        PhiT, *_ = np.linalg.lstsq(A, Y, rcond=None)
        assert rel(res["out"][0, 0, t], PhiT.T @ q[0, 0, t]) < 1e-9, t
    # zero gradient of the objective at the final token: Phi (H_T + Lambda) = G_T
    sz = np.sqrt(zeta(gam, T - 1))
    A = np.vstack([sz[:, None] * K, np.diag(np.sqrt(lam[0]))])
    Y = np.vstack([sz[:, None] * V, np.zeros((dk, dv))])
    PhiT, *_ = np.linalg.lstsq(A, Y, rcond=None)
    Phi = PhiT.T
    assert rel(Phi @ (res["final_H"][0, 0] + np.diag(lam[0])), res["final_G"][0, 0]) < 1e-10


# --------------------------------------------------------------------------
# P3: gamma == 1, Lambda = lam I  ->  kernel-ridge form (a t x t solve)
# --------------------------------------------------------------------------
def test_ridge_kernel_form_without_forgetting():
    rng = np.random.default_rng(3)
    T, dk, dv, lamv = 12, 7, 4, 0.7
    q, k, v, _, _ = rand_problem(rng, T, dk, dv)
    g = np.ones((1, 1, T))
    lam = np.full((1, dk), lamv)
    res = oracle.forward(q, k, v, g, lam, max_iters=4 * dk, tol=1e-14)
    K, V = k[0, 0], v[0, 0]
    for t in range(T):
        Kt, Vt = K[:t + 1], V[:t + 1]
        o = Vt.T @ np.linalg.solve(Kt @ Kt.T + lamv * np.eye(t + 1), Kt @ q[0, 0, t])
        assert rel(res["out"][0, 0, t], o) < 1e-10, t


# --------------------------------------------------------------------------
# P4: first token, Sherman-Morrison; Lambda = lam I reached in two CG steps
# --------------------------------------------------------------------------
def test_first_token_sherman_morrison():
    rng = np.random.default_rng(4)
    dk, dv = 9, 5
    for lam_iso in (True, False):
        q, k, v, g, lam = rand_problem(rng, 3, dk, dv)
        if lam_iso:
            lam = np.full((1, dk), 1.3)
        iters = 2 if lam_iso else 3 * dk
        res = oracle.forward(q, k, v, g, lam, max_iters=iters, tol=0.0 if lam_iso else 1e-14)
        k1, v1, q1, li = k[0, 0, 0], v[0, 0, 0], q[0, 0, 0], 1.0 / lam[0]
        o1 = v1 * (k1 @ (li * q1)) / (1.0 + k1 @ (li * k1))
        assert rel(res["out"][0, 0, 0], o1) < 1e-12


# --------------------------------------------------------------------------
# P5: the k-step CG iterate is the A-orthogonal projection onto the Krylov
#     space span{b, Ab, ..., A^{k-1} b} (exact rational arithmetic)
# --------------------------------------------------------------------------
def _frac_solve(M, y):
    n = len(M)
    M = [row[:] + [y[i]] for i, row in enumerate(M)]
    for c in range(n):
        p = next(r for r in range(c, n) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        for r in range(n):
            if r != c and M[r][c] != 0:
                f = M[r][c] / M[c][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [M[i][n] / M[i][i] for i in range(n)]


def _krylov_iterate(A, b, kk):
    n = len(b)
    cols = [b]
    for _ in range(kk - 1):
        prev = cols[-1]
        cols.append([sum(A[i][j] * prev[j] for j in range(n)) for i in range(n)])
    AK = [[sum(A[i][j] * cols[c][j] for j in range(n)) for i in range(n)] for c in range(kk)]
    KtAK = [[sum(cols[a][i] * AK[c][i] for i in range(n)) for c in range(kk)] for a in range(kk)]
    Ktb = [sum(cols[a][i] * b[i] for i in range(n)) for a in range(kk)]
    y = _frac_solve(KtAK, Ktb)
    return [sum(cols[c][i] * y[c] for c in range(kk)) for i in range(n)]


def test_k_step_iterate_is_krylov_projection():
    rng = np.random.default_rng(5)
    n = 5
    for trial in range(3):
        ints = rng.integers(-3, 4, size=(n + 2, n))
        Hq = [[Fraction(int(sum(ints[r, i] * ints[r, j] for r in range(n + 2))), 4)
               for j in range(n)] for i in range(n)]
        lam = [Fraction(int(x), 2) for x in rng.integers(1, 6, size=n)]
        b = [Fraction(int(x)) for x in rng.integers(-4, 5, size=n)]
        if all(x == 0 for x in b):
            b[0] = Fraction(1)
        A = [[Hq[i][j] + (lam[i] if i == j else 0) for j in range(n)] for i in range(n)]
        Hf = np.array([[float(x) for x in row] for row in Hq])
        lf = np.array([float(x) for x in lam])
        bf = np.array([float(x) for x in b])
        for kk in range(1, n + 1):
            exact = np.array([float(x) for x in _krylov_iterate(A, b, kk)])
            x, it, *_ = oracle.cg_solve(Hf, lf, bf, kk, 0.0)
            if it < kk:      # exact convergence before kk steps: iterate is A^-1 b
                exact = np.array([float(x) for x in _frac_solve(A, b)])
            assert rel(x, exact) < 1e-11, (trial, kk)


# --------------------------------------------------------------------------
# P6: finite termination on the tiny workload (Lambda = I, k = 10):
#     H_t has rank <= t (1-based), so A_t has <= t+1 distinct eigenvalues and
#     10 CG steps are exact for t <= 9.
# --------------------------------------------------------------------------
def test_finite_termination_tiny_workload():
    w = inputs.WORKLOADS["tiny_f32_d16_T256"]
    x = inputs.forward_inputs(w, T=12)
    q, k, v = (inputs.as_f64(x[n], w.dtype) for n in ("q", "k", "v"))
    g, lam = x["gamma"].astype(np.float64), x["lam"].astype(np.float64)
    assert np.all(lam == 1.0)
    res = oracle.forward(q, k, v, g, lam, w.max_iters, 0.0)
    for t in range(9):
        Hm, Gm = brute_states(k[0, 0], v[0, 0], g[0, 0], t)
        xs = scipy.linalg.solve(Hm + np.eye(w.d), q[0, 0, t], assume_a="pos")
        assert rel(res["out"][0, 0, t], Gm @ xs) < 1e-12, t
    # a later token is NOT exact after 10 steps (the pin has teeth)
    t = 11
    Hm, Gm = brute_states(k[0, 0], v[0, 0], g[0, 0], t)
    xs = scipy.linalg.solve(Hm + np.eye(w.d), q[0, 0, t], assume_a="pos")
    assert rel(res["out"][0, 0, t], Gm @ xs) > 1e-12


# --------------------------------------------------------------------------
# P7: d = 1 closed form
# --------------------------------------------------------------------------
def test_scalar_closed_form():
    rng = np.random.default_rng(7)
    T = 30
    q, k, v, g, lam = rand_problem(rng, T, 1, 1)
    res = oracle.forward(q, k, v, g, lam, max_iters=1, tol=0.0)
    K, V, gam = k[0, 0, :, 0], v[0, 0, :, 0], g[0, 0]
    for t in range(T):
        z = zeta(gam, t)
        o = q[0, 0, t, 0] * np.sum(z * V[:t + 1] * K[:t + 1]) / (np.sum(z * K[:t + 1] ** 2) + lam[0, 0])
        assert abs(res["out"][0, 0, t, 0] - o) <= 1e-13 * max(1.0, abs(o)), t


# --------------------------------------------------------------------------
# P8: dynamic stopping bookkeeping, with residuals recomputed from the
#     definition (q - A x_j, A built from explicit zeta sums)
# --------------------------------------------------------------------------
def test_dynamic_stop_matches_true_residuals():
    rng = np.random.default_rng(8)
    T, dk, dv, tol, cap = 40, 12, 6, 1e-3, 9
    q, k, v, g, lam = rand_problem(rng, T, dk, dv, glo=0.9)
    res = oracle.forward(q, k, v, g, lam, max_iters=cap, tol=tol)
    checked = 0
    for t in range(T):
        n = int(res["iters"][0, 0, t])
        Hm, _ = brute_states(k[0, 0], v[0, 0], g[0, 0], t)
        A = Hm + np.diag(lam[0])
        qt = q[0, 0, t]

        def rho(j):
            x, *_ = oracle.cg_solve(Hm, lam[0], qt, j, 0.0)
            return np.linalg.norm(qt - A @ x) / np.linalg.norm(qt)
        rhos = [rho(j) for j in range(n + 1)]
        if any(abs(r / tol - 1.0) < 1e-9 for r in rhos):
            continue
        assert all(r >= tol for r in rhos[:n]), t
        if n < cap:
            assert res["reason"][0, 0, t] == oracle.STOP_TOL
            assert rhos[n] < tol, t
        else:
            assert res["reason"][0, 0, t] == oracle.STOP_CAP
        assert abs(res["rho_stop"][0, 0, t] - rhos[n]) <= 1e-9 * max(rhos[n], 1e-12) + 1e-13
        checked += 1
    assert checked >= T - 2
    assert len(set(res["iters"][0, 0].tolist())) > 1   # counts do vary per token


# --------------------------------------------------------------------------
# P9: count bound for Lambda = lam I:  iters_t <= t + 1 (1-based t)
# --------------------------------------------------------------------------
def test_iteration_count_bound_isotropic():
    rng = np.random.default_rng(9)
    T, dk, dv = 20, 16, 4
    q, k, v, g, _ = rand_problem(rng, T, dk, dv, glo=0.9)
    lam = np.full((1, dk), 0.8)
    res = oracle.forward(q, k, v, g, lam, max_iters=40, tol=1e-10)
    it = res["iters"][0, 0]
    for t in range(T):
        assert it[t] <= t + 2, (t, it[t])     # 0-based t: rank <= t+1
    assert it[0] <= 2 and it[T - 1] > 2


# --------------------------------------------------------------------------
# P10: CG internals -- residuals mutually orthogonal, A-norm error decreasing
# --------------------------------------------------------------------------
def test_cg_residual_orthogonality_and_energy_decrease():
    rng = np.random.default_rng(10)
    n = 24
    M = rng.standard_normal((2 * n, n)) / np.sqrt(n)
    Hm = M.T @ M
    lam = rng.uniform(0.2, 1.0, n)
    A = Hm + np.diag(lam)
    b = rng.standard_normal(n)
    xs = np.linalg.solve(A, b)
    res, errs = [], []
    for j in range(8):
        x, *_ = oracle.cg_solve(Hm, lam, b, j, 0.0)
        res.append(b - A @ x)
        e = xs - x
        errs.append(np.sqrt(e @ A @ e))
    for i in range(8):
        for j in range(i):
            c = res[i] @ res[j] / (np.linalg.norm(res[i]) * np.linalg.norm(res[j]))
            assert abs(c) < 1e-8, (i, j, c)
    assert all(errs[j + 1] < errs[j] for j in range(7))


# --------------------------------------------------------------------------
# internal consistency: decode continues the forward recurrence; selecting
# tokens does not change them; zero query -> zero output and count
# --------------------------------------------------------------------------
def test_decode_continues_forward():
    rng = np.random.default_rng(11)
    T, S, dk, dv, cap, tol = 30, 5, 8, 8, 12, 1e-6
    q, k, v, g, lam = rand_problem(rng, T, dk, dv, glo=0.8)
    full = oracle.forward(q, k, v, g, lam, cap, tol)
    pre = oracle.forward(q[:, :, :T - S], k[:, :, :T - S], v[:, :, :T - S], g[:, :, :T - S],
                         lam, cap, tol, final_state=True)
    Hs, Gs = pre["final_H"][:, :].copy(), pre["final_G"][:, :].copy()
    for s in range(T - S, T):
        r = oracle.decode_step(q[:, :, s], k[:, :, s], v[:, :, s], g[:, :, s], lam, Hs, Gs, cap, tol)
        np.testing.assert_allclose(r["out"][0, 0], full["out"][0, 0, s], rtol=1e-12, atol=1e-13)
        assert r["iters"][0, 0] == full["iters"][0, 0, s]


def test_want_mask_and_zero_query():
    rng = np.random.default_rng(12)
    T, dk, dv = 25, 6, 6
    q, k, v, g, lam = rand_problem(rng, T, dk, dv)
    q[0, 0, 4] = 0.0
    full = oracle.forward(q, k, v, g, lam, 7, 1e-5)
    want = np.zeros((1, 1, T), bool)
    want[0, 0, [2, 4, 20]] = True
    part = oracle.forward(q, k, v, g, lam, 7, 1e-5, want=want)
    for t in [2, 4, 20]:
        np.testing.assert_array_equal(part["out"][0, 0, t], full["out"][0, 0, t])
    assert np.isnan(part["out"][0, 0, 3]).all()
    assert full["iters"][0, 0, 4] == 0 and np.all(full["out"][0, 0, 4] == 0)
    assert full["reason"][0, 0, 4] == oracle.STOP_Q_ZERO


def test_generator_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(13).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3.0e38]   # ties to even, sign, large
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# --------------------------------------------------------------------------
# Warm start (the page names warm-start strategies as future work, section
# "Significancia e Alegacoes").  W1: from x0 the k-step CG iterate is x0 plus
# the Krylov projection of the initial residual r0 = b - A x0 (exact
# rationals).  W2: an exact start needs no update.  W3: the projected start
# c x_prev minimises the A-norm error over multiples of x_prev (brute-force
# scan) and is exact when x_prev is an eigenvector parallel to q.  W4: cold
# and degenerate warm modes reproduce the cold decode step bit for bit.
# --------------------------------------------------------------------------
def test_warm_start_iterate_is_shifted_krylov_projection():
    rng = np.random.default_rng(21)
    n = 5
    for trial in range(3):
        ints = rng.integers(-3, 4, size=(n + 2, n))
        Hq = [[Fraction(int(sum(ints[r, i] * ints[r, j] for r in range(n + 2))), 4)
               for j in range(n)] for i in range(n)]
        lam = [Fraction(int(x), 2) for x in rng.integers(1, 6, size=n)]
        b = [Fraction(int(x)) for x in rng.integers(-4, 5, size=n)]
        x0 = [Fraction(int(x), 3) for x in rng.integers(-3, 4, size=n)]
        A = [[Hq[i][j] + (lam[i] if i == j else 0) for j in range(n)] for i in range(n)]
        r0 = [b[i] - sum(A[i][j] * x0[j] for j in range(n)) for i in range(n)]
        if all(x == 0 for x in r0):
            continue
        Hf = np.array([[float(x) for x in row] for row in Hq])
        lf = np.array([float(x) for x in lam])
        bf = np.array([float(x) for x in b])
        x0f = np.array([float(x) for x in x0])
        for kk in range(1, n + 1):
            e = _krylov_iterate(A, r0, kk)
            exact = np.array([float(x0[i] + e[i]) for i in range(n)])
            x, it, *_ = oracle.cg_solve(Hf, lf, bf, kk, 0.0, x0=x0f)
            if it < kk:
                exact = np.array([float(x) for x in _frac_solve(A, b)])
            assert rel(x, exact) < 1e-11, (trial, kk)
        # the start point matters: the 1-step iterates from x0 and from 0 differ
        x_cold, *_ = oracle.cg_solve(Hf, lf, bf, 1, 0.0)
        x_warm, *_ = oracle.cg_solve(Hf, lf, bf, 1, 0.0, x0=x0f)
        assert rel(x_warm, x_cold) > 1e-6


def test_warm_start_from_the_solution_makes_no_update():
    rng = np.random.default_rng(22)
    n = 12
    K = rng.standard_normal((20, n)) / np.sqrt(n)
    Hm, lam, b = K.T @ K, rng.uniform(0.5, 2.0, n), rng.standard_normal(n)
    xs = scipy.linalg.solve(Hm + np.diag(lam), b, assume_a="pos")
    x, it, why, rho, _ = oracle.cg_solve(Hm, lam, b, 30, 1e-8, x0=xs)
    assert it == 0 and why == oracle.STOP_TOL and rho < 1e-12
    np.testing.assert_array_equal(x, xs)
    # a zero query gives x = 0 whatever the start
    x, it, why, *_ = oracle.cg_solve(Hm, lam, np.zeros(n), 30, 1e-8, x0=xs)
    assert it == 0 and why == oracle.STOP_Q_ZERO and not x.any()


def _decode_problem(rng, dk, dv, T):
    k = rng.standard_normal((T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(0.8, 1.0, T)
    Hm, Gm = brute_states(k, v, g, T - 1)
    return Hm, Gm


def test_projected_warm_start_minimises_energy_error():
    rng = np.random.default_rng(23)
    dk = dv = 10
    for trial in range(4):
        Hm, Gm = _decode_problem(rng, dk, dv, 15)
        lam = rng.uniform(0.5, 2.0, (1, dk))
        q = rng.standard_normal((1, 1, dk))
        kn = rng.standard_normal((1, 1, dk)) / np.sqrt(dk)
        vn = rng.standard_normal((1, 1, dv))
        g = np.array([[0.9]])
        x_prev = rng.standard_normal(dk)
        # A after this step's state update, built from the recurrence's definition
        A = 0.9 * Hm + np.outer(kn[0, 0], kn[0, 0]) + np.diag(lam[0])
        xs = scipy.linalg.solve(A, q[0, 0], assume_a="pos")
        SH, SG = Hm[None, None].copy(), Gm[None, None].copy()
        SX = x_prev[None, None].copy()
        oracle.decode_step_warm(q, kn, vn, g, lam, SH, SG, SX, 0, 0.0, oracle.WARM_PROJECTED)
        c = SX[0, 0] @ x_prev / (x_prev @ x_prev)
        np.testing.assert_allclose(SX[0, 0], c * x_prev, rtol=1e-12, atol=1e-14)

        def energy(cc):
            e = xs - cc * x_prev
            return e @ A @ e
        grid = np.linspace(c - 1.0, c + 1.0, 2001)
        assert energy(c) <= min(energy(cc) for cc in grid) + 1e-12
        assert energy(c) <= energy(0.0) + 1e-12   # never worse than the cold start


def test_projected_warm_start_exact_for_parallel_eigenvector():
    rng = np.random.default_rng(24)
    dk = dv = 8
    Hm, Gm = _decode_problem(rng, dk, dv, 12)
    lam = np.full((1, dk), 0.7)               # Lambda = lambda I keeps eigenvectors of H
    kn = np.zeros((1, 1, dk))                 # no new key: A = g Hm + Lambda
    vn = rng.standard_normal((1, 1, dv))
    g = np.array([[1.0]])
    w, U = np.linalg.eigh(Hm)
    u = U[:, 3]
    q = (2.5 * u)[None, None]
    SH, SG, SX = Hm[None, None].copy(), Gm[None, None].copy(), (-0.3 * u)[None, None].copy()
    r = oracle.decode_step_warm(q, kn, vn, g, lam, SH, SG, SX, 30, 1e-9, oracle.WARM_PROJECTED)
    assert r["iters"][0, 0] == 0
    np.testing.assert_allclose(SX[0, 0], 2.5 / (w[3] + 0.7) * u, rtol=1e-12, atol=1e-14)
    # the plain previous-solution start is not exact here and needs updates
    SH, SG, SX = Hm[None, None].copy(), Gm[None, None].copy(), (-0.3 * u)[None, None].copy()
    r = oracle.decode_step_warm(q, kn, vn, g, lam, SH, SG, SX, 30, 1e-9, oracle.WARM_PREVIOUS)
    assert r["iters"][0, 0] >= 1


def test_warm_decode_degenerate_modes_equal_cold():
    rng = np.random.default_rng(25)
    N, H, dk, dv = 2, 3, 6, 6
    base_H = np.stack([np.stack([_decode_problem(rng, dk, dv, 9)[0] for _ in range(H)]) for _ in range(N)])
    base_G = rng.standard_normal((N, H, dv, dk))
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk)) / np.sqrt(dk)
    v = rng.standard_normal((N, H, dv))
    g = rng.uniform(0.9, 1.0, (N, H))
    lam = rng.uniform(0.5, 2.0, (H, dk))
    cold_H, cold_G = base_H.copy(), base_G.copy()
    cold = oracle.decode_step(q, k, v, g, lam, cold_H, cold_G, 9, 1e-7)
    cases = [(oracle.WARM_COLD, rng.standard_normal((N, H, dk))),
             (oracle.WARM_PREVIOUS, np.zeros((N, H, dk))),
             (oracle.WARM_PROJECTED, np.zeros((N, H, dk)))]
    for mode, x_prev in cases:
        SH, SG, SX = base_H.copy(), base_G.copy(), x_prev.copy()
        r = oracle.decode_step_warm(q, k, v, g, lam, SH, SG, SX, 9, 1e-7, mode)
        np.testing.assert_array_equal(r["out"], cold["out"])
        np.testing.assert_array_equal(r["iters"], cold["iters"])
        np.testing.assert_array_equal(SH, cold_H)
        np.testing.assert_array_equal(SG, cold_G)
        # this step's solution is left in state_x: G x reproduces the output
        np.testing.assert_allclose(np.einsum("nhij,nhj->nhi", SG, SX), cold["out"], rtol=1e-12, atol=1e-13)


def test_warm_previous_start_is_the_previous_solution():
    rng = np.random.default_rng(26)
    dk = dv = 7
    Hm, Gm = _decode_problem(rng, dk, dv, 10)
    lam = rng.uniform(0.5, 2.0, (1, dk))
    q = rng.standard_normal((1, 1, dk))
    kn = rng.standard_normal((1, 1, dk)) / np.sqrt(dk)
    vn = rng.standard_normal((1, 1, dv))
    g = np.array([[0.95]])
    x_prev = rng.standard_normal(dk)
    # no update allowed: the solution left behind is the start point itself
    SH, SG, SX = Hm[None, None].copy(), Gm[None, None].copy(), x_prev[None, None].copy()
    r = oracle.decode_step_warm(q, kn, vn, g, lam, SH, SG, SX, 0, 0.0, oracle.WARM_PREVIOUS)
    np.testing.assert_array_equal(SX[0, 0], x_prev)
    A = 0.95 * Hm + np.outer(kn[0, 0], kn[0, 0])
    Gn = 0.95 * Gm + np.outer(vn[0, 0], kn[0, 0])
    np.testing.assert_allclose(r["out"][0, 0], Gn @ x_prev, rtol=1e-12, atol=1e-13)
    # with updates, the residual that decides the stop is measured from x_prev
    SH, SG, SX = Hm[None, None].copy(), Gm[None, None].copy(), x_prev[None, None].copy()
    r = oracle.decode_step_warm(q, kn, vn, g, lam, SH, SG, SX, 3, 0.0, oracle.WARM_PREVIOUS)
    res = q[0, 0] - (A + np.diag(lam[0])) @ SX[0, 0]
    assert abs(r["rho_stop"][0, 0] - np.linalg.norm(res) / np.linalg.norm(q[0, 0])) < 1e-10


# --------------------------------------------------------------------------
# q/k pre-processing (section "Arquitetura (MesaNet)", bullet
# "Pre-processamento": keys and queries are normalised and convolved with a
# small window before the layer).  C1: a hand-worked example (width 2,
# d = 2).  C2: each channel's convolution equals numpy.convolve truncated to
# the causal part, then unit-normalised.  C3: a sequence cut into pieces with
# the carried history gives the same result as one piece.  C4: width 1 with
# unit weights is plain L2 normalisation; zero rows stay zero.
# --------------------------------------------------------------------------
def test_preprocess_hand_worked_example():
    x = np.array([[3.0, 0.0], [1.0, 4.0], [0.0, -4.0]])[None, None]
    w = np.array([[[1.0, 1.0], [2.0, 0.5]]])         # w[h][j][f], j = 0 is the current token
    # c_0 = (3, 0); c_1 = (1 + 6, 4 + 0) = (7, 4); c_2 = (0 + 2, -4 + 2) = (2, -2)
    want = np.array([[1.0, 0.0], [7.0, 4.0] / np.sqrt(65.0), [2.0, -2.0] / np.sqrt(8.0)])
    y = oracle.qk_preprocess(x, w)
    np.testing.assert_allclose(y[0, 0], want, rtol=1e-15, atol=1e-15)


def test_preprocess_matches_numpy_convolve():
    rng = np.random.default_rng(31)
    B, H, T, d, W = 2, 3, 17, 5, 4
    x = rng.standard_normal((B, H, T, d))
    w = rng.standard_normal((H, W, d))
    y = oracle.qk_preprocess(x, w)
    for b in range(B):
        for h in range(H):
            c = np.stack([np.convolve(x[b, h, :, f], w[h, :, f])[:T] for f in range(d)], axis=-1)
            want = c / np.linalg.norm(c, axis=-1, keepdims=True)
            assert rel(y[b, h], want) < 1e-13
    # the order matters: normalising first and convolving after is different
    xn = x / np.linalg.norm(x, axis=-1, keepdims=True)
    c = np.stack([np.convolve(xn[0, 0, :, f], w[0, :, f])[:T] for f in range(d)], axis=-1)
    assert rel(y[0, 0], c) > 1e-3


def test_preprocess_history_continues_the_sequence():
    rng = np.random.default_rng(32)
    B, H, d = 2, 2, 6
    for W, cuts in ((4, (5, 1, 2, 9)), (3, (1, 1, 1, 4)), (2, (7,)), (1, (3, 3))):
        T = sum(cuts)
        x = rng.standard_normal((B, H, T, d))
        w = rng.standard_normal((H, W, d))
        whole = oracle.qk_preprocess(x, w)
        hist, t0, parts = None, 0, []
        for n in cuts:
            y, hist = oracle.qk_preprocess(x[:, :, t0:t0 + n], w, hist=hist, want_hist=True)
            parts.append(y)
            t0 += n
        np.testing.assert_allclose(np.concatenate(parts, axis=2), whole, rtol=1e-13, atol=1e-14)
        # the carried rows are the last W-1 inputs
        np.testing.assert_array_equal(hist, x[:, :, T - (W - 1):])


def test_preprocess_width_one_is_normalisation():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((1, 2, 9, 7)) * rng.uniform(0.1, 10, (1, 2, 9, 1))
    x[0, 1, 4] = 0.0
    y = oracle.qk_preprocess(x, np.ones((2, 1, 7)))
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    np.testing.assert_allclose(y, np.where(n > 0, x / np.where(n > 0, n, 1), 0), rtol=1e-15)
    assert not y[0, 1, 4].any()


# --------------------------------------------------------------------------
# Backward pass (the page says the layer trains in parallel but gives no
# gradient; section "A Camada Mesa", bullet "Paralelizacao").  The oracle
# differentiates o_t = G_t (H_t + Lambda)^{-1} q_t implicitly with a k-step
# adjoint CG.  B1: with the solves converged, every gradient equals central
# finite differences of the oracle's own forward (a different route: no
# adjoint, no reverse sums).  B2: gamma at the first token has no effect, so
# its gradient is zero.  B3: the adjoint solve is the k-step CG of G_t^T g_t.
# --------------------------------------------------------------------------
def _loss(q, k, v, g, lam, gout, cap, tol):
    return float(np.sum(oracle.forward(q, k, v, g, lam, cap, tol)["out"] * gout))


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(41)
    B, H, T, dk, dv = 1, 2, 6, 3, 2
    q, k, v, g, lam = rand_problem(rng, T, dk, dv, glo=0.7)
    q, k, v, g = (np.repeat(a, H, axis=1) + rng.standard_normal((B, H) + a.shape[2:]) * 0.3 for a in (q, k, v, g))
    g = np.clip(g, 0.5, 1.0)
    lam = rng.uniform(0.4, 1.5, (H, dk))
    gout = rng.standard_normal((B, H, T, dv))
    cap, tol = 4 * dk, 1e-13
    r = oracle.backward(q, k, v, g, lam, gout, cap, tol)
    args = dict(q=q, k=k, v=v, g=g, lam=lam)
    grads = dict(q=r["dq"], k=r["dk"], v=r["dv"], g=r["dgamma"], lam=r["dlam"])
    for name, a in args.items():
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            hstep = 1e-6 * max(1.0, abs(a[idx]))
            ap, am = a.copy(), a.copy()
            ap[idx] += hstep
            am[idx] -= hstep
            kw_p = dict(args, **{name: ap})
            kw_m = dict(args, **{name: am})
            fd[idx] = (_loss(kw_p["q"], kw_p["k"], kw_p["v"], kw_p["g"], kw_p["lam"], gout, cap, tol)
                       - _loss(kw_m["q"], kw_m["k"], kw_m["v"], kw_m["g"], kw_m["lam"], gout, cap, tol)) / (2 * hstep)
        if name == "g":
            fd[:, :, 0] = 0.0       # gamma_1 has no effect
        err = np.abs(grads[name] - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 2e-6, (name, err)


def test_backward_first_gate_gradient_is_zero_and_adjoint_is_cg():
    rng = np.random.default_rng(42)
    B, H, T, dk, dv = 2, 1, 9, 4, 4
    q, k, v, g, lam = rand_problem(rng, T, dk, dv, glo=0.8)
    q, k, v, g = (np.concatenate([a, a[:, :, ::-1]], axis=0) for a in (q, k, v, g))
    gout = rng.standard_normal((B, H, T, dv))
    cap, tol = 3, 0.0
    r = oracle.backward(q, k, v, g, lam, gout, cap, tol)
    assert np.abs(r["dgamma"][:, :, 0]).max() < 1e-10 * np.abs(r["dgamma"]).max()
    # the adjoint: z_t = 3-step CG on (H_t + Lambda) z = G_t^T gout_t, states from their definition
    for b in range(B):
        for t in (0, 4, 8):
            Hm, Gm = brute_states(k[b, 0], v[b, 0], g[b, 0], t)
            z, it, *_ = oracle.cg_solve(Hm, lam[0], Gm.T @ gout[b, 0, t], cap, 0.0)
            assert it == cap
            np.testing.assert_allclose(r["dq"][b, 0, t], z, rtol=1e-10, atol=1e-12)
            xs, *_ = oracle.cg_solve(Hm, lam[0], q[b, 0, t], cap, 0.0)
            np.testing.assert_allclose(r["x"][b, 0, t], xs, rtol=1e-10, atol=1e-12)
    # dlambda sums -z (.) x over the batch and tokens
    np.testing.assert_allclose(r["dlam"][0], -np.sum(r["dq"][:, 0] * r["x"][:, 0], axis=(0, 1)), rtol=1e-12)


# --------------------------------------------------------------------------
# Hawk layer recurrence (section "Arquitetura (MesaNet)", bullet "Variante
# Hibrida": the hybrid alternates LRU (Hawk) layers with Mesa layers; the
# recurrence is the published real-gated LRU of Hawk).  H1: a hand-worked
# example.  H2: constant gates reduce to a first-order filter, checked with
# scipy.signal.lfilter.  H3: time-varying gates against the explicit
# sum of products.  H4: pieces with the carried state equal one pass.
# H5: closed gates keep the state.
# --------------------------------------------------------------------------
def test_hawk_hand_worked_example():
    # c = 1, lam = 0, ga = gx = +50 (r = i = 1): a = sigmoid(0) = 1/2, sqrt(1 - a^2) = sqrt(3)/2
    x = np.array([2.0, 4.0]).reshape(1, 2, 1)
    big = np.full((1, 2, 1), 50.0)
    y, hf = oracle.hawk_scan(x, big, big, np.zeros(1), c=1.0)
    s3 = np.sqrt(3.0)
    np.testing.assert_allclose(y[0, :, 0], [s3, 2.5 * s3], rtol=1e-15)
    np.testing.assert_allclose(hf[0], [2.5 * s3], rtol=1e-15)


def test_hawk_constant_gates_is_a_first_order_filter():
    import scipy.signal
    rng = np.random.default_rng(51)
    B, T, D, c = 2, 40, 3, 8.0
    x = rng.standard_normal((B, T, D))
    ga0 = rng.standard_normal((1, 1, D))
    gx0 = rng.standard_normal((1, 1, D))
    lam = rng.standard_normal(D)
    h0 = rng.standard_normal((B, D))
    y, hf = oracle.hawk_scan(x, np.broadcast_to(ga0, x.shape), np.broadcast_to(gx0, x.shape), lam, c, h0)
    for b in range(B):
        for d in range(D):
            r = 1 / (1 + np.exp(-ga0[0, 0, d]))
            i = 1 / (1 + np.exp(-gx0[0, 0, d]))
            a = (1 / (1 + np.exp(-lam[d]))) ** (c * r)
            u = np.sqrt(1 - a * a) * i * x[b, :, d]
            want, _ = scipy.signal.lfilter([1.0], [1.0, -a], u, zi=[a * h0[b, d]])
            assert rel(y[b, :, d], want) < 1e-13


def test_hawk_time_varying_gates_explicit_sum():
    rng = np.random.default_rng(52)
    B, T, D, c = 1, 25, 4, 8.0
    x, ga, gx = (rng.standard_normal((B, T, D)) for _ in range(3))
    lam = rng.standard_normal(D) + 2.0
    h0 = rng.standard_normal((B, D))
    y, _ = oracle.hawk_scan(x, ga, gx, lam, c, h0)
    sig = lambda z: 1 / (1 + np.exp(-z))
    a = np.exp(c * sig(ga) * np.log(sig(lam)))          # a^{c r_t}
    u = np.sqrt(1 - a * a) * sig(gx) * x
    for t in range(T):
        # h_t = (prod_{s<=t} a_s) h0 + sum_{s<=t} (prod_{s<u<=t} a_u) u_s
        want = np.prod(a[0, :t + 1], axis=0) * h0[0]
        for s_ in range(t + 1):
            want = want + np.prod(a[0, s_ + 1:t + 1], axis=0) * u[0, s_]
        assert rel(y[0, t], want) < 1e-12, t


def test_hawk_pieces_and_closed_gates():
    rng = np.random.default_rng(53)
    B, T, D = 2, 30, 5
    x, ga, gx = (rng.standard_normal((B, T, D)) for _ in range(3))
    lam = rng.standard_normal(D)
    y, hf = oracle.hawk_scan(x, ga, gx, lam)
    y1, h1 = oracle.hawk_scan(x[:, :11], ga[:, :11], gx[:, :11], lam)
    y2, h2 = oracle.hawk_scan(x[:, 11:], ga[:, 11:], gx[:, 11:], lam, h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(h2, hf, rtol=1e-14)
    # closed gates (r = 0 -> a = 1, no input) keep the state
    h0 = rng.standard_normal((B, D))
    yc, hc = oracle.hawk_scan(x, np.full_like(x, -60.0), gx, lam, h0=h0)
    np.testing.assert_allclose(yc, np.broadcast_to(h0[:, None, :], x.shape), rtol=1e-12)
