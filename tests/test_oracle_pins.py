"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Every pin is an independent route to a value: a hand-worked example, exact
rational brute force through the unrolled transition product, closed forms of
special cases, invariants proved in the paper ("Kaczmarz Linear Attention",
arXiv 2605.08587), and the chunkwise solve of Propositions 3-4.  A dropped
term, a wrong sign, a swapped decay/write order or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunkwise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand_problem(rng, T, H, dk, dv, eps=1e-6, g_low=-0.5, s0=True, key_scale=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if key_scale:
        k *= 10.0 ** rng.uniform(-1, 1, size=(T, H, 1))
    v = rng.standard_normal((T, H, dv))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    g = rng.uniform(g_low, 0.0, size=(T, H))
    S0 = rng.standard_normal((1, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, g, eta, eps, S0


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------- golden
def test_golden_hand_worked(oracle_lib):
    """Hand-derived values (Algorithm 1 left panel + Eq. (3)), stored with derivations."""
    data = json.load(open(GOLDEN))
    for case in data["cases"]:
        k = np.array(case["k"], float)[:, None, :]
        v = np.array(case["v"], float)[:, None, :]
        q = np.array(case["q"], float)[:, None, :]
        g = np.log(np.array(case["alpha"], float))[:, None]
        eta = np.array(case["eta"], float)[:, None]
        S0 = np.array(case["S0"], float)[None, None]
        o, ST = oracle.prefill(q, k, v, g, eta, case["eps"], S0=S0)
        np.testing.assert_allclose(o[:, 0], np.array(case["o"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(ST[0, 0], np.array(case["S_T"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- brute force
def _frac_matmul(A, B):
    return [[sum((A[i][t] * B[t][j] for t in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _brute_force(q, k, v, alpha, eta, eps, S0):
    """Exact rational unrolled form S_t = Phi(t,0) S0 + sum_j Phi(t,j) b_j k_j^T v_j,
    Phi(t,j) = M_t ... M_{j+1}, M_s = alpha_s (I - b_s k_s^T k_s); o_t = q_t S_t.
    (The recurrent form of the paper's Table 6 KLA row, with the b_j and S0 terms of
    Appendix B's H_i written out.)"""
    T, dk, dv = len(k), len(k[0]), len(v[0])
    I = [[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)]

    def beta(t):
        den = sum(x * x for x in k[t]) + eps
        return Fraction(0) if den == 0 else eta[t] / den

    def M(s):
        b = beta(s)
        return [[alpha[s] * (I[i][j] - b * k[s][i] * k[s][j]) for j in range(dk)] for i in range(dk)]

    outs = []
    for t in range(T):
        Phi = I
        S = [[Fraction(0)] * dv for _ in range(dk)]
        # contributions j = t, t-1, ..., 0, then S0 with Phi(t, -1)
        for j in range(t, -1, -1):
            b = beta(j)
            w = [[b * k[j][i] * v[j][c] for c in range(dv)] for i in range(dk)]
            contrib = _frac_matmul(Phi, w)
            S = [[S[i][c] + contrib[i][c] for c in range(dv)] for i in range(dk)]
            Phi = _frac_matmul(Phi, M(j))
        base = _frac_matmul(Phi, S0)
        S = [[S[i][c] + base[i][c] for c in range(dv)] for i in range(dk)]
        outs.append([sum((q[t][i] * S[i][c] for i in range(dk)), Fraction(0)) for c in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_rational(oracle_lib, seed):
    rnd = random.Random(seed)
    T = rnd.randint(1, 8)
    dk, dv = rnd.randint(1, 4), rnd.randint(1, 4)
    fr = lambda: Fraction(rnd.randint(-4, 4), rnd.choice([1, 2, 3, 4]))
    k = [[fr() for _ in range(dk)] for _ in range(T)]
    if seed == 5:  # a zero key with eps = 0 exercises the b = 0 reading
        k[T // 2] = [Fraction(0)] * dk
    q = [[fr() for _ in range(dk)] for _ in range(T)]
    v = [[fr() for _ in range(dv)] for _ in range(T)]
    alpha = [rnd.choice([Fraction(1), Fraction(1, 2), Fraction(3, 4), Fraction(1, 8)]) for _ in range(T)]
    eta = [rnd.choice([Fraction(1), Fraction(1, 2), Fraction(1, 3), Fraction(9, 10)]) for _ in range(T)]
    eps = [Fraction(0), Fraction(1, 10), Fraction(0), Fraction(1), Fraction(1, 1000), Fraction(0)][seed]
    S0 = [[fr() for _ in range(dv)] for _ in range(dk)]
    o_ref, S_ref = _brute_force(q, k, v, alpha, eta, eps, S0)
    f = lambda M: np.array([[float(x) for x in row] for row in M])
    o, ST = oracle.prefill(f(q)[:, None], f(k)[:, None], f(v)[:, None],
                           np.log(np.array([float(a) for a in alpha]))[:, None],
                           np.array([float(e) for e in eta])[:, None], float(eps),
                           S0=f(S0)[None, None])
    scale = max(np.max(np.abs(f(o_ref))), 1e-300)
    assert np.max(np.abs(o[:, 0] - f(o_ref))) <= 1e-12 * scale
    scaleS = max(np.max(np.abs(f(S_ref))), 1e-300)
    assert np.max(np.abs(ST[0, 0] - f(S_ref))) <= 1e-12 * scaleS


# --------------------------------------------------------------------------- tokenwise theory
def _step_states(q, k, v, g, eta, eps, S0):
    """Run the oracle one token at a time (decode) and return per-token (S~, S_t)."""
    S = S0.copy()
    out = []
    for t in range(k.shape[0]):
        S_tilde = math.exp(g[t, 0]) * S
        _, Sn = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], eta[t:t + 1], eps, S)
        out.append((S_tilde[0, 0], Sn[0, 0]))
        S = Sn
    return out


def test_hard_projection_constraint(oracle_lib):
    """eta = 1, a = 1, eps = 0: every write satisfies k_t S_t = v_t (Eq. (2), Theorem 1 / Eq. (11))."""
    rng = np.random.default_rng(1)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 96, 2, 16, 8)
    # q := k makes the readout o_t = k_t S_t
    o, _ = oracle.prefill(k, k, v, np.zeros_like(g), np.ones_like(eta), 0.0, S0=S0)
    assert _rel(o, v) < 1e-9


def test_relaxed_update_interpolates(oracle_lib):
    """Prop. 2 / Eq. (5), (17): k S_t = (1 - eta rho) k S~ + eta rho v, rho = |k|^2/(|k|^2+eps)."""
    rng = np.random.default_rng(2)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 24, 1, 8, 5)
    for eps in (0.0, 1e-6, 0.5, 30.0):
        for t, (St, Sn) in enumerate(_step_states(q, k, v, g, eta, eps, S0)):
            kt, vt, et = k[t, 0], v[t, 0], eta[t, 0]
            rho = kt @ kt / (kt @ kt + eps)
            want = (1 - et * rho) * (kt @ St) + et * rho * vt
            np.testing.assert_allclose(kt @ Sn, want, rtol=1e-11, atol=1e-11 * np.abs(vt).max())
            # residual contraction factor of Eq. (5)
            np.testing.assert_allclose(vt - kt @ Sn, (1 - et * rho) * (vt - kt @ St), rtol=1e-9,
                                       atol=1e-11 * np.abs(vt).max())


def test_proximal_optimality(oracle_lib):
    """Prop. 1: S_t minimises 1/2|S - S~|^2 + mu/2 |k S - v|^2, mu = eta/((1-eta)|k|^2 + eps).
    Its gradient (S - S~) + mu k^T (k S - v) vanishes at S_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 20, 1, 6, 4)
    eta = np.minimum(eta, 0.95)
    for eps in (0.0, 1e-3, 2.0):
        for t, (St, Sn) in enumerate(_step_states(q, k, v, g, eta, eps, S0)):
            kt, vt, et = k[t, 0], v[t, 0], eta[t, 0]
            mu = et / ((1 - et) * (kt @ kt) + eps)
            grad = (Sn - St) + mu * np.outer(kt, kt @ Sn - vt)
            assert np.max(np.abs(grad)) <= 1e-9 * max(1.0, np.max(np.abs(Sn - St)))


def test_rank_one_orthogonal_correction(oracle_lib):
    """Eq. (12): the correction S_t - S~ is k^T w and is Frobenius-orthogonal to every H with k H = 0;
    along S~ + tau k^T e the loss is 1/2 (1 - tau |k|^2)^2 |e|^2 (Eq. (4), (10))."""
    rng = np.random.default_rng(4)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 12, 1, 7, 3)
    for t, (St, Sn) in enumerate(_step_states(q, k, v, g, eta, 1e-6, S0)):
        kt = k[t, 0]
        D = Sn - St
        w = kt @ D / (kt @ kt)
        np.testing.assert_allclose(D, np.outer(kt, w), atol=1e-12 * np.abs(D).max())
        H = rng.standard_normal(D.shape)
        H -= np.outer(kt, kt @ H) / (kt @ kt)
        assert abs(np.sum(D * H)) <= 1e-10 * np.abs(D).sum() * np.abs(H).max()
        e = v[t, 0] - kt @ St
        for tau in (0.0, 0.3 / (kt @ kt), 1.0 / (kt @ kt), 1.7 / (kt @ kt)):
            loss = 0.5 * np.sum((kt @ (St + tau * np.outer(kt, e)) - v[t, 0]) ** 2)
            assert math.isclose(loss, 0.5 * (1 - tau * (kt @ kt)) ** 2 * (e @ e), rel_tol=1e-9,
                                abs_tol=1e-12)


def test_zero_key_means_no_write(oracle_lib):
    """|k|^2 + eps = 0 is read as b = 0: the state is only decayed."""
    rng = np.random.default_rng(5)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 3, 1, 4, 4)
    k[1] = 0.0
    out = _step_states(q, k, v, g, eta, 0.0, S0)
    St, Sn = out[1]
    np.testing.assert_array_equal(St, Sn)
    assert np.all(np.isfinite(Sn))


# --------------------------------------------------------------------------- closed forms
def test_one_hot_keys_closed_form(oracle_lib):
    """Keys c_t e_{i_t}: KLA reduces to independent per-slot updates.  Every row of S decays by
    a_t; the written row becomes (1 - rho) x + rho v / c with rho = eta c^2/(c^2 + eps)."""
    rng = np.random.default_rng(6)
    T, dk, dv = 3000, 8, 5
    slots = rng.integers(0, dk, size=T)
    c = 10.0 ** rng.uniform(-5, 1, size=T)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, slots] = c
    v = rng.standard_normal((T, 1, dv))
    q = rng.standard_normal((T, 1, dk))
    eta = rng.uniform(0.05, 1.0, size=(T, 1))
    g = rng.uniform(-0.05, 0.0, size=(T, 1))
    eps = 1e-6
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.prefill(q, k, v, g, eta, eps, S0=S0)
    X = S0[0, 0].copy()
    o_ref = np.zeros((T, dv))
    for t in range(T):
        X *= math.exp(g[t, 0])
        rho = eta[t, 0] * c[t] ** 2 / (c[t] ** 2 + eps)
        X[slots[t]] = (1 - rho) * X[slots[t]] + rho * v[t, 0] / c[t]
        o_ref[t] = q[t, 0] @ X
    assert _rel(ST[0, 0], X) < 1e-9
    assert _rel(o[:, 0], o_ref) < 1e-9


def test_classical_kaczmarz_orthonormal_sweep(oracle_lib):
    """a = 1, eta = 1, eps = 0, S0 = 0 and d_k orthonormal keys: one sweep gives S = sum k_i^T v_i
    (orthogonal rows are solved in one Kaczmarz sweep)."""
    rng = np.random.default_rng(7)
    dk, dv = 16, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, None, :]
    v = rng.standard_normal((dk, 1, dv))
    o, ST = oracle.prefill(k, k, v, np.zeros((dk, 1)), np.ones((dk, 1)), 0.0)
    np.testing.assert_allclose(ST[0, 0], Qm.T @ v[:, 0], atol=1e-12)


def test_key_scaling_invariance(oracle_lib):
    """eps = 0: (c_t k_t, v_t) writes the same state as (k_t, v_t / c_t) (Eq. (1)-(2):
    S^T (c k) = v  <=>  S^T k = v / c) -- the property that separates KLA from GDN."""
    rng = np.random.default_rng(8)
    q, k, v, g, eta, _, S0 = _rand_problem(rng, 50, 2, 8, 6)
    c = 10.0 ** rng.uniform(-2, 2, size=(50, 2, 1))
    o1, S1 = oracle.prefill(q, k * c, v, g, eta, 0.0, S0=S0)
    o2, S2 = oracle.prefill(q, k, v / c, g, eta, 0.0, S0=S0)
    assert _rel(S1, S2) < 1e-10
    assert _rel(o1, o2) < 1e-10


def test_linearity_in_state_and_values(oracle_lib):
    """For fixed K, g, eta the map (S0, V) -> (O, S_T) is linear (Eq. (7)-(9))."""
    rng = np.random.default_rng(9)
    q, k, v, g, eta, eps, S0 = _rand_problem(rng, 70, 2, 8, 4)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    a, b = 0.7, -1.9
    oA, SA = oracle.prefill(q, k, v, g, eta, eps, S0=S0)
    oB, SB = oracle.prefill(q, k, v2, g, eta, eps, S0=S02)
    oC, SC = oracle.prefill(q, k, a * v + b * v2, g, eta, eps, S0=a * S0 + b * S02)
    assert _rel(oC, a * oA + b * oB) < 1e-11
    assert _rel(SC, a * SA + b * SB) < 1e-11


# --------------------------------------------------------------------------- chunkwise == tokenwise
@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64, 200])
def test_tokenwise_equals_chunkwise(oracle_lib, chunk):
    """Props. 3-4: the chunkwise solve equals the tokenwise recurrence, for any chunk length
    (partial last chunks included) and across packed sequences."""
    rng = np.random.default_rng(10 + chunk)
    lens = [37, 1, 130]
    T = sum(lens)
    q, k, v, g, eta, eps, _ = _rand_problem(rng, T, 2, 8, 6)
    S0 = rng.standard_normal((3, 2, 8, 6))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ST = oracle.prefill(q, k, v, g, eta, eps, S0=S0, cu_seqlens=cu)
    oc, STc, _ = chunkwise.prefill(q, k, v, g, eta, eps, S0=S0, cu_seqlens=cu, chunk=chunk)
    assert _rel(oc, o) < 1e-11
    assert _rel(STc, ST) < 1e-11


def test_chunkwise_intermediates(oracle_lib):
    """b and G follow Eq. (3) and the inclusive log-decay sum; T = (I+L)^{-1} Diag(b) is lower
    triangular with diagonal b."""
    rng = np.random.default_rng(11)
    q, k, v, g, eta, eps, S0 = _rand_problem(rng, 64, 1, 8, 4)
    _, _, inter = chunkwise.prefill(q, k, v, g, eta, eps, S0=S0, chunk=64)
    d = inter[(0, 0, 0)]
    np.testing.assert_allclose(d["b"], eta[:, 0] / (np.sum(k[:, 0] ** 2, -1) + eps), rtol=1e-14)
    np.testing.assert_allclose(d["G"], np.cumsum(g[:, 0]), rtol=1e-13, atol=1e-15)
    assert np.all(np.triu(d["T"], 1) == 0)
    np.testing.assert_allclose(np.diag(d["T"]), d["b"], rtol=1e-14)


# --------------------------------------------------------------------------- chaining
def test_split_resume_and_decode_chain(oracle_lib):
    """prefill(T) == prefill(T1) then prefill(rest, S0=S_T1); prefill(T) + m decode steps ==
    prefill(T+m); packed == per-sequence calls."""
    rng = np.random.default_rng(12)
    q, k, v, g, eta, eps, S0 = _rand_problem(rng, 100, 2, 8, 5)
    o, ST = oracle.prefill(q, k, v, g, eta, eps, S0=S0)
    o1, S1 = oracle.prefill(q[:41], k[:41], v[:41], g[:41], eta[:41], eps, S0=S0)
    o2, S2 = oracle.prefill(q[41:], k[41:], v[41:], g[41:], eta[41:], eps, S0=S1)
    assert _rel(np.concatenate([o1, o2]), o) < 1e-13
    assert _rel(S2, ST) < 1e-13
    o3, S3 = oracle.prefill(q[:90], k[:90], v[:90], g[:90], eta[:90], eps, S0=S0)
    for t in range(90, 100):
        od, S3 = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], eta[t:t + 1], eps, S3)
        assert _rel(od, o[t:t + 1]) < 1e-12
    assert _rel(S3, ST) < 1e-12
    # packed vs per-sequence
    lens = [30, 0, 70]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0p = rng.standard_normal((3, 2, 8, 5))
    op, STp = oracle.prefill(q, k, v, g, eta, eps, S0=S0p, cu_seqlens=cu)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], eta[a:b], eps, S0=S0p[n:n + 1])
        assert np.array_equal(op[a:b], on)
        assert np.array_equal(STp[n:n + 1], Sn)
    np.testing.assert_array_equal(STp[1], S0p[1])  # empty sequence keeps its state
