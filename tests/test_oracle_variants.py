"""Pins of the oracle's write-coefficient and readout variants (CPU only).

The variants are the pages' ablations of the coefficient (paper section 2 for the gated
delta rule's b_t = eta_t; Table 5 and Appendix D for key-norm only and the sequence
factors on the Kaczmarz coefficient, t the absolute position) and the readout divided by
||q_t|| (section 3.3, Algorithm 1's readout).  Each test ties a variant either to a closed
form or to the pinned default method under the substitution the variant's definition
implies, so that a wrong position base, a dropped eta or a misplaced norm fails.
"""
import math

import numpy as np
import pytest

import oracle


def draw(seed, T, H=2, dk=16, dv=8, unit_keys=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k *= 10.0 ** rng.uniform(-1, 1, (T, H, 1))
    v = rng.standard_normal((T, H, dv))
    g = -rng.uniform(0.0, 0.5, (T, H))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, eta


def close(a, b, tol=1e-11):
    a, b = np.asarray(a), np.asarray(b)
    assert np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b))), np.max(np.abs(a - b))


def test_gated_coefficient_closed_form():
    # orthogonal keys of norm 2, no decay: each write meets a state that has no component
    # along its key, so S_t = sum_s b_s k_s^T v_s and the read with q_t = k_t / 2 gives
    # o_t = 2 b_t v_t: b_t = eta_t for the gated rule, eta_t / 4 for the Kaczmarz step
    T, dk, dv = 6, 8, 3
    rng = np.random.default_rng(7)
    k = np.zeros((T, 1, dk))
    for t in range(T):
        k[t, 0, t] = 2.0
    q = k / 2.0
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1))
    eta = np.full((T, 1), 0.5)
    o_g, _ = oracle.prefill(q, k, v, g, eta, 0.0, beta_mode="gated")
    o_k, _ = oracle.prefill(q, k, v, g, eta, 0.0, beta_mode="kaczmarz")
    close(o_g, 2 * 0.5 * v)
    close(o_k, 2 * (0.5 / 4.0) * v)


def test_gated_equals_kaczmarz_on_unit_keys():
    q, k, v, g, eta = draw(1, 90, unit_keys=True)
    og, Sg = oracle.prefill(q, k, v, g, eta, 0.0, beta_mode="gated")
    ok, Sk = oracle.prefill(q, k, v, g, eta, 0.0, beta_mode="kaczmarz")
    close(og, ok)
    close(Sg, Sk)


def test_key_norm_is_kaczmarz_with_unit_eta():
    q, k, v, g, eta = draw(2, 90)
    on, Sn = oracle.prefill(q, k, v, g, eta, 1e-6, beta_mode="key_norm")
    ok, Sk = oracle.prefill(q, k, v, g, np.ones_like(eta), 1e-6, beta_mode="kaczmarz")
    close(on, ok)
    close(Sn, Sk)


@pytest.mark.parametrize("mode,factor", [("inv_t", lambda t: 1.0 / t),
                                         ("inv_sqrt_t", lambda t: 1.0 / math.sqrt(t)),
                                         ("inv_log_t", lambda t: 1.0 / math.log(t + 1.0))])
def test_sequence_factor_is_kaczmarz_with_scaled_eta(mode, factor):
    # two packed sequences; the first starts at absolute position 5 + 1, the second at 1
    q, k, v, g, eta = draw(3, 70 + 45)
    cu = np.array([0, 70, 115])
    pos = np.array([5, 0])
    om, Sm = oracle.prefill(q, k, v, g, eta, 1e-6, cu_seqlens=cu, beta_mode=mode, pos_offset=pos)
    eta2 = eta.copy()
    for n in range(2):
        for i in range(cu[n], cu[n + 1]):
            eta2[i] *= factor(pos[n] + (i - cu[n]) + 1)
    ok, Sk = oracle.prefill(q, k, v, g, eta2, 1e-6, cu_seqlens=cu, beta_mode="kaczmarz")
    close(om, ok)
    close(Sm, Sk)


def test_position_offset_continues_a_split_sequence():
    q, k, v, g, eta = draw(4, 100)
    o1, S1 = oracle.prefill(q, k, v, g, eta, 1e-6, beta_mode="inv_sqrt_t")
    oa, Sa = oracle.prefill(q[:60], k[:60], v[:60], g[:60], eta[:60], 1e-6, beta_mode="inv_sqrt_t")
    ob, Sb = oracle.prefill(q[60:], k[60:], v[60:], g[60:], eta[60:], 1e-6, S0=Sa,
                            beta_mode="inv_sqrt_t", pos_offset=np.array([60]))
    close(np.concatenate([oa, ob]), o1)
    close(Sb, S1)


def test_normalised_readout_divides_by_query_norm():
    q, k, v, g, eta = draw(5, 80)
    q[7, 1] = 0.0  # a zero query reads out zero
    on, Sn = oracle.prefill(q, k, v, g, eta, 1e-6, normalize_q=True)
    qn = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-300)
    ok, Sk = oracle.prefill(qn, k, v, g, eta, 1e-6)
    close(on, ok)
    close(Sn, Sk)  # the readout does not touch the state
    assert np.all(on[7, 1] == 0.0)


@pytest.mark.parametrize("mode", ["kaczmarz", "gated", "key_norm", "inv_t", "inv_sqrt_t",
                                  "inv_log_t"])
def test_decode_variant_matches_one_token_prefill(mode):
    rng = np.random.default_rng(6)
    B, H, dk, dv = 3, 2, 16, 8
    q, k, v, g, eta = draw(6, B, H, dk, dv, unit_keys=(mode == "gated"))
    S = 0.2 * rng.standard_normal((B, H, dk, dv))
    pos = np.array([0, 9, 40])
    od, Sd = oracle.decode(q, k, v, g, eta, 1e-6, S, beta_mode=mode, normalize_q=True,
                           pos_offset=pos)
    op, Sp = oracle.prefill(q, k, v, g, eta, 1e-6, S0=S, cu_seqlens=np.arange(B + 1),
                            beta_mode=mode, normalize_q=True, pos_offset=pos)
    close(od, op)
    close(Sd, Sp)
