"""Pins of the oracle's diagonal-gated variant (CPU only).

Paper "Kaczmarz Linear Attention", Appendix B.5 ("Extension to diagonal gating"): the decay
becomes Diag(alpha_t), one factor per key channel, and the Kaczmarz coefficient is kept as
it is.  The tests tie the variant to (i) the scalar-gated oracle when every channel decays
alike, (ii) a closed form of the forget step, (iii) the projection properties of the write
(Eq. (2) / Theorem 1 and Eq. (5)), which hold whatever the decay, and (iv) an independent
chunkwise evaluation (oracle.chunkwise.prefill_diag).  Applying the decay to the value
columns instead of the key rows, reading the wrong token's decay, or leaving the decay out
of the residual fails one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import chunkwise


def draw(seed, T, H=2, dk=12, dv=7):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk)) * 10.0 ** rng.uniform(-1, 1, (T, H, 1))
    v = rng.standard_normal((T, H, dv))
    g = -rng.uniform(0.0, 0.6, (T, H, dk))          # one log-decay per key channel
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = 0.1 * rng.standard_normal((1, H, dk, dv))
    return q, k, v, g, eta, S0


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


def test_equal_channels_reduce_to_scalar_gating():
    q, k, v, g, eta, S0 = draw(0, 150)
    gs = g[:, :, 0]
    gd = np.repeat(gs[:, :, None], k.shape[-1], axis=2)
    o1, S1 = oracle.prefill(q, k, v, gs, eta, 1e-6, S0=S0)
    o2, S2 = oracle.prefill(q, k, v, gd, eta, 1e-6, S0=S0)
    assert rel(o2, o1) < 1e-13 and rel(S2, S1) < 1e-13
    d1 = oracle.decode(q[:1], k[:1], v[:1], gs[:1], eta[:1], 1e-6, S0)
    d2 = oracle.decode(q[:1], k[:1], v[:1], gd[:1], eta[:1], 1e-6, S0)
    assert rel(d2[0], d1[0]) < 1e-13 and rel(d2[1], d1[1]) < 1e-13


def test_forget_step_scales_key_rows():
    # eta = 0: no write, so one step is exactly S' = Diag(exp(g_t)) S (rows = key channels),
    # and the readout is q_t S'
    q, k, v, g, _, S0 = draw(1, 1, H=3, dk=9, dv=5)
    eta = np.zeros((1, 3))
    o, Sn = oracle.decode(q[0][None], k[0][None], v[0][None], g[0][None], eta, 1e-6, S0)
    want = np.exp(g[0])[:, :, None] * S0[0]
    assert rel(Sn[0], want) < 1e-15
    assert rel(o[0], np.einsum("hi,hij->hj", q[0], want)) < 1e-14


def test_hard_projection_under_diagonal_decay():
    # eta = 1, eps = 0, q := k: every write meets its constraint k_t S_t = v_t (Eq. (2)),
    # whatever the per-channel decay applied before it
    q, k, v, g, eta, S0 = draw(2, 80)
    o, _ = oracle.prefill(k, k, v, g, np.ones_like(eta), 0.0, S0=S0)
    assert rel(o, v) < 1e-9


def test_relaxed_step_under_diagonal_decay():
    # Eq. (5): k S_t = (1 - eta rho) k S~ + eta rho v with S~ = Diag(alpha_t) S_{t-1},
    # rho = |k|^2 / (|k|^2 + eps)
    q, k, v, g, eta, S0 = draw(3, 20, H=1, dk=8, dv=5)
    S = S0.copy()
    for eps in (0.0, 0.3):
        S = S0.copy()
        for t in range(20):
            _, Sn = oracle.decode(q[t][None], k[t][None], v[t][None], g[t][None], eta[t][None],
                                  eps, S)
            St = np.exp(g[t, 0])[:, None] * S[0, 0]
            kt, vt, et = k[t, 0], v[t, 0], eta[t, 0]
            rho = kt @ kt / (kt @ kt + eps)
            want = (1 - et * rho) * (kt @ St) + et * rho * vt
            np.testing.assert_allclose(kt @ Sn[0, 0], want, rtol=1e-11,
                                       atol=1e-11 * np.abs(vt).max())
            S = Sn


@pytest.mark.parametrize("chunk", [64, 16, 5])
def test_tokenwise_equals_chunkwise_diagonal(chunk):
    rng = np.random.default_rng(4)
    lens = [70, 1, 129, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    H, dk, dv = 2, 10, 6
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk)) * 10.0 ** rng.uniform(-1, 1, (T, H, 1))
    v = rng.standard_normal((T, H, dv))
    g = -rng.uniform(0.0, 2.0, (T, H, dk))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = 0.1 * rng.standard_normal((len(lens), H, dk, dv))
    o1, S1 = oracle.prefill(q, k, v, g, eta, 1e-6, S0=S0, cu_seqlens=cu)
    o2, S2 = chunkwise.prefill_diag(q, k, v, g, eta, 1e-6, S0=S0, cu_seqlens=cu, chunk=chunk)
    assert rel(o2, o1) < 1e-10 and rel(S2, S1) < 1e-10


def test_decode_chain_equals_prefill_diagonal():
    q, k, v, g, eta, S0 = draw(5, 12)
    o, ST = oracle.prefill(q, k, v, g, eta, 1e-6, S0=S0)
    S = S0.copy()
    for t in range(12):
        od, S = oracle.decode(q[t][None], k[t][None], v[t][None], g[t][None], eta[t][None],
                              1e-6, S)
        assert rel(od[0], o[t]) < 1e-12
    assert rel(S, ST) < 1e-12
