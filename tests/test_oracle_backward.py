"""Pins of the fp64 backward oracle (oracle/backward.py), all on the CPU.

The gradients come from automatic differentiation of the tokenwise recurrence, so they are
pinned against things that do not use it: central differences of the C oracle's forward
pass, a one-token closed form worked by hand from Algorithm 1 and Eq. (3), the invariance of
the write under scaling (k_t, v_t) together at eps = 0 (Eq. (1)-(2)), and the closed form
of a sequence with no writes.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob


def draw(seed, n_tok, H=2, dk=4, dv=3, n_seq=1, g_low=-0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_tok, H, dk))
    k = rng.standard_normal((n_tok, H, dk)) * 10.0 ** rng.uniform(-0.5, 0.5, (n_tok, H, 1))
    v = rng.standard_normal((n_tok, H, dv))
    g = rng.uniform(g_low, 0.0, (n_tok, H))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((n_tok, H))))
    S0 = 0.3 * rng.standard_normal((n_seq, H, dk, dv))
    dO = rng.standard_normal((n_tok, H, dv))
    dST = rng.standard_normal((n_seq, H, dk, dv))
    return q, k, v, g, eta, S0, dO, dST


def loss_c(q, k, v, g, eta, eps, S0, dO, dST, cu=None):
    """<dO, O> + <dS_T, S_T> from the C oracle's forward pass."""
    O, ST = oracle.prefill(q, k, v, g, eta, eps, S0=S0, cu_seqlens=cu)
    return float((O * dO).sum() + (ST * dST).sum())


def test_forward_matches_c_oracle():
    q, k, v, g, eta, S0, _, _ = draw(0, 40, H=3, dk=5, dv=4, n_seq=2)
    cu = np.array([0, 17, 40])
    O1, S1 = ob.prefill_forward(q, k, v, g, eta, 1e-6, S0=S0, cu_seqlens=cu)
    O2, S2 = oracle.prefill(q, k, v, g, eta, 1e-6, S0=S0, cu_seqlens=cu)
    assert np.abs(O1 - O2).max() < 1e-12 * np.abs(O2).max()
    assert np.abs(S1 - S2).max() < 1e-12 * np.abs(S2).max()


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_gradients_match_central_differences_of_c_oracle(eps):
    # every input element of a small packed case (two sequences, one of length 1)
    q, k, v, g, eta, S0, dO, dST = draw(1, 7, H=2, dk=3, dv=2, n_seq=2)
    cu = np.array([0, 6, 7])
    grads = ob.prefill_backward(q, k, v, g, eta, eps, dO, S0=S0, dS_T=dST, cu_seqlens=cu)
    inputs = [q, k, v, g, eta, S0]
    h = 1e-6
    for which, (x, gx) in enumerate(zip(inputs, grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in inputs]
            xm = [a.copy() for a in inputs]
            xp[which][idx] += h
            xm[which][idx] -= h
            num[idx] = (loss_c(*xp[:5], eps, xp[5], dO, dST, cu) -
                        loss_c(*xm[:5], eps, xm[5], dO, dST, cu)) / (2 * h)
        err = np.abs(num - gx).max() / max(np.abs(num).max(), 1e-300)
        assert err < 1e-6, (which, err)


def test_one_token_closed_form():
    # S0 = 0, one token: S_1 = b k^T v and o = b (q.k) v, so with
    # c = (q.k)(v.dO) + k dS_T v^T  (the loss divided by b):
    #   dv = b ((q.k) dO + k dS_T),   dq = b (v.dO) k,   deta = c / den,   dg = 0,
    #   dk = b ((v.dO) q + dS_T v^T) - 2 b c k / den,    den = ||k||^2 + eps
    q, k, v, g, eta, _, dO, dST = draw(2, 1, H=3, dk=4, dv=5)
    eps = 0.25
    grads = ob.prefill_backward(q, k, v, g, eta, eps, dO, S0=None, dS_T=dST)
    for h in range(3):
        qh, kh, vh, oh, Sh = q[0, h], k[0, h], v[0, h], dO[0, h], dST[0, h]
        den = kh @ kh + eps
        b = eta[0, h] / den
        c = (qh @ kh) * (vh @ oh) + kh @ Sh @ vh
        want = {
            "dq": b * (vh @ oh) * kh,
            "dk": b * ((vh @ oh) * qh + Sh @ vh) - 2 * b * c * kh / den,
            "dv": b * ((qh @ kh) * oh + kh @ Sh),
            "dg": 0.0,
            "deta": c / den,
        }
        got = {"dq": grads[0][0, h], "dk": grads[1][0, h], "dv": grads[2][0, h],
               "dg": grads[3][0, h], "deta": grads[4][0, h]}
        for key in want:
            assert np.allclose(got[key], want[key], rtol=1e-12, atol=1e-14), key
    assert np.abs(grads[5]).max() > 0  # dS0 is the state gradient, decayed by exp(g)


def test_key_scale_invariance_at_zero_eps():
    # at eps = 0 the write of token t depends on (k_t, v_t) only through the constraint
    # k_t S = v_t (Eq. (1)-(2)), which scaling both by c leaves unchanged; the derivative
    # along that direction vanishes: k_t . dk_t + v_t . dv_t = 0 for every token-head
    q, k, v, g, eta, S0, dO, dST = draw(3, 30, H=2, dk=4, dv=3)
    _, dk, dv, _, _, _ = ob.prefill_backward(q, k, v, g, eta, 0.0, dO, S0=S0, dS_T=dST)
    proj = np.einsum("thi,thi->th", k, dk) + np.einsum("thi,thi->th", v, dv)
    scale = np.abs(np.einsum("thi,thi->th", v, dv)).max()
    assert np.abs(proj).max() < 1e-11 * scale


def test_state_gradient_through_zero_write():
    # eta = 0: no write, so S_T = exp(sum g) S0 and O_t = exp(G_t) q_t S0; then
    # dS0 = exp(G_T) dS_T + sum_t exp(G_t) q_t^T dO_t and dg_t = sum_{s >= t} of the loss terms
    q, k, v, g, _, S0, dO, dST = draw(4, 6, H=1, dk=3, dv=2)
    eta = np.zeros((6, 1))
    dq, dk, dv, dg, deta, dS0 = ob.prefill_backward(q, k, v, g, eta, 1e-6, dO, S0=S0, dS_T=dST)
    G = np.cumsum(g[:, 0])
    want = np.exp(G[-1]) * dST[0, 0] + sum(
        np.exp(G[t]) * np.outer(q[t, 0], dO[t, 0]) for t in range(6))
    assert np.allclose(dS0[0, 0], want, rtol=1e-12)
    terms = np.array([np.exp(G[t]) * q[t, 0] @ S0[0, 0] @ dO[t, 0] for t in range(6)])
    final = np.exp(G[-1]) * (S0[0, 0] * dST[0, 0]).sum()
    want_dg = np.array([terms[t:].sum() + final for t in range(6)])
    assert np.allclose(dg[:, 0], want_dg, rtol=1e-12)
    assert np.abs(dv).max() == 0.0


def test_packed_equals_per_sequence():
    q, k, v, g, eta, S0, dO, dST = draw(5, 25, H=2, dk=3, dv=3, n_seq=2)
    cu = np.array([0, 11, 25])
    packed = ob.prefill_backward(q, k, v, g, eta, 1e-6, dO, S0=S0, dS_T=dST, cu_seqlens=cu)
    for n in range(2):
        s, e = cu[n], cu[n + 1]
        one = ob.prefill_backward(q[s:e], k[s:e], v[s:e], g[s:e], eta[s:e], 1e-6, dO[s:e],
                                  S0=S0[n:n + 1], dS_T=dST[n:n + 1])
        for a, b in zip(packed[:5], one[:5]):
            assert np.allclose(a[s:e], b, rtol=1e-13, atol=1e-15)
        assert np.allclose(packed[5][n], one[5][0], rtol=1e-13)


def test_dense_sequences_equal_packed():
    q, k, v, g, eta, S0, dO, dST = draw(6, 24, H=2, dk=3, dv=2, n_seq=3)
    dense = ob.prefill_backward(q, k, v, g, eta, 1e-6, dO, S0=S0, dS_T=dST, n_seq=3)
    packed = ob.prefill_backward(q, k, v, g, eta, 1e-6, dO, S0=S0, dS_T=dST,
                                 cu_seqlens=np.array([0, 8, 16, 24]))
    for a, b in zip(dense, packed):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["gated", "key_norm", "inv_t", "inv_sqrt_t", "inv_log_t"])
def test_variant_gradients_match_central_differences(mode):
    # the coefficient variants, each against central differences of the C oracle run in the
    # same mode (packed, with position offsets for the sequence factors)
    q, k, v, g, eta, S0, dO, dST = draw(7, 5, H=2, dk=3, dv=2, n_seq=2)
    cu = np.array([0, 3, 5])
    pos = np.array([4, 0], dtype=np.int32)
    eps = 0.1
    grads = ob.prefill_backward(q, k, v, g, eta, eps, dO, S0=S0, dS_T=dST, cu_seqlens=cu,
                                beta_mode=mode, pos_offset=pos)

    def loss(xs):
        O, ST = oracle.prefill(*xs[:5], eps, S0=xs[5], cu_seqlens=cu, beta_mode=mode,
                               pos_offset=pos)
        return float((O * dO).sum() + (ST * dST).sum())
    inputs = [q, k, v, g, eta, S0]
    h = 1e-6
    for which, (x, gx) in enumerate(zip(inputs, grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in inputs]
            xm = [a.copy() for a in inputs]
            xp[which][idx] += h
            xm[which][idx] -= h
            num[idx] = (loss(xp) - loss(xm)) / (2 * h)
        err = np.abs(num - gx).max() / max(np.abs(num).max(), 1e-300)
        assert err < 1e-6, (mode, which, err)
    if mode == "key_norm":
        assert np.abs(grads[4]).max() == 0.0  # b does not depend on eta


def test_normalised_readout_gradients_match_central_differences():
    # o_t = q_t S_t / ||q_t|| against central differences of the C oracle's normalised readout
    q, k, v, g, eta, S0, dO, dST = draw(8, 6, H=2, dk=3, dv=2, n_seq=2)
    cu = np.array([0, 4, 6])
    grads = ob.prefill_backward(q, k, v, g, eta, 0.2, dO, S0=S0, dS_T=dST, cu_seqlens=cu,
                                normalize_q=True)

    def loss(xs):
        O, ST = oracle.prefill(*xs[:5], 0.2, S0=xs[5], cu_seqlens=cu, normalize_q=True)
        return float((O * dO).sum() + (ST * dST).sum())
    inputs = [q, k, v, g, eta, S0]
    h = 1e-6
    for which, (x, gx) in enumerate(zip(inputs, grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in inputs]
            xm = [a.copy() for a in inputs]
            xp[which][idx] += h
            xm[which][idx] -= h
            num[idx] = (loss(xp) - loss(xm)) / (2 * h)
        err = np.abs(num - gx).max() / max(np.abs(num).max(), 1e-300)
        assert err < 1e-6, (which, err)
    # the readout depends on q_t only through its direction: q_t . dq_t = 0
    assert np.abs(np.einsum("thi,thi->th", q, grads[0])).max() < 1e-12 * np.abs(grads[0]).max()


def test_normalised_readout_zero_query():
    # a zero query reads out 0; its gradient is taken as 0 (the direction is undefined there)
    q, k, v, g, eta, S0, dO, dST = draw(9, 5, H=1, dk=3, dv=2)
    q[2] = 0.0
    dq = ob.prefill_backward(q, k, v, g, eta, 1e-6, dO, S0=S0, dS_T=dST, normalize_q=True)[0]
    assert np.all(np.isfinite(dq)) and np.abs(dq[2]).max() == 0.0
    assert np.abs(dq[1]).max() > 0


def draw_diag(seed, n_tok, H=2, dk=3, dv=2, n_seq=1):
    """draw() with one log-decay per key channel (diagonal gating), channels decaying at
    rates that differ by an order of magnitude"""
    q, k, v, _, eta, S0, dO, dST = draw(seed, n_tok, H=H, dk=dk, dv=dv, n_seq=n_seq)
    rng = np.random.default_rng(seed + 1000)
    g = rng.uniform(-1.0, 0.0, (n_tok, H, dk)) * 10.0 ** rng.uniform(-1.0, 0.0, (1, 1, dk))
    return q, k, v, g, eta, S0, dO, dST


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_diagonal_gate_gradients_match_central_differences(eps):
    # Appendix B.5: every input element of a small packed case against central differences of
    # the C oracle's diagonal-gate forward pass (g per key channel)
    q, k, v, g, eta, S0, dO, dST = draw_diag(11, 7, H=2, dk=3, dv=2, n_seq=2)
    cu = np.array([0, 5, 7])
    grads = ob.prefill_backward(q, k, v, g, eta, eps, dO, S0=S0, dS_T=dST, cu_seqlens=cu)
    assert grads[3].shape == g.shape
    inputs = [q, k, v, g, eta, S0]
    h = 1e-6
    for which, (x, gx) in enumerate(zip(inputs, grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in inputs]
            xm = [a.copy() for a in inputs]
            xp[which][idx] += h
            xm[which][idx] -= h
            num[idx] = (loss_c(*xp[:5], eps, xp[5], dO, dST, cu) -
                        loss_c(*xm[:5], eps, xm[5], dO, dST, cu)) / (2 * h)
        err = np.abs(num - gx).max() / max(np.abs(num).max(), 1e-300)
        assert err < 1e-6, (which, err)


def test_diagonal_gate_with_equal_channels_is_the_scalar_gate():
    # a per-channel gate equal across channels is the scalar gate (Appendix B.5 with
    # Diag(alpha_t) = alpha_t I): the same gradients of q, k, v, eta and S0, and the scalar
    # gate's dg_t is the sum of the channels' dg_t (chain rule through g_t -> (g_t, .., g_t))
    q, k, v, g, eta, S0, dO, dST = draw(12, 9, H=2, dk=4, dv=3, n_seq=1)
    gd = np.repeat(g[:, :, None], 4, axis=2)
    gs = ob.prefill_backward(q, k, v, g, eta, 1e-3, dO, S0=S0, dS_T=dST)
    gdg = ob.prefill_backward(q, k, v, gd, eta, 1e-3, dO, S0=S0, dS_T=dST)
    for which in (0, 1, 2, 4, 5):
        assert np.abs(gs[which] - gdg[which]).max() < 1e-12 * np.abs(gs[which]).max()
    assert np.abs(gdg[3].sum(-1) - gs[3]).max() < 1e-12 * np.abs(gs[3]).max()


def test_diagonal_gate_dead_channel_blocks_the_state():
    # a channel whose gate is -inf at the first token forgets row c of S0 before anything
    # reads it (Diag(alpha_1) with alpha_{1,c} = 0), so the gradients of that row of S0
    # vanish, while the other rows keep theirs
    q, k, v, g, eta, S0, dO, dST = draw_diag(13, 6, H=1, dk=3, dv=2)
    g[0, 0, 1] = -np.inf
    dS0 = ob.prefill_backward(q, k, v, g, eta, 1e-3, dO, S0=S0, dS_T=dST)[5]
    assert np.abs(dS0[0, 0, 1]).max() == 0.0
    assert np.abs(dS0[0, 0, 0]).max() > 0 and np.abs(dS0[0, 0, 2]).max() > 0
