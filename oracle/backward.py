"""fp64 gradients of the KLA prefill -- TEST INFRASTRUCTURE ONLY (parity oracle).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this module; the HIP library shares no code with it.

The paper ("Kaczmarz Linear Attention", arXiv 2605.08587) trains with the chunkwise
algorithm but derives no backward pass.  The gradients here are those of the tokenwise
recurrence of Algorithm 1 (left panel) with the coefficient of Eq. (3), taken by reverse-mode
automatic differentiation in plain PyTorch CPU ops in float64:

    a_t = exp(g_t),  S~ = a_t S_{t-1},  e_t = v_t - k_t S~,
    b_t = eta_t / (||k_t||^2 + eps)  (0 when that denominator is 0),
    S_t = S~ + b_t k_t^T e_t,  o_t = q_t S_t,

for the scalar loss  L = <dO, O> + <dS_T, S_T>, so that the returned tensors are the
vector-Jacobian products (dq, dk, dv, dg, deta, dS0) of the forward map
(q, k, v, g, eta, S0) -> (O, S_T) with the cotangents (dO, dS_T).  Sequences are independent;
packed input follows ``cu_seqlens`` as in the forward oracle.  The coefficient variants of
the forward oracle are covered (``beta_mode``: the gated delta rule's b_t = eta_t, section 2;
key-norm only b_t = 1/(||k_t||^2 + eps) and the sequence factors 1/t, 1/sqrt(t),
1/log(t + 1) on the Kaczmarz coefficient, Appendix D and Table 5; t the absolute 1-based
position, sequence n starting at pos_offset[n] + 1) and the readout divided by ||q_t||
(section 3.3; 0 for a zero query), with one scalar gate per token-head, or one gate per key
channel (Appendix B.5, diagonal gating: g of shape [n_tok, H, d_k], S~ = Diag(exp(g_t)) S_{t-1},
the rows of S being key channels).
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


MODES = ("kaczmarz", "gated", "key_norm", "inv_t", "inv_sqrt_t", "inv_log_t")


def _coef(mode, eta_t, den, pos):
    """b_t for one token of every head; a zero denominator gives 0 wherever b_t divides by it."""
    if mode == "gated":
        return eta_t
    nz = den != 0
    rden = torch.where(nz, 1.0 / torch.where(nz, den, torch.ones_like(den)), torch.zeros_like(den))
    if mode == "key_norm":
        return rden
    b = eta_t * rden
    if mode == "inv_t":
        b = b / pos
    elif mode == "inv_sqrt_t":
        b = b / np.sqrt(pos)
    elif mode == "inv_log_t":
        b = b / np.log(pos + 1.0)
    elif mode != "kaczmarz":
        raise ValueError(f"unknown beta_mode {mode}")
    return b


def _sequence(q, k, v, g, eta, eps, S0, mode="kaczmarz", pos0=0, normalize_q=False):
    """The tokenwise recurrence over one sequence, all heads at once: (O [T, H, dv], S_T).
    Token t of the sequence is at absolute position pos0 + t + 1."""
    S = S0
    outs = []
    for t in range(q.shape[0]):
        kt, qt = k[t], q[t]                                   # [H, dk]
        a = torch.exp(g[t])                                   # [H], or [H, dk] per key channel
        den = (kt * kt).sum(-1) + eps                         # [H]
        b = _coef(mode, eta[t], den, float(pos0 + t + 1))
        St = (a[:, :, None] if a.dim() == 2 else a[:, None, None]) * S   # forget
        e = v[t] - torch.einsum("hi,hij->hj", kt, St)         # residual
        S = St + b[:, None, None] * kt[:, :, None] * e[:, None, :]   # Kaczmarz write
        if normalize_q:                                       # readout q_t / ||q_t||
            qq = (qt * qt).sum(-1)                            # a zero query reads out 0, with
            nzq = qq > 0                                      # a zero gradient
            r = torch.where(nzq, 1.0 / torch.where(nzq, qq, torch.ones_like(qq)).sqrt(),
                            torch.zeros_like(qq))
            qt = qt * r[:, None]
        outs.append(torch.einsum("hi,hij->hj", qt, S))        # readout
    O = torch.stack(outs) if outs else q.new_zeros((0,) + v.shape[1:])
    return O, S


def prefill_backward(q, k, v, g, eta, eps, dO, S0=None, dS_T=None, cu_seqlens=None, n_seq=1,
                     beta_mode="kaczmarz", pos_offset=None, normalize_q=False):
    """Gradients of the prefill for the cotangents dO [n_tok, H, dv] and dS_T [n_seq, H, dk, dv].

    Inputs as for :func:`oracle.prefill` (q, k [n_tok, H, dk]; v [n_tok, H, dv];
    g, eta [n_tok, H], or g [n_tok, H, dk] for diagonal gating; S0 [n_seq, H, dk, dv] or
    None = zeros; dS_T None = zeros);
    without cu_seqlens the tokens are n_seq sequences of equal length.  beta_mode,
    pos_offset ([n_seq] or None) and normalize_q select the variant as in the forward oracle.
    Returns numpy float64 arrays (dq, dk, dv, dg, deta, dS0), shaped like the inputs.
    """
    q, k, v, g, eta, dO = (_t(x) for x in (q, k, v, g, eta, dO))
    n_tok, H, dk = q.shape
    dv_ = v.shape[-1]
    if cu_seqlens is None:
        if n_tok % n_seq:
            raise ValueError("dense input needs n_tok divisible by n_seq")
        cu = np.arange(n_seq + 1, dtype=np.int64) * (n_tok // n_seq)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    n_seq = len(cu) - 1
    S0 = torch.zeros(n_seq, H, dk, dv_, dtype=torch.float64) if S0 is None else _t(S0)
    dS_T = torch.zeros(n_seq, H, dk, dv_, dtype=torch.float64) if dS_T is None else _t(dS_T)
    for x in (q, k, v, g, eta, S0):
        x.requires_grad_(True)
    loss = q.new_zeros(())
    for n in range(n_seq):
        s, e = int(cu[n]), int(cu[n + 1])
        pos0 = 0 if pos_offset is None else int(pos_offset[n])
        O, ST = _sequence(q[s:e], k[s:e], v[s:e], g[s:e], eta[s:e], float(eps), S0[n],
                          beta_mode, pos0, normalize_q)
        loss = loss + (O * dO[s:e]).sum() + (ST * dS_T[n]).sum()
    grads = torch.autograd.grad(loss, (q, k, v, g, eta, S0), allow_unused=True)
    out = []
    for x, gr in zip((q, k, v, g, eta, S0), grads):
        out.append(np.zeros(tuple(x.shape)) if gr is None else gr.detach().numpy())
    return tuple(out)


def prefill_forward(q, k, v, g, eta, eps, S0=None, cu_seqlens=None):
    """The same recurrence's forward values (O, S_T) in float64 (used to pin this module
    against the C oracle)."""
    q, k, v, g, eta = (_t(x) for x in (q, k, v, g, eta))
    n_tok, H, dk = q.shape
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens)
    n_seq = len(cu) - 1
    S0 = torch.zeros(n_seq, H, dk, v.shape[-1], dtype=torch.float64) if S0 is None else _t(S0)
    Os, Ss = [], []
    with torch.no_grad():
        for n in range(n_seq):
            s, e = int(cu[n]), int(cu[n + 1])
            O, ST = _sequence(q[s:e], k[s:e], v[s:e], g[s:e], eta[s:e], float(eps), S0[n])
            Os.append(O)
            Ss.append(ST)
    return torch.cat(Os).numpy(), torch.stack(Ss).numpy()
