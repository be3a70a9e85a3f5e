"""Seeded synthetic inputs for the KLA forward pass (shared by tests, smoke and bench).

This module only draws numbers: it holds none of the method's arithmetic.  The
same stored tensors feed the HIP library and, widened to float64, the oracle.

Workloads (value distributions follow the workload list of the benchmark
specification; the pages' own timing runs use a trained 0.4B model on
SlimPajama, which these synthetic tensors stand in for):

  0  tiny fp32      N=1, H=1,  T=256,   d_k=d_v=64,  S0=0
  1  layer bf16     N=4, H=16, T=4096,  d_k=d_v=128, S0 ~ N(0, var 0.01)
  2  long bf16      N=1, H=16, T=65536, d_k=d_v=128, unit keys x loguniform[0.5, 2]
  3  decode         B=256, H=16, d_k=d_v=128, fp32 state ~ N(0, var 0.05), 512 steps
  4  packed mixed   N=16, H=8, d_k=128, d_v=256, T_n ~ U{1024..16384}, g ~ U(-2, 0),
                    5% of keys rescaled to norm 10^U(-5,-3), then 128 decode steps

Common draws (unless a workload overrides them): q, k ~ N(0, 1) with every key
row multiplied by s = 10^U(-1, 1) (log-uniform in [0.1, 10]); v ~ N(0, 1);
eta = sigmoid(N(0, 1)); g ~ U(-0.5, 0); eps = 1e-6.  "N(0, s)" in the workload
list is read as variance s.  The seed is 42 + workload index.  Draws are made in
fp32 and cast to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BASE_SEED = 42


@dataclass
class Workload:
    index: int
    name: str
    n_seq: int
    H: int
    d_k: int
    d_v: int
    dtype: torch.dtype
    T: int = 0                       # dense length (0 = packed, see lens)
    lens: tuple = ()                 # packed lengths
    g_low: float = -0.5
    s0_var: float = 0.0
    key_mode: str = "loguniform"     # "loguniform" | "unit_loguniform"
    tiny_key_frac: float = 0.0
    eps: float = 1e-6
    decode_steps: int = 0
    extra: dict = field(default_factory=dict)


def _packed_lens(n: int, lo: int, hi: int, seed: int) -> tuple:
    gen = torch.Generator().manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen))


WORKLOADS = {
    0: Workload(0, "tiny-fp32-T256-d64", 1, 1, 64, 64, torch.float32, T=256),
    1: Workload(1, "prefill-bf16-B4-H16-T4096-d128", 4, 16, 128, 128, torch.bfloat16, T=4096,
                s0_var=0.01),
    2: Workload(2, "prefill-bf16-B1-H16-T65536-d128", 1, 16, 128, 128, torch.bfloat16, T=65536,
                key_mode="unit_loguniform"),
    3: Workload(3, "decode-B256-H16-d128-ctx32K", 256, 16, 128, 128, torch.bfloat16, T=1,
                s0_var=0.05, decode_steps=512),
    4: Workload(4, "packed-bf16-B16-H8-dk128-dv256", 16, 8, 128, 256, torch.bfloat16,
                lens=_packed_lens(16, 1024, 16384, BASE_SEED + 4), g_low=-2.0,
                tiny_key_frac=0.05, decode_steps=128),
}


def _gen(device, seed):
    return torch.Generator(device=device).manual_seed(int(seed))


def _keys(n_tok, H, dk, w: Workload, gen, device):
    k = torch.randn(n_tok, H, dk, generator=gen, device=device, dtype=torch.float32)
    if w.key_mode == "unit_loguniform":
        k = k / k.norm(dim=-1, keepdim=True)
        lo, hi = math.log10(0.5), math.log10(2.0)
    else:
        lo, hi = -1.0, 1.0
    s = 10.0 ** (lo + (hi - lo) * torch.rand(n_tok, H, 1, generator=gen, device=device))
    k = k * s
    if w.tiny_key_frac > 0:
        pick = torch.rand(n_tok, H, generator=gen, device=device) < w.tiny_key_frac
        target = 10.0 ** (-5.0 + 2.0 * torch.rand(n_tok, H, generator=gen, device=device))
        scale = target / k.norm(dim=-1)
        k = torch.where(pick[..., None], k * scale[..., None], k)
    return k


def prefill_inputs(w, device="cpu", seed=None, T=None, lens=None, n_seq=None, H=None,
                   diag=False):
    """Draw one prefill problem for workload ``w`` (a Workload or its index).

    Optional overrides shrink the problem (T for dense, lens for packed, n_seq, H)
    while keeping the workload's distributions.  Returns a dict with q, k, v
    ([n_tok, H, d]), g, eta ([n_tok, H] fp32), S0 ([n_seq, H, d_k, d_v] fp32 or
    None), cu_seqlens (int32 [n_seq+1] or None for dense), n_seq, eps, dtype.
    diag=True draws g per key channel ([n_tok, H, d_k], each entry from the workload's
    log-decay range) for the diagonal-gated variant.
    """
    if not isinstance(w, Workload):
        w = WORKLOADS[int(w)]
    seed = BASE_SEED + w.index if seed is None else seed
    Hh = w.H if H is None else H
    if lens is None and (w.lens and T is None):
        lens = w.lens if n_seq is None else w.lens[:n_seq]
    if lens is not None:
        lens = tuple(int(x) for x in lens)
        ns = len(lens)
        n_tok = sum(lens)
        cu = torch.zeros(ns + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    else:
        ns = w.n_seq if n_seq is None else n_seq
        Tt = w.T if T is None else T
        n_tok = ns * Tt
        cu = None
    gen = _gen(device, seed)
    q = torch.randn(n_tok, Hh, w.d_k, generator=gen, device=device)
    k = _keys(n_tok, Hh, w.d_k, w, gen, device)
    v = torch.randn(n_tok, Hh, w.d_v, generator=gen, device=device)
    eta = torch.sigmoid(torch.randn(n_tok, Hh, generator=gen, device=device))
    g = w.g_low * torch.rand(n_tok, Hh, generator=gen, device=device)
    if diag:
        g = w.g_low * torch.rand(n_tok, Hh, w.d_k, generator=gen, device=device)
    S0 = None
    if w.s0_var > 0:
        S0 = math.sqrt(w.s0_var) * torch.randn(ns, Hh, w.d_k, w.d_v, generator=gen, device=device)
    return dict(q=q.to(w.dtype).contiguous(), k=k.to(w.dtype).contiguous(),
                v=v.to(w.dtype).contiguous(), g=g.contiguous(), eta=eta.contiguous(),
                S0=S0, cu_seqlens=None if cu is None else cu.to(device), n_seq=ns, eps=w.eps,
                dtype=w.dtype)


def cotangents(inp: dict, seed: int, device="cpu") -> dict:
    """Seeded cotangents for a backward call on the inputs `inp`: dO ~ N(0, 1) shaped like
    the output o (in the inputs' dtype) and dS_T ~ N(0, 1) shaped like the final state
    (fp32)."""
    n_tok, H, _ = inp["q"].shape
    d_k, d_v = inp["k"].shape[-1], inp["v"].shape[-1]
    gen = _gen(device, seed)
    dO = torch.randn(n_tok, H, d_v, generator=gen, device=device)
    dST = torch.randn(inp["n_seq"], H, d_k, d_v, generator=gen, device=device)
    return dict(dO=dO.to(inp["q"].dtype).contiguous(), dS_T=dST.contiguous())


def hard_variant(inp: dict) -> dict:
    """Hard-projection variant: eta = 1, g = 0, eps = 0, and q := k (so o_t must equal v_t)."""
    out = dict(inp)
    out["eta"] = torch.ones_like(inp["eta"])
    out["g"] = torch.zeros_like(inp["g"])
    out["eps"] = 0.0
    out["q"] = inp["k"].clone()
    return out


def decode_inputs(w, steps=None, device="cpu", seed=None, B=None, H=None, S=None, diag=False):
    """Draw ``steps`` decode tokens per sequence plus a start state.

    Returns dict with q, k ([steps, B, H, d_k]), v ([steps, B, H, d_v]),
    g, eta ([steps, B, H] fp32), S ([B, H, d_k, d_v] fp32, drawn with the
    workload's state variance unless given), eps, dtype.  diag=True: g is [steps, B, H, d_k].
    """
    if not isinstance(w, Workload):
        w = WORKLOADS[int(w)]
    seed = BASE_SEED + w.index + 1000 if seed is None else seed
    steps = w.decode_steps if steps is None else steps
    Bb = w.n_seq if B is None else B
    Hh = w.H if H is None else H
    gen = _gen(device, seed)
    n = steps * Bb
    q = torch.randn(n, Hh, w.d_k, generator=gen, device=device)
    k = _keys(n, Hh, w.d_k, w, gen, device)
    v = torch.randn(n, Hh, w.d_v, generator=gen, device=device)
    eta = torch.sigmoid(torch.randn(n, Hh, generator=gen, device=device))
    g = w.g_low * torch.rand(n, Hh, generator=gen, device=device)
    if diag:
        g = w.g_low * torch.rand(n, Hh, w.d_k, generator=gen, device=device)
    if S is None:
        var = w.s0_var if w.s0_var > 0 else 0.05
        S = math.sqrt(var) * torch.randn(Bb, Hh, w.d_k, w.d_v, generator=gen, device=device)
    shp = lambda x, d: x.reshape(steps, Bb, Hh, d) if d else x.reshape(steps, Bb, Hh)
    return dict(q=shp(q.to(w.dtype), w.d_k).contiguous(), k=shp(k.to(w.dtype), w.d_k).contiguous(),
                v=shp(v.to(w.dtype), w.d_v).contiguous(),
                g=(shp(g, w.d_k) if diag else shp(g, 0)).contiguous(),
                eta=shp(eta, 0).contiguous(), S=S.contiguous(), eps=w.eps, dtype=w.dtype)
