"""Parity of the diagonal-gate backward pass (kla_prefill_backward with g per key channel,
paper Appendix B.5, through the C ABI) with the fp64 oracle's reverse-mode gradients of the
tokenwise recurrence S~ = Diag(exp(g_t)) S (oracle/backward.py).

Bars as for the scalar gate (per tensor, err = max|x - y| / max|y|): fp32 inputs 1e-4, bf16
inputs 2e-2.  dg is [n_tok, H, d_k].  The gradient kernel forms its per-channel decay
products on the matrix cores when every row's cumulative log-decay stays within 2^64 of the
chunk's row 32 on the 16 channels of an output tile, and term by term otherwise (and always
for fp32 inputs): the cases below cover both, and both in one call.
"""
import numpy as np
import pytest
import torch

import kla_inputs as ki
from oracle import backward as ob

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dg", "deta", "dS0")


def err(x, y):
    x = x.detach().double().cpu().numpy()
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    assert np.all(np.isfinite(x)), "non-finite values in device output"
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30))


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_delta_rule_kla_amd as m
    m.load_library()
    return m


def with_state(inp, seed):
    if inp["S0"] is None:  # give every case a nonzero incoming state
        gen = torch.Generator().manual_seed(seed)
        inp["S0"] = 0.3 * torch.randn(inp["n_seq"], inp["q"].shape[1], inp["k"].shape[-1],
                                      inp["v"].shape[-1], generator=gen)
    return inp


def run_case(kla, inp, ct, tol, **variant):
    assert inp["g"].shape == inp["k"].shape
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dev_variant = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in variant.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     cu_seqlens=d["cu_seqlens"], n_seq=d["n_seq"], **dev_variant)
    torch.cuda.synchronize()
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    f64 = lambda t: None if t is None else t.double().numpy()
    ov = {k: (v.numpy() if isinstance(v, torch.Tensor) else v) for k, v in variant.items()}
    ref = ob.prefill_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                              f64(inp["eta"]), inp["eps"], f64(ct["dO"]), S0=f64(inp["S0"]),
                              dS_T=f64(ct["dS_T"]), cu_seqlens=cu, n_seq=inp["n_seq"], **ov)
    for name, x, y in zip(NAMES, grads, ref):
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {tol:g})", flush=True)
        assert e < tol, f"{name}: err {e:.3e} >= {tol:g}"
    return grads


CASES = {
    # name: (workload, overrides, dtype override or None)
    "tiny_fp32_T256_d64": (0, dict(), None),
    "fp32_ragged_packed": (0, dict(lens=(150, 64, 5, 0, 1, 70), H=2), None),
    "fp32_d128_T200": (1, dict(T=200, n_seq=1, H=2), torch.float32),
    "bf16_d64_T260": (0, dict(T=260, H=2), torch.bfloat16),
    "bf16_d128_T300": (1, dict(T=300, n_seq=2, H=3), None),
    # g ~ U(-2, 0) per channel: many channels leave the 2^64 window within a chunk
    "bf16_packed_dv256_strong": (4, dict(lens=(100, 0, 200, 33), H=2), None),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_diagonal_backward_matches_oracle(kla, case):
    w, over, dt = CASES[case]
    inp = ki.prefill_inputs(w, diag=True, **over)
    if dt is not None:
        for name in ("q", "k", "v"):
            inp[name] = inp[name].to(dt).contiguous()
        inp["dtype"] = dt
    inp = with_state(inp, 7)
    ct = ki.cotangents(inp, seed=3000 + len(case))
    print(f"case {case}", flush=True)
    run_case(kla, inp, ct, TOL[inp["dtype"]])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_diagonal_backward_extreme_decay(kla, dtype):
    # log-decays down to -8 per token and channel: every tile takes the term-by-term path
    inp = ki.prefill_inputs(1, T=200, n_seq=1, H=2, diag=True)
    gen = torch.Generator().manual_seed(41)
    inp["g"] = (-8.0 * torch.rand(inp["g"].shape, generator=gen)).contiguous()
    for name in ("q", "k", "v"):
        inp[name] = inp[name].to(dtype).contiguous()
    inp["dtype"] = dtype
    inp = with_state(inp, 42)
    ct = ki.cotangents(inp, seed=43)
    print(f"extreme decay {dtype}", flush=True)
    run_case(kla, inp, ct, TOL[dtype])


def test_diagonal_backward_mixed_channel_decay(kla):
    # channels 0..47 decay slowly, 48..79 at up to -6 per token, the rest not at all: the
    # matrix-core and term-by-term paths run in one call, on tiles of one chunk
    inp = ki.prefill_inputs(1, T=256, n_seq=2, H=2, diag=True)
    gen = torch.Generator().manual_seed(51)
    g = -0.05 * torch.rand(inp["g"].shape, generator=gen)
    g[..., 48:80] = -6.0 * torch.rand(g[..., 48:80].shape, generator=gen)
    g[..., 80:] = 0.0
    inp["g"] = g.contiguous()
    inp = with_state(inp, 52)
    ct = ki.cotangents(inp, seed=53)
    run_case(kla, inp, ct, TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_diagonal_backward_variants(kla, dtype):
    # the 1/sqrt(t) coefficient with position offsets and the readout divided by ||q_t||
    # (one query row exactly zero), packed
    inp = ki.prefill_inputs(0, lens=(130, 61, 3), H=2, diag=True)
    q = inp["q"].clone()
    q[7] = 0.0
    inp["q"] = q.to(dtype).contiguous()
    inp["k"], inp["v"] = inp["k"].to(dtype).contiguous(), inp["v"].to(dtype).contiguous()
    inp["dtype"] = dtype
    inp = with_state(inp, 61)
    ct = ki.cotangents(inp, seed=62)
    pos = torch.tensor([5, 0, 300], dtype=torch.int32)
    print(f"variants {dtype}", flush=True)
    grads = run_case(kla, inp, ct, TOL[dtype], beta_mode="inv_sqrt_t", normalize_q=True,
                     pos_offset=pos)
    assert torch.count_nonzero(grads[0][7]) == 0


def test_diagonal_backward_gated_rule(kla):
    # the gated delta rule's b = eta (no key-norm dependence of b), unit-norm keys
    inp = ki.prefill_inputs(0, lens=(150, 40, 77), H=2, diag=True)
    kf = inp["k"].float()
    inp["k"] = (kf / kf.norm(dim=-1, keepdim=True)).contiguous()
    inp = with_state(inp, 71)
    ct = ki.cotangents(inp, seed=72)
    run_case(kla, inp, ct, TOL[torch.float32], beta_mode="gated")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_diagonal_backward_equal_channels_is_the_scalar_gate(kla, dtype):
    # a per-channel gate equal across channels is the scalar gate: the two backward paths
    # agree on dq, dk, dv, deta and dS0, and the scalar dg is the channels' dg summed
    inp = ki.prefill_inputs(1, T=320, n_seq=2, H=2)
    for name in ("q", "k", "v"):
        inp[name] = inp[name].to(dtype).contiguous()
    inp = with_state(inp, 81)
    ct = ki.cotangents(inp, seed=82)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    gd = d["g"][:, :, None].expand(-1, -1, d["k"].shape[-1]).contiguous()
    args = lambda g: (d["q"], d["k"], d["v"], g, d["eta"], d["eps"], ct["dO"].to(DEV))
    gs = kla.kla_prefill_backward(*args(d["g"]), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                  n_seq=d["n_seq"])
    gg = kla.kla_prefill_backward(*args(gd), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                  n_seq=d["n_seq"])
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for name, x, y in zip(NAMES, gg, gs):
        if name == "dg":
            x = x.sum(-1)
        e = err(x, y.double().cpu().numpy())
        print(f"  {name}: diagonal vs scalar {e:.3e} (bar {tol:g})", flush=True)
        assert e < tol, name


def test_diagonal_backward_full_workload_sampled(kla):
    # the prefill workload with g per key channel (4 x 4096 tokens x 16 heads, d = 128, bf16)
    # in the launch configuration bench.py times; two sampled (sequence, head) pairs
    inp = ki.prefill_inputs(1, diag=True)
    ct = ki.cotangents(inp, seed=2026)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     n_seq=d["n_seq"])
    torch.cuda.synchronize()
    T = inp["q"].shape[0] // inp["n_seq"]
    f64 = lambda t: t.double().numpy()
    for n, h in ((1, 3), (2, 14)):
        sl = slice(n * T, (n + 1) * T)
        pick = lambda t: f64(t[sl, h:h + 1])
        ref = ob.prefill_backward(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                  pick(inp["g"]), pick(inp["eta"]), inp["eps"], pick(ct["dO"]),
                                  S0=f64(inp["S0"][n:n + 1, h:h + 1]),
                                  dS_T=f64(ct["dS_T"][n:n + 1, h:h + 1]))
        got = [x[sl, h:h + 1] for x in grads[:5]] + [grads[5][n:n + 1, h:h + 1]]
        print(f"sequence {n}, head {h}", flush=True)
        for name, x, y in zip(NAMES, got, ref):
            e = err(x, y)
            print(f"  {name}: err {e:.3e} (bar {TOL[torch.bfloat16]:g})", flush=True)
            assert e < TOL[torch.bfloat16], f"{name}: err {e:.3e}"
