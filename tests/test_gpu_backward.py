"""Parity of the backward pass (kla_prefill_backward, through the C ABI) with the fp64
oracle's reverse-mode gradients of the tokenwise recurrence (oracle/backward.py), on seeded
inputs and cotangents.

Bars (per tensor, err = max|x - y| / max|y| with y the oracle), for each of dq, dk, dv, dg,
deta and dS0, the forward's bars: fp32 inputs 1e-4; bf16 inputs 2e-2 (dq, dk, dv are rounded
to bf16 on output, and the stored forward tiles T and P are bf16).  The last test runs the
full prefill workload (4 sequences x 4096 tokens x 16 heads, d = 128, bf16) in the launch
configuration bench.py times and checks two sampled (sequence, head) pairs: sequences and
heads are independent, so the oracle runs on those alone.
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


def run_case(kla, inp, ct, tol, with_state=True, with_dst=True):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    S0 = d["S0"] if with_state else None
    dST = ct["dS_T"].to(DEV) if with_dst else None
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=S0, dS_T=dST,
                                     cu_seqlens=d["cu_seqlens"], n_seq=d["n_seq"])
    torch.cuda.synchronize()
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    f64 = lambda t: None if t is None else t.double().numpy()
    ref = ob.prefill_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                              f64(inp["eta"]), inp["eps"], f64(ct["dO"]),
                              S0=f64(inp["S0"]) if with_state else None,
                              dS_T=f64(ct["dS_T"]) if with_dst else None, cu_seqlens=cu,
                              n_seq=inp["n_seq"])
    for name, x, y in zip(NAMES, grads, ref):
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {tol:g})", flush=True)
        assert e < tol, f"{name}: err {e:.3e} >= {tol:g}"


CASES = {
    # name: (workload, overrides, dtype override or None)
    "tiny_fp32_T256_d64": (0, dict(), None),
    "fp32_ragged_packed": (0, dict(lens=(150, 64, 5, 0, 1, 70), H=2), None),
    "fp32_d128_T200": (1, dict(T=200, n_seq=1, H=2), torch.float32),
    "bf16_d64_T260": (0, dict(T=260, H=2), torch.bfloat16),
    "bf16_d128_T300": (1, dict(T=300, n_seq=2, H=3), None),
    "bf16_packed_dv256": (4, dict(lens=(100, 0, 200, 33), H=2), None),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_matches_oracle(kla, case):
    w, over, dt = CASES[case]
    inp = ki.prefill_inputs(w, **over)
    if dt is not None:
        for name in ("q", "k", "v"):
            inp[name] = inp[name].to(dt).contiguous()
        inp["dtype"] = dt
    if inp["S0"] is None:  # give every case a nonzero incoming state
        gen = torch.Generator().manual_seed(7)
        inp["S0"] = 0.3 * torch.randn(inp["n_seq"], inp["q"].shape[1], inp["k"].shape[-1],
                                      inp["v"].shape[-1], generator=gen)
    ct = ki.cotangents(inp, seed=1000 + len(case))
    print(f"case {case}", flush=True)
    run_case(kla, inp, ct, TOL[inp["dtype"]])


def test_backward_without_state_or_final_cotangent(kla):
    inp = ki.prefill_inputs(0, T=200)
    ct = ki.cotangents(inp, seed=5)
    run_case(kla, inp, ct, TOL[torch.float32], with_state=False, with_dst=False)


def test_backward_strong_decay(kla):
    # log-decays down to -8 per token: exp(G) spans many decades inside one chunk
    inp = ki.prefill_inputs(0, T=192)
    gen = torch.Generator().manual_seed(9)
    inp["g"] = (-8.0 * torch.rand(inp["g"].shape, generator=gen)).contiguous()
    ct = ki.cotangents(inp, seed=6)
    run_case(kla, inp, ct, TOL[torch.float32])


def test_backward_beyond_2g_elements(kla):
    """Packed input whose second sequence starts past element 2^31 of q, k, v, dO and the
    gradients (8,388,736 + 200 tokens x 2 heads x d = 128, bf16): the far sequence's
    gradients against the oracle (sequences are independent)."""
    L0, L1, H = 8388736, 200, 2
    assert L0 * H * 128 > 2 ** 31
    w = ki.Workload(99, "far", 2, H, 128, 128, torch.bfloat16, lens=(L0, L1), s0_var=0.01)
    inp = ki.prefill_inputs(w, device=DEV)
    ct = ki.cotangents(inp, seed=4242, device=DEV)
    grads = kla.kla_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["eta"],
                                     inp["eps"], ct["dO"], S0=inp["S0"], dS_T=ct["dS_T"],
                                     cu_seqlens=inp["cu_seqlens"], n_seq=2)
    torch.cuda.synchronize()
    sl = slice(L0, L0 + L1)
    f64 = lambda t: t.double().cpu().numpy()
    pick = lambda t: f64(t[sl])
    ref = ob.prefill_backward(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"]),
                              pick(inp["eta"]), inp["eps"], pick(ct["dO"]),
                              S0=f64(inp["S0"][1:2]), dS_T=f64(ct["dS_T"][1:2]))
    got = [x[sl] for x in grads[:5]] + [grads[5][1:2]]
    for name, x, y in zip(NAMES, got, ref):
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {TOL[torch.bfloat16]:g})", flush=True)
        assert e < TOL[torch.bfloat16], f"{name}: err {e:.3e}"


def test_backward_full_workload_sampled(kla):
    inp = ki.prefill_inputs(1)
    ct = ki.cotangents(inp, seed=2024)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     n_seq=d["n_seq"])
    torch.cuda.synchronize()
    T = inp["q"].shape[0] // inp["n_seq"]
    f64 = lambda t: t.double().numpy()
    for n, h in ((0, 0), (3, 15)):
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


def test_backward_is_deterministic(kla):
    # no atomics: two calls on the same inputs give the same bits
    inp = ki.prefill_inputs(1, T=200, n_seq=2, H=2)
    ct = ki.cotangents(inp, seed=8)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    run = lambda: kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                           ct["dO"].to(DEV), S0=d["S0"],
                                           dS_T=ct["dS_T"].to(DEV), n_seq=d["n_seq"])
    a, b = run(), run()
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y), name


def test_backward_all_sequences_empty(kla):
    # no tokens: the state gradient passes through unchanged, dS0 = dS_T
    H, dk, dv = 2, 64, 64
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    e = torch.empty(0, H, dk, device=DEV)
    ev = torch.empty(0, H, dv, device=DEV)
    s = torch.empty(0, H, device=DEV)
    dST = torch.randn(3, H, dk, dv, device=DEV)
    grads = kla.kla_prefill_backward(e, e, ev, s, s, 1e-6, ev, S0=None, dS_T=dST,
                                     cu_seqlens=cu, n_seq=3)
    torch.cuda.synchronize()
    assert torch.equal(grads[5], dST)
    assert all(x.numel() == 0 for x in grads[:5])


def test_backward_zero_keys_at_zero_eps(kla):
    # eps = 0 and some keys exactly zero: b = 0 there (no write), and the gradients through
    # the coefficient vanish at those tokens (deta = 0)
    inp = ki.prefill_inputs(0, T=160)
    inp["eps"] = 0.0
    k = inp["k"].clone()
    k[::7] = 0.0
    inp["k"] = k.contiguous()
    ct = ki.cotangents(inp, seed=12)
    run_case(kla, inp, ct, TOL[torch.float32])


def test_backward_hard_projection(kla):
    # eta = 1, g = 0, eps = 0, q := k: every write is an exact projection (Theorem 1)
    inp = ki.hard_variant(ki.prefill_inputs(0, T=128))
    ct = ki.cotangents(inp, seed=13)
    run_case(kla, inp, ct, TOL[torch.float32])


@pytest.mark.parametrize("mode", ["gated", "key_norm", "inv_t", "inv_sqrt_t", "inv_log_t"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_coefficient_modes(kla, mode, dtype):
    # packed sequences with position offsets; unit-norm keys keep the gated rule bounded
    # (b ||k||^2 = eta < 2)
    inp = ki.prefill_inputs(0, lens=(150, 40, 77), H=2)
    kf = inp["k"].float()
    inp["k"] = (kf / kf.norm(dim=-1, keepdim=True)).to(dtype).contiguous()
    inp["q"], inp["v"] = inp["q"].to(dtype).contiguous(), inp["v"].to(dtype).contiguous()
    inp["dtype"] = dtype
    gen = torch.Generator().manual_seed(21)
    inp["S0"] = 0.3 * torch.randn(3, 2, 64, 64, generator=gen)
    pos = torch.tensor([5, 0, 300], dtype=torch.int32)
    ct = ki.cotangents(inp, seed=22)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     cu_seqlens=d["cu_seqlens"], n_seq=d["n_seq"],
                                     beta_mode=mode, pos_offset=pos.to(DEV))
    torch.cuda.synchronize()
    f64 = lambda t: t.double().numpy()
    ref = ob.prefill_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                              f64(inp["eta"]), inp["eps"], f64(ct["dO"]), S0=f64(inp["S0"]),
                              dS_T=f64(ct["dS_T"]), cu_seqlens=inp["cu_seqlens"].numpy(),
                              beta_mode=mode, pos_offset=pos.numpy())
    print(f"mode {mode} {dtype}", flush=True)
    for name, x, y in zip(NAMES, grads, ref):
        if name == "deta" and mode == "key_norm":
            assert torch.count_nonzero(x) == 0, "deta must vanish: b does not depend on eta"
            continue
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {TOL[dtype]:g})", flush=True)
        assert e < TOL[dtype], f"{name}: err {e:.3e} >= {TOL[dtype]:g}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_normalised_readout(kla, dtype):
    # o = q S / ||q||, with one query row exactly zero (its output and gradient are 0)
    inp = ki.prefill_inputs(0, lens=(130, 61), H=2)
    q = inp["q"].clone()
    q[7] = 0.0
    inp["q"] = q.to(dtype).contiguous()
    inp["k"], inp["v"] = inp["k"].to(dtype).contiguous(), inp["v"].to(dtype).contiguous()
    inp["dtype"] = dtype
    gen = torch.Generator().manual_seed(31)
    inp["S0"] = 0.3 * torch.randn(2, 2, 64, 64, generator=gen)
    ct = ki.cotangents(inp, seed=32)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     cu_seqlens=d["cu_seqlens"], n_seq=d["n_seq"],
                                     normalize_q=True)
    torch.cuda.synchronize()
    f64 = lambda t: t.double().numpy()
    ref = ob.prefill_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                              f64(inp["eta"]), inp["eps"], f64(ct["dO"]), S0=f64(inp["S0"]),
                              dS_T=f64(ct["dS_T"]), cu_seqlens=inp["cu_seqlens"].numpy(),
                              normalize_q=True)
    print(f"normalised readout {dtype}", flush=True)
    for name, x, y in zip(NAMES, grads, ref):
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {TOL[dtype]:g})", flush=True)
        assert e < TOL[dtype], f"{name}: err {e:.3e} >= {TOL[dtype]:g}"
    assert torch.count_nonzero(grads[0][7]) == 0


def test_backward_variant_full_workload_sampled(kla):
    # the 1/sqrt(t) coefficient with position offsets and the readout divided by ||q_t||, on
    # the full prefill workload; one sampled (sequence, head) pair against the oracle
    inp = ki.prefill_inputs(1)
    ct = ki.cotangents(inp, seed=2025)
    pos = torch.tensor([0, 4096, 100000, 7], dtype=torch.int32)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grads = kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                     ct["dO"].to(DEV), S0=d["S0"], dS_T=ct["dS_T"].to(DEV),
                                     n_seq=d["n_seq"], beta_mode="inv_sqrt_t", normalize_q=True,
                                     pos_offset=pos.to(DEV))
    torch.cuda.synchronize()
    T = inp["q"].shape[0] // inp["n_seq"]
    f64 = lambda t: t.double().numpy()
    n, h = 2, 9
    sl = slice(n * T, (n + 1) * T)
    pick = lambda t: f64(t[sl, h:h + 1])
    ref = ob.prefill_backward(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"]),
                              pick(inp["eta"]), inp["eps"], pick(ct["dO"]),
                              S0=f64(inp["S0"][n:n + 1, h:h + 1]),
                              dS_T=f64(ct["dS_T"][n:n + 1, h:h + 1]), beta_mode="inv_sqrt_t",
                              pos_offset=pos[n:n + 1].numpy(), normalize_q=True)
    got = [x[sl, h:h + 1] for x in grads[:5]] + [grads[5][n:n + 1, h:h + 1]]
    print(f"sequence {n}, head {h}", flush=True)
    for name, x, y in zip(NAMES, got, ref):
        e = err(x, y)
        print(f"  {name}: err {e:.3e} (bar {TOL[torch.bfloat16]:g})", flush=True)
        assert e < TOL[torch.bfloat16], f"{name}: err {e:.3e}"
