"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded inputs.

Bars (per tensor, err = max|x - y| / max|y| with y the oracle):
  fp32 inputs: 1e-4;  bf16 inputs with fp32 accumulation and state: 2e-2.
Both o and the final state are checked.  Sizes span several chunks and a ragged
tail, packed sequences with empty and one-token members, the workloads' full
sizes (whole, or sampled where the oracle would take too long), and the method's
degenerate cases.
"""
import math

import numpy as np
import pytest
import torch

import kla_inputs as ki
import oracle
from oracle import chunkwise

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda"


def err(x, y):
    """Per-tensor error max|x - y| / max|y| (y is the reference)."""
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    y = y.detach().double().cpu().numpy() if hasattr(y, "detach") else np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    assert np.all(np.isfinite(x)), "non-finite values in device output"
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30))


def check(x, y, tol, what=""):
    e = err(x, y)
    print(f"  {what}: err {e:.3e} (bar {tol:g})", flush=True)
    assert e < tol, f"{what}: err {e:.3e} >= {tol:g}"


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_delta_rule_kla_amd as m
    m.load_library()
    oracle.build(force=False)
    return m


def to_dev(inp):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(DEV) if isinstance(val, torch.Tensor) else val
    return out


def run_prefill(kla, d, S0=True):
    o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                    S0=d["S0"] if S0 else None, cu_seqlens=d["cu_seqlens"],
                                    n_seq=d["n_seq"])
    torch.cuda.synchronize()
    return o, ST


def oracle_prefill(d, S0=True):
    cu = d["cu_seqlens"]
    if cu is None:
        T = d["q"].shape[0] // d["n_seq"]
        cu = np.arange(d["n_seq"] + 1) * T
    else:
        cu = cu.cpu().numpy()
    return oracle.prefill(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                          S0=d["S0"] if S0 else None, cu_seqlens=cu)


# ------------------------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 256), (64, 256)])
def test_decode_step_parity(kla, dtype, dk, dv):
    w = ki.Workload(90, "decode-unit", 6, 3, dk, dv, dtype, T=1, s0_var=0.05, decode_steps=5)
    d = to_dev(ki.decode_inputs(w))
    S = d["S"].clone()
    So = d["S"].double().cpu().numpy()
    for t in range(5):
        o, S = kla.kla_decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                                   d["eps"], S, inplace=(t % 2 == 1))
        oo, So = oracle.decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t], d["eps"], So)
        torch.cuda.synchronize()
        check(o, oo, TOL[dtype], "o t")
        check(S, So, TOL[dtype], "S t")


def test_decode_full_batch(kla):
    """Decode workload: B=256, H=16, d=128 from an N(0, 0.05) state, 4 steps, in place."""
    w = ki.WORKLOADS[3]
    d = to_dev(ki.decode_inputs(w, steps=4))
    S = d["S"].clone()
    So = d["S"].double().cpu().numpy()
    for t in range(4):
        o, _ = kla.kla_decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                                   d["eps"], S, inplace=True)
        oo, So = oracle.decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t], d["eps"], So)
        torch.cuda.synchronize()
        check(o, oo, 2e-2, "o")
        check(S, So, 2e-2, "S")


def test_decode_from_prefill_built_32k_state(kla):
    """Workload 3 with its state built by the prefill over 32768 tokens of workload 1's
    distributions (from a zero state), on a 2-sequence subset: the device prefill's state
    and last-chunk outputs against the oracle's, then 8 decode steps of workload 3's draws
    from each state."""
    B, T = 2, 32768
    pre = to_dev(ki.prefill_inputs(1, T=T, n_seq=B))
    o, ST = run_prefill(kla, pre, S0=False)
    oo, So = oracle_prefill(pre, S0=False)
    check(ST, So, 2e-2, "S after 32768 tokens")
    for n in range(B):
        check(o[(n + 1) * T - 64:(n + 1) * T], oo[(n + 1) * T - 64:(n + 1) * T], 2e-2,
              "o, last chunk")
    dd = to_dev(ki.decode_inputs(3, steps=8, B=B, S=ST))
    S, Sd = ST.clone(), So
    for t in range(8):
        od, S = kla.kla_decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["eta"][t],
                                    dd["eps"], S, inplace=True)
        ood, Sd = oracle.decode(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["eta"][t],
                                dd["eps"], Sd)
        torch.cuda.synchronize()
        check(od, ood, 2e-2, "decode o")
    check(S, Sd, 2e-2, "decode S")


def test_decode_state_beyond_2g_elements(kla):
    """131,200 (sequence, head) items of d = 128 (an 8.6 GB fp32 state, 2^31 elements end
    inside item 131,072), two in-place steps: the last 64 items against the oracle."""
    B, H = 8200, 16
    assert B * H * 128 * 128 > 2 ** 31
    w = ki.Workload(93, "decode-far", B, H, 128, 128, torch.bfloat16, T=1, s0_var=0.05,
                    decode_steps=2)
    d = ki.decode_inputs(w, device=DEV)
    tail = slice(B - 4, B)  # 4 sequences x 16 heads
    So = d["S"][tail].double().cpu().numpy()
    S = d["S"]
    for t in range(2):
        o, S = kla.kla_decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                                   d["eps"], S, inplace=True)
        cpu = lambda x: x[t][tail].cpu()
        oo, So = oracle.decode(cpu(d["q"]), cpu(d["k"]), cpu(d["v"]), cpu(d["g"]),
                               cpu(d["eta"]), d["eps"], So)
        torch.cuda.synchronize()
        check(o[tail], oo, 2e-2, "o, last items")
        check(S[tail], So, 2e-2, "S, last items")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_many_items(kla, dtype):
    """6144 (sequence, head) items: the launch shape with one 512-lane workgroup per item (the
    smaller cases above take four 128-lane workgroups per item at d_k = 128 and d_v >= 128,
    two otherwise).  Every output and state element against the oracle."""
    w = ki.Workload(91, "decode-many", 64, 96, 64, 128, dtype, T=1, s0_var=0.05, decode_steps=2)
    d = to_dev(ki.decode_inputs(w))
    S = d["S"].clone()
    So = d["S"].double().cpu().numpy()
    for t in range(2):
        o, S = kla.kla_decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                                   d["eps"], S, inplace=(t == 1))
        oo, So = oracle.decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                               d["eps"], So)
        torch.cuda.synchronize()
        check(o, oo, TOL[dtype], "o t")
        check(S, So, TOL[dtype], "S t")


# ------------------------------------------------------------------------------------ prefill
def test_prefill_tiny_fp32(kla):
    """Workload 0 (fp32, T=256, d=64) at the 1e-4 bar."""
    d = to_dev(ki.prefill_inputs(0))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 1e-4, "o")
    check(ST, So, 1e-4, "ST")


def test_prefill_tiny_fp32_hard_projection(kla):
    """Workload 0, hard variant (eta=1, g=0, eps=0, q := k): every o_t must be v_t
    (Theorem 1: k_t S_t = v_t), and the whole output must match the oracle."""
    d = to_dev(ki.hard_variant(ki.prefill_inputs(0)))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(oo, d["v"].double().cpu().numpy(), 1e-9, "oo")   # the oracle itself
    check(o, d["v"].double().cpu().numpy(), 1e-4, "o")
    check(o, oo, 1e-4, "o")
    check(ST, So, 1e-4, "ST")


@pytest.mark.parametrize("n_seq,T,H,dk,dv", [
    (2, 200, 3, 128, 128),   # 3 full chunks + ragged tail of 8
    (1, 64, 2, 64, 64),      # exactly one chunk
    (3, 130, 2, 128, 256),   # wide heads, tail of 2
    (1, 1, 1, 128, 128),     # a single token
    (2, 127, 2, 64, 128),
])
def test_prefill_bf16_shapes(kla, n_seq, T, H, dk, dv):
    w = ki.Workload(91, "unit", n_seq, H, dk, dv, torch.bfloat16, T=T, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 2e-2, "o")
    check(ST, So, 2e-2, "ST")


@pytest.mark.parametrize("n_seq,T,H,dk,dv", [(2, 200, 2, 128, 128), (1, 150, 1, 64, 256)])
def test_prefill_fp32_shapes(kla, n_seq, T, H, dk, dv):
    w = ki.Workload(92, "unit", n_seq, H, dk, dv, torch.float32, T=T, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 1e-4, "o")
    check(ST, So, 1e-4, "ST")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk", [64, 128])
def test_prefill_wide_workgroups(kla, dtype, dk):
    """Enough (sequence, head, 32-column) blocks to exceed the chip's compute units, so the
    scan runs its 64-column workgroup shape; ragged tail, random S0."""
    w = ki.Workload(99, "unit", 3, 24, dk, 128, dtype, T=130, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, TOL[dtype], "o")
    check(ST, So, TOL[dtype], "ST")


def test_prefill_packed_ragged(kla):
    """Packed sequences with empty, one-token, chunk-edge and multi-chunk members, strong
    decay and 5% near-zero keys (the eps guard)."""
    lens = [1, 0, 63, 64, 65, 200, 0, 129]
    w = ki.Workload(93, "packed-unit", len(lens), 2, 128, 256, torch.bfloat16, lens=tuple(lens),
                    g_low=-2.0, tiny_key_frac=0.05, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 2e-2, "o")
    check(ST, So, 2e-2, "ST")
    # empty sequences keep their state
    assert torch.equal(ST[1], d["S0"][1]) and torch.equal(ST[6], d["S0"][6])


def test_prefill_many_sequences(kla):
    """100 packed sequences (more than one wavefront can plan inside the prep kernel, so the
    separate planning kernel runs) with empty, one-token and multi-chunk members."""
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.choice([0, 1, 7, 63, 64, 65, 130], size=100)]
    w = ki.Workload(94, "packed-unit", len(lens), 2, 64, 64, torch.bfloat16, lens=tuple(lens),
                    s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 2e-2, "o")
    check(ST, So, 2e-2, "ST")


@pytest.mark.parametrize("n_seq", [5, 63, 64, 90])
def test_prefill_malformed_offsets_are_sanitised(kla, n_seq):
    """Offsets outside [0, total] or decreasing are clamped and made non-decreasing (running
    maximum): the result equals, bit for bit, the run with the sanitised offsets, both where
    the prep kernel plans the sequences itself (n_seq <= 63) and where the plan kernel does."""
    rng = np.random.default_rng(n_seq)
    total = 40 * n_seq
    raw = np.sort(rng.integers(0, total, n_seq + 1)).astype(np.int64)
    raw[0], raw[-1] = 0, total
    bad = raw.copy()
    bad[1::3] = bad[1::3] - 100      # dips below the previous offset (or below 0)
    bad[-2] = total + 77             # past the end
    clean = np.maximum.accumulate(np.clip(bad, 0, total))
    assert clean[-1] == total and np.any(bad != clean)
    w = ki.Workload(95, "unit", 1, 2, 64, 64, torch.bfloat16, T=total, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    S0 = torch.randn(n_seq, 2, 64, 64, device=DEV) * 0.1
    outs = []
    for cu in (bad, clean):
        o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                        S0=S0, n_seq=n_seq,
                                        cu_seqlens=torch.tensor(cu, dtype=torch.int32,
                                                                device=DEV))
        torch.cuda.synchronize()
        outs.append((o.clone(), ST.clone()))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0], outs[1][0])


def test_prefill_layer_workload_full(kla):
    """Workload 1 (B=4, H=16, T=4096, d=128, bf16, random S0) at full size, every output."""
    d = to_dev(ki.prefill_inputs(1))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 2e-2, "o")
    check(ST, So, 2e-2, "ST")


def test_prefill_long_context_full(kla):
    """Workload 2 (T=65536, H=16, bf16) at full size, every output and S_T."""
    d = to_dev(ki.prefill_inputs(2))
    o, ST = run_prefill(kla, d)
    oo, So = oracle_prefill(d)
    check(o, oo, 2e-2, "o")
    check(o[-64:], oo[-64:], 2e-2, "o[-64:]")  # the last chunk on its own scale
    check(ST, So, 2e-2, "ST")


def test_prefill_beyond_2g_elements(kla):
    """Packed input whose second sequence starts past element 2^31 of q, k, v and o
    (1,048,768 + 200 tokens x 16 heads x d = 128, bf16, about 4.3 GB per token tensor): every
    index into the token tensors, the workspace and the states must be 64-bit there.  The far
    sequence's outputs and final state against the oracle, and the long sequence's last chunk
    (also past element 2^31) against the oracle started from the state a device prefill of
    the chunks before it leaves."""
    L0, L1, H = 1048768, 200, 16
    assert L0 * H * 128 > 2 ** 31
    w = ki.Workload(98, "far", 2, H, 128, 128, torch.bfloat16, lens=(L0, L1), s0_var=0.01)
    d = ki.prefill_inputs(w, device=DEV)
    o, ST = run_prefill(kla, d)
    sl = slice(L0, L0 + L1)
    cpu = lambda t: t[sl].cpu()
    oo, So = oracle.prefill(cpu(d["q"]), cpu(d["k"]), cpu(d["v"]), cpu(d["g"]), cpu(d["eta"]),
                            d["eps"], S0=d["S0"][1:2].cpu())
    check(o[sl], oo, 2e-2, "o, far sequence")
    check(ST[1:2], So, 2e-2, "S_T, far sequence")
    head = slice(0, L0 - 64)
    _, S_mid = kla.kla_prefill_chunked(d["q"][head], d["k"][head], d["v"][head], d["g"][head],
                                       d["eta"][head], d["eps"], S0=d["S0"][0:1], n_seq=1)
    tail = slice(L0 - 64, L0)
    ct = lambda t: t[tail].cpu()
    ot, St = oracle.prefill(ct(d["q"]), ct(d["k"]), ct(d["v"]), ct(d["g"]), ct(d["eta"]),
                            d["eps"], S0=S_mid.cpu())
    check(o[tail], ot, 2e-2, "o, long sequence's last chunk")
    check(ST[0:1], St, 2e-2, "S_T, long sequence")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n_seq,T,H,dk,dv,G,S0,weak", [
    (1, 64 * 9 + 13, 2, 128, 128, 3, True, False),   # ragged last segment
    (2, 64 * 8, 1, 64, 256, 2, True, False),
    (1, 64 * 7, 2, 128, 64, 7, False, False),        # one chunk per segment, zero S0
    (3, 64 * 5 + 1, 2, 64, 64, 4, True, False),      # 3 segments of 2 chunks, one-token tail
    (1, 64 * 6, 40, 128, 128, 3, True, False),       # enough workgroups for the 64-column shape
    (1, 64 * 9 + 13, 2, 128, 128, 3, True, True),    # the same without decay and with weak
    (3, 64 * 5 + 1, 2, 64, 64, 4, True, True),       # writes: the transitions M_g matter
    (1, 64 * 6, 40, 128, 128, 6, True, True),
    # segments longer than the 8-chunk warm-up: with the workloads' gates every boundary's
    # warm-up contracts by far more than 2^-150 (segments start early from zero); without
    # decay none does (map, combine and segment phases); both in one call ('head0': head 0
    # without decay)
    (1, 64 * 40 + 7, 2, 128, 128, 4, True, False),
    (2, 64 * 33, 2, 64, 128, 3, True, False),
    (1, 64 * 40 + 7, 2, 128, 128, 4, True, True),
    (1, 64 * 40 + 7, 3, 128, 128, 4, True, "head0"),
])
def test_prefill_two_level_scan(kla, dtype, n_seq, T, H, dk, dv, G, S0, weak):
    """The two-level scan (segments' transitions, chained incoming states, segments rerun)
    against the oracle and against the sequential scan on the same inputs.  With the
    workloads' gates a state fades within a few chunks, so the segments' transitions
    M_g are near zero; weak=True sets g = 0 and eta to 5% of its draw, so that a state
    carries across whole segments and the chained states depend on M_g."""
    w = ki.Workload(97, "unit", n_seq, H, dk, dv, dtype, T=T, s0_var=0.01)
    inp = ki.prefill_inputs(w)
    if weak == "head0":
        inp["g"][:, 0] = 0.0
        inp["eta"][:, 0] = inp["eta"][:, 0] * 0.05
    elif weak:
        inp["g"] = torch.zeros_like(inp["g"])
        inp["eta"] = inp["eta"] * 0.05
    d = to_dev(inp)
    outs = []
    for segs in (G, 1):
        o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                        S0=d["S0"] if S0 else None, n_seq=n_seq,
                                        scan_segments=segs)
        torch.cuda.synchronize()
        outs.append((o, ST))
    oo, So = oracle_prefill(d, S0=S0)
    for (o, ST), name in zip(outs, ("two-level", "sequential")):
        check(o, oo, TOL[dtype], f"o {name}")
        check(ST, So, TOL[dtype], f"ST {name}")
    check(outs[0][0], outs[1][0], TOL[dtype], "o two-level vs sequential")
    check(outs[0][1], outs[1][1], TOL[dtype], "ST two-level vs sequential")


def test_packed_workload_full_with_decode(kla):
    """Workload 4 (16 packed sequences of 1024..16384 tokens, H=8, d_v=256, g ~ U(-2,0),
    tiny keys) at full size: every output and final state of the prefill, then all 128
    decode steps that continue from the prefill state (every output and the final state),
    each sequence also on its own scale."""
    d = to_dev(ki.prefill_inputs(4))
    o, ST = run_prefill(kla, d, S0=False)
    cu = d["cu_seqlens"].cpu().numpy()
    steps = 128
    dd = to_dev(ki.decode_inputs(4, steps=steps, S=ST))
    S = ST.clone()
    outs = []
    for t in range(steps):
        od, S = kla.kla_decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["eta"][t],
                                    dd["eps"], S, inplace=True)
        outs.append(od.clone())
    torch.cuda.synchronize()
    oo, So = oracle_prefill(d, S0=False)
    check(o, oo, 2e-2, "o")
    check(ST, So, 2e-2, "ST")
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        worst = max(worst, err(o[a:b], oo[a:b]), err(ST[n], So[n]))
    print(f"  worst per-sequence err {worst:.3e}", flush=True)
    assert worst < 2e-2
    Sd = So
    od_all, oo_all = [], []
    for t in range(steps):
        od, Sd = oracle.decode(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["eta"][t],
                               dd["eps"], Sd)
        oo_all.append(od)
        od_all.append(outs[t].double().cpu().numpy())
    check(np.stack(od_all), np.stack(oo_all), 2e-2, f"decode o, {steps} steps")
    check(S, Sd, 2e-2, "decode S")


# ------------------------------------------------------------------------------------ invariants
def test_one_hot_keys_long_context_closed_form(kla):
    """Keys c e_i (exact in bf16): every slot is an independent relaxed update, so the
    state after 65536 tokens has a closed form (no oracle run needed at this length)."""
    T, dk, dv = 65536, 128, 128
    gen = torch.Generator().manual_seed(7)
    slots = torch.randint(0, dk, (T,), generator=gen)
    c = torch.tensor([0.5, 1.0, 2.0, 4.0])[torch.randint(0, 4, (T,), generator=gen)]
    k = torch.zeros(T, 1, dk)
    k[torch.arange(T), 0, slots] = c
    v = torch.randn(T, 1, dv, generator=gen).to(torch.bfloat16)
    q = torch.randn(T, 1, dk, generator=gen).to(torch.bfloat16)
    eta = torch.rand(T, 1, generator=gen) * 0.9 + 0.1
    g = -0.01 * torch.rand(T, 1, generator=gen)
    eps = 1e-6
    d = dict(q=q, k=k.to(torch.bfloat16), v=v, g=g, eta=eta, eps=eps, S0=None, cu_seqlens=None,
             n_seq=1)
    o, ST = run_prefill(kla, to_dev(d), S0=False)
    X = np.zeros((dk, dv))
    vv, gg, ee = v[:, 0].double().numpy(), g[:, 0].double().numpy(), eta[:, 0].double().numpy()
    ss, cc = slots.numpy(), c.double().numpy()
    for t in range(T):
        X *= math.exp(gg[t])
        rho = ee[t] * cc[t] ** 2 / (cc[t] ** 2 + eps)
        X[ss[t]] = (1 - rho) * X[ss[t]] + rho * vv[t] / cc[t]
    check(ST[0, 0], X, 2e-2, "ST[0, 0]")


def test_hard_projection_bf16_reads_back_values(kla):
    """eta = 1, g = 0, eps = 0 and q := k on bf16 inputs: o_t = v_t (Theorem 1).

    Keys are unit vectors scaled by loguniform[0.5, 2] (the long-context workload's keys).
    With keys whose norms span 100x, o_t = k_t S~ + e_t cancels terms ~||k|| |S| down to
    |v|, which amplifies bf16 operand rounding (2^-9) past the bar; that spread is covered
    in fp32 by the tiny-workload hard case above."""
    w = ki.Workload(94, "unit", 1, 4, 128, 128, torch.bfloat16, T=300, key_mode="unit_loguniform")
    d = to_dev(ki.hard_variant(ki.prefill_inputs(w)))
    o, _ = run_prefill(kla, d, S0=False)
    check(o, d["v"].double().cpu().numpy(), 2e-2, "o")


def _spread_keys_hard_bf16(T, H, dk, dv):
    """The tiny workload's draws (keys with norms 10^U(-1, 1)) in bf16, hard variant."""
    w = ki.Workload(0, "spread-bf16", 1, H, dk, dv, torch.bfloat16, T=T)
    return to_dev(ki.hard_variant(ki.prefill_inputs(w)))


@pytest.mark.parametrize("T,H,dk,dv", [(256, 1, 64, 64), (300, 2, 128, 128)])
def test_hard_projection_bf16_spread_key_norms_split_precision(kla, T, H, dk, dv):
    """Theorem 1 on bf16 inputs with keys whose norms span 100x: with split precision (T R,
    P U and the state update on hi/lo bf16 operand pairs) o_t = v_t, and o matches the
    oracle."""
    d = _spread_keys_hard_bf16(T, H, dk, dv)
    o, _ = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                   n_seq=1, precision="split")
    torch.cuda.synchronize()
    check(o, d["v"].double().cpu().numpy(), 2e-2, "o vs v")
    oo, _ = oracle_prefill(d, S0=False)
    check(o, oo, 2e-2, "o vs oracle")


@pytest.mark.xfail(strict=True, reason="bf16 operand mode on keys whose norms span 100x: o = "
                   "k S~ + e cancels terms of size ||k|| |S| down to |v|, and bf16 operands "
                   "(2^-9) leave a measured error of 0.10-0.20 against the 2e-2 bar; the split "
                   "precision mode holds it")
def test_hard_projection_bf16_spread_key_norms_bf16_operands(kla):
    d = _spread_keys_hard_bf16(300, 2, 128, 128)
    o, _ = run_prefill(kla, d, S0=False)
    check(o, d["v"].double().cpu().numpy(), 2e-2, "o vs v")


@pytest.mark.parametrize("n_seq,T,H,dk,dv,S0", [
    (2, 200, 3, 128, 128, True),   # ragged tail
    (3, 130, 2, 128, 256, True),
    (1, 1, 1, 128, 128, False),    # a single token
    (2, 127, 2, 64, 128, True),
    (3, 130, 24, 128, 128, True),  # the 64-column workgroup shape
])
def test_prefill_split_precision_shapes(kla, n_seq, T, H, dk, dv, S0):
    """Split precision against the oracle on the workloads' draws; never worse than the
    bf16 operand mode beyond rounding."""
    w = ki.Workload(96, "unit", n_seq, H, dk, dv, torch.bfloat16, T=T, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    outs = {}
    for prec in ("split", "bf16"):
        o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                        S0=d["S0"] if S0 else None, n_seq=n_seq, precision=prec)
        torch.cuda.synchronize()
        outs[prec] = (o, ST)
    oo, So = oracle_prefill(d, S0=S0)
    check(outs["split"][0], oo, 2e-2, "o split")
    check(outs["split"][1], So, 2e-2, "ST split")
    assert err(outs["split"][0], oo) <= err(outs["bf16"][0], oo) + 4e-3
    assert err(outs["split"][1], So) <= err(outs["bf16"][1], So) + 4e-3


def test_split_resume_and_prefill_decode_chain(kla):
    """prefill(T) == prefill(T1) + prefill(rest, S0 = S_T1) for a split inside a chunk, and
    prefill(T) + m decode steps == prefill(T + m)."""
    w = ki.Workload(95, "unit", 1, 4, 128, 128, torch.bfloat16, T=300, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    sl = lambda x, a, b: x[a:b].contiguous()
    o1, S1 = kla.kla_prefill_chunked(sl(d["q"], 0, 101), sl(d["k"], 0, 101), sl(d["v"], 0, 101),
                                     sl(d["g"], 0, 101), sl(d["eta"], 0, 101), d["eps"], S0=d["S0"])
    o2, S2 = kla.kla_prefill_chunked(sl(d["q"], 101, 300), sl(d["k"], 101, 300),
                                     sl(d["v"], 101, 300), sl(d["g"], 101, 300),
                                     sl(d["eta"], 101, 300), d["eps"], S0=S1)
    ref = lambda x: x.double().cpu().numpy()
    check(torch.cat([o1, o2]), ref(o), 2e-2, "torch.cat([o1, o2])")
    check(S2, ref(ST), 2e-2, "S2")
    o3, S3 = kla.kla_prefill_chunked(sl(d["q"], 0, 290), sl(d["k"], 0, 290), sl(d["v"], 0, 290),
                                     sl(d["g"], 0, 290), sl(d["eta"], 0, 290), d["eps"], S0=d["S0"])
    for t in range(290, 300):
        od, S3 = kla.kla_decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1],
                                     d["g"][t:t + 1], d["eta"][t:t + 1], d["eps"], S3, inplace=True)
        check(od, ref(o[t:t + 1]), 2e-2, "od")
    check(S3, ref(ST), 2e-2, "S3")


def test_packed_equals_per_sequence_and_deterministic(kla):
    lens = [70, 0, 129, 5]
    w = ki.Workload(96, "unit", 4, 2, 128, 128, torch.bfloat16, lens=tuple(lens), s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o, ST = run_prefill(kla, d)
    o_again, ST_again = run_prefill(kla, d)
    assert torch.equal(o, o_again) and torch.equal(ST, ST_again)  # run-to-run bitwise
    cu = d["cu_seqlens"].cpu().tolist()
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        if a == b:
            continue
        on, Sn = kla.kla_prefill_chunked(d["q"][a:b].contiguous(), d["k"][a:b].contiguous(),
                                         d["v"][a:b].contiguous(), d["g"][a:b].contiguous(),
                                         d["eta"][a:b].contiguous(), d["eps"],
                                         S0=d["S0"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(on, o[a:b]) and torch.equal(Sn[0], ST[n])


def test_in_place_state_and_null_state(kla):
    w = ki.Workload(97, "unit", 2, 2, 64, 64, torch.float32, T=100, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o_ref, ST_ref = run_prefill(kla, d)
    S = d["S0"].clone()
    o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], S0=S,
                                    n_seq=2, S_T=S)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    assert torch.equal(S, ST_ref) and torch.equal(o, o_ref)
    o0, _ = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], n_seq=2,
                                    output_final_state=False)
    oo, _ = oracle_prefill(d, S0=False)
    check(o0, oo, 1e-4, "o0")


def test_zero_tokens(kla):
    """No tokens at all: S_T = S0."""
    S0 = torch.randn(3, 2, 128, 128, device=DEV)
    e = torch.empty(0, 2, 128, device=DEV, dtype=torch.bfloat16)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    o, ST = kla.kla_prefill_chunked(e, e, e, torch.empty(0, 2, device=DEV),
                                    torch.empty(0, 2, device=DEV), 1e-6, S0=S0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and torch.equal(ST, S0)


def test_chunk_stage_intermediates(kla):
    """Per-chunk b, G and T = (I + L)^{-1} Diag(b), and the WY factors W, U~, against the
    chunkwise fp64 reference (fp32 inputs, so the bar is fp32-level)."""
    lens = [150, 64, 3]
    w = ki.Workload(98, "unit", 3, 2, 64, 64, torch.float32, lens=tuple(lens))
    d = to_dev(ki.prefill_inputs(w))
    r = kla.kla_prefill_chunk_stage(d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                    cu_seqlens=d["cu_seqlens"], want_wy=True)
    torch.cuda.synchronize()
    q, k, v, g, eta = (d[x].double().cpu().numpy() for x in ("q", "k", "v", "g", "eta"))
    cu = d["cu_seqlens"].cpu().numpy()
    _, _, inter = chunkwise.prefill(q, k, v, g, eta, d["eps"], cu_seqlens=cu, chunk=64)
    ci = 0
    for n in range(3):
        for c, t0 in enumerate(range(int(cu[n]), int(cu[n + 1]), 64)):
            t1 = min(t0 + 64, int(cu[n + 1]))
            m = t1 - t0
            for h in range(2):
                ref = inter[(n, h, c)]
                check(r["beta"][t0:t1, h], ref["b"], 1e-5, "r['beta'][t0:t1, h]")
                check(r["G"][t0:t1, h], ref["G"], 1e-5, "r['G'][t0:t1, h]")
                Tdev = r["T"][ci, h]
                check(Tdev[:m, :m], ref["T"], 1e-4, "Tdev[:m, :m]")
                assert torch.count_nonzero(Tdev[m:, :]) == 0 and torch.count_nonzero(Tdev[:, m:]) == 0
                gam = np.exp(ref["G"])
                W_ref = ref["T"] @ (gam[:, None] * k[t0:t1, h])
                U_ref = ref["T"] @ v[t0:t1, h]
                check(r["W"][t0:t1, h], W_ref, 1e-4, "r['W'][t0:t1, h]")
                check(r["Ut"][t0:t1, h], U_ref, 1e-4, "r['Ut'][t0:t1, h]")
            ci += 1
