"""Parity of the coefficient and readout variants (kla_options) with the fp64 oracle.

The variants are the pages' ablations of the write coefficient (gated delta rule's
b_t = eta_t; key-norm only; the Kaczmarz coefficient times 1/t, 1/sqrt(t), 1/log(t + 1)
with t the absolute position) and the readout divided by ||q_t||.  Same bars as the main
parity suite: 1e-4 for fp32 inputs, 2e-2 for bf16 (per tensor, relative to max|oracle|).
Inputs come from the seeded generators with packed ragged sequences and position offsets;
the gated rule is run on unit-norm keys, where its update stays bounded.
"""
import numpy as np
import pytest
import torch

import kla_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
MODES = ["kaczmarz", "gated", "key_norm", "inv_t", "inv_sqrt_t", "inv_log_t"]


def err(x, y):
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    assert np.all(np.isfinite(x)), "non-finite values in device output"
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30))


def check(x, y, tol, what):
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


def to_dev(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def unit_keys(d):
    d = dict(d)
    d["k"] = (d["k"].float() / d["k"].float().norm(dim=-1, keepdim=True)).to(d["k"].dtype)
    return d


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("normq", [False, True])
def test_prefill_variant_parity(kla, dtype, mode, normq):
    w = ki.WORKLOADS[0]
    d = ki.prefill_inputs(w, lens=(70, 1, 130, 64), H=2)
    if dtype == torch.bfloat16:
        d = {key: (val.to(torch.bfloat16) if key in ("q", "k", "v") else val)
             for key, val in d.items()}
    if mode == "gated":
        d = unit_keys(d)
    d["q"][5, 1] = 0  # a zero query (reads out zero under the normalised readout)
    pos = torch.tensor([0, 7, 1000, 3], dtype=torch.int32)
    dev = {key: (val.cuda() if isinstance(val, torch.Tensor) else val) for key, val in d.items()}
    S0 = torch.randn(d["n_seq"], 2, w.d_k, w.d_v, generator=torch.Generator().manual_seed(9)) * 0.1
    print(f"prefill variant {mode} normq={normq} {dtype}", flush=True)
    o, ST = kla.kla_prefill_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["eta"], d["eps"],
                                    S0=S0.cuda(), cu_seqlens=dev["cu_seqlens"], n_seq=d["n_seq"],
                                    beta_mode=mode, normalize_q=normq, pos_offset=pos.cuda())
    torch.cuda.synchronize()
    oref, Sref = oracle.prefill(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], S0=S0,
                                cu_seqlens=d["cu_seqlens"].numpy(), beta_mode=mode,
                                normalize_q=normq, pos_offset=pos.numpy())
    check(o, oref, TOL[dtype], "o")
    check(ST, Sref, TOL[dtype], "S_T")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_decode_variant_parity(kla, dtype, mode):
    w = ki.WORKLOADS[3]
    d = ki.decode_inputs(w, steps=3, B=6, H=4)
    if dtype == torch.float32:
        d = {key: (val.float() if key in ("q", "k", "v") else val) for key, val in d.items()}
    pos = torch.tensor([0, 1, 2, 100, 5000, 31], dtype=torch.int32)
    S = d["S"].clone()
    Sd = S.cuda()
    print(f"decode variant {mode} {dtype}", flush=True)
    for i in range(3):
        k = d["k"][i]
        if mode == "gated":
            k = (k.float() / k.float().norm(dim=-1, keepdim=True)).to(k.dtype)
        o, Sd = kla.kla_decode_step(d["q"][i].cuda(), k.cuda(), d["v"][i].cuda(), d["g"][i].cuda(),
                                    d["eta"][i].cuda(), d["eps"], Sd, beta_mode=mode,
                                    normalize_q=True, pos_offset=(pos + i).cuda())
        torch.cuda.synchronize()
        oref, Sref = oracle.decode(d["q"][i], k, d["v"][i], d["g"][i], d["eta"][i], d["eps"], S,
                                   beta_mode=mode, normalize_q=True, pos_offset=(pos + i).numpy())
        check(o, oref, TOL[dtype], f"o step {i}")
        check(Sd, Sref, TOL[dtype], f"S step {i}")
        S = torch.from_numpy(Sref).float()
        Sd = S.cuda()


# ------------------------------------------------------------------ diagonal gating (decode)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv,B,H", [(64, 64, 6, 3), (128, 128, 4, 5), (128, 256, 3, 2),
                                       (64, 128, 64, 96)])
def test_decode_diagonal_gate(kla, dtype, dk, dv, B, H):
    """Diagonal gating (paper Appendix B.5): g holds one log-decay per key channel.  The last
    case has 6144 (sequence, head) items, the launch shape with one 512-lane workgroup each."""
    w = ki.Workload(92, "decode-diag", B, H, dk, dv, dtype, T=1, s0_var=0.05, decode_steps=3,
                    g_low=-1.0)
    d = to_dev(ki.decode_inputs(w, diag=True))
    S = d["S"].clone()
    So = d["S"].double().cpu().numpy()
    for t in range(3):
        o, S = kla.kla_decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                                   d["eps"], S, inplace=(t == 1))
        oo, So = oracle.decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["eta"][t],
                               d["eps"], So)
        torch.cuda.synchronize()
        check(o, oo, TOL[dtype], "o t")
        check(S, So, TOL[dtype], "S t")


# ------------------------------------------------------------------ diagonal gating (prefill)
def run_prefill_diag(kla, d, **kw):
    o, ST = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                    S0=d["S0"], cu_seqlens=d["cu_seqlens"], n_seq=d["n_seq"], **kw)
    torch.cuda.synchronize()
    return o, ST


def oracle_prefill_diag(d, **kw):
    cu = d["cu_seqlens"]
    if cu is None:
        T = d["q"].shape[0] // d["n_seq"]
        cu = np.arange(d["n_seq"] + 1) * T
    else:
        cu = cu.cpu().numpy()
    return oracle.prefill(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], S0=d["S0"],
                          cu_seqlens=cu, **kw)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", ["tiny", "ragged128", "dk64_dv256", "strong_decay",
                                  "extreme_decay", "extreme_decay_dk64", "wide"])
def test_prefill_diagonal_gate(kla, dtype, case):
    """Diagonal gating (paper Appendix B.5): g [n_tok, H, d_k], one log-decay per key channel,
    through kla_prefill_chunked_ex, against the fp64 tokenwise oracle.  'wide' has 3 x 24 x 4
    column slices, more than the compute units, so the 64-column workgroups run.  With
    g ~ U(-8, 0) ('extreme_decay') a chunk's channels decay by far more than 2^64 around its
    middle row, so the prep takes its blockwise-anchored products."""
    spec = {
        "tiny": dict(H=1, dk=64, dv=64, lens=None, T=256, n_seq=1, g_low=-0.5),
        "ragged128": dict(H=3, dk=128, dv=128, lens=(70, 1, 129, 200), g_low=-0.5),
        "dk64_dv256": dict(H=2, dk=64, dv=256, lens=(64, 190, 5), g_low=-0.5),
        "strong_decay": dict(H=2, dk=128, dv=128, lens=(300, 77), g_low=-2.0),
        "extreme_decay": dict(H=2, dk=128, dv=128, lens=(200, 64, 3), g_low=-8.0),
        "extreme_decay_dk64": dict(H=2, dk=64, dv=128, lens=(150, 70), g_low=-8.0),
        "wide": dict(H=24, dk=128, dv=128, lens=None, T=130, n_seq=3, g_low=-0.5),
    }[case]
    w = ki.Workload(93, "prefill-diag", spec.get("n_seq", len(spec["lens"] or ())), spec["H"],
                    spec["dk"], spec["dv"], dtype, T=spec.get("T", 0), lens=spec["lens"] or (),
                    g_low=spec["g_low"], s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w, diag=True))
    assert d["g"].shape == d["k"].shape
    o, ST = run_prefill_diag(kla, d)
    oo, So = oracle_prefill_diag(d)
    check(o, oo, TOL[dtype], "o")
    check(ST, So, TOL[dtype], "S_T")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_diagonal_gate_mixed_channel_decay(kla, dtype):
    """Key channels 32..63 decay with g ~ U(-8, 0), the others with g ~ U(-0.5, 0): the prep's
    wavefront over those 32 channels takes the blockwise-anchored products while the others
    take the one-anchor products, and their partial A and P sums meet in one chunk solve."""
    w = ki.Workload(96, "prefill-diag-mixed", 2, 2, 128, 128, dtype, lens=(190, 64),
                    g_low=-0.5, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w, diag=True))
    g = d["g"].clone()
    g[:, :, 32:64] *= 16.0
    d["g"] = g.contiguous()
    o, ST = run_prefill_diag(kla, d)
    oo, So = oracle_prefill_diag(d)
    check(o, oo, TOL[dtype], "o")
    check(ST, So, TOL[dtype], "S_T")


def test_prefill_diagonal_gate_normalised_readout(kla):
    """Diagonal gating together with the readout divided by ||q_t|| and the GDN coefficient
    (on unit keys, where that coefficient keeps the recurrence bounded)."""
    w = ki.Workload(94, "prefill-diag-nq", 2, 2, 128, 128, torch.float32, T=150, s0_var=0.01)
    d = unit_keys(to_dev(ki.prefill_inputs(w, diag=True)))
    o, ST = run_prefill_diag(kla, d, normalize_q=True, beta_mode="gated")
    oo, So = oracle_prefill_diag(d, normalize_q=True, beta_mode="gated")
    check(o, oo, 1e-4, "o")
    check(ST, So, 1e-4, "S_T")


def test_prefill_diagonal_equal_channels_match_scalar_gate(kla):
    """A per-channel g that is the same on every channel gives the scalar-gated result."""
    w = ki.Workload(95, "prefill-diag-eq", 2, 3, 128, 128, torch.float32, T=200, s0_var=0.01)
    d = to_dev(ki.prefill_inputs(w))
    o1, S1 = run_prefill_diag(kla, d)
    dd = dict(d)
    dd["g"] = d["g"][:, :, None].expand(-1, -1, 128).contiguous()
    o2, S2 = run_prefill_diag(kla, dd)
    check(o2, o1.double().cpu().numpy(), 1e-5, "o")
    check(S2, S1.double().cpu().numpy(), 1e-5, "S_T")


# ------------------------------------------------------------- variants at the full layer size
@pytest.mark.parametrize("variant", ["diagonal_gate", "gated_unit_keys", "normalised_inv_sqrt_t"])
def test_variants_full_workload(kla, variant):
    """The prefill workload at full size (4 sequences x 4096 tokens x 16 heads, d = 128, bf16,
    random S0) in the bench launch configuration, once per variant: the diagonal gate (g per
    key channel), the gated delta rule on unit-norm keys, and the readout divided by ||q_t||
    with the 1/sqrt(t) coefficient and position offsets.  Every output and final state
    against the oracle, and each (sequence, head) on its own scale."""
    d = ki.prefill_inputs(1, diag=(variant == "diagonal_gate"))
    kw = {}
    if variant == "gated_unit_keys":
        d = unit_keys(d)
        kw = dict(beta_mode="gated")
    elif variant == "normalised_inv_sqrt_t":
        kw = dict(beta_mode="inv_sqrt_t", normalize_q=True)
    pos = torch.tensor([0, 4096, 100000, 7], dtype=torch.int32)
    if kw:
        kw["pos_offset"] = pos
    dev = to_dev(d)
    print(f"full-size variant {variant}", flush=True)
    o, ST = run_prefill_diag(kla, dev, **{key: (val.cuda() if isinstance(val, torch.Tensor)
                                                else val) for key, val in kw.items()})
    T = d["q"].shape[0] // d["n_seq"]
    okw = dict(kw)
    if "pos_offset" in okw:
        okw["pos_offset"] = pos.numpy()
    oo, So = oracle.prefill(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], S0=d["S0"],
                            cu_seqlens=np.arange(d["n_seq"] + 1) * T, **okw)
    check(o, oo, TOL[torch.bfloat16], "o")
    check(ST, So, TOL[torch.bfloat16], "S_T")
    oh = o.double().cpu().numpy()
    worst = 0.0
    for n in range(d["n_seq"]):
        sl = slice(n * T, (n + 1) * T)
        for h in range(d["q"].shape[1]):
            worst = max(worst, err(oh[sl, h], oo[sl, h]), err(ST[n, h], So[n, h]))
    print(f"  worst per-(sequence, head) err {worst:.3e}", flush=True)
    assert worst < TOL[torch.bfloat16]
