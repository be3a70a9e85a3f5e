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
