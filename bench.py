#!/usr/bin/env python3
"""Benchmark of the KLA forward hot path on one MI355X (prints ONE JSON line).

A step is one chunkwise prefill (plan + prep/UT kernel, then the chunk-scan kernel
with the fused output) over the layer-scale workload: B=4 sequences, H=16 heads,
T=4096 tokens, d_k=d_v=128, bf16 q/k/v, fp32 g/eta/state, chunk 64, random S0.
``value`` is prefill tokens/s over the timed steps.  Four copies of the inputs and
workspace are rotated so the 256 MB last-level cache cannot serve them from one
step to the next.

The same run measures the decode step (the other half of the metric) on the
decode workload (B=256, H=16, d=128, fp32 state from N(0, 0.05), 512 consecutive
in-place steps with fresh bf16 q/k/v and fp32 g/eta per step), and times the fp64
CPU oracle on the host cores as a reported baseline.

Per-kernel durations come from HIP events recorded on the launch stream inside the
timed loop: the prefill is issued as its two halves (kla_prefill_prepare, then
kla_prefill_scan), which is exactly what kla_prefill_chunked enqueues.

Algorithmic work (per token-head, C = 64, d = d_k = d_v):
  scan kernel bytes  = 2 d_k e (q, k) + d_v e (v) + d_v e (o)
                       + 2 x 40 e (T and P: the ten 16 x 16 blocks on and below the diagonal
                         of each 64 x 64 matrix, 2560 entries per 64 tokens)
                       + 12 (three fp32 decay factors)
                       + 8 d_k d_v per (sequence, head) for S0 in / S_T out,  e = 2 (bf16)
  prefill MFMA flops = 6 d_k d_v + (C-1) d_k + (C+1)(2 d_k + 2 d_v)
  decode bytes       = 8 d_k d_v + 2 (2 d_k + d_v) + 2 d_v + 8
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic_prefill_B4_H16_T4096_d128.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# what the chunk-scan kernel is compiled from (its sources and the compiler flags): a change to
# any of them voids its counters
SCAN_SOURCES = ("csrc/kla_scan.hip", "csrc/kla_device.h", "csrc/kla_launch.h", "build.py")


def csrc_digest() -> str:
    h = hashlib.sha256()
    pdir = os.path.join(ROOT, "gated_delta_rule_kla_amd")
    for name in SCAN_SOURCES:
        with open(os.path.join(pdir, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per scan launch from the committed rocprofv3 counter summary, or None if
    the kernels changed since the counters were taken."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("csrc_digest") != csrc_digest():
            return None
        return float(fields["hbm_bytes_per_scan_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="timed steps of the backward pass (0 = skip)")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant-steps", type=int, default=10,
                    help="steps timed for each coefficient / readout variant (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="finally copy this many MiB device to device once: a kernel of known "
                         "traffic for scaling hardware byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); sequences and heads shard across GPUs with no exchange, "
              f"so the path is timed on one GPU's share", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import gated_delta_rule_kla_amd as kla
    import kla_inputs as ki

    kla.load_library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = ki.WORKLOADS[1]
    log(f"prefill workload {w.name}: generating inputs")
    base = ki.prefill_inputs(w, device=dev)
    n_seq, H, dk, dv = base["n_seq"], w.H, w.d_k, w.d_v
    n_tok = base["q"].shape[0]
    ws_bytes = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv)
    sets = []
    for _ in range(4):
        sets.append(dict(q=base["q"].clone(), k=base["k"].clone(), v=base["v"].clone(),
                         g=base["g"].clone(), eta=base["eta"].clone(), S0=base["S0"].clone(),
                         o=torch.empty(n_tok, H, dv, dtype=w.dtype, device=dev),
                         S_T=torch.empty(n_seq, H, dk, dv, dtype=torch.float32, device=dev),
                         ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)))

    def step(s, ev_mid=None):
        kla.kla_prefill_prepare(s["q"], s["k"], s["g"], s["eta"], base["eps"], s["ws"], n_seq=n_seq, d_v=dv)
        if ev_mid is not None:
            ev_mid.record()
        kla.kla_prefill_scan(s["q"], s["k"], s["v"], s["ws"], n_seq=n_seq, S0=s["S0"], o=s["o"],
                             S_T=s["S_T"])

    for i in range(args.warmup):
        step(sets[i % 4])
    torch.cuda.synchronize()
    K = args.steps
    # the timed region: K back-to-back steps between one pair of events
    log(f"timing {K} prefill steps")
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for i in range(K):
        step(sets[i % 4])
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e_start.elapsed_time(e_end)
    ms_per_step = total_ms / K
    # a second pass with events around each kernel, for the prep / scan split and the scan's
    # launch duration (the extra event records make it slightly slower than the pass above)
    ev_start = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_mid = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev_start[i].record()
        step(sets[i % 4], ev_mid[i])
        ev_end[i].record()
    torch.cuda.synchronize()
    prep_ms = sum(ev_start[i].elapsed_time(ev_mid[i]) for i in range(K)) / K
    scan_ms = sum(ev_mid[i].elapsed_time(ev_end[i]) for i in range(K)) / K
    tok_per_s = n_tok / (ms_per_step * 1e-3)
    th = n_tok * H
    # per token-head: q, k, v rows, o row, one row each of T and P, three decay factors
    tp_per_token = 10 * 256 // CHUNK  # lower 16 x 16 blocks of T (and of P) per token
    scan_bytes = (th * (2 * dk * 2 + dv * 2 + dv * 2 + 2 * tp_per_token * 2 + 12)
                  + 2 * n_seq * H * dk * dv * 4)
    scan_gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    flops_prefill = th * (6 * dk * dv + (CHUNK - 1) * dk + (CHUNK + 1) * (2 * dk + 2 * dv))
    mfma_frac = flops_prefill / (ms_per_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    prefill_bytes_min = th * (2 * (2 * dk + dv) + 8 + 2 * dv) + 2 * n_seq * H * dk * dv * 4
    log(f"prefill {ms_per_step:.3f} ms/step (prep {prep_ms:.3f}, scan {scan_ms:.3f}); "
        f"{tok_per_s:.3e} tok/s; wall {wall:.2f}s")

    # ---------------------------------------------------------------- coefficient / readout
    # variants on the same kernels: the gated delta rule's b = eta against the Kaczmarz
    # coefficient, and the readout divided by ||q|| (unit-norm keys keep the gated rule bounded)
    variants = None
    if args.variant_steps > 0:
        s0 = sets[0]
        ku = (s0["k"].float() / s0["k"].float().norm(dim=-1, keepdim=True)).to(s0["k"].dtype)
        variants = {}
        for name, kw in (("kaczmarz", {}), ("gated", {"beta_mode": "gated"}),
                         ("kaczmarz_normalized_readout", {"normalize_q": True})):
            def vstep():
                kla.kla_prefill_chunked(s0["q"], ku, s0["v"], s0["g"], s0["eta"], base["eps"],
                                        S0=s0["S0"], n_seq=n_seq, o=s0["o"], S_T=s0["S_T"],
                                        workspace=s0["ws"], **kw)
            for _ in range(2):
                vstep()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.variant_steps):
                vstep()
            e1.record()
            torch.cuda.synchronize()
            variants[name + "_ms_per_step"] = e0.elapsed_time(e1) / args.variant_steps
        # diagonal gating (one log-decay per key channel, drawn like the scalar g), with its
        # own larger workspace
        gen = torch.Generator(device=dev).manual_seed(ki.BASE_SEED + 77)
        gd = (w.g_low * torch.rand(*s0["k"].shape, generator=gen, device=dev)).contiguous()
        wsd = torch.empty(kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv,
                                                          diagonal_gate=True),
                          dtype=torch.uint8, device=dev)

        def dstep():
            kla.kla_prefill_chunked(s0["q"], ku, s0["v"], gd, s0["eta"], base["eps"],
                                    S0=s0["S0"], n_seq=n_seq, o=s0["o"], S_T=s0["S_T"],
                                    workspace=wsd)
        for _ in range(2):
            dstep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.variant_steps):
            dstep()
        e1.record()
        torch.cuda.synchronize()
        variants["diagonal_gate_ms_per_step"] = dg_ms = e0.elapsed_time(e1) / args.variant_steps
        # algorithmic HBM bytes of the diagonal-gated prefill: q, k, v read, o written, g read
        # per key channel, eta read; S0 read and S_T written
        es = s0["q"].element_size()
        dg_bytes = n_tok * H * (es * (2 * dk + 2 * dv) + 4 * dk + 4) + 2 * n_seq * H * dk * dv * 4
        dg_gbs = dg_bytes / (dg_ms * 1e-3) / 1e9
        variants["diagonal_gate_roofline"] = {
            "bound": "hbm", "achieved": dg_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": dg_gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_step": dg_bytes}
        del wsd, gd
        variants["note"] = ("same workload, one input set (cache-warm, unlike the headline), "
                            "unit-norm keys; one kla_prefill_chunked call per step; "
                            "diagonal_gate: g per key channel [n_tok, H, d_k]")
        log(f"variants: {variants}")

    # backward pass on the same workload: gradients for seeded cotangents dO, dS_T
    backward = None
    if args.backward_steps > 0:
        s0 = sets[0]
        ct = ki.cotangents({"q": s0["q"], "k": s0["k"], "v": s0["v"], "n_seq": n_seq},
                           seed=ki.BASE_SEED + 99, device=dev)
        wsb = torch.empty(kla.kla_prefill_backward_workspace_bytes(n_seq, n_tok, H, dk, dv,
                                                                   s0["q"].dtype),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return kla.kla_prefill_backward(s0["q"], s0["k"], s0["v"], s0["g"], s0["eta"],
                                            base["eps"], ct["dO"], S0=s0["S0"],
                                            dS_T=ct["dS_T"], n_seq=n_seq, workspace=wsb)
        for _ in range(2):
            bstep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.backward_steps):
            bstep()
        e1.record()
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / args.backward_steps
        # algorithmic HBM bytes: q, k, v, dO, g, eta read and dq, dk, dv, dg, deta written once
        # per token-head, S0 and dS_T read and dS0 written once per (sequence, head)
        es = s0["q"].element_size()
        bwd_bytes = (n_tok * H * (es * (4 * dk + 3 * dv) + 16)
                     + 3 * n_seq * H * dk * dv * 4)
        bwd_gbs = bwd_bytes / (bwd_ms * 1e-3) / 1e9
        backward = {"ms_per_step": bwd_ms, "tokens_per_s": n_tok / (bwd_ms * 1e-3),
                    "roofline": {"bound": "hbm", "achieved": bwd_gbs, "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": bwd_gbs / PEAK_HBM_GBS,
                                 "algorithmic_bytes_per_step": bwd_bytes},
                    "steps": args.backward_steps, "workspace_bytes": wsb.numel(),
                    "note": "kla_prefill_backward (dq, dk, dv, dg, deta, dS0) on the prefill "
                            "workload, one input set; each step runs the prep, the chunk scan "
                            "storing every chunk's state, the adjoint scan and the per-chunk "
                            "gradients"}
        log(f"backward: {bwd_ms:.3f} ms/step")
        del wsb, ct
    del sets

    # ---------------------------------------------------------------- decode
    wd = ki.WORKLOADS[3]
    nd = args.decode_steps
    log(f"decode workload {wd.name}: generating {nd} steps of inputs")
    d = ki.decode_inputs(wd, steps=nd, device=dev)
    S = d["S"].clone()
    od = torch.empty(wd.n_seq, wd.H, wd.d_v, dtype=wd.dtype, device=dev)
    for i in range(min(8, nd)):
        kla.kla_decode_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["eta"][i], d["eps"], S,
                            o=od, inplace=True)
    S.copy_(d["S"])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(nd):
        kla.kla_decode_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["eta"][i], d["eps"], S,
                            o=od, inplace=True)
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / nd
    dec_th = wd.n_seq * wd.H
    dec_bytes = dec_th * (8 * wd.d_k * wd.d_v + 2 * (2 * wd.d_k + wd.d_v) + 2 * wd.d_v + 8)
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    log(f"decode {dec_ms * 1e3:.1f} us/step, {dec_gbs:.0f} GB/s")
    # diagonal gating: the same steps with one log-decay per key channel (the g read grows
    # by 4 d_k bytes per token-head)
    gdd = (wd.g_low * torch.rand(nd, wd.n_seq, wd.H, wd.d_k, device=dev)).contiguous()
    S.copy_(d["S"])
    for i in range(min(8, nd)):
        kla.kla_decode_step(d["q"][i], d["k"][i], d["v"][i], gdd[i], d["eta"][i], d["eps"], S,
                            o=od, inplace=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(nd):
        kla.kla_decode_step(d["q"][i], d["k"][i], d["v"][i], gdd[i], d["eta"][i], d["eps"], S,
                            o=od, inplace=True)
    e1.record()
    torch.cuda.synchronize()
    dec_diag_ms = e0.elapsed_time(e1) / nd
    dec_diag_gbs = (dec_bytes + dec_th * 4 * (wd.d_k - 1)) / (dec_diag_ms * 1e-3) / 1e9
    log(f"decode, diagonal gate: {dec_diag_ms * 1e3:.1f} us/step, {dec_diag_gbs:.0f} GB/s")
    del gdd
    del d, S

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        qc, kc, vc = (base[x].cpu() for x in ("q", "k", "v"))
        gc, ec, sc = base["g"].cpu(), base["eta"].cpu(), base["S0"].cpu()
        cu = [i * (n_tok // n_seq) for i in range(n_seq + 1)]
        log("timing the fp64 oracle on the host")
        t0 = time.perf_counter()
        oracle.prefill(qc, kc, vc, gc, ec, base["eps"], S0=sc, cu_seqlens=cu)
        cpu_s = time.perf_counter() - t0
        cpu = {"value": n_tok / cpu_s, "unit": "tokens/s", "cores": oracle.max_threads(),
               "kind": "oracle",
               "sample": f"the whole prefill workload ({n_seq} seq x {H} heads x "
                         f"{n_tok // n_seq} tokens, d=128) through the fp64 tokenwise oracle, "
                         f"{cpu_s:.2f} s wall"}

    if args.copy_calibration_mib > 0:
        a = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration_mib} MiB done")
        del a, b

    traffic = measured_traffic()
    line = {
        "metric": "prefill tokens/s (%MFMA peak) + decode tokens/s (%HBM peak), 1 MI355X",
        "value": tok_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": n_seq, "heads": H, "seq_len": n_tok // n_seq,
                   "d_k": dk, "d_v": dv, "chunk": CHUNK, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "kla_scan_kernel", "bound": "hbm", "achieved": scan_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": scan_gbs / PEAK_HBM_GBS,
                     "traffic": traffic, "avg_launch_ms": scan_ms,
                     "algorithmic_bytes_per_launch": scan_bytes},
        "prefill": {"mfma_frac": mfma_frac, "algorithmic_flops_per_step": flops_prefill,
                    "hbm_frac_at_min_bytes": prefill_bytes_min / (ms_per_step * 1e-3) / 1e9
                    / PEAK_HBM_GBS,
                    "prep_ms": prep_ms, "scan_ms": scan_ms},
        "decode": {"workload": wd.name, "tokens_per_s": wd.n_seq / (dec_ms * 1e-3),
                   "ms_per_step": dec_ms, "steps": nd,
                   "roofline": {"kernel": "kla_decode_kernel", "bound": "hbm",
                                "achieved": dec_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": dec_gbs / PEAK_HBM_GBS},
                   "diagonal_gate": {"ms_per_step": dec_diag_ms,
                                     "tokens_per_s": wd.n_seq / (dec_diag_ms * 1e-3),
                                     "achieved_GBs": dec_diag_gbs,
                                     "frac": dec_diag_gbs / PEAK_HBM_GBS}},
        "variants": variants,
        "backward": backward,
        "cpu_baseline": cpu,
        "context": "the pages report 3.54 vs 1.65 tok/s decode at 32K context (2.1x KLA/GDN) for "
                   "a whole 0.4B model at batch 1 on NVIDIA A100 80GB (FLA library); not this "
                   "metric or workload",
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
