#!/usr/bin/env python3
"""Benchmark of the KLA forward hot path on one MI355X (prints ONE JSON line).

A step is one chunkwise prefill (the prep/UT kernel, then the chunk-scan kernel
with the fused output) over the layer-scale workload: B=4 sequences, H=16 heads,
T=4096 tokens, d_k=d_v=128, bf16 q/k/v, fp32 g/eta/state, chunk 64, random S0.
``value`` is prefill tokens/s over the timed steps.  Four copies of the inputs and
workspace are rotated so the 256 MB last-level cache cannot serve them from one
step to the next.

The same run measures the decode step (the other half of the metric) on the
decode workload (B=256, H=16, d=128, fp32 state from N(0, 0.05), 512 consecutive
in-place steps with fresh bf16 q/k/v and fp32 g/eta per step), and times the fp64
CPU oracle on the host cores as a reported baseline.

Per-kernel durations come from HIP events recorded on the launch stream in a pass right
after the timed loop, over the same rotating inputs: each call issued as its two halves
(kla_prefill_prepare, then kla_prefill_scan, exactly what kla_prefill_chunked enqueues)
with an event before, between and after them.  A third pass times the same calls one by
one (an event pair each) for the median and minimum call time.

Algorithmic work (per token-head, C = 64; the minimum any chunkwise implementation moves and
multiplies):
  prefill bytes      = 2 (2 d_k + d_v) e + 8 + 2 d_v e        (q, k, v, g, eta read; o written)
                       + 8 d_k d_v per (sequence, head)        (S0 read, S_T written), e = 2 (bf16)
                     = 1064 B per token-head on the layer workload (d = 128, T = 4096)
  prefill MFMA flops = 6 d_k d_v + (C-1) d_k + (C+1)(2 d_k + 2 d_v)
  decode bytes       = 8 d_k d_v + 2 (2 d_k + d_v) + 2 d_v + 8
The roofline object is for the dominant kernel (the chunk scan): the prefill's algorithmic
bytes per launch over the scan's mean event-timed duration.  ``step`` gives the same bytes
and flops over the whole step (prep + scan).  The long-context (T = 65536) and packed
wide-head workloads are timed the same way on one input set each (their inputs exceed the
256 MB last-level cache), the packed one followed by 128 decode steps from its state.
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
TRAFFIC_NOTE = ("rocprofv3 read-request and WRITE_SIZE counters of this scan kernel build, "
                "committed under profiles/ (not measured in this run)")


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


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    ap.add_argument("--workload-steps", type=int, default=5,
                    help="timed calls of the long-context and packed workloads (0 = skip)")
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
    def prefill_bytes_flops(n_tok, n_seq, H, dk, dv, es):
        """The algorithmic bytes and MFMA flops of one prefill call (the formulas above)."""
        th = n_tok * H
        nb = th * (es * (2 * dk + dv) + 8 + es * dv) + 2 * n_seq * H * dk * dv * 4
        nf = th * (6 * dk * dv + (CHUNK - 1) * dk + (CHUNK + 1) * (2 * dk + 2 * dv))
        return nb, nf

    def time_prefill(sets, meta, steps, warmup):
        """Time `steps` kla_prefill_chunked calls rotating over `sets` (one event pair around
        the back-to-back calls), then split them into the prep kernel and the scan: with
        the sequential scan by a pass of prepare + scan calls (what kla_prefill_chunked
        enqueues) with an event between the halves; with the two-level scan (reachable
        through kla_prefill_chunked only) by a pass of prepare calls alone, the scan phases
        taking the rest."""
        n_seq, dv, eps = meta["n_seq"], meta["d_v"], meta["eps"]

        def whole(s):
            kla.kla_prefill_chunked(s["q"], s["k"], s["v"], s["g"], s["eta"], eps,
                                    S0=s.get("S0"), cu_seqlens=s.get("cu"), n_seq=n_seq,
                                    o=s["o"], S_T=s["S_T"], workspace=s["ws"])

        def prepare(s):
            kla.kla_prefill_prepare(s["q"], s["k"], s["g"], s["eta"], eps, s["ws"], n_seq=n_seq,
                                    d_v=dv, cu_seqlens=s.get("cu"))

        def scan(s):
            kla.kla_prefill_scan(s["q"], s["k"], s["v"], s["ws"], n_seq=n_seq, S0=s.get("S0"),
                                 o=s["o"], S_T=s["S_T"])
        for i in range(warmup):
            whole(sets[i % len(sets)])
        torch.cuda.synchronize()
        e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_start.record()
        for i in range(steps):
            whole(sets[i % len(sets)])
        e_end.record()
        torch.cuda.synchronize()
        ms = e_start.elapsed_time(e_end) / steps
        # the same calls timed one by one (an event pair around each), for the median and min
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            evc[i][0].record()
            whole(sets[i % len(sets)])
            evc[i][1].record()
        torch.cuda.synchronize()
        per_call = sorted(e[0].elapsed_time(e[1]) for e in evc)
        calls = {"median_ms": per_call[len(per_call) // 2], "min_ms": per_call[0]}
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            s = sets[i % len(sets)]
            ev[i][0].record()
            prepare(s)
            ev[i][1].record()
            if not meta.get("two_level"):
                scan(s)
            ev[i][2].record()
        torch.cuda.synchronize()
        prep = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        if meta.get("two_level"):
            return ms, prep, ms - prep, calls
        return ms, prep, sum(e[1].elapsed_time(e[2]) for e in ev) / steps, calls

    def make_set(inp, dev, ws_bytes, dtype):
        n_tok, H, dk = inp["q"].shape
        dv = inp["v"].shape[-1]
        return dict(q=inp["q"], k=inp["k"], v=inp["v"], g=inp["g"], eta=inp["eta"],
                    S0=inp["S0"], cu=inp["cu_seqlens"],
                    o=torch.empty(n_tok, H, dv, dtype=dtype, device=dev),
                    S_T=torch.empty(inp["n_seq"], H, dk, dv, dtype=torch.float32, device=dev),
                    ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev))

    def workload_leg(widx, steps, warmup):
        """One of the long-context or packed workloads: timing and roofline fractions."""
        wl = ki.WORKLOADS[widx]
        inp = ki.prefill_inputs(wl, device=dev)
        n_tok, H_, dk_, dv_ = inp["q"].shape[0], wl.H, wl.d_k, wl.d_v
        es = inp["q"].element_size()
        ws_b = kla.kla_prefill_workspace_bytes(inp["n_seq"], n_tok, H_, dk_, dv_, wl.dtype)
        s = make_set(inp, dev, ws_b, wl.dtype)
        # dense input whose workspace holds the two-level scan's scratch runs that scan
        two_level = inp["cu_seqlens"] is None and ws_b != kla.kla_prefill_workspace_bytes(
            inp["n_seq"], n_tok, H_, dk_, dv_, wl.dtype, scan_segments=1)
        meta = {"n_seq": inp["n_seq"], "d_v": dv_, "eps": inp["eps"], "two_level": two_level}
        ms, prep, scan, _ = time_prefill([s], meta, steps, warmup)
        nb, nf = prefill_bytes_flops(n_tok, inp["n_seq"], H_, dk_, dv_, es)
        out = {"workload": wl.name, "tokens": n_tok, "ms_per_call": ms, "prep_ms": prep,
               "scan_ms": scan, "scan": "two-level" if two_level else "sequential",
               "tokens_per_s": n_tok / (ms * 1e-3),
               "mfma_frac": nf / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
               "hbm_frac": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "scan_hbm_frac": nb / (scan * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "algorithmic_bytes": nb, "algorithmic_flops": nf, "steps": steps}
        if wl.decode_steps:
            nd = wl.decode_steps
            dd = ki.decode_inputs(wl, steps=nd, device=dev, S=s["S_T"])
            S = s["S_T"].clone()
            od = torch.empty(inp["n_seq"], H_, dv_, dtype=wl.dtype, device=dev)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(nd):
                kla.kla_decode_step(dd["q"][i], dd["k"][i], dd["v"][i], dd["g"][i], dd["eta"][i],
                                    dd["eps"], S, o=od, inplace=True)
            e1.record()
            torch.cuda.synchronize()
            dms = e0.elapsed_time(e1) / nd
            dbytes = inp["n_seq"] * H_ * (8 * dk_ * dv_ + es * (2 * dk_ + dv_) + es * dv_ + 8)
            out["decode"] = {"steps": nd, "ms_per_step": dms,
                             "tokens_per_s": inp["n_seq"] / (dms * 1e-3),
                             "hbm_frac": dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "note": "state of 16.8 MB stays in the last-level cache"}
            # the same steps captured once into a HIP graph and replayed (no per-call host
            # work): what a serving loop gets at this small batch, where launches dominate
            S.copy_(s["S_T"])

            def loop():
                for i in range(nd):
                    kla.kla_decode_step(dd["q"][i], dd["k"][i], dd["v"][i], dd["g"][i],
                                        dd["eta"][i], dd["eps"], S, o=od, inplace=True)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                loop()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                loop()
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            gms = e0.elapsed_time(e1) / nd
            out["decode"]["graph_ms_per_step"] = gms
            out["decode"]["graph_tokens_per_s"] = inp["n_seq"] / (gms * 1e-3)
            del graph, dd, S
        log(f"{wl.name}: {ms:.3f} ms/call (prep {prep:.3f}, scan {scan:.3f}), "
            f"{n_tok / (ms * 1e-3):.3e} tok/s")
        del inp, s
        return out

    w = ki.WORKLOADS[1]
    log(f"prefill workload {w.name}: generating inputs")
    base = ki.prefill_inputs(w, device=dev)
    n_seq, H, dk, dv = base["n_seq"], w.H, w.d_k, w.d_v
    n_tok = base["q"].shape[0]
    ws_bytes = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, w.dtype)
    sets = []
    for _ in range(4):
        cp = {key: (val.clone() if isinstance(val, torch.Tensor) else val)
              for key, val in base.items()}
        sets.append(make_set(cp, dev, ws_bytes, w.dtype))
    K = args.steps
    log(f"timing {K} prefill steps")
    t0 = time.perf_counter()
    ms_per_step, prep_ms, scan_ms, call_stats = time_prefill(sets, {"n_seq": n_seq, "d_v": dv,
                                                        "eps": base["eps"]}, K, args.warmup)
    wall = time.perf_counter() - t0
    tok_per_s = n_tok / (ms_per_step * 1e-3)
    prefill_bytes, flops_prefill = prefill_bytes_flops(n_tok, n_seq, H, dk, dv, 2)
    scan_gbs = prefill_bytes / (scan_ms * 1e-3) / 1e9
    step_gbs = prefill_bytes / (ms_per_step * 1e-3) / 1e9
    mfma_frac = flops_prefill / (ms_per_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    log(f"prefill {ms_per_step:.3f} ms/step (prep {prep_ms:.3f}, scan {scan_ms:.3f}); "
        f"{tok_per_s:.3e} tok/s; wall {wall:.2f}s")
    others = {}
    if args.workload_steps > 0:
        for widx, key in ((2, "long_context"), (4, "packed")):
            others[key] = workload_leg(widx, args.workload_steps, 1)

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
        # split operand precision (T R, P U and the state update on hi/lo bf16 pairs) on the
        # headline's keys, with its own larger workspace
        wss = torch.empty(kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv,
                                                          precision="split"),
                          dtype=torch.uint8, device=dev)

        def sstep():
            kla.kla_prefill_chunked(s0["q"], s0["k"], s0["v"], s0["g"], s0["eta"], base["eps"],
                                    S0=s0["S0"], n_seq=n_seq, o=s0["o"], S_T=s0["S_T"],
                                    workspace=wss, precision="split")
        for _ in range(2):
            sstep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.variant_steps):
            sstep()
        e1.record()
        torch.cuda.synchronize()
        variants["split_precision_ms_per_step"] = e0.elapsed_time(e1) / args.variant_steps
        del wss
        variants["note"] = ("same workload, one input set (cache-warm, unlike the headline), "
                            "unit-norm keys (split precision: the headline's keys); one "
                            "kla_prefill_chunked call per step; diagonal_gate: g per key "
                            "channel [n_tok, H, d_k]")
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
        del wsb
        # the same under diagonal gating (g per key channel, Appendix B.5), its own workspace
        gen = torch.Generator(device=dev).manual_seed(ki.BASE_SEED + 78)
        gd = (w.g_low * torch.rand(*s0["k"].shape, generator=gen, device=dev)).contiguous()
        wsbd = torch.empty(kla.kla_prefill_backward_workspace_bytes(
            n_seq, n_tok, H, dk, dv, s0["q"].dtype, diagonal_gate=True),
            dtype=torch.uint8, device=dev)

        def bdstep():
            return kla.kla_prefill_backward(s0["q"], s0["k"], s0["v"], gd, s0["eta"],
                                            base["eps"], ct["dO"], S0=s0["S0"],
                                            dS_T=ct["dS_T"], n_seq=n_seq, workspace=wsbd)
        for _ in range(2):
            bdstep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.backward_steps):
            bdstep()
        e1.record()
        torch.cuda.synchronize()
        bwdd_ms = e0.elapsed_time(e1) / args.backward_steps
        # g read and dg written per key channel (fp32) instead of per token-head
        bwdd_bytes = (n_tok * H * (es * (4 * dk + 3 * dv) + 8 * dk + 8)
                      + 3 * n_seq * H * dk * dv * 4)
        bwdd_gbs = bwdd_bytes / (bwdd_ms * 1e-3) / 1e9
        backward["diagonal_gate"] = {
            "ms_per_step": bwdd_ms, "tokens_per_s": n_tok / (bwdd_ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": bwdd_gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": bwdd_gbs / PEAK_HBM_GBS,
                         "algorithmic_bytes_per_step": bwdd_bytes},
            "workspace_bytes": wsbd.numel(),
            "note": "g per key channel [n_tok, H, d_k] ~ U(g_low, 0); dg of that shape"}
        log(f"backward (diagonal gate): {bwdd_ms:.3f} ms/step")
        del wsbd, ct, gd
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
               "kind": "oracle", "host_cpus": len(os.sched_getaffinity(0)),
               "cpu_model": cpu_model(),
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
                     "traffic": traffic, "traffic_source": TRAFFIC_NOTE if traffic else None,
                     "avg_launch_ms": scan_ms, "algorithmic_bytes_per_launch": prefill_bytes},
        "step": {"hbm_frac": step_gbs / PEAK_HBM_GBS, "mfma_frac": mfma_frac,
                 "algorithmic_bytes": prefill_bytes, "algorithmic_flops": flops_prefill,
                 "note": "prep + scan, the same algorithmic bytes and flops over the step time"},
        "prefill": {"mfma_frac": mfma_frac, "prep_ms": prep_ms, "scan_ms": scan_ms,
                    "call_ms_median": call_stats["median_ms"], "call_ms_min": call_stats["min_ms"],
                    "call_note": "the same calls timed one by one (an event pair each); "
                                 "ms_per_step is one event pair around all of them"},
        "workloads": others,
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
