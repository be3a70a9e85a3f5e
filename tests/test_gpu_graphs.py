"""The entry points under HIP graph capture (through torch.cuda.graph).

The library only enqueues kernels on the caller's stream: no allocation, memset, copy or
synchronisation inside a call once the caller supplies the workspace and outputs.  So a decode
loop or a prefill can be captured once and replayed.  Each test captures, then replays several
times with eager work of the program between the replays and new inputs copied into the
captured buffers, and checks every replay against the eager calls on the same inputs bit for
bit (the kernels are deterministic: fixed reduction order, no atomics).
"""
import pytest
import torch

import kla_inputs as ki

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_delta_rule_kla_amd as m
    m.load_library()
    return m


def capture(fn):
    """Warm up `fn` on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("diag", [False, True])
def test_decode_loop_graph_replay(kla, diag):
    """Sixteen in-place decode steps of the packed workload's shape (16 sequences x 8 heads,
    d_k = 128, d_v = 256, bf16) as one graph, replayed three times from new start states."""
    steps = 16
    w = ki.WORKLOADS[4]
    dd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
          for k, v in ki.decode_inputs(w, steps=steps, diag=diag).items()}
    S = dd["S"].clone()
    outs = [torch.empty(w.n_seq, w.H, w.d_v, dtype=w.dtype, device=DEV) for _ in range(steps)]

    def loop():
        for t in range(steps):
            kla.kla_decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["eta"][t],
                                dd["eps"], S, o=outs[t], inplace=True)

    graph = capture(loop)
    gen = torch.Generator(device=DEV).manual_seed(77)
    for rep in range(3):
        S0 = 0.2 * torch.randn(S.shape, generator=gen, device=DEV)
        # eager reference from S0, on buffers of its own
        Se = S0.clone()
        ref = []
        for t in range(steps):
            o, _ = kla.kla_decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t],
                                       dd["eta"][t], dd["eps"], Se, inplace=True)
            ref.append(o)
        torch.cuda.synchronize()
        S.copy_(S0)
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        for t in range(steps):
            assert torch.equal(outs[t], ref[t]), f"replay {rep}, step {t}: o differs"
        assert torch.equal(S, Se), f"replay {rep}: state differs"


@pytest.mark.parametrize("segments", [0, 4])
def test_prefill_graph_replay(kla, segments):
    """A bf16 prefill (2 sequences x 2048 tokens x 4 heads, d = 128) with the caller's
    workspace as one graph, replayed three times on new inputs copied into the captured
    buffers; segments=4 takes the two-level scan (map, combine and segment phases)."""
    n_seq, T, H = 2, 2048, 4
    base = ki.prefill_inputs(1, T=T, n_seq=n_seq, H=H)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
    n_tok, dk, dv = n_seq * T, 128, 128
    ws = torch.empty(kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv,
                                                     scan_segments=segments),
                     dtype=torch.uint8, device=DEV)
    o = torch.empty(n_tok, H, dv, dtype=torch.bfloat16, device=DEV)
    ST = torch.empty(n_seq, H, dk, dv, dtype=torch.float32, device=DEV)

    def call(out, st):
        kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"], S0=d["S0"],
                                n_seq=n_seq, o=out, S_T=st, workspace=ws,
                                scan_segments=segments)

    graph = capture(lambda: call(o, ST))
    for rep in range(3):
        new = ki.prefill_inputs(1, T=T, n_seq=n_seq, H=H, seed=5000 + rep)
        for name in ("q", "k", "v", "g", "eta", "S0"):
            d[name].copy_(new[name])
        oe = torch.empty_like(o)
        Se = torch.empty_like(ST)
        call(oe, Se)  # eager, on the same inputs and workspace
        torch.cuda.synchronize()
        o.zero_()
        ST.zero_()
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        assert torch.equal(o, oe), f"replay {rep}: o differs"
        assert torch.equal(ST, Se), f"replay {rep}: S_T differs"


def test_noalloc_prefill_graph_replay(kla):
    """The allocation-free prefill entry point (its scratch a static array per GPU) captured into
    a graph on packed input with a ragged tail, replayed three times on new inputs; each
    replay against an eager call of the same entry point on the same inputs."""
    import ctypes
    lib = kla.load_library()
    lens, H, dk, dv = (700, 0, 1300, 64, 333), 4, 128, 128
    n_seq, n_tok = len(lens), sum(lens)

    def draw(seed):
        w = ki.Workload(seed, "graph-noalloc", n_seq, H, dk, dv, torch.bfloat16, lens=lens,
                        s0_var=0.01)
        return ki.prefill_inputs(w)

    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in draw(71).items()}
    o = torch.empty(n_tok, H, dv, dtype=torch.bfloat16, device=DEV)
    ST = torch.empty(n_seq, H, dk, dv, dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def call(out, st):
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.kla_prefill_chunked_noalloc(
            p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["eta"]), d["eps"], p(d["S0"]),
            p(out), p(st), p(d["cu_seqlens"]), None, n_seq, n_tok, H, dk, dv, 1, None, stream)
        assert rc == 0, lib.kla_last_error().decode()

    graph = capture(lambda: call(o, ST))
    for rep in range(3):
        new = draw(7100 + rep)
        for name in ("q", "k", "v", "g", "eta", "S0"):
            d[name].copy_(new[name])
        oe, Se = torch.empty_like(o), torch.empty_like(ST)
        call(oe, Se)
        torch.cuda.synchronize()
        o.zero_()
        ST.zero_()
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        assert torch.equal(o, oe), f"replay {rep}: o differs"
        assert torch.equal(ST, Se), f"replay {rep}: S_T differs"


@pytest.mark.parametrize("diag", [False, True])
def test_backward_graph_replay(kla, diag):
    """The backward pass (2 sequences x 640 tokens x 2 heads, d = 128, bf16; scalar or
    per-channel gate) captured with its outputs and workspace allocated inside the capture
    (torch's graph pool), replayed three times on new inputs and cotangents; every gradient
    against an eager call on the same inputs bit for bit."""
    n_seq, T, H = 2, 640, 2
    base = ki.prefill_inputs(1, T=T, n_seq=n_seq, H=H, diag=diag)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
    ct = {k: v.to(DEV) for k, v in ki.cotangents(base, seed=900).items()}
    out = {}

    def call():
        return kla.kla_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["eta"], d["eps"],
                                        ct["dO"], S0=d["S0"], dS_T=ct["dS_T"], n_seq=n_seq)

    def captured():
        out["grads"] = call()

    graph = capture(captured)
    for rep in range(3):
        new = ki.prefill_inputs(1, T=T, n_seq=n_seq, H=H, diag=diag, seed=6000 + rep)
        for name in ("q", "k", "v", "g", "eta", "S0"):
            d[name].copy_(new[name])
        nct = ki.cotangents(new, seed=6100 + rep)
        ct["dO"].copy_(nct["dO"])
        ct["dS_T"].copy_(nct["dS_T"])
        ref = [x.clone() for x in call()]
        torch.cuda.synchronize()
        for x in out["grads"]:
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        for name, x, y in zip(("dq", "dk", "dv", "dg", "deta", "dS0"), out["grads"], ref):
            assert torch.equal(x, y), f"replay {rep}: {name} differs"
