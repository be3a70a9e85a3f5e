"""The allocation-free prefill entry point (kla_prefill_chunked_noalloc), called through the C
ABI: its output must equal, bit for bit, that of kla_prefill_chunked_ex with a workspace on the
same inputs (both run the same kernels), on two calls in a row whose second is smaller, so the
static scratch holding the first call's contents cannot leak into the second."""
import ctypes

import pytest
import torch

import kla_inputs as ki

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = 1


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_delta_rule_kla_amd as kla
    return kla, kla.load_library()


def _call_noalloc(lib, d, n_seq, o, S_T):
    n_tok, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.kla_prefill_chunked_noalloc(
        p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["eta"]), d["eps"], p(d["S0"]), p(o),
        p(S_T), p(d["cu_seqlens"]), None, n_seq, n_tok, H, dk, dv, BF16, None, stream)


def _case(seed, lens, H, dk, dv):
    w = ki.Workload(seed, "noalloc", len(lens), H, dk, dv, torch.bfloat16, lens=tuple(lens),
                    s0_var=0.01)
    d = ki.prefill_inputs(w)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_noalloc_matches_workspace_entry_point_twice(lib):
    kla, L = lib
    # a larger packed call, then a smaller one with fewer sequences, heads and a ragged tail
    for seed, lens, H in ((61, (700, 0, 1300, 64, 333), 8), (62, (130, 5), 2)):
        d = _case(seed, lens, H, 128, 128)
        n_seq = len(lens)
        print(f"noalloc case seed={seed} lens={lens} H={H}", flush=True)
        o_ref, S_ref = kla.kla_prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["eta"],
                                               d["eps"], S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                                               n_seq=n_seq)
        o = torch.full_like(o_ref, float("nan"))
        S_T = torch.full_like(S_ref, float("nan"))
        st = _call_noalloc(L, d, n_seq, o, S_T)
        assert st == 0, L.kla_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "output differs from the workspace entry point"
        assert torch.equal(S_T, S_ref), "final state differs from the workspace entry point"


def test_noalloc_rejects_a_problem_beyond_its_scratch(lib):
    kla, L = lib
    n_seq, n_tok, H = 1, 1 << 20, 64  # fp32 inputs: ~1 GB of per-chunk tiles
    need = L.kla_prefill_workspace_bytes_ex(n_seq, n_tok, H, 128, 128, 0, None)
    assert need > (64 << 20)
    FAKE = 1 << 32
    st = L.kla_prefill_chunked_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1e-6, None,
                                       FAKE * 6, None, None, None, n_seq, n_tok, H, 128, 128,
                                       0, None, None)
    assert st == 3  # KLA_ERR_WORKSPACE, nothing enqueued
    assert "static scratch" in L.kla_last_error().decode()
