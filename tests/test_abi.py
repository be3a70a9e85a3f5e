"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol that
include/kla.h declares, and rejects bad arguments with the documented status before any
HIP call is made (validation happens on the host before the first launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_kla_amd as kla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kla.load_library()


def test_header_declares_the_two_calls():
    names = declared_functions()
    assert "kla_prefill_chunked" in names and "kla_decode_step" in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kla.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(kla_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR):
        assert lib.kla_status_string(st).decode().startswith("KLA_")
    assert lib.kla_version() >= 100


def test_workspace_bytes_formula(lib):
    # cu + chunk offsets + G (fp32 per token-head) + decays (3 x 64 fp32 per chunk-head)
    # + T and P as ten 16 x 16 blocks each per chunk-head in the element type; the chunk
    # count is bounded by ceil(n/64) + n_seq, and each part is padded to 256 bytes
    n_seq, n_tok, H = 4, 16384, 16
    nch = (n_tok + 63) // 64 + n_seq
    pad = lambda x: (x + 255) // 256 * 256
    for torch_dt, es in ((kla.torch.bfloat16, 2), (kla.torch.float32, 4)):
        nb = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, 128, 128, torch_dt)
        want = (2 * pad(4 * (n_seq + 1)) + pad(4 * n_tok * H) + pad(4 * nch * H * 192)
                + 2 * pad(es * nch * H * 2560))
        assert nb == want, (torch_dt, nb, want)
    # bf16 halves the tiles against fp32
    assert (kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, 128, 128, kla.torch.float32)
            - kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, 128, 128)) == 2 * 2 * nch * H * 2560
    assert kla.kla_prefill_workspace_bytes(4, 100, 16, 96, 128) == 0
    assert kla.kla_prefill_workspace_bytes(0, 100, 16, 128, 128) == 0
    assert lib.kla_prefill_workspace_bytes(4, 100, 16, 128, 128, 7) == 0  # unknown dtype


def test_workspace_two_level_scratch(lib):
    """Dense input of few long sequences adds the two-level scan's fp32 scratch: per
    (sequence, segment but the last, head) [N_g | M_g] ([d_k][d_v + d_k]) and the chained
    incoming state ([d_k][d_v]), and per chunk-head the log contraction bound of the warm-up
    test.  The shape rule: n_seq H d_v / 32 workgroups of the sequential scan below 128 and
    G = min(512 / that, chunks per sequence / 32)."""
    pad = lambda x: (x + 255) // 256 * 256
    n_seq, n_tok, H, dk, dv = 1, 65536, 16, 128, 128
    nch = (n_tok + 63) // 64 + n_seq
    seq = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, scan_segments=1)
    G = min(512 // (n_seq * H * dv // 32), (n_tok // 64) // 32)
    assert G == 8
    units = n_seq * (G - 1) * H * dk
    want = seq + pad(4 * units * (dv + dk)) + pad(4 * units * dv) + pad(4 * nch * H)
    assert kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv) == want
    assert kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, scan_segments=8) == want
    # an explicit count: segments of ceil(chunks / G) chunks, G recounted over what holds tokens
    units7 = n_seq * 6 * H * dk
    assert (kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, scan_segments=7)
            == seq + pad(4 * units7 * (dv + dk)) + pad(4 * units7 * dv) + pad(4 * nch * H))
    # 5 chunks in 4 requested segments: 2 chunks each, so 3 segments
    units3 = 1 * 2 * H * dk
    assert (kla.kla_prefill_workspace_bytes(1, 300, H, dk, dv, scan_segments=4)
            == kla.kla_prefill_workspace_bytes(1, 300, H, dk, dv, scan_segments=1)
            + pad(4 * units3 * (dv + dk)) + pad(4 * units3 * dv) + pad(4 * (5 + 1) * H))
    # no scratch: enough sequences to fill the chip, short sequences, uneven totals (packed
    # input only), the diagonal gate
    for args in ((4, n_tok, H, dk, dv), (1, 64 * 63, H, dk, dv), (3, 3 * 4096 + 1, 2, dk, dv)):
        assert (kla.kla_prefill_workspace_bytes(*args)
                == kla.kla_prefill_workspace_bytes(*args, scan_segments=1)), args
    assert (kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, diagonal_gate=True)
            == kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, diagonal_gate=True,
                                               scan_segments=1))


FAKE = 1 << 32  # 16-byte aligned non-NULL addresses 4 GiB apart; never dereferenced on error paths


def _prefill(lib, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, eps=1e-6, S0=None, o=FAKE * 6,
             S_T=None, cu=None, cu_host=None, n_seq=2, total=256, H=4, dk=128, dv=128, dtype=BF16,
             ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return lib.kla_prefill_chunked(a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["S0"],
                                   a["o"], a["S_T"], a["cu"], a["cu_host"], a["n_seq"], a["total"],
                                   a["H"], a["dk"], a["dv"], a["dtype"], a["ws"], a["ws_bytes"],
                                   a["stream"])


def _decode(lib, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, eps=1e-6, S=FAKE * 7,
             o=FAKE * 6, S_new=FAKE * 7, B=4, H=2, dk=128, dv=128, dtype=BF16, stream=None)
    a.update(over)
    return lib.kla_decode_step(a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["S"], a["o"],
                               a["S_new"], a["B"], a["H"], a["dk"], a["dv"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(n_seq=0), INVALID),
    (dict(H=0), INVALID),
    (dict(total=-1), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(eps=float("inf")), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(dk=96), UNSUPPORTED),
    (dict(dv=512), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED),
    (dict(total=255), INVALID),          # dense: not divisible by n_seq
    (dict(q=FAKE + 4), INVALID),         # misaligned (16-byte vector loads)
    (dict(o=FAKE * 6 + 8), INVALID),     # o is written with vector stores
    (dict(g=FAKE * 4 + 2), INVALID),     # fp32 needs 4-byte alignment
    (dict(o=FAKE), INVALID),             # o overlaps q
    (dict(ws=None), WORKSPACE),
    (dict(ws=FAKE * 64, ws_bytes=16), WORKSPACE),
    # one 64-token chunk of o would span 64 * 40000 * 256 * 4 bytes > 2^31
    (dict(dtype=0, H=40000, dv=256, total=2, n_seq=2), UNSUPPORTED),
])
def test_prefill_argument_errors(lib, over, status):
    assert _prefill(lib, **over) == status
    assert lib.kla_last_error().decode() != ""


def test_prefill_host_cu_seqlens_validated(lib):
    bad = [(0, 100, 90), (1, 100, 256), (0, 100, 200)]
    for cu in bad:
        arr = (ctypes.c_int32 * 3)(*cu)
        st = _prefill(lib, cu=FAKE * 8, cu_host=ctypes.cast(arr, ctypes.c_void_p), total=256)
        assert st == INVALID, cu
    # a good table gets past the host checks and stops at the missing workspace
    arr = (ctypes.c_int32 * 3)(0, 100, 256)
    assert _prefill(lib, cu=FAKE * 8, cu_host=ctypes.cast(arr, ctypes.c_void_p)) == WORKSPACE


@pytest.mark.parametrize("over,status", [
    (dict(S=None), INVALID),
    (dict(B=-1), INVALID),
    (dict(dk=32), UNSUPPORTED),
    (dict(dv=100), UNSUPPORTED),
    (dict(eps=-0.5), INVALID),
    (dict(dtype=3), UNSUPPORTED),
    (dict(S_new=FAKE * 7 + 16), INVALID),  # partial overlap with S
    (dict(v=FAKE * 3 + 1), INVALID),      # bf16 needs 2-byte alignment
    (dict(S=FAKE * 9 + 4, S_new=FAKE * 10), INVALID),  # the state streams as float4
])
def test_decode_argument_errors(lib, over, status):
    assert _decode(lib, **over) == status


def test_last_error_is_thread_local_text(lib):
    _decode(lib, dk=32)
    assert "d_k" in lib.kla_last_error().decode()


def _opts(mode=0, normq=0, pos=None, diag=0, prec=0):
    return ctypes.pointer(kla.KlaOptions(mode, normq, pos, diag, 0, prec))


@pytest.mark.parametrize("opts,status", [
    (lambda: _opts(mode=6), UNSUPPORTED),       # unknown coefficient mode
    (lambda: _opts(mode=-1), UNSUPPORTED),
    (lambda: _opts(mode=3, pos=FAKE + 2), INVALID),   # int32 offsets need 4-byte alignment
    (lambda: _opts(prec=2), UNSUPPORTED),       # unknown precision
    (lambda: _opts(prec=-1), UNSUPPORTED),
])
def test_options_errors(lib, opts, status):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, o=FAKE * 6)
    ws = FAKE * 64
    nb = kla.kla_prefill_workspace_bytes(2, 256, 4, 128, 128)
    st = lib.kla_prefill_chunked_ex(a["q"], a["k"], a["v"], a["g"], a["eta"], 1e-6, None, a["o"],
                                    None, None, None, 2, 256, 4, 128, 128, BF16, ws, nb, opts(),
                                    None)
    assert st == status
    st = lib.kla_prefill_prepare_ex(a["q"], a["k"], a["g"], a["eta"], 1e-6, None, None, 2, 256, 4,
                                    128, 128, BF16, ws, nb, opts(), None)
    assert st == status
    st = lib.kla_decode_step_ex(a["q"], a["k"], a["v"], a["g"], a["eta"], 1e-6, FAKE * 7, a["o"],
                                FAKE * 7, 4, 2, 128, 128, BF16, opts(), None)
    assert st == status
    assert lib.kla_last_error().decode() != ""


def test_split_precision_workspace_and_entry_points(lib):
    """Split precision stores T and P as hi and lo bf16 blocks: twice their region for bf16
    inputs, nothing for fp32 ones (exact fp32 products already).  It runs through
    kla_prefill_chunked_ex with the scalar gate only."""
    pad = lambda x: (x + 255) // 256 * 256
    n_seq, n_tok, H, dk, dv = 4, 16384, 16, 128, 128
    nch = (n_tok + 63) // 64 + n_seq
    base = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv)
    split = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, precision="split")
    assert split - base == 2 * pad(2 * nch * H * 2560)
    assert (kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, kla.torch.float32,
                                            precision="split")
            == kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, kla.torch.float32))
    # split precision takes no two-level scan: no segment scratch for a long sequence
    assert (kla.kla_prefill_workspace_bytes(1, 65536, 16, dk, dv, precision="split")
            - kla.kla_prefill_workspace_bytes(1, 65536, 16, dk, dv, scan_segments=1)
            == 2 * pad(2 * ((65536 + 63) // 64 + 1) * 16 * 2560))
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, o=FAKE * 6)
    ws = FAKE * 64
    nb = kla.kla_prefill_workspace_bytes(2, 256, 4, 128, 128, precision="split")
    # the staged entry point and the backward refuse it
    st = lib.kla_prefill_prepare_ex(a["q"], a["k"], a["g"], a["eta"], 1e-6, None, None, 2, 256, 4,
                                    128, 128, BF16, ws, nb, _opts(prec=1), None)
    assert st == UNSUPPORTED
    st = lib.kla_prefill_backward_ex(
        FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1e-6, None, FAKE * 6, None, FAKE * 7,
        FAKE * 8, FAKE * 9, FAKE * 10, FAKE * 11, FAKE * 12, None, None, 2, 256, 4, 128, 128,
        BF16, FAKE * 64, lib.kla_prefill_backward_workspace_bytes(2, 256, 4, 128, 128, BF16),
        _opts(prec=1), None)
    assert st == UNSUPPORTED
    # with the diagonal gate
    st = lib.kla_prefill_chunked_ex(a["q"], a["k"], a["v"], a["g"], a["eta"], 1e-6, None, a["o"],
                                    None, None, None, 2, 256, 4, 128, 128, BF16, ws, nb,
                                    _opts(diag=1, prec=1), None)
    assert st == UNSUPPORTED
    # a workspace sized for the bf16 mode is too small for it
    st = lib.kla_prefill_chunked_ex(a["q"], a["k"], a["v"], a["g"], a["eta"], 1e-6, None, a["o"],
                                    None, None, None, 2, 256, 4, 128, 128, BF16, ws,
                                    kla.kla_prefill_workspace_bytes(2, 256, 4, 128, 128),
                                    _opts(prec=1), None)
    assert st == WORKSPACE


def test_options_default_pointer_is_accepted_up_to_the_workspace_check(lib):
    # NULL options are the defaults: argument checking proceeds to the missing workspace
    st = lib.kla_prefill_chunked_ex(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1e-6, None,
                                    FAKE * 6, None, None, None, 2, 256, 4, 128, 128, BF16, None, 0,
                                    None, None)
    assert st == WORKSPACE


def test_diagonal_gate_workspace_and_entry_points(lib):
    # the diagonal-gated variant needs the decayed key and query tiles: three [64, d_k]
    # tiles in the element type and d_k fp32 decays per chunk-head on top of the default
    # workspace
    n_seq, n_tok, H, dk, dv = 4, 16384, 16, 128, 128
    base = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv)
    diag = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv, diagonal_gate=True)
    nch = (n_tok + 63) // 64 + n_seq
    assert diag >= base + nch * H * (2 * 3 * 64 * dk + 4 * dk) and diag % 256 == 0
    # NULL options give the default size
    assert lib.kla_prefill_workspace_bytes_ex(n_seq, n_tok, H, dk, dv, BF16, None) == base
    # the default-size workspace is too small for the diagonal-gated prefill
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, o=FAKE * 6)
    st = lib.kla_prefill_chunked_ex(a["q"], a["k"], a["v"], a["g"], a["eta"], 1e-6, None,
                                    a["o"], None, None, None, 2, 256, 4, 128, 128, BF16, FAKE * 64,
                                    kla.kla_prefill_workspace_bytes(2, 256, 4, 128, 128),
                                    _opts(diag=1), None)
    assert st == WORKSPACE
    # the two-call prefill does not take the diagonal gate
    nb = kla.kla_prefill_workspace_bytes(2, 256, 4, 128, 128, diagonal_gate=True)
    st = lib.kla_prefill_prepare_ex(a["q"], a["k"], a["g"], a["eta"], 1e-6, None, None, 2, 256,
                                    4, 128, 128, BF16, FAKE * 64, nb, _opts(diag=1), None)
    assert st == UNSUPPORTED
    assert "chunked_ex" in lib.kla_last_error().decode()


def _bwd_call(lib, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, eta=FAKE * 5, eps=1e-6, S0=None,
             dO=FAKE * 6, dST=None, dq=FAKE * 7, dk=FAKE * 8, dv=FAKE * 9, dg=FAKE * 10,
             deta=FAKE * 11, dS0=FAKE * 12, cu=None, cu_host=None, n_seq=2, n_tok=256, H=4,
             dk_=128, dv_=128, dtype=BF16, ws=FAKE * 64, ws_bytes=None)
    a.update(over)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.kla_prefill_backward_workspace_bytes(a["n_seq"], a["n_tok"], a["H"],
                                                                 128, 128, BF16)
    return lib.kla_prefill_backward(
        a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["S0"], a["dO"], a["dST"], a["dq"],
        a["dk"], a["dv"], a["dg"], a["deta"], a["dS0"], a["cu"], a["cu_host"], a["n_seq"],
        a["n_tok"], a["H"], a["dk_"], a["dv_"], a["dtype"], a["ws"], a["ws_bytes"], None)


def test_backward_workspace_and_errors(lib):
    # the backward workspace holds the forward one plus, per chunk-head, the incoming state
    # and the outgoing state's cotangent (d_k x d_v each), dU (64 x d_v) and (I + L)^{-1} (ten
    # 16 x 16 blocks), all in the operand type (bf16 by default); dR goes to dv
    n_seq, n_tok, H, dk, dv = 4, 16384, 16, 128, 128
    nch = (n_tok + 63) // 64 + n_seq
    nb = kla.kla_prefill_backward_workspace_bytes(n_seq, n_tok, H, dk, dv)
    base = kla.kla_prefill_workspace_bytes(n_seq, n_tok, H, dk, dv)
    assert nb >= base + nch * H * 2 * (2 * dk * dv + 64 * dv + 10 * 256)
    assert nb < base + nch * H * 2 * (2 * dk * dv + 64 * dv + 10 * 256) + 8 * 256
    assert nb % 256 == 0
    assert kla.kla_prefill_backward_workspace_bytes(n_seq, n_tok, H, 96, dv) == 0
    cases = [
        (dict(ws_bytes=1024), WORKSPACE),
        (dict(dk_=96), UNSUPPORTED),
        (dict(dO=None), INVALID),
        (dict(dq=None), INVALID),
        (dict(dk=FAKE + 4), INVALID),                 # misaligned (16-byte vector access)
        (dict(dg=FAKE * 10 + 2), INVALID),            # misaligned (4-byte scalars)
        (dict(dg=FAKE * 5), INVALID),                 # dg overlaps eta
        (dict(dv=FAKE * 7), INVALID),                 # two gradients in one buffer
        (dict(n_tok=255), INVALID),                   # dense: 255 tokens over 2 sequences
        (dict(eps=-1.0), INVALID),
        (dict(dtype=7), UNSUPPORTED),
    ]
    for over, want in cases:
        assert _bwd_call(lib, **over) == want, (over, lib.kla_last_error())


def _bwd_ex_call(lib, opts, ws_bytes, **over):
    a = dict(n_seq=2, n_tok=256, H=4, dk_=128, dv_=128, dg=FAKE * 10)
    a.update(over)
    return lib.kla_prefill_backward_ex(
        FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1e-6, None, FAKE * 6, None, FAKE * 7,
        FAKE * 8, FAKE * 9, a["dg"], FAKE * 11, FAKE * 12, None, None, a["n_seq"], a["n_tok"],
        a["H"], a["dk_"], a["dv_"], BF16, FAKE * 64, ws_bytes,
        None if opts is None else ctypes.pointer(opts), None)


def test_backward_diagonal_gate_workspace_and_errors(lib):
    # Appendix B.5 (diagonal gating): the backward workspace adds the forward's decayed tiles
    # K o exp(G), Q o exp(G), K o exp(G_last - G) ([64][d_k] per chunk-head, operand type) and
    # exp(G_last) ([d_k] fp32), and every chunk's A (ten 16 x 16 blocks, operand type)
    n_seq, n_tok, H, dk, dv = 2, 256, 4, 128, 128
    nch = (n_tok + 63) // 64 + n_seq
    diag = kla.KlaOptions(0, 0, None, 1)
    nb = lib.kla_prefill_backward_workspace_bytes(n_seq, n_tok, H, dk, dv, BF16)
    assert lib.kla_prefill_backward_workspace_bytes_ex(n_seq, n_tok, H, dk, dv, BF16, None) == nb
    nd = lib.kla_prefill_backward_workspace_bytes_ex(n_seq, n_tok, H, dk, dv, BF16,
                                                     ctypes.pointer(diag))
    assert nd >= nb + nch * H * (3 * 64 * dk * 2 + 4 * dk + 2 * 10 * 256)
    assert nd % 256 == 0
    assert lib.kla_prefill_backward_workspace_bytes_ex(n_seq, n_tok, H, 96, dv, BF16,
                                                       ctypes.pointer(diag)) == 0
    # the scalar-gate workspace is too small for the diagonal gate
    assert _bwd_ex_call(lib, diag, nb) == WORKSPACE
    # dg is [n_tok, H, d_k] fp32 under diagonal gating: 512 KiB here, so a dg starting 256 KiB
    # below eta overlaps it (a scalar gate's 4 KiB dg would not)
    assert _bwd_ex_call(lib, diag, nd, dg=FAKE * 5 - (256 << 10)) == INVALID
    assert "overlap" in lib.kla_last_error().decode()
    # unknown coefficient mode, and a precision the backward does not take
    assert _bwd_ex_call(lib, kla.KlaOptions(9, 0, None, 0), nb) == UNSUPPORTED
    assert _bwd_ex_call(lib, kla.KlaOptions(0, 0, None, 1, 0, 1), nd) == UNSUPPORTED


def test_noalloc_rejects_a_problem_beyond_its_static_scratch(lib):
    # the size check runs on the host before any HIP call; fp32 inputs take the staged path,
    # whose workspace holds every chunk's T and P
    n_seq, n_tok, H = 1, 1 << 20, 64
    assert lib.kla_prefill_workspace_bytes_ex(n_seq, n_tok, H, 128, 128, F32, None) > (64 << 20)
    st = lib.kla_prefill_chunked_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1e-6, None,
                                         FAKE * 6, None, None, None, n_seq, n_tok, H, 128, 128,
                                         F32, None, None)
    assert st == WORKSPACE
    assert "static scratch" in lib.kla_last_error().decode()
