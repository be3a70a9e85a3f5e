"""Kaczmarz Linear Attention forward pass on MI355X (gfx950): Python binding of libkla.so.

The binding only marshals arguments: it checks tensor placement, dtypes and
shapes, allocates outputs and the workspace with torch, and calls the C ABI of
``include/kla.h`` on torch's current HIP stream.  Every step of the computation
runs in the HIP kernels of ``csrc/``; there is no fallback.  If libkla.so is
missing the first call raises an error naming the build step.

Functions mirror the C entry points:

* :func:`kla_prefill_chunked` -- chunkwise prefill (q, k, v, g, eta, eps, S0) -> (o, S_T)
* :func:`kla_prefill_prepare` / :func:`kla_prefill_scan` -- its two halves
* :func:`kla_decode_step`     -- one decode step (q, k, v, g, eta, eps, S) -> (o, S')
* :func:`kla_prefill_chunk_stage` -- per-chunk b, G, T (and W, U~) for unit checks
* :func:`kla_prefill_backward` -- gradients (dq, dk, dv, dg, deta, dS0) of the prefill
* :func:`kla_prefill_workspace_bytes`, :func:`kla_prefill_backward_workspace_bytes`
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["kla_prefill_chunked", "kla_prefill_prepare", "kla_prefill_scan", "kla_decode_step",
           "kla_prefill_chunk_stage", "kla_prefill_workspace_bytes", "kla_prefill_backward",
           "kla_prefill_backward_workspace_bytes", "library_path",
           "load_library", "CHUNK", "KlaError"]

CHUNK = 64
_PKG = os.path.dirname(os.path.abspath(__file__))
# KLA_LIBRARY names another build of the same C ABI (the sanitized host build of the CPU
# tests); the default is the in-tree libkla.so
_LIB_PATH = os.environ.get("KLA_LIBRARY") or os.path.join(_PKG, "libkla.so")
_lib = None

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class KlaError(RuntimeError):
    """A non-OK kla_status returned by libkla.so."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkla.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python gated_delta_rule_kla_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kla_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kla_prefill_workspace_bytes.restype = sz
    lib.kla_prefill_chunked.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i32, i32, i32,
                                        i32, i32, ctypes.c_int, vp, sz, vp]
    lib.kla_prefill_chunked.restype = ctypes.c_int
    lib.kla_prefill_prepare.argtypes = [vp, vp, vp, vp, f32, vp, vp, i32, i32, i32, i32, i32,
                                        ctypes.c_int, vp, sz, vp]
    lib.kla_prefill_prepare.restype = ctypes.c_int
    lib.kla_prefill_scan.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                     vp, sz, vp]
    lib.kla_prefill_scan.restype = ctypes.c_int
    lib.kla_prefill_chunk_stage.argtypes = [vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, i32,
                                            i32, i32, i32, i32, ctypes.c_int, vp, sz, vp]
    lib.kla_prefill_chunk_stage.restype = ctypes.c_int
    lib.kla_decode_step.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, i32, i32, i32,
                                    ctypes.c_int, vp]
    lib.kla_decode_step.restype = ctypes.c_int
    opt_p = ctypes.POINTER(KlaOptions)
    lib.kla_prefill_workspace_bytes_ex.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, opt_p]
    lib.kla_prefill_workspace_bytes_ex.restype = sz
    lib.kla_prefill_chunked_ex.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i32, i32,
                                           i32, i32, i32, ctypes.c_int, vp, sz, opt_p, vp]
    lib.kla_prefill_chunked_ex.restype = ctypes.c_int
    lib.kla_prefill_prepare_ex.argtypes = [vp, vp, vp, vp, f32, vp, vp, i32, i32, i32, i32, i32,
                                           ctypes.c_int, vp, sz, opt_p, vp]
    lib.kla_prefill_prepare_ex.restype = ctypes.c_int
    lib.kla_decode_step_ex.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, i32, i32, i32,
                                       ctypes.c_int, opt_p, vp]
    lib.kla_decode_step_ex.restype = ctypes.c_int
    lib.kla_prefill_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i32,
                                                i32, i32, i32, i32, ctypes.c_int, opt_p, vp]
    lib.kla_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.kla_prefill_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kla_prefill_backward_workspace_bytes.restype = sz
    lib.kla_prefill_backward_workspace_bytes_ex.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int,
                                                            opt_p]
    lib.kla_prefill_backward_workspace_bytes_ex.restype = sz
    lib.kla_prefill_backward.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp,
                                         sz, vp]
    lib.kla_prefill_backward.restype = ctypes.c_int
    lib.kla_prefill_backward_ex.argtypes = lib.kla_prefill_backward.argtypes[:-1] + [opt_p, vp]
    lib.kla_prefill_backward_ex.restype = ctypes.c_int
    lib.kla_status_string.argtypes = [ctypes.c_int]
    lib.kla_status_string.restype = ctypes.c_char_p
    lib.kla_last_error.argtypes = []
    lib.kla_last_error.restype = ctypes.c_char_p
    lib.kla_version.argtypes = []
    lib.kla_version.restype = i32
    _lib = lib
    return lib


# Write-coefficient variants (kla_beta_mode in include/kla.h).
BETA_MODES = {"kaczmarz": 0, "gated": 1, "key_norm": 2, "inv_t": 3, "inv_sqrt_t": 4,
              "inv_log_t": 5}


class KlaOptions(ctypes.Structure):
    """Mirror of ``kla_options``: the write-coefficient mode, the normalised readout, the
    per-sequence position offsets (device int32 or NULL), the diagonal gate and the
    segment count of the two-level scan (0 = by shape, 1 = sequential scan) and the operand
    precision (PRECISIONS)."""
    _fields_ = [("beta_mode", ctypes.c_int32), ("normalize_q", ctypes.c_int32),
                ("pos_offset", ctypes.c_void_p), ("diagonal_gate", ctypes.c_int32),
                ("scan_segments", ctypes.c_int32), ("precision", ctypes.c_int32)]


# Operand precision of the bf16 prefill's products (kla_precision in include/kla.h).
PRECISIONS = {"bf16": 0, "split": 1}


def _options(beta_mode, normalize_q, pos_offset, n_rows, dev, diagonal_gate=False,
             scan_segments=0, precision="bf16"):
    """ctypes pointer to a KlaOptions (None = the defaults).  beta_mode is a name from
    BETA_MODES or its integer code; pos_offset an int32 device tensor of n_rows entries;
    diagonal_gate: g holds one log-decay per key channel; scan_segments as in kla_options;
    precision a name from PRECISIONS or its code."""
    mode = BETA_MODES[beta_mode] if isinstance(beta_mode, str) else int(beta_mode)
    prec = PRECISIONS[precision] if isinstance(precision, str) else int(precision)
    if (mode == 0 and not normalize_q and pos_offset is None and not diagonal_gate
            and not scan_segments and prec == 0):
        return None
    if pos_offset is not None:
        _need(pos_offset, "pos_offset", torch.int32, dev)
        if pos_offset.numel() != n_rows:
            raise ValueError(f"pos_offset must have {n_rows} entries")
    return ctypes.pointer(KlaOptions(mode, 1 if normalize_q else 0,
                                     None if pos_offset is None else pos_offset.data_ptr(),
                                     1 if diagonal_gate else 0, int(scan_segments), prec))


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise KlaError(status, f"{lib.kla_status_string(status).decode()}: "
                               f"{lib.kla_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kla_prefill_workspace_bytes(n_seq: int, total_tokens: int, n_heads: int, d_k: int,
                                d_v: int, dtype=torch.bfloat16, diagonal_gate: bool = False,
                                scan_segments: int = 0, precision="bf16") -> int:
    """Workspace bytes a prefill of this size and element type needs (0 for unsupported
    sizes); diagonal_gate sizes it for the diagonal-gated variant, scan_segments and
    precision for those choices (kla_options)."""
    prec = PRECISIONS[precision] if isinstance(precision, str) else int(precision)
    opts = (ctypes.pointer(KlaOptions(0, 0, None, 1 if diagonal_gate else 0, int(scan_segments),
                                      prec))
            if diagonal_gate or scan_segments or prec else None)
    return int(load_library().kla_prefill_workspace_bytes_ex(n_seq, total_tokens, n_heads, d_k,
                                                             d_v, _DTYPES[dtype], opts))


def _flatten_tokens(q, k, v, g, eta, cu_seqlens, n_seq):
    """Accept dense [B, T, H, d] or flat [n_tok, H, d] token-major tensors."""
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs flat [n_tok, H, d] inputs")
        B, T = q.shape[:2]
        n_seq = B
        q, k, v = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v))
        g = g.reshape(B * T, *g.shape[2:])
        eta = eta.reshape(B * T, eta.shape[-1])
    elif q.dim() != 3:
        raise ValueError("q must be [n_tok, H, d_k] or [B, T, H, d_k]")
    if n_seq is None:
        n_seq = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    return q, k, v, g, eta, n_seq


def kla_prefill_chunked(q, k, v, g, eta, eps: float = 1e-6, S0=None, cu_seqlens=None,
                        n_seq=None, *, cu_seqlens_host=None, output_final_state=True, o=None,
                        S_T=None, workspace=None, beta_mode="kaczmarz", normalize_q=False,
                        pos_offset=None, scan_segments=0, precision="bf16"):
    """Chunkwise KLA prefill (paper section 4, Eq. (7)-(9); chunk = 64 tokens).

    q, k: [n_tok, H, d_k] or [B, T, H, d_k] (fp32 or bf16); v like q with d_v;
    g, eta: [n_tok, H] / [B, T, H] fp32 (a g shaped like k selects diagonal gating: one
    log-decay per key channel, paper Appendix B.5); S0: [n_seq, H, d_k, d_v] fp32 or None;
    cu_seqlens: int32 device [n_seq + 1] for packed sequences, or None (dense;
    n_seq sequences of equal length).  Returns (o, S_T); S_T is None when
    output_final_state is False.  Pass S_T=S0 to update the state in place.
    beta_mode / normalize_q / pos_offset select the variants of kla_options; scan_segments
    the chunk scan of dense input (0: by shape, 1: sequential, G >= 2: two-level with G
    segments per sequence); precision the operand precision of bf16 products ("bf16" or
    "split", kla_precision).
    """
    shape_v = v.shape
    q, k, v, g, eta, n_seq = _flatten_tokens(q, k, v, g, eta, cu_seqlens, n_seq)
    dev = q.device
    _need(q, "q", device=dev)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(k, "k", dt, dev)
    _need(v, "v", dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(eta, "eta", torch.float32, dev)
    n_tok, H, d_k = q.shape
    d_v = v.shape[-1]
    diag = tuple(g.shape) == (n_tok, H, d_k)
    if (k.shape != q.shape or v.shape[:2] != (n_tok, H) or (g.shape != (n_tok, H) and not diag)
            or eta.shape != (n_tok, H)):
        raise ValueError("inconsistent q/k/v/g/eta shapes")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if cu_seqlens.numel() != n_seq + 1:
            raise ValueError("cu_seqlens must have n_seq + 1 entries")
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
    if S0 is not None:
        _need(S0, "S0", torch.float32, dev)
        if S0.shape != (n_seq, H, d_k, d_v):
            raise ValueError(f"S0 must be [{n_seq}, {H}, {d_k}, {d_v}]")
    if o is None:
        o = torch.empty((n_tok, H, d_v), dtype=dt, device=dev)
    else:
        _need(o, "o", dt, dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((n_seq, H, d_k, d_v), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need(S_T, "S_T", torch.float32, dev)
    lib = load_library()
    opts = _options(beta_mode, normalize_q, pos_offset, n_seq, dev, diagonal_gate=diag,
                    scan_segments=scan_segments, precision=precision)
    ws_bytes = int(lib.kla_prefill_workspace_bytes_ex(n_seq, n_tok, H, d_k, d_v, _DTYPES[dt],
                                                      opts))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    host_ptr = None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr())
    _check(lib.kla_prefill_chunked_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(S0), _ptr(o), _ptr(S_T),
        _ptr(cu_seqlens), host_ptr, n_seq, n_tok, H, d_k, d_v, _DTYPES[dt], _ptr(workspace),
        workspace.numel(), opts, _stream(dev)))
    return o.reshape(shape_v), S_T


def kla_prefill_backward_workspace_bytes(n_seq: int, total_tokens: int, n_heads: int, d_k: int,
                                         d_v: int, dtype=torch.bfloat16,
                                         diagonal_gate: bool = False) -> int:
    """Workspace bytes kla_prefill_backward needs (0 for unsupported sizes); diagonal_gate
    sizes it for the diagonal-gated variant."""
    opts = (ctypes.pointer(KlaOptions(0, 0, None, 1, 0, 0)) if diagonal_gate else None)
    return int(load_library().kla_prefill_backward_workspace_bytes_ex(
        n_seq, total_tokens, n_heads, d_k, d_v, _DTYPES[dtype], opts))


def kla_prefill_backward(q, k, v, g, eta, eps: float, dO, S0=None, dS_T=None, cu_seqlens=None,
                         n_seq=None, *, cu_seqlens_host=None, workspace=None,
                         need_dS0=True, beta_mode="kaczmarz", normalize_q=False,
                         pos_offset=None):
    """Gradients of the prefill for the cotangents dO (like o) and dS_T (like S_T, or None).

    Inputs as for :func:`kla_prefill_chunked`: a g shaped like k selects diagonal gating (one
    log-decay per key channel); beta_mode / normalize_q / pos_offset select the variant of the
    forward call.  Returns (dq, dk, dv, dg, deta, dS0), shaped like q, k, v, g, eta and S0
    ([n_seq, H, d_k, d_v]; None when need_dS0 is False).
    """
    shape_q, shape_v, shape_g, shape_eta = q.shape, v.shape, g.shape, eta.shape
    q, k, v, g, eta, n_seq = _flatten_tokens(q, k, v, g, eta, cu_seqlens, n_seq)
    dev = q.device
    _need(q, "q", device=dev)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(k, "k", dt, dev)
    _need(v, "v", dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(eta, "eta", torch.float32, dev)
    n_tok, H, d_k = q.shape
    d_v = v.shape[-1]
    diag = tuple(g.shape) == (n_tok, H, d_k)
    if (k.shape != q.shape or v.shape[:2] != (n_tok, H) or (g.shape != (n_tok, H) and not diag)
            or eta.shape != (n_tok, H)):
        raise ValueError("inconsistent q/k/v/g/eta shapes")
    dO = dO.reshape(n_tok, H, d_v)
    _need(dO, "dO", dt, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if cu_seqlens.numel() != n_seq + 1:
            raise ValueError("cu_seqlens must have n_seq + 1 entries")
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
    for t, name in ((S0, "S0"), (dS_T, "dS_T")):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if t.shape != (n_seq, H, d_k, d_v):
                raise ValueError(f"{name} must be [{n_seq}, {H}, {d_k}, {d_v}]")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(g)
    deta = torch.empty_like(eta)
    dS0 = torch.empty((n_seq, H, d_k, d_v), dtype=torch.float32, device=dev) if need_dS0 else None
    lib = load_library()
    opts = _options(beta_mode, normalize_q, pos_offset, n_seq, dev, diagonal_gate=diag)
    ws_bytes = int(lib.kla_prefill_backward_workspace_bytes_ex(n_seq, n_tok, H, d_k, d_v,
                                                               _DTYPES[dt], opts))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    host_ptr = None if host_cu is None else ctypes.c_void_p(host_cu.data_ptr())
    _check(lib.kla_prefill_backward_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(S0), _ptr(dO),
        _ptr(dS_T), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(deta), _ptr(dS0),
        _ptr(cu_seqlens), host_ptr, n_seq, n_tok, H, d_k, d_v, _DTYPES[dt], _ptr(workspace),
        workspace.numel(), opts, _stream(dev)))
    return (dq.reshape(shape_q), dk.reshape(shape_q), dv.reshape(shape_v), dg.reshape(shape_g),
            deta.reshape(shape_eta), dS0)


def kla_prefill_prepare(q, k, g, eta, eps, workspace, *, n_seq, d_v, cu_seqlens=None,
                        beta_mode="kaczmarz", normalize_q=False, pos_offset=None):
    """First half of the prefill: sequence tables, decays, T and P of every chunk into
    ``workspace`` (a uint8 device tensor of at least kla_prefill_workspace_bytes(...) bytes).
    q, k: [n_tok, H, d_k]; g, eta: [n_tok, H]; variants as in kla_prefill_chunked."""
    dev = k.device
    _need(k, "k", device=dev)
    if k.dtype not in _DTYPES:
        raise TypeError("k must be float32 or bfloat16")
    _need(q, "q", k.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(eta, "eta", torch.float32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    n_tok, H, d_k = k.shape
    opts = _options(beta_mode, normalize_q, pos_offset, n_seq, dev)
    _check(load_library().kla_prefill_prepare_ex(
        _ptr(q), _ptr(k), _ptr(g), _ptr(eta), float(eps), _ptr(cu_seqlens), None, n_seq, n_tok,
        H, d_k, d_v, _DTYPES[k.dtype], _ptr(workspace), workspace.numel(), opts, _stream(dev)))


def kla_prefill_scan(q, k, v, workspace, *, n_seq, S0=None, o=None, S_T=None):
    """Second half of the prefill: the chunk scan with outputs, reading the workspace that
    kla_prefill_prepare filled for the same k, g, eta and sizes.  Returns (o, S_T)."""
    dev = q.device
    dt = q.dtype
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, dt, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    n_tok, H, d_k = q.shape
    d_v = v.shape[-1]
    if o is None:
        o = torch.empty((n_tok, H, d_v), dtype=dt, device=dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, dev)
    if S_T is not None:
        _need(S_T, "S_T", torch.float32, dev)
    _check(load_library().kla_prefill_scan(
        _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(o), _ptr(S_T), n_seq, n_tok, H, d_k, d_v,
        _DTYPES[dt], _ptr(workspace), workspace.numel(), _stream(dev)))
    return o, S_T


def kla_decode_step(q, k, v, g, eta, eps: float, S, *, o=None, S_new=None, inplace=False,
                    beta_mode="kaczmarz", normalize_q=False, pos_offset=None):
    """One KLA decode step per sequence (paper Algorithm 1, tokenwise panel).

    q, k: [B, H, d_k]; v: [B, H, d_v] (fp32 or bf16); g, eta: [B, H] fp32;
    S: [B, H, d_k, d_v] fp32.  Returns (o, S_new); inplace=True writes S' into S.
    A g shaped like k ([B, H, d_k]) selects diagonal gating (one log-decay per key channel).
    Variants as in kla_prefill_chunked (pos_offset: int32 [B], this token is at
    position pos_offset + 1).
    """
    dev = q.device
    _need(q, "q", device=dev)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(k, "k", dt, dev)
    _need(v, "v", dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(eta, "eta", torch.float32, dev)
    _need(S, "S", torch.float32, dev)
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    diag = tuple(g.shape) == (B, H, d_k)
    if S.shape != (B, H, d_k, d_v) or (g.shape != (B, H) and not diag) or eta.shape != (B, H):
        raise ValueError("inconsistent decode shapes")
    if o is None:
        o = torch.empty((B, H, d_v), dtype=dt, device=dev)
    if inplace:
        S_new = S
    elif S_new is None:
        S_new = torch.empty_like(S)
    _need(S_new, "S_new", torch.float32, dev)
    opts = _options(beta_mode, normalize_q, pos_offset, B, dev, diagonal_gate=diag)
    _check(load_library().kla_decode_step_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(S), _ptr(o), _ptr(S_new),
        B, H, d_k, d_v, _DTYPES[dt], opts, _stream(dev)))
    return o, S_new


def kla_prefill_chunk_stage(k, v, g, eta, eps: float = 1e-6, cu_seqlens=None, n_seq=None, *,
                            want_wy=False):
    """Per-chunk stage of the prefill (b, G, T; optionally W and U~), for unit checks.

    Returns dict(beta [n_tok, H], G [n_tok, H], T [n_chunks, H, 64, 64], W, Ut).
    """
    dev = k.device
    if k.dim() == 4:
        B, T = k.shape[:2]
        n_seq = B
        k, v = (x.reshape(B * T, *x.shape[2:]) for x in (k, v))
        g, eta = (x.reshape(B * T, x.shape[-1]) for x in (g, eta))
    dt = k.dtype
    _need(k, "k", device=dev)
    _need(v, "v", dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(eta, "eta", torch.float32, dev)
    n_tok, H, d_k = k.shape
    d_v = v.shape[-1]
    if n_seq is None:
        n_seq = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is None:
        Tn = n_tok // n_seq
        n_chunks = n_seq * ((Tn + CHUNK - 1) // CHUNK)
    else:
        cu = cu_seqlens.cpu().tolist()
        n_chunks = sum((cu[i + 1] - cu[i] + CHUNK - 1) // CHUNK for i in range(n_seq))
    lib = load_library()
    beta = torch.zeros((n_tok, H), dtype=torch.float32, device=dev)
    G = torch.zeros((n_tok, H), dtype=torch.float32, device=dev)
    T = torch.zeros((max(n_chunks, 1), H, CHUNK, CHUNK), dtype=torch.float32, device=dev)
    W = torch.zeros((n_tok, H, d_k), dtype=torch.float32, device=dev) if want_wy else None
    Ut = torch.zeros((n_tok, H, d_v), dtype=torch.float32, device=dev) if want_wy else None
    ws_bytes = int(lib.kla_prefill_workspace_bytes(n_seq, n_tok, H, d_k, d_v, _DTYPES[dt]))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # chunk indices written by the kernel are below the true chunk count, which sizes T
    _check(lib.kla_prefill_chunk_stage(
        _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(beta), _ptr(G), _ptr(T), _ptr(W),
        _ptr(Ut), _ptr(cu_seqlens), None, n_seq, n_tok, H, d_k, d_v, _DTYPES[dt], _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return dict(beta=beta, G=G, T=T[:n_chunks], W=W, Ut=Ut)
