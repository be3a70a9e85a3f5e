"""fp64 CPU oracle of the Kaczmarz Linear Attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  The HIP library never loads it, and it shares no code
with the HIP path.

Two independent routes to the same function (paper "Kaczmarz Linear
Attention", arXiv 2605.08587):

* :func:`prefill` / :func:`decode` -- the tokenwise recurrence of Algorithm 1
  (left panel) with the coefficient of Eq. (3), in plain C (``kla_oracle.c``),
  fp64, OpenMP over (sequence, head).  This is THE oracle.
* :mod:`oracle.chunkwise` -- the chunkwise solve of Propositions 3 and 4
  (Eq. (7)-(9)) in numpy fp64, used only to pin the oracle (tokenwise ==
  chunkwise) and to expose the per-chunk intermediates (b, G, T).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kla_oracle.c")
# KLA_ORACLE_LIBRARY names another build of kla_oracle.c (the sanitized build of the CPU
# tests); the default is the one build() writes next to the source
_LIB = os.environ.get("KLA_ORACLE_LIBRARY") or os.path.join(_HERE, "libkla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``kla_oracle.c`` with gcc (-O3, no fast-math, OpenMP) into ``libkla_oracle.so``."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile ``kla_oracle.c`` with gcc under AddressSanitizer and UndefinedBehaviorSanitizer
    into ``path`` (loading it needs gcc's libasan preloaded)."""
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c99", "-fopenmp", "-fPIC",
         "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", _SRC,
         "-o", path, "-lm"])
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kla_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double, dp,
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp,
                                           ctypes.c_int]
        lib.kla_oracle_prefill.restype = ctypes.c_int
        lib.kla_oracle_decode.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double, dp,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          dp, dp, ctypes.c_int]
        lib.kla_oracle_decode.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.kla_oracle_prefill_v.argtypes = lib.kla_oracle_prefill.argtypes + [
            ctypes.c_int, ctypes.c_int, i64p, ctypes.c_int]
        lib.kla_oracle_prefill_v.restype = ctypes.c_int
        lib.kla_oracle_decode_v.argtypes = lib.kla_oracle_decode.argtypes + [
            ctypes.c_int, ctypes.c_int, i64p, ctypes.c_int]
        lib.kla_oracle_decode_v.restype = ctypes.c_int
        lib.kla_oracle_max_threads.argtypes = []
        lib.kla_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Widen a tensor/array to a C-contiguous float64 numpy array (lossless for bf16/fp32)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU or device): widen on the CPU
        x = x.detach().to("cpu")
        import torch  # local: the oracle itself needs only numpy
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kla_oracle_max_threads())


# Write-coefficient variants (the C oracle's `mode`; see the header of kla_oracle.c).
MODES = {"kaczmarz": 0, "gated": 1, "key_norm": 2, "inv_t": 3, "inv_sqrt_t": 4, "inv_log_t": 5}


def _mode(beta_mode) -> int:
    return MODES[beta_mode] if isinstance(beta_mode, str) else int(beta_mode)


def _i64(x, n):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int64))
    if a.shape != (n,):
        raise ValueError(f"pos_offset must have {n} entries")
    return a


def prefill(q, k, v, g, eta, eps, S0=None, cu_seqlens=None, n_seq=None, nthreads=0,
            beta_mode="kaczmarz", normalize_q=False, pos_offset=None):
    """Tokenwise fp64 prefill.

    q, k: [n_tok, H, d_k]; v: [n_tok, H, d_v]; g, eta: [n_tok, H];
    g: [n_tok, H, d_k] instead for diagonal gating (one log-decay per key channel, paper
    Appendix B.5; shaped like k);
    S0: [n_seq, H, d_k, d_v] or None (zeros); cu_seqlens: [n_seq+1] token offsets,
    or None for one sequence per leading batch row when q is [B, T, H, d_k].
    beta_mode / normalize_q / pos_offset ([n_seq]: the first token of sequence n is at
    position pos_offset[n] + 1) select the variants.
    Returns (o [n_tok, H, d_v], S_T [n_seq, H, d_k, d_v]) as float64 numpy arrays,
    with o shaped like v.
    """
    q, k, v, g, eta = (_f64(x) for x in (q, k, v, g, eta))
    gdiag = g.shape == q.shape
    out_shape = v.shape
    if cu_seqlens is None and q.ndim == 4:  # dense [B, T, H, d]
        B, T = q.shape[0], q.shape[1]
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if cu_seqlens is None:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
        else:
            cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                            dtype=np.int64)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    q = q.reshape(-1, H, dk)
    k = k.reshape(-1, H, dk)
    v = v.reshape(-1, H, dv)
    g = g.reshape(-1, H, dk) if gdiag else g.reshape(-1, H)
    eta = eta.reshape(-1, H)
    ns = len(cu) - 1
    if n_seq is not None and n_seq != ns:
        raise ValueError("n_seq does not match cu_seqlens")
    if int(cu[-1]) != q.shape[0]:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    S0a = None if S0 is None else _f64(S0).reshape(ns, H, dk, dv)
    cu = np.ascontiguousarray(cu)
    o = np.empty((q.shape[0], H, dv), dtype=np.float64)
    ST = np.empty((ns, H, dk, dv), dtype=np.float64)
    po = _i64(pos_offset, ns)
    rc = _load().kla_oracle_prefill_v(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(S0a),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ns, H, dk, dv, _ptr(o), _ptr(ST),
        int(nthreads), _mode(beta_mode), 1 if normalize_q else 0,
        None if po is None else po.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        1 if gdiag else 0)
    if rc != 0:
        raise RuntimeError("kla_oracle_prefill failed")
    return o.reshape(out_shape), ST


def decode(q, k, v, g, eta, eps, S, nthreads=0, beta_mode="kaczmarz", normalize_q=False,
           pos_offset=None):
    """One tokenwise fp64 step per sequence.

    q, k: [B, H, d_k]; v: [B, H, d_v]; g, eta: [B, H]; S: [B, H, d_k, d_v].
    g: [B, H, d_k] instead for diagonal gating (shaped like k).
    Variants as in prefill (pos_offset [B]: this token is at position pos_offset + 1).
    Returns (o [B, H, d_v], S_new [B, H, d_k, d_v]) as float64 numpy arrays.
    """
    q, k, v, g, eta, S = (_f64(x) for x in (q, k, v, g, eta, S))
    gdiag = g.shape == q.shape
    B, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, H, dv), dtype=np.float64)
    Sn = np.empty((B, H, dk, dv), dtype=np.float64)
    po = _i64(pos_offset, B)
    rc = _load().kla_oracle_decode_v(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(eta), float(eps), _ptr(S), B, H, dk, dv,
        _ptr(o), _ptr(Sn), int(nthreads), _mode(beta_mode), 1 if normalize_q else 0,
        None if po is None else po.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        1 if gdiag else 0)
    if rc != 0:
        raise RuntimeError("kla_oracle_decode failed")
    return o, Sn
