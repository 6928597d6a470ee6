"""float64 CPU oracle of the matrix-state affine scan (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``scan_sequence_models_amd``) and never imports it; the GPU library never
imports this package.

``oracle.c`` holds the arithmetic (the token-by-token recurrence and its
reverse-mode gradient, see its comments for the passages they follow); this
module compiles it with gcc and marshals numpy arrays.  The functions here are
pinned by the CPU tests in ``tests/test_oracle_pins.py``,
``tests/test_oracle_diag.py`` and ``tests/test_oracle_bwd.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           "-std=c11", "-Wall", "-Wextra"]
_lib = None

GDN, GLA, GDN_EW, GDN_DIAG, GLA_DIAG = 0, 1, 2, 3, 4


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it; returns the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized() -> str:
    """``liboracle_san.so``: the same source under AddressSanitizer and
    UndefinedBehaviorSanitizer, built with clang so that it shares one sanitizer
    runtime (clang's, preloaded by the process) with the library's sanitizer
    build.  Load it by setting ORACLE_LIB to its path."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    tmp = _LIB_SAN + f".tmp{os.getpid()}"
    subprocess.run([clang, *_CFLAGS, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-g", _SRC, "-o", tmp], check=True)
    os.replace(tmp, _LIB_SAN)
    return _LIB_SAN


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        lib.oracle_scan_f64.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, p, p, p, p, p, p, p, p, ctypes.c_int]
        lib.oracle_scan_f64.restype = ctypes.c_int
        lib.oracle_decode_f64.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          p, p, p, p, p, p, p, ctypes.c_int]
        lib.oracle_decode_f64.restype = ctypes.c_int
        lib.oracle_scan_bwd_f64.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int] + [p] * 14 + [ctypes.c_int]
        lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _mode(mode) -> int:
    if mode in (GDN, "gdn"):
        return GDN
    if mode in (GLA, "gla"):
        return GLA
    if mode in (GDN_EW, "gdn_ew"):
        return GDN_EW
    if mode in (GDN_DIAG, "gdn_diag"):
        return GDN_DIAG
    if mode in (GLA_DIAG, "gla_diag"):
        return GLA_DIAG
    raise ValueError(f"unknown mode {mode!r}")


def scan(mode, q, k, v, alpha, beta=None, S0=None, threads: int | None = None,
         store_o: bool = True, return_threads: bool = False):
    """Token-by-token scan in float64.

    q, k: [..., T, dk]; v: [..., T, dv]; alpha: [..., T], or [..., T, dk] (one
    decay per key channel) for "gdn_diag" and "gla_diag"; beta: [..., T] for
    "gdn" and "gdn_diag", None for "gla" and "gla_diag", [2, ..., T] (erase
    strengths, then write strengths) for "gdn_ew"; S0: [..., dv, dk] or None (zero).  Leading dimensions are
    independent heads.  Inputs are taken as float32 (exact for bfloat16
    values), S0 as float64.
    Returns (o [..., T, dv] float64 or None, ST [..., dv, dk] float64).
    """
    m = _mode(mode)
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    diag = m in (GDN_DIAG, GLA_DIAG)
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or \
            alpha.shape != (q.shape if diag else q.shape[:-1]):
        raise ValueError("shape mismatch among q, k, v, alpha")
    if m not in (GLA, GLA_DIAG):
        if beta is None:
            raise ValueError("gdn modes need beta")
        beta = _f32(beta)
        if beta.shape != ((2, *q.shape[:-1]) if m == GDN_EW else q.shape[:-1]):
            raise ValueError("beta shape mismatch")
    else:
        beta = None
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        if S0.shape != (*lead, dv, dk):
            raise ValueError("S0 shape mismatch")
    o = np.empty((*lead, T, dv), np.float64) if store_o else None
    ST = np.empty((*lead, dv, dk), np.float64)
    n = _load().oracle_scan_f64(m, BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                                threads or default_threads())
    if n < 0:
        raise RuntimeError("oracle_scan_f64 failed")
    return (o, ST, n) if return_threads else (o, ST)


def decode_step(mode, q, k, v, alpha, beta, S, threads: int | None = None):
    """One token per state, S ([N, dv, dk] float64, C-contiguous) updated in place.

    alpha: [N], or [N, dk] for "gdn_diag" and "gla_diag"; beta: [N] ("gdn",
    "gdn_diag"), None ("gla", "gla_diag") or [2, N] ("gdn_ew": erase, write).
    Returns o [N, dv] float64 = S_new q.
    """
    m = _mode(mode)
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)
    if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous):
        raise ValueError("S must be a C-contiguous float64 array (updated in place)")
    N, dk = q.shape
    dv = v.shape[1]
    if S.shape != (N, dv, dk):
        raise ValueError("S shape mismatch")
    if alpha.shape != ((N, dk) if m in (GDN_DIAG, GLA_DIAG) else (N,)):
        raise ValueError("alpha shape mismatch")
    if m not in (GLA, GLA_DIAG):
        beta = _f32(beta)
        if beta.shape != ((2, N) if m == GDN_EW else (N,)):
            raise ValueError("beta shape mismatch")
    else:
        beta = None
    o = np.empty((N, dv), np.float64)
    n = _load().oracle_decode_f64(m, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(S), _ptr(o), threads or default_threads())
    if n < 0:
        raise RuntimeError("oracle_decode_f64 failed")
    return o


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def scan_bwd(mode, q, k, v, alpha, beta=None, S0=None, dO=None, dST=None,
             threads: int | None = None):
    """Gradients of L = sum <dO, o> + <dST, S_T> of ``scan`` with respect to
    every input, in float64 (inputs are taken as float64, unrounded).

    Shapes as in ``scan`` (every mode; "gdn_ew" takes beta [2, ..., T], erase
    then write strengths, and returns dbeta in the same layout); dO like o
    ([..., T, dv]) or None (zero), dST like S_T or None (zero).
    Returns (dq, dk, dv, dalpha, dbeta or None, dS0).
    """
    m = _mode(mode)
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    diag = m in (GDN_DIAG, GLA_DIAG)
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or \
            alpha.shape != (q.shape if diag else q.shape[:-1]):
        raise ValueError("shape mismatch among q, k, v, alpha")
    delta = m in (GDN, GDN_DIAG, GDN_EW)
    bshape = (2, *q.shape[:-1]) if m == GDN_EW else q.shape[:-1]
    if delta:
        beta = _f64(beta)
        if beta is None or beta.shape != bshape:
            raise ValueError("beta shape mismatch")
    else:
        beta = None
    S0, dO, dST = _f64(S0), _f64(dO), _f64(dST)
    if S0 is not None and S0.shape != (*lead, dv, dk):
        raise ValueError("S0 shape mismatch")
    if dO is not None and dO.shape != v.shape:
        raise ValueError("dO shape mismatch")
    if dST is not None and dST.shape != (*lead, dv, dk):
        raise ValueError("dST shape mismatch")
    gq, gk, gv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    ga = np.empty_like(alpha)
    gb = np.empty(bshape, np.float64) if delta else None
    gS0 = np.empty((*lead, dv, dk), np.float64)
    n = _load().oracle_scan_bwd_f64(m, BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(gq), _ptr(gk),
                                    _ptr(gv), _ptr(ga), _ptr(gb), _ptr(gS0),
                                    threads or default_threads())
    if n < 0:
        raise RuntimeError("oracle_scan_bwd_f64 failed")
    return gq, gk, gv, ga, gb, gS0


def rel_err_per_head(x, ref, head_dims: int):
    """Relative Frobenius error per head: ||x - ref||_F / ||ref||_F.

    The first ``head_dims`` axes index heads; the norm runs over the rest.  A
    head whose reference norm is zero reports the absolute norm instead.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    axes = tuple(range(head_dims, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
