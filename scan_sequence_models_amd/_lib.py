"""ctypes binding of ``libgdscan.so`` (include/gdscan.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch when the caller does not pass them, and the C entry points
of the same names are called on torch's current HIP stream.  Every step of the
scan runs in the library's kernels; there is no other implementation to fall
back on, so a missing or unloadable library is an error.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

# GDSCAN_LIB names another build of the same library (the sanitizer build)
LIB_PATH = os.environ.get("GDSCAN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libgdscan.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "gdscan.h")

SCAN_GDN, SCAN_GLA, SCAN_GDN_EW, SCAN_GDN_DIAG, SCAN_GLA_DIAG = 0, 1, 2, 3, 4
SCAN_F32, SCAN_BF16 = 0, 1
SCAN_OK, SCAN_EINVAL, SCAN_EUNSUPPORTED, SCAN_EWORKSPACE, SCAN_EALIGN, SCAN_EHIP = range(6)
SCAN_NOALLOC_MAX_WORKSPACE = 64 << 20
PATHS = {"auto": 0, "sequential": 1, "blelloch": 2}
STATUS_NAMES = {0: "SCAN_OK", 1: "SCAN_EINVAL", 2: "SCAN_EUNSUPPORTED", 3: "SCAN_EWORKSPACE",
                4: "SCAN_EALIGN", 5: "SCAN_EHIP"}


class ScanOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("leaf_chunks", ctypes.c_int)]


class ScanError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m scan_sequence_models_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.scan_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(ScanOpts)]
        L.scan_fwd_workspace_size.restype = sz
        L.scan_fwd.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, p, sz,
                               ctypes.POINTER(ScanOpts), p]
        L.scan_fwd.restype = i
        L.scan_fwd_noalloc.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p,
                                       ctypes.POINTER(ScanOpts), p]
        L.scan_fwd_noalloc.restype = i
        L.decode_step.argtypes = [i, i, i, i, i, p, p, p, p, p, p, p, p]
        L.decode_step.restype = i
        L.prism_expand.argtypes = [i] * 8 + [p] * 15 + [p]
        L.prism_expand.restype = i
        L.lact_fwd_workspace_size.argtypes = [i] * 7
        L.lact_fwd_workspace_size.restype = sz
        L.lact_fwd.argtypes = [i] * 8 + [p] * 7 + [p, sz, p]
        L.lact_fwd.restype = i
        L.prism_scan_workspace_size.argtypes = [i] * 7
        L.prism_scan_workspace_size.restype = sz
        L.prism_scan.argtypes = [i] * 8 + [p] * 13 + [p, sz, p]
        L.prism_scan.restype = i
        L.scan_bwd_workspace_size.argtypes = [i] * 7
        L.scan_bwd_workspace_size.restype = sz
        L.scan_bwd.argtypes = [i] * 7 + [p] * 15 + [sz, p]
        L.scan_bwd.restype = i
        L.scan_last_error.restype = ctypes.c_char_p
        L.scan_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/gdscan.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def last_error() -> str:
    return lib().scan_last_error().decode()


def version() -> str:
    return lib().scan_version().decode()


def _check(status: int):
    if status != SCAN_OK:
        raise ScanError(status, last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SCAN_F32
    if t.dtype == torch.bfloat16:
        return SCAN_BF16
    raise TypeError(f"q, k, v must be float32 or bfloat16 (got {t.dtype})")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def scan_fwd_workspace_size(mode: int, dtype: int, B: int, H: int, T: int, dk: int, dv: int,
                            chunk: int, path: str = "auto", leaf_chunks: int = 0) -> int:
    opts = ScanOpts(PATHS[path], leaf_chunks)
    n = lib().scan_fwd_workspace_size(mode, dtype, B, H, T, dk, dv, chunk, ctypes.byref(opts))
    if n == ctypes.c_size_t(-1).value:
        raise ScanError(SCAN_EINVAL, last_error())
    return n


def _scan_args(q, k, v, alpha, beta, S0, o, ST, write_state):
    """Checks the tensors of a forward scan and allocates missing outputs;
    returns (mode, B, H, T, dk, dv, o, ST)."""
    _need(q, "q")
    dev = q.device
    dt = q.dtype
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (B, H, T, dk), dev)
    _need(v, "v", dt, (B, H, T, dv), dev)
    diag = alpha.dim() == 4
    _need(alpha, "alpha", torch.float32, (B, H, T, dk) if diag else (B, H, T), dev)
    if diag:
        mode = SCAN_GLA_DIAG if beta is None else SCAN_GDN_DIAG
    else:
        mode = SCAN_GLA if beta is None else SCAN_GDN_EW if beta.dim() == 4 else SCAN_GDN
    if beta is not None:
        _need(beta, "beta", torch.float32, (2, B, H, T) if mode == SCAN_GDN_EW else (B, H, T), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (B, H, T, dv), dev)
    if ST is None and write_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if ST is not None:
        _need(ST, "ST", torch.float32, (B, H, dv, dk), dev)
    return mode, B, H, T, dk, dv, o, ST


def scan_fwd(q, k, v, alpha, beta=None, S0=None, *, chunk: int = 64, path: str = "auto",
             leaf_chunks: int = 0, o=None, ST=None, workspace=None, write_state: bool = True):
    """Forward scan over [B, H, T, d] tensors; returns (o, ST).

    ``beta is None`` selects gated linear attention (E = alpha I, f = v k^T),
    a [B, H, T] ``beta`` the gated delta rule, and a [2, B, H, T] ``beta``
    (erase strengths, then write strengths) the gated delta rule with split
    strengths (SCAN_GDN_EW).  A [B, H, T, dk] ``alpha`` (one decay per key
    channel) selects the diagonal-gate modes (SCAN_GDN_DIAG with beta,
    SCAN_GLA_DIAG without).  ``S0=None`` is the zero state.  ``ST`` may
    be ``S0`` itself (in-place carry).  ``write_state=False`` skips S_T.
    """
    mode, B, H, T, dk, dv, o, ST = _scan_args(q, k, v, alpha, beta, S0, o, ST, write_state)
    dev = q.device
    dcode = _dtype_code(q)
    ws_bytes = scan_fwd_workspace_size(mode, dcode, B, H, T, dk, dv, chunk, path, leaf_chunks)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, dev)
    opts = ScanOpts(PATHS[path], leaf_chunks)
    with torch.cuda.device(dev):
        st = lib().scan_fwd(mode, dcode, B, H, T, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v),
                            _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST), _ptr(workspace),
                            0 if workspace is None else workspace.numel(), ctypes.byref(opts),
                            _stream(dev))
    _check(st)
    return o, ST


def scan_fwd_noalloc(q, k, v, alpha, beta=None, S0=None, *, o, ST=None, chunk: int = 64,
                     path: str = "auto", leaf_chunks: int = 0):
    """``scan_fwd`` through the C entry point of the same name, which takes no
    workspace: the library's fixed per-GPU scratch stands in for it (at most
    SCAN_NOALLOC_MAX_WORKSPACE bytes).  The caller passes the outputs (``o``,
    and ``ST`` unless S_T is not wanted), so nothing is allocated here either."""
    if o is None:
        raise ValueError("scan_fwd_noalloc: pass the output tensor o")
    mode, B, H, T, dk, dv, o, ST = _scan_args(q, k, v, alpha, beta, S0, o, ST, False)
    dev = q.device
    opts = ScanOpts(PATHS[path], leaf_chunks)
    with torch.cuda.device(dev):
        st = lib().scan_fwd_noalloc(mode, _dtype_code(q), B, H, T, dk, dv, chunk, _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                                    ctypes.byref(opts), _stream(dev))
    _check(st)
    return o, ST


def decode_step(q, k, v, alpha, beta, S, o=None):
    """One token per state: S [N, dv, dk] float32 updated in place; returns o [N, dv].

    ``beta is None`` selects gated linear attention; a [2, N] ``beta`` (erase,
    write) the split-strength mode; an [N, dk] ``alpha`` the diagonal gates.
    """
    _need(q, "q")
    dev, dt = q.device, q.dtype
    if q.dim() != 2:
        raise ValueError("q must be [N, dk]")
    N, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (N, dk), dev)
    _need(v, "v", dt, (N, dv), dev)
    diag = alpha.dim() == 2
    _need(alpha, "alpha", torch.float32, (N, dk) if diag else (N,), dev)
    if diag:
        mode = SCAN_GLA_DIAG if beta is None else SCAN_GDN_DIAG
    else:
        mode = SCAN_GLA if beta is None else SCAN_GDN_EW if beta.dim() == 2 else SCAN_GDN
    if beta is not None:
        _need(beta, "beta", torch.float32, (2, N) if mode == SCAN_GDN_EW else (N,), dev)
    _need(S, "S", torch.float32, (N, dv, dk), dev)
    if o is None:
        o = torch.empty((N, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (N, dv), dev)
    with torch.cuda.device(dev):
        st = lib().decode_step(mode, _dtype_code(q), N, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(alpha), _ptr(beta), _ptr(S), _ptr(o), _stream(dev))
    _check(st)
    return o


def prism_expand(q, k, v, alpha, beta, x=None, beta_l=None, conv=None, Wk=None, Wp=None, *,
                 out=None):
    """PRISM write factors expanded into a split-strength scan stream.

    q, k [B, H, T, dk] and v, x [B, H, T, dv] (float32 or bfloat16); alpha, beta
    [B, H, T] float32; beta_l [B, H, T, L] float32; conv [H, W, dv] float32; Wk
    [H, L, dk, dv] and Wp [H, L, dv, dv] in the data type.  ``beta_l=None``
    means L = 0.  Returns (q2, k2, v2, alpha2, beta2) with T (L+1) elements per
    head; beta2 is [2, B, H, T (L+1)] (erase, write), ready for ``scan_fwd``.
    ``out`` may pass those five tensors preallocated.
    """
    _need(q, "q")
    dev, dt = q.device, q.dtype
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (B, H, T, dk), dev)
    _need(v, "v", dt, (B, H, T, dv), dev)
    _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    _need(beta, "beta", torch.float32, (B, H, T), dev)
    L = 0 if beta_l is None else beta_l.shape[-1]
    W = 1
    if L > 0:
        _need(x, "x", dt, (B, H, T, dv), dev)
        _need(beta_l, "beta_l", torch.float32, (B, H, T, L), dev)
        _need(conv, "conv", torch.float32, None, dev)
        if conv.dim() != 3 or conv.shape[0] != H or conv.shape[2] != dv:
            raise ValueError(f"conv must be [H, W, dv] = [{H}, W, {dv}]")
        W = conv.shape[1]
        _need(Wk, "Wk", dt, (H, L, dk, dv), dev)
        _need(Wp, "Wp", dt, (H, L, dv, dv), dev)
    T2 = T * (L + 1)
    if out is None:
        out = (torch.empty((B, H, T2, dk), dtype=dt, device=dev),
               torch.empty((B, H, T2, dk), dtype=dt, device=dev),
               torch.empty((B, H, T2, dv), dtype=dt, device=dev),
               torch.empty((B, H, T2), dtype=torch.float32, device=dev),
               torch.empty((2, B, H, T2), dtype=torch.float32, device=dev))
    q2, k2, v2, a2, b2 = out
    _need(q2, "q2", dt, (B, H, T2, dk), dev)
    _need(k2, "k2", dt, (B, H, T2, dk), dev)
    _need(v2, "v2", dt, (B, H, T2, dv), dev)
    _need(a2, "alpha2", torch.float32, (B, H, T2), dev)
    _need(b2, "beta2", torch.float32, (2, B, H, T2), dev)
    with torch.cuda.device(dev):
        st = lib().prism_expand(_dtype_code(q), B, H, T, dk, dv, L, W, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(x) if L else None, _ptr(alpha), _ptr(beta),
                                _ptr(beta_l) if L else None, _ptr(conv) if L else None,
                                _ptr(Wk) if L else None, _ptr(Wp) if L else None, _ptr(q2),
                                _ptr(k2), _ptr(v2), _ptr(a2), _ptr(b2), _stream(dev))
    _check(st)
    return q2, k2, v2, a2, b2


def prism_scan_workspace_size(dtype: int, B: int, H: int, T: int, dk: int, dv: int, L: int) -> int:
    n = lib().prism_scan_workspace_size(dtype, B, H, T, dk, dv, L)
    if n == ctypes.c_size_t(-1).value:
        raise ScanError(SCAN_EINVAL, last_error())
    return n


def prism_scan(q, k, v, alpha, beta, x=None, beta_l=None, conv=None, Wk=None, Wp=None, S0=None, *,
               o=None, ST=None, workspace=None, write_state: bool = True):
    """The PRISM layer's scan without a materialised element stream (bfloat16,
    d = 128): the arguments of ``prism_expand`` plus S0; returns (o, ST) with o
    [B, H, T, dv].  Equal bit for bit to ``scan_fwd`` over ``prism_expand``'s
    stream, read at each token's last element."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (B, H, T, dk), dev)
    _need(v, "v", dt, (B, H, T, dv), dev)
    _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    _need(beta, "beta", torch.float32, (B, H, T), dev)
    L = 0 if beta_l is None else beta_l.shape[-1]
    W = 1
    if L > 0:
        _need(x, "x", dt, (B, H, T, dv), dev)
        _need(beta_l, "beta_l", torch.float32, (B, H, T, L), dev)
        _need(conv, "conv", torch.float32, None, dev)
        if conv.dim() != 3 or conv.shape[0] != H or conv.shape[2] != dv:
            raise ValueError(f"conv must be [H, W, dv] = [{H}, W, {dv}]")
        W = conv.shape[1]
        _need(Wk, "Wk", dt, (H, L, dk, dv), dev)
        _need(Wp, "Wp", dt, (H, L, dv, dv), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (B, H, T, dv), dev)
    if ST is None and write_state:
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if ST is not None:
        _need(ST, "ST", torch.float32, (B, H, dv, dk), dev)
    dcode = _dtype_code(q)
    ws_bytes = prism_scan_workspace_size(dcode, B, H, T, dk, dv, L)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, dev)
    with torch.cuda.device(dev):
        st = lib().prism_scan(dcode, B, H, T, dk, dv, L, W, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(x) if L else None, _ptr(alpha), _ptr(beta),
                              _ptr(beta_l) if L else None, _ptr(conv) if L else None,
                              _ptr(Wk) if L else None, _ptr(Wp) if L else None, _ptr(S0), _ptr(o),
                              _ptr(ST), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                              _stream(dev))
    _check(st)
    return o, ST


def prism_scan_fwd(q, k, v, alpha, beta, x=None, beta_l=None, conv=None, Wk=None, Wp=None,
                   S0=None, *, chunk: int = 64, path: str = "auto", leaf_chunks: int = 0,
                   write_state: bool = True, stream: bool = False):
    """PRISM layer forward.  bfloat16 with d = 128 (unless ``stream``) runs
    ``prism_scan``; otherwise ``prism_expand`` then the split-strength
    ``scan_fwd``.  Returns (o, ST) with o [B, H, T, dv] (on the stream path a
    view of the expanded output: every (L+1)-th element, the last of each
    token's group).
    """
    if (not stream and q.dtype == torch.bfloat16 and q.shape[-1] == 128 and v.shape[-1] == 128
            and path == "auto" and chunk == 64):
        return prism_scan(q, k, v, alpha, beta, x, beta_l, conv, Wk, Wp, S0, write_state=write_state)
    q2, k2, v2, a2, b2 = prism_expand(q, k, v, alpha, beta, x, beta_l, conv, Wk, Wp)
    o2, ST = scan_fwd(q2, k2, v2, a2, b2, S0, chunk=chunk, path=path, leaf_chunks=leaf_chunks,
                      write_state=write_state)
    B, H, T, _ = q.shape
    G = q2.shape[2] // T
    return o2.view(B, H, T, G, o2.shape[-1])[:, :, :, G - 1], ST


LACT_ORDERS = {"update_then_apply": 0, "apply_then_update": 1}


def lact_fwd_workspace_size(dtype: int, B: int, H: int, T: int, dk: int, dv: int, chunk: int) -> int:
    n = lib().lact_fwd_workspace_size(dtype, B, H, T, dk, dv, chunk)
    if n == ctypes.c_size_t(-1).value:
        raise ScanError(SCAN_EINVAL, last_error())
    return n


def lact_fwd(q, k, v, eta, W0=None, *, chunk: int, order: str = "update_then_apply", o=None,
             WT=None, workspace=None, write_state: bool = True):
    """Large-chunk fast-weight update over [B, H, T, d] tensors; returns (o, WT).

    eta [B, H, T] float32; W0 [B, H, dv, dk] float32 or None (zero); ``order``
    is "update_then_apply" or "apply_then_update".
    """
    _need(q, "q")
    dev, dt = q.device, q.dtype
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (B, H, T, dk), dev)
    _need(v, "v", dt, (B, H, T, dv), dev)
    _need(eta, "eta", torch.float32, (B, H, T), dev)
    if W0 is not None:
        _need(W0, "W0", torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (B, H, T, dv), dev)
    if WT is None and write_state:
        WT = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if WT is not None:
        _need(WT, "WT", torch.float32, (B, H, dv, dk), dev)
    dcode = _dtype_code(q)
    ws_bytes = lact_fwd_workspace_size(dcode, B, H, T, dk, dv, chunk)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, dev)
    with torch.cuda.device(dev):
        st = lib().lact_fwd(dcode, B, H, T, dk, dv, chunk, LACT_ORDERS[order], _ptr(q), _ptr(k),
                            _ptr(v), _ptr(eta), _ptr(W0), _ptr(o), _ptr(WT), _ptr(workspace),
                            0 if workspace is None else workspace.numel(), _stream(dev))
    _check(st)
    return o, WT


def scan_bwd_workspace_size(mode: int, dtype: int, B: int, H: int, T: int, dk: int, dv: int) -> int:
    n = lib().scan_bwd_workspace_size(mode, dtype, B, H, T, dk, dv)
    if n == ctypes.c_size_t(-1).value:
        raise ScanError(SCAN_EINVAL, last_error())
    return n


def scan_bwd(q, k, v, alpha, beta=None, S0=None, dO=None, dST=None, *, workspace=None, out=None):
    """Gradients of a scan_fwd call (gated delta rule when ``beta`` is a
    [B, H, T] tensor, with split strengths when it is [2, B, H, T], gated linear
    attention when it is None) for incoming gradients dO (at o, dtype of q;
    None: zero) and dST (at S_T, float32; None: zero).

    Returns (dq, dk, dv, dalpha, dbeta or None, dS0), all float32; ``out`` may
    give those six tensors preallocated.
    """
    _need(q, "q")
    dev, dt = q.device, q.dtype
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", dt, (B, H, T, dk), dev)
    _need(v, "v", dt, (B, H, T, dv), dev)
    _need(alpha, "alpha", torch.float32, (B, H, T), dev)
    mode = SCAN_GLA if beta is None else SCAN_GDN_EW if beta.dim() == 4 else SCAN_GDN
    bshape = (2, B, H, T) if mode == SCAN_GDN_EW else (B, H, T)
    if beta is not None:
        _need(beta, "beta", torch.float32, bshape, dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dv, dk), dev)
    if dO is not None:
        _need(dO, "dO", dt, (B, H, T, dv), dev)
    if dST is not None:
        _need(dST, "dST", torch.float32, (B, H, dv, dk), dev)
    f32 = torch.float32
    shapes = [(B, H, T, dk), (B, H, T, dk), (B, H, T, dv), (B, H, T), bshape, (B, H, dv, dk)]
    if out is None:
        out = [None if (i == 4 and beta is None) else torch.empty(sh, dtype=f32, device=dev)
               for i, sh in enumerate(shapes)]
    out = list(out)
    for i, (name, sh) in enumerate(zip(["dq", "dk", "dv", "dalpha", "dbeta", "dS0"], shapes)):
        if i == 4 and beta is None:
            if out[i] is not None:
                raise ValueError("dbeta must be None for gated linear attention")
            continue
        _need(out[i], name, f32, sh, dev)
    dcode = _dtype_code(q)
    ws_bytes = scan_bwd_workspace_size(mode, dcode, B, H, T, dk, dv)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    with torch.cuda.device(dev):
        st = lib().scan_bwd(mode, dcode, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                            _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dST), *[_ptr(x) for x in out],
                            _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st)
    return tuple(out)

