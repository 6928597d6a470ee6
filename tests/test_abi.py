"""The C-ABI library loads and exports what include/gdscan.h declares, and its
host-side validation rejects bad calls before anything is launched.

Every call here fails validation on the host, so no pointer is dereferenced
and no GPU is needed (the pointers are fake integers that are never used)."""
import ctypes

import pytest

from scan_sequence_models_amd import _lib as L

FAKE = 1 << 40          # a 256-byte aligned "device pointer" that is never touched
STEP = 1 << 32          # spacing of fake buffers so they never overlap


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = L.header_functions()
    assert set(names) == {"scan_fwd_workspace_size", "scan_fwd", "scan_fwd_noalloc", "decode_step",
                          "prism_expand", "prism_scan_workspace_size", "prism_scan",
                          "lact_fwd_workspace_size", "lact_fwd", "scan_bwd_workspace_size", "scan_bwd",
                          "scan_last_error", "scan_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert "gfx950" in L.version()


def _opts(path=1, leaf=0):
    return ctypes.byref(L.ScanOpts(path, leaf))


def _scan(lib, mode=0, dtype=1, B=1, H=2, T=64, dk=128, dv=128, chunk=64, q=FAKE, k=FAKE + STEP,
          v=FAKE + 2 * STEP, alpha=FAKE + 3 * STEP, beta=FAKE + 4 * STEP, S0=None,
          o=FAKE + 6 * STEP, ST=FAKE + 7 * STEP, ws=None, wsb=0, opts=None):
    return lib.scan_fwd(mode, dtype, B, H, T, dk, dv, chunk, q, k, v, alpha, beta, S0, o, ST, ws,
                        wsb, opts if opts is not None else _opts(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=7), L.SCAN_EINVAL),
    (dict(dtype=3), L.SCAN_EINVAL),
    (dict(T=0), L.SCAN_EINVAL),
    (dict(B=-1), L.SCAN_EINVAL),
    (dict(chunk=48), L.SCAN_EUNSUPPORTED),
    (dict(dk=24), L.SCAN_EUNSUPPORTED),
    (dict(dv=20), L.SCAN_EUNSUPPORTED),
    (dict(q=None), L.SCAN_EINVAL),
    (dict(o=None), L.SCAN_EINVAL),
    (dict(beta=None), L.SCAN_EINVAL),                 # gdn needs beta
    (dict(mode=1), L.SCAN_EINVAL),                    # gla takes no beta
    (dict(k=FAKE + STEP + 8), L.SCAN_EALIGN),
    (dict(alpha=FAKE + 3 * STEP + 2), L.SCAN_EALIGN),
    (dict(o=FAKE + 256), L.SCAN_EINVAL),              # o overlaps q
    (dict(ST=FAKE + 2 * STEP), L.SCAN_EINVAL),        # ST overlaps v
    (dict(S0=FAKE + 5 * STEP, ST=FAKE + 5 * STEP + 256), L.SCAN_EINVAL),  # partial alias
    (dict(opts=_opts(path=9)), L.SCAN_EINVAL),
    (dict(opts=_opts(path=1, leaf=3)), L.SCAN_EINVAL),
    (dict(mode=2, beta=None), L.SCAN_EINVAL),         # split strengths need beta
    # split strengths: beta holds two planes (2 x B*H*T floats = 1 KB here), so
    # an output starting 768 bytes after beta overlaps its write plane (with
    # one plane counted it would not)
    (dict(mode=2, o=FAKE + 4 * STEP + 768), L.SCAN_EINVAL),
    (dict(mode=3, beta=None), L.SCAN_EINVAL),
    (dict(mode=4), L.SCAN_EINVAL),                    # diagonal gla takes no beta
    (dict(mode=3, alpha=FAKE + 3 * STEP + 8), L.SCAN_EALIGN),
    (dict(mode=3, opts=_opts(path=2)), L.SCAN_EUNSUPPORTED),   # sequential path only
    (dict(mode=3, dk=96), L.SCAN_EUNSUPPORTED),
    # per-channel alpha is B*H*T*dk floats (64 KB here): o 32 KB after its start
    # overlaps it (a scalar alpha would end at 512 bytes)
    (dict(mode=3, o=FAKE + 3 * STEP + 32768), L.SCAN_EINVAL),
])
def test_scan_fwd_rejects(lib, kw, code):
    assert _scan(lib, **kw) == code
    assert len(L.last_error()) > 0


def test_scan_fwd_workspace_size_invalid(lib):
    n = lib.scan_fwd_workspace_size(0, 1, 1, 1, 64, 24, 128, 64, None)
    assert n == ctypes.c_size_t(-1).value
    assert "dk" in L.last_error()


def test_sequential_path_needs_no_workspace(lib):
    assert lib.scan_fwd_workspace_size(0, 1, 8, 16, 8192, 128, 128, 64, _opts(1)) == 0
    assert lib.scan_fwd_workspace_size(0, 0, 1, 1, 64, 16, 16, 16, _opts(1)) == 0


def _noalloc(lib, B=1, H=2, T=64, opts=None, q=FAKE, o=FAKE + 6 * STEP):
    return lib.scan_fwd_noalloc(0, 1, B, H, T, 128, 128, 64, q, FAKE + STEP, FAKE + 2 * STEP,
                                FAKE + 3 * STEP, FAKE + 4 * STEP, None, o, FAKE + 7 * STEP,
                                opts if opts is not None else _opts(), None)


def test_noalloc_rejects_workspace_above_its_scratch(lib):
    """128 heads x 64 leaves need about 3 GB of tree workspace: above the fixed
    scratch, so the call is refused before anything is launched."""
    need = lib.scan_fwd_workspace_size(0, 1, 8, 16, 65536, 128, 128, 64, _opts(2, 16))
    assert need > L.SCAN_NOALLOC_MAX_WORKSPACE
    assert _noalloc(lib, B=8, H=16, T=65536, opts=_opts(2, 16)) == L.SCAN_EWORKSPACE
    assert "scratch" in L.last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), L.SCAN_EINVAL),
    (dict(q=None), L.SCAN_EINVAL),
    (dict(o=FAKE + 256), L.SCAN_EINVAL),   # o overlaps q
    (dict(opts=_opts(path=9)), L.SCAN_EINVAL),
])
def test_noalloc_validates_like_scan_fwd(lib, kw, code):
    assert _noalloc(lib, **kw) == code


def test_noalloc_limit_matches_header():
    text = open(L.HEADER).read()
    assert "#define SCAN_NOALLOC_MAX_WORKSPACE (64u << 20)" in text
    assert L.SCAN_NOALLOC_MAX_WORKSPACE == 64 << 20


def _decode(lib, mode=0, dtype=1, N=4, dk=128, dv=128, q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP,
            alpha=FAKE + 3 * STEP, beta=FAKE + 4 * STEP, S=FAKE + 5 * STEP, o=FAKE + 6 * STEP):
    return lib.decode_step(mode, dtype, N, dk, dv, q, k, v, alpha, beta, S, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=7), L.SCAN_EINVAL),
    (dict(mode=2, beta=None), L.SCAN_EINVAL),
    (dict(mode=3, beta=None), L.SCAN_EINVAL),               # diagonal gdn needs beta
    (dict(mode=4), L.SCAN_EINVAL),                          # diagonal gla takes no beta
    (dict(mode=3, alpha=FAKE + 3 * STEP + 4), L.SCAN_EALIGN),  # per-channel alpha: 16 bytes
    (dict(mode=3, o=FAKE + 3 * STEP + 1024), L.SCAN_EINVAL),   # o inside alpha [N, dk] (2 KB)
    (dict(mode=2, o=FAKE + 4 * STEP + 16), L.SCAN_EINVAL),  # o inside beta's write plane
    (dict(N=0), L.SCAN_EINVAL),
    (dict(dk=96), L.SCAN_EUNSUPPORTED),
    (dict(S=None), L.SCAN_EINVAL),
    (dict(beta=None), L.SCAN_EINVAL),
    (dict(mode=1), L.SCAN_EINVAL),
    (dict(S=FAKE + 5 * STEP + 4), L.SCAN_EALIGN),
    (dict(o=FAKE + 5 * STEP + 1024), L.SCAN_EINVAL),  # o inside S
    (dict(S=FAKE + 64), L.SCAN_EINVAL),               # S overlaps q
])
def test_decode_step_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def _prism(lib, dtype=1, B=1, H=2, T=64, dk=128, dv=128, Lsteps=2, W=4, q=FAKE, k=FAKE + STEP,
           v=FAKE + 2 * STEP, x=FAKE + 3 * STEP, alpha=FAKE + 4 * STEP, beta=FAKE + 5 * STEP,
           beta_l=FAKE + 6 * STEP, conv=FAKE + 7 * STEP, Wk=FAKE + 8 * STEP, Wp=FAKE + 9 * STEP,
           q2=FAKE + 10 * STEP, k2=FAKE + 11 * STEP, v2=FAKE + 12 * STEP, a2=FAKE + 13 * STEP,
           b2=FAKE + 14 * STEP):
    # a valid argument set would launch with fake pointers: only invalid ones are passed
    return lib.prism_expand(dtype, B, H, T, dk, dv, Lsteps, W, q, k, v, x, alpha, beta, beta_l,
                            conv, Wk, Wp, q2, k2, v2, a2, b2, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), L.SCAN_EINVAL),
    (dict(T=0), L.SCAN_EINVAL),
    (dict(Lsteps=-1), L.SCAN_EINVAL),
    (dict(Lsteps=9), L.SCAN_EINVAL),
    (dict(W=0), L.SCAN_EINVAL),
    (dict(W=9), L.SCAN_EINVAL),
    (dict(dk=96), L.SCAN_EUNSUPPORTED),
    (dict(dv=48), L.SCAN_EUNSUPPORTED),
    (dict(q=None), L.SCAN_EINVAL),
    (dict(beta=None), L.SCAN_EINVAL),
    (dict(b2=None), L.SCAN_EINVAL),
    (dict(Wk=None), L.SCAN_EINVAL),                   # L > 0 needs the weights
    (dict(x=None), L.SCAN_EINVAL),
    (dict(conv=FAKE + 7 * STEP + 8), L.SCAN_EALIGN),
    (dict(Wp=FAKE + 9 * STEP + 2), L.SCAN_EALIGN),
    (dict(beta_l=FAKE + 6 * STEP + 2), L.SCAN_EALIGN),
    (dict(q2=FAKE + 512), L.SCAN_EINVAL),             # q2 overlaps q
    (dict(v2=FAKE + 11 * STEP + 4096), L.SCAN_EINVAL),  # v2 overlaps k2
    (dict(b2=FAKE + 5 * STEP + 256), L.SCAN_EINVAL),  # beta2 overlaps beta
])
def test_prism_expand_rejects(lib, kw, code):
    assert _prism(lib, **kw) == code
    assert len(L.last_error()) > 0


def _lact(lib, dtype=1, B=1, H=2, T=4096, dk=128, dv=128, chunk=2048, order=0, q=FAKE,
          k=FAKE + STEP, v=FAKE + 2 * STEP, eta=FAKE + 3 * STEP, W0=None, o=FAKE + 5 * STEP,
          WT=FAKE + 6 * STEP, ws=FAKE + 7 * STEP, wsb=1 << 30):
    # a valid argument set would launch with fake pointers: only invalid ones are passed
    return lib.lact_fwd(dtype, B, H, T, dk, dv, chunk, order, q, k, v, eta, W0, o, WT, ws, wsb, None)


def _prism_scan(lib, dtype=1, B=1, H=2, T=64, dk=128, dv=128, L=2, W=4, q=FAKE, o=FAKE + 6 * STEP,
                ws=FAKE + 9 * STEP, wsb=1 << 30, x=FAKE + 10 * STEP):
    return lib.prism_scan(dtype, B, H, T, dk, dv, L, W, q, FAKE + STEP, FAKE + 2 * STEP, x,
                          FAKE + 3 * STEP, FAKE + 4 * STEP, FAKE + 11 * STEP, FAKE + 12 * STEP,
                          FAKE + 13 * STEP, FAKE + 14 * STEP, None, o, FAKE + 7 * STEP, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), L.SCAN_EUNSUPPORTED),       # bfloat16 only
    (dict(dk=64), L.SCAN_EUNSUPPORTED),
    (dict(L=9), L.SCAN_EINVAL),
    (dict(W=0), L.SCAN_EINVAL),
    (dict(T=0), L.SCAN_EINVAL),
    (dict(x=None), L.SCAN_EINVAL),              # L > 0 needs the anchor source
    (dict(ws=None), L.SCAN_EWORKSPACE),
    (dict(wsb=1024), L.SCAN_EWORKSPACE),
    (dict(ws=FAKE + 9 * STEP + 8), L.SCAN_EALIGN),
    (dict(o=FAKE + 256), L.SCAN_EINVAL),        # o overlaps q
    (dict(T=1 << 30), L.SCAN_EUNSUPPORTED),     # element index range
])
def test_prism_scan_rejects(lib, kw, code):
    assert _prism_scan(lib, **kw) == code
    assert len(L.last_error()) > 0


def test_prism_scan_workspace_sizes(lib):
    # the factor rows: B H T L (dk + dv) bfloat16 values; none without corrections
    assert lib.prism_scan_workspace_size(1, 8, 16, 8192, 128, 128, 2) == 8 * 16 * 8192 * 2 * 256 * 2
    assert lib.prism_scan_workspace_size(1, 8, 16, 8192, 128, 128, 0) == 0
    assert lib.prism_scan_workspace_size(0, 1, 1, 64, 128, 128, 2) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), L.SCAN_EINVAL),
    (dict(T=0), L.SCAN_EINVAL),
    (dict(chunk=0), L.SCAN_EINVAL),
    (dict(chunk=100), L.SCAN_EUNSUPPORTED),           # bf16 d=128 needs a multiple of 64
    (dict(dk=96), L.SCAN_EUNSUPPORTED),
    (dict(dtype=0), L.SCAN_EUNSUPPORTED),             # float32 has no d = 128 path
    (dict(order=2), L.SCAN_EINVAL),
    (dict(q=None), L.SCAN_EINVAL),
    (dict(eta=None), L.SCAN_EINVAL),
    (dict(ws=None), L.SCAN_EWORKSPACE),
    (dict(wsb=1024), L.SCAN_EWORKSPACE),
    (dict(ws=FAKE + 7 * STEP + 64), L.SCAN_EALIGN),
    (dict(k=FAKE + STEP + 8), L.SCAN_EALIGN),
    (dict(eta=FAKE + 3 * STEP + 2), L.SCAN_EALIGN),
    (dict(o=FAKE + 1024), L.SCAN_EINVAL),             # o overlaps q
    (dict(WT=FAKE + 2 * STEP), L.SCAN_EINVAL),        # WT overlaps v
])
def test_lact_fwd_rejects(lib, kw, code):
    assert _lact(lib, **kw) == code
    assert len(L.last_error()) > 0


def test_lact_workspace_sizes(lib):
    # plain path (d <= 64): none; MFMA path: partial statistics and bf16 weights
    assert lib.lact_fwd_workspace_size(0, 1, 1, 64, 16, 16, 16) == 0
    n = lib.lact_fwd_workspace_size(1, 8, 16, 8192, 128, 128, 2048)
    assert n == 128 * 4 * (2 * 128 * 128 * 4 + 128 * 128 * 2)
    assert lib.lact_fwd_workspace_size(1, 1, 1, 64, 128, 128, 100) == ctypes.c_size_t(-1).value


def _bwd(lib, mode=0, dtype=1, B=1, H=2, T=64, dk=128, dv=128, q=FAKE, k=FAKE + STEP,
         v=FAKE + 2 * STEP, alpha=FAKE + 3 * STEP, beta=FAKE + 4 * STEP, S0=None, dO=FAKE + 6 * STEP,
         dST=None, dq=FAKE + 8 * STEP, dk_=FAKE + 9 * STEP, dv_=FAKE + 10 * STEP,
         dalpha=FAKE + 11 * STEP, dbeta=FAKE + 12 * STEP, dS0=FAKE + 13 * STEP, ws=FAKE + 14 * STEP,
         wsb=1 << 31):
    # a valid argument set would launch with fake pointers: only invalid ones are passed
    return lib.scan_bwd(mode, dtype, B, H, T, dk, dv, q, k, v, alpha, beta, S0, dO, dST, dq, dk_, dv_,
                        dalpha, dbeta, dS0, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=3), L.SCAN_EUNSUPPORTED),
    (dict(dtype=2), L.SCAN_EINVAL),
    (dict(T=0), L.SCAN_EINVAL),
    (dict(dk=96), L.SCAN_EUNSUPPORTED),
    (dict(dv=96), L.SCAN_EUNSUPPORTED),
    (dict(q=None), L.SCAN_EINVAL),
    (dict(beta=None), L.SCAN_EINVAL),                  # the delta rule needs beta
    (dict(mode=1), L.SCAN_EINVAL),                     # linear attention takes no beta
    (dict(dbeta=None), L.SCAN_EINVAL),
    # split strengths: dbeta holds two planes of B*H*T floats (512 bytes each here), so
    # its second plane would overlap dS0 (one plane would end right where dS0 starts)
    (dict(mode=2, dbeta=FAKE + 13 * STEP - 512), L.SCAN_EINVAL),
    (dict(dS0=None), L.SCAN_EINVAL),
    (dict(ws=None), L.SCAN_EWORKSPACE),
    (dict(wsb=1024), L.SCAN_EWORKSPACE),
    (dict(ws=FAKE + 14 * STEP + 64), L.SCAN_EALIGN),
    (dict(k=FAKE + STEP + 8), L.SCAN_EALIGN),
    (dict(alpha=FAKE + 3 * STEP + 2), L.SCAN_EALIGN),
    (dict(dq=FAKE + 1024), L.SCAN_EINVAL),             # dq overlaps q
    (dict(dS0=FAKE + 10 * STEP + 4096), L.SCAN_EINVAL),  # dS0 overlaps dv
])
def test_scan_bwd_rejects(lib, kw, code):
    assert _bwd(lib, **kw) == code
    assert len(L.last_error()) > 0


def test_scan_bwd_workspace_sizes(lib):
    # the state entering every 32-token chunk; with more than two 64-row value
    # slices also per-slice partials of dq, dk (dk floats per token) and of
    # d ln alpha and the two strength planes (one float each); with one or two
    # slices the sums go straight into the outputs
    n = lib.scan_bwd_workspace_size(0, 1, 8, 16, 8192, 128, 128)
    assert n == 4 * (128 * 256 * 128 * 128)
    assert lib.scan_bwd_workspace_size(1, 0, 1, 1, 33, 32, 64) == 4 * (2 * 64 * 32)
    assert lib.scan_bwd_workspace_size(2, 1, 1, 1, 64, 128, 128) == 4 * (2 * 128 * 128)
    assert lib.scan_bwd_workspace_size(0, 0, 1, 1, 70, 128, 192) == 4 * (3 * 192 * 128 + 3 * 70 * 259)
    assert lib.scan_bwd_workspace_size(0, 1, 1, 1, 64, 128, 96) == ctypes.c_size_t(-1).value
    assert lib.scan_bwd_workspace_size(3, 1, 1, 1, 64, 128, 128) == ctypes.c_size_t(-1).value

