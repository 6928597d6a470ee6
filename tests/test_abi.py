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
    assert set(names) == {"scan_fwd_workspace_size", "scan_fwd", "decode_step",
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


def _decode(lib, mode=0, dtype=1, N=4, dk=128, dv=128, q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP,
            alpha=FAKE + 3 * STEP, beta=FAKE + 4 * STEP, S=FAKE + 5 * STEP, o=FAKE + 6 * STEP):
    return lib.decode_step(mode, dtype, N, dk, dv, q, k, v, alpha, beta, S, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), L.SCAN_EINVAL),
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
