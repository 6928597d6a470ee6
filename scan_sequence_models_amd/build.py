"""Build ``libgdscan.so`` (the gfx950 C-ABI library) in-tree with hipcc.

Usage: ``python -m scan_sequence_models_amd.build`` (or ``build()`` from Python).
Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` in parallel
and the objects are linked into ``scan_sequence_models_amd/libgdscan.so``.

``python -m scan_sequence_models_amd.build --sanitize`` builds
``libgdscan_san.so`` instead (objects under ``_build_san/``): the host code is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer, the device code
is built as usual.  The library leaves the sanitizer runtime unresolved; the
process preloads clang's ``libclang_rt.asan-x86_64.so`` (see
``tests/sanitize.sh``, which runs the CPU suite that way).  It is a CPU-side
check of the host code: validation, planning and the ABI.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdscan.so")
OBJ_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libgdscan_san.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed-fp32 instructions are kept out of every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


# host-only sanitizer flags: each -fsanitize= applies to the host pass alone
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(OBJ_SAN if sanitize else OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; that is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every HIP source and link ``libgdscan.so`` (``libgdscan_san.so``
    with ``sanitize``); returns its path."""
    os.makedirs(OBJ_SAN if sanitize else OBJ, exist_ok=True)
    lib = LIB_SAN if sanitize else LIB
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = lib + f".tmp{os.getpid()}"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv[1:]))
