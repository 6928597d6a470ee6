#!/bin/bash
# CPU-only sanitizer run: builds the oracle (oracle/oracle.c) and the host code
# of the library (csrc/*.hip; device code unchanged) with AddressSanitizer and
# UndefinedBehaviorSanitizer, then runs the CPU test suite against those builds
# with clang's sanitizer runtime preloaded.  No GPU is used.
#   usage: bash tests/sanitize.sh [extra pytest arguments]
set -euo pipefail
ROOT="$(cd "$(dirname "${BASH_SOURCE[0]}")/.." && pwd)"
cd "$ROOT"
LIB=$(python3 -m scan_sequence_models_amd.build --sanitize)
ORA=$(python3 -c "import oracle; print(oracle.build_sanitized())")
RT=$("${ROCM_PATH:-/opt/rocm}/llvm/bin/clang" -print-file-name=libclang_rt.asan-x86_64.so)
echo "sanitizer builds: $LIB $ORA (runtime $RT)"
# leak checking is off: the Python interpreter itself keeps memory until exit
GDSCAN_LIB="$LIB" ORACLE_LIB="$ORA" LD_PRELOAD="$RT" \
ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1" \
UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1" \
    python3 -m pytest tests -m "not gpu" -q -x -p no:cacheprovider "$@"
