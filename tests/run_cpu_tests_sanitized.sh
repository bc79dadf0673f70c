#!/bin/bash
# The CPU test suite (-m "not gpu") against host-sanitizer builds of the HIP library (its C ABI's
# argument checks, planning and launch code; device code as usual) and of the oracle, both with
# AddressSanitizer + UndefinedBehaviorSanitizer from ROCm's clang, whose shared ASan runtime is
# preloaded into Python.  Leak reports are off (the interpreter itself keeps allocations alive).
set -euo pipefail
cd "$(dirname "$0")/.."
python3 sparse_attention_flash_amd/build.py --sanitize
python3 -c "import oracle; oracle.build(force=True, sanitize=True)"
ASAN_RT=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)
export LD_PRELOAD="$ASAN_RT"
export ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1"
export UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"
export SA_HIP_LIB="$PWD/sparse_attention_flash_amd/libsa_hip_san.so"
export SA_ORACLE_LIB="$PWD/oracle/libsa_oracle_san.so"
exec python3 -m pytest tests -m "not gpu" -x -q -p no:cacheprovider "$@"
