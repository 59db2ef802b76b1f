#!/bin/bash
# Host-side sanitizer run of the CPU test suite: the oracle and the library's
# host code (layout, validation, pool carving, bit allocation) built with
# AddressSanitizer and UndefinedBehaviorSanitizer, any finding fatal.  The
# device code is the release code and is not run here (no GPU).
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
cd "$ROOT"
python -c 'import __graft_entry__ as g; g.build()' > /dev/null
python linear_attention_recurrent_stq_amd/build.py --sanitize > /dev/null
python -c 'import oracle; print(oracle.build_sanitized())' > /dev/null
RT="$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)"
LD_PRELOAD="$RT" \
ASAN_OPTIONS=detect_leaks=0:halt_on_error=1:abort_on_error=1 \
UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
STQ_LIBRARY="$ROOT/linear_attention_recurrent_stq_amd/libstq_san.so" \
ORACLE_LIBRARY="$ROOT/oracle/liboracle_san.so" \
python -m pytest tests -q -x -m "not gpu" -p no:cacheprovider "$@"
