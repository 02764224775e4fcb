#!/bin/bash
# The CPU test suite with AddressSanitizer and UndefinedBehaviorSanitizer on host code: the
# oracle (C) and the library's host side (argument checks, workspace and launch code; its GPU
# code is built as usual) are rebuilt with clang's sanitizers into a temporary directory, the
# tests load those builds (SPECVERIFY_ORACLE_LIB, SPECVERIFY_LIB), and Python runs with the
# sanitizer runtime preloaded.  Any report fails the run (UBSan does not recover).
#   bash tests/run_sanitized.sh [pytest arguments]
set -euo pipefail
ROOT="$(cd "$(dirname "${BASH_SOURCE[0]}")/.." && pwd)"
LLVM=/opt/rocm/llvm
OUT="$(mktemp -d)"
trap 'rm -rf "$OUT"' EXIT
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -shared-libsan"
"$LLVM/bin/clang" -O1 -g -fno-omit-frame-pointer $SAN -std=c11 -fPIC -shared \
    -ffp-contract=off -o "$OUT/liboracle.so" "$ROOT/oracle/specverify_oracle.c" -lm
CSRC="$ROOT/rejection_sampling_verification_row_amd/csrc"
/opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared -ffp-contract=off \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -shared-libsan \
    -Xarch_host -fno-omit-frame-pointer \
    -I"$ROOT/include" -I"$CSRC" "$CSRC/sv_kernels.hip" "$CSRC/specverify.cpp" \
    -o "$OUT/libspecverify.so" 2>&1 | grep -v "packed-fp32-ops" || true
test -s "$OUT/libspecverify.so"
RT="$(ls "$LLVM"/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
cd "$ROOT"
SPECVERIFY_ORACLE_LIB="$OUT/liboracle.so" SPECVERIFY_LIB="$OUT/libspecverify.so" \
    LD_PRELOAD="$RT" ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1" \
    UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1" \
    python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
