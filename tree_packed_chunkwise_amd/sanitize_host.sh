#!/bin/bash
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer check of the library
# (CPU only; device code is built as usual, every -fsanitize applies to the
# host pass alone).  Copies the package, oracle, header and tests into OUT,
# builds the library there with the sanitizers, and runs the CPU tests that
# drive the host planner, the L1 planner, the C-ABI argument checks and the
# window bookkeeping against it.
#
#   bash tree_packed_chunkwise_amd/sanitize_host.sh [OUT]    (default: _build/sanitize)
set -e
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-$ROOT/_build/sanitize}
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
rm -rf "$OUT"; mkdir -p "$OUT/_objs"
(cd "$ROOT" && tar cf - tree_packed_chunkwise_amd oracle include tests) | (cd "$OUT" && tar xf -)
rm -f "$OUT/tree_packed_chunkwise_amd/libkda_tree.so"
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=undefined"
FL="--offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops -O1 -g -fPIC -std=c++17 -I$OUT/include -I$OUT/tree_packed_chunkwise_amd/csrc"
objs=""
for f in "$OUT"/tree_packed_chunkwise_amd/csrc/*.hip "$OUT"/tree_packed_chunkwise_amd/csrc/*.cpp; do
  o="$OUT/_objs/$(basename "$f").o"
  case "$f" in *.cpp) X="-x hip" ;; *) X="" ;; esac
  $HIPCC $FL $SAN $X -c "$f" -o "$o" 2>/dev/null &
  objs="$objs $o"
done
wait
for o in $objs; do [ -f "$o" ] || { echo "compile failed: $o"; exit 1; }; done
$HIPCC --offload-arch=gfx950 -shared -fPIC $SAN -shared-libsan $objs -o "$OUT/tree_packed_chunkwise_amd/libkda_tree.so"
ASAN_RT=$($HIPCC -print-file-name=libclang_rt.asan-x86_64.so)
[ -f "$ASAN_RT" ] || ASAN_RT=$(dirname "$($HIPCC -print-libgcc-file-name)")/libclang_rt.asan-x86_64.so
nm -D "$OUT/tree_packed_chunkwise_amd/libkda_tree.so" | grep -q __asan_report || { echo "library not instrumented"; exit 1; }
cd "$OUT"
LD_PRELOAD="$ASAN_RT" ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 \
  UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
  python -m pytest -x -q -m "not gpu" -p no:cacheprovider \
    tests/test_planner_lib.py tests/test_l1_lib.py tests/test_binding_checks.py tests/test_window.py
