#!/bin/bash
# Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU test suite
# (no GPU): the oracle (oracle/oracle.c) and the host side of libmoe.so (the
# argument validation of every entry point in csrc/api.hip) are rebuilt with
# both sanitizers, and `pytest -m "not gpu"` runs against those builds.  GPU
# code is built exactly as usual: every -fsanitize= on the hipcc line applies
# to the host pass only (-Xarch_host).  Any sanitizer report aborts the run.
#
#   bash tests/sanitize/run_host_sanitizers.sh
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/../.." && pwd)"
OUT="$(mktemp -d /tmp/moe_sanitize.XXXXXX)"
trap 'rm -rf "$OUT"' EXIT
LLVM=/opt/rocm/llvm
RT="$(ls "$LLVM"/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
echo "building sanitized copies in $OUT"
"$LLVM/bin/clang" -O1 -g -std=c11 -ffp-contract=off -fno-omit-frame-pointer \
  -fsanitize=address,undefined -fno-sanitize-recover=undefined -shared-libsan \
  -fPIC -shared "$ROOT/oracle/oracle.c" -lm -o "$OUT/liboracle_san.so"
/opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared \
  -fno-omit-frame-pointer -I "$ROOT/include" \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -shared-libsan \
  -Xclang -target-feature -Xclang -packed-fp32-ops \
  "$ROOT"/moe_token_routing_router_amd/csrc/*.hip -o "$OUT/libmoe_san.so" 2>&1 \
  | grep -v "is not a recognized feature for this target" || true
test -f "$OUT/libmoe_san.so"
echo "running the CPU suite under ASan + UBSan"
cd "$ROOT"
LD_PRELOAD="$RT" \
ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1" \
UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1" \
MOE_ORACLE_LIB="$OUT/liboracle_san.so" MOE_LIB="$OUT/libmoe_san.so" \
  python -m pytest tests -q -m "not gpu" -p no:cacheprovider \
  --ignore tests/test_oracle_mutants.py "$@"
