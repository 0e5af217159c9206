#!/bin/bash
# CPU-only AddressSanitizer + UndefinedBehaviorSanitizer run of the host
# side: the library's host code (pool bookkeeping, validation, planning,
# offline helpers, C ABI) and the oracle's C codec are rebuilt with both
# sanitizers in a scratch copy of the tree, and the "not gpu" test suite runs
# against them.  Device code is compiled as usual (sanitizers apply to the
# host pass only).  Usage: bash tests/sanitize_host.sh [pytest args]
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
WORK="$(mktemp -d /tmp/oscar_sanitize.XXXXXX)"
trap 'rm -rf "$WORK"' EXIT
tar -C "$ROOT" --exclude=.git --exclude=_work --exclude=_build --exclude=gpurun_out --exclude=__pycache__ \
  --exclude='*.so' -cf - . | tar -C "$WORK" -xf -
CLANG=/opt/rocm/llvm/bin/clang
HIPCC=/opt/rocm/bin/hipcc
RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g -O1"

# oracle codec (same semantics flags as its normal build, plus the sanitizers)
$CLANG $SAN -shared-libsan -fno-fast-math -ffp-contract=off -mfma -fPIC -shared -std=c11 \
  -o "$WORK/oracle/liboscar_oracle.so" "$WORK/oracle/oscar_oracle.c" -lm

# library: host pass sanitized, device pass unchanged
HFLAGS="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined"
DEV="-O1 -g -std=c++17 -fPIC --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops -I $WORK/include"
mkdir -p "$WORK/_san"
for src in oscar_host.cpp kernels_encode.hip kernels_decode.hip kernels_bf16.hip kernels_calib.hip kernels_prefill.hip; do
  $HIPCC -x hip $DEV $HFLAGS -shared-libsan -c "$WORK/bit_kv_cache_segment_amd/csrc/$src" -o "$WORK/_san/$src.o" 2>&1 \
    | grep -v "packed-fp32-ops" || true
done
$HIPCC --offload-arch=gfx950 -shared -fPIC $HFLAGS -shared-libsan -o "$WORK/bit_kv_cache_segment_amd/liboscar.so" "$WORK"/_san/*.o

# both libraries really carry the sanitizers
for so in "$WORK/oracle/liboscar_oracle.so" "$WORK/bit_kv_cache_segment_amd/liboscar.so"; do
  nm -D "$so" | grep -q "__asan_init" || { echo "not instrumented: $so"; exit 1; }
  nm -D "$so" | grep -q "__ubsan_handle" || { echo "not instrumented (UBSan): $so"; exit 1; }
done

cd "$WORK"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
LD_PRELOAD="$RT" python -m pytest tests -q -m "not gpu" -x -p no:cacheprovider "$@"
LD_PRELOAD="$RT" python -c "import bit_kv_cache_segment_amd as ok, oracle; ok.lib(); oracle.lib(); print('checked:', ok.LIB_PATH, oracle._LIB)"
