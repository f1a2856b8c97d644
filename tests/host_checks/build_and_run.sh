#!/bin/bash
# Builds the C-ABI host code (csrc/pa_api.hip) with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host side only, links it with launcher
# stand-ins and the driver, and runs the driver (no GPU needed: every call
# returns before a device access or reaches a stubbed launch).
# Usage: build_and_run.sh OUT_DIR
set -euo pipefail
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="$1"
mkdir -p "$OUT"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
INC=(-I "$ROOT/include" -I "$ROOT/paged_kv_cache_pa_amd/csrc")
SAN=(-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined
     -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer)
# pa_api.hip with its device part (the allocation-free entry point's scratch
# array has no kernels, but the host code registers it); sanitizers apply to
# the host side only.
"$HIPCC" --offload-arch=gfx950 -O1 -g -std=c++17 "${SAN[@]}" "${INC[@]}" \
  -c "$ROOT/paged_kv_cache_pa_amd/csrc/pa_api.hip" -o "$OUT/pa_api.o"
"$HIPCC" --offload-arch=gfx950 --cuda-host-only -O1 -g -std=c++17 "${SAN[@]}" "${INC[@]}" \
  -x hip -c "$HERE/stubs.cpp" -o "$OUT/stubs.o"
"$HIPCC" --offload-arch=gfx950 --cuda-host-only -O1 -g -std=c++17 "${SAN[@]}" "${INC[@]}" \
  -x hip -c "$HERE/driver.cpp" -o "$OUT/driver.o"
"$HIPCC" --offload-arch=gfx950 "${SAN[@]}" -o "$OUT/host_checks" "$OUT/pa_api.o" "$OUT/stubs.o" \
  "$OUT/driver.o"
ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0" \
UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1" "$OUT/host_checks"
