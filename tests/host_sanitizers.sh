#!/usr/bin/env bash
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the library's
# argument validation, on the CPU (no GPU, no device code executed).
#
# Builds the sanitizer copy of the library (host code instrumented, device
# code unchanged), then runs the host-only ABI tests with the sanitizer
# runtime preloaded ahead of anything else the environment preloads. Any
# sanitizer report aborts the process, so a pass means no report.
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
cd "$ROOT"
python latent_sparse_moe_amd/build.py --sanitize
RT="$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -n 1)"
export MOE_LATENT_LIB="$ROOT/_build/san/libmoe_latent.so"
# leaks: the HIP runtime and CPython keep allocations until exit by design
export ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1:verify_asan_link_order=0"
export UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"
LD_PRELOAD="$RT${LD_PRELOAD:+:$LD_PRELOAD}" \
  python -m pytest -q -p no:cacheprovider tests/test_abi.py "$@"
