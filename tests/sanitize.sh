#!/bin/bash
# AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU tests (no GPU used):
#  1. the oracle and the input generators built by gcc with both sanitizers, under the
#     oracle's pin tests, the golden fixtures and the workload tests;
#  2. the host code of libibp.so (argument checks, launch set-up) built by hipcc with
#     both sanitizers on the host side only, under the C-ABI tests.
# The two runs load different sanitizer runtimes (gcc's, clang's), so they are
# separate processes.  Any report aborts the run (-fno-sanitize-recover=all).
set -euo pipefail
cd "$(dirname "$0")/.."
python -c "import oracle, workloads; oracle.build(sanitize=True); workloads.build(sanitize=True)"
IBP_SANITIZE_ORACLE=1 ASAN_OPTIONS=detect_leaks=0 \
  LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
  python -m pytest -q -p no:cacheprovider -m "not gpu" tests/test_oracle_pins.py tests/test_golden.py \
  tests/test_workloads.py
python -c "from bit_packing_amd.build import build_library; build_library(sanitize=True)"
RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
IBP_SANITIZE_LIB=1 ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD="$RT" \
  python -m pytest -q -p no:cacheprovider -m "not gpu" tests/test_abi.py
