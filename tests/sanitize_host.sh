#!/bin/bash
# Host-code sanitizer run (CPU only, no GPU needed): builds the C oracle with
# gcc and the library (host parts only instrumented; device code unchanged)
# with clang through hipcc, both under AddressSanitizer and
# UndefinedBehaviorSanitizer with recovery off, then runs the CPU tests that
# exercise them: the oracle pins against the instrumented oracle, and the
# ABI validation and the expert cache slot planner against the instrumented
# library.  Usage: tests/sanitize_host.sh [output dir]
set -euo pipefail
R=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-/tmp/moe_sanitize}
mkdir -p "$OUT"
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
SAN="-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"

gcc -O1 -g -std=c11 -fPIC -shared -fopenmp -ffp-contract=off $SAN \
    -o "$OUT/liboracle.so" "$R/oracle/oracle.c" -lm

SRCS="abi.cpp route.hip permute.hip quant.hip ffn.hip ffn_decode.hip ffn_bitplane.hip \
      ffn_prefill.hip combine.hip alloc.hip cache.hip cache.cpp noalloc.hip retile.hip"
ARGS=()
for s in $SRCS; do ARGS+=("$R/quantized_mixture_experts_fp32_amd/csrc/$s"); done
"$HIPCC" --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared \
    -Xclang -target-feature -Xclang -packed-fp32-ops -mllvm -amdgpu-mfma-vgpr-form=1 \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer \
    -I "$R/include" -o "$OUT/libmoe_wq.so" "${ARGS[@]}"

export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1
cd "$R"
LD_PRELOAD=$(gcc -print-file-name=libasan.so) python3 -c "
import sys, oracle, pytest
oracle.LIB = sys.argv[1]
sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',
                      'tests/test_oracle_pins.py']))" "$OUT/liboracle.so"
RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
LD_PRELOAD="$RT" python3 -c "
import sys, pytest
import quantized_mixture_experts_fp32_amd as moe
moe.LIB_PATH = sys.argv[1]
sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',
                      'tests/test_abi_host.py', 'tests/test_cache_plan.py']))" "$OUT/libmoe_wq.so"
echo "sanitized host run: clean"
