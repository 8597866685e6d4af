#!/bin/bash
# The CPU test suite (-m "not gpu") against AddressSanitizer + UndefinedBehaviorSanitizer builds of
# the oracle, the input generator and the host code of libmoe_int4.so (argument validation, the
# workspace layout, launch set-up; the device code is built as usual). It runs on a copy of the
# tree in a temporary directory, so the in-tree libraries are left alone. CPU only: it makes no GPU
# call. Usage: bash tests/sanitize.sh [extra pytest arguments]
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
LLVM=/opt/rocm/llvm
RT="$(ls "$LLVM"/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
WORK="$(mktemp -d)"
trap 'rm -rf "$WORK"' EXIT
tar -C "$ROOT" --exclude=./_work --exclude=./.git --exclude=./gpurun_out --exclude=./_build -cf - . | tar -C "$WORK" -xf -
SAN=(-fsanitize=address -fsanitize=undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g)
COMMON=(-O1 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared -Wall -Wno-unknown-pragmas)
"$LLVM"/bin/clang -std=c11 "${COMMON[@]}" "${SAN[@]}" "$WORK"/oracle/moe_oracle.c -o "$WORK"/oracle/libmoe_oracle.so -lm
"$LLVM"/bin/clang "${COMMON[@]}" "${SAN[@]}" "$WORK"/workload/moe_gen.c -o "$WORK"/workload/libmoe_gen.so -lm
CS="$WORK/bit_moe_expert_amd/csrc"
HOST_SAN=()
for f in "${SAN[@]}"; do HOST_SAN+=(-Xarch_host "$f"); done
mkdir -p "$WORK/obj"
for s in moe_abi.cpp route.hip gemv.hip gemm.hip gemm_b3.hip gemm_b2.hip dequant.hip vocab_topk.hip noalloc.hip; do
  lang=(); case $s in *.hip) lang=(-x hip);; esac
  /opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -fPIC -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
    "${HOST_SAN[@]}" -I "$WORK/include" -I "$CS" "${lang[@]}" -c "$CS/$s" -o "$WORK/obj/$s.o" 2>/dev/null &
done
wait
/opt/rocm/bin/hipcc --offload-arch=gfx950 -shared -fPIC -o "$WORK/bit_moe_expert_amd/libmoe_int4.so" "$WORK"/obj/*.o
# the libraries' sanitizer hooks resolve against the preloaded runtime (Python itself is not
# instrumented, so leak reports would be about the interpreter and are off)
cd "$WORK"
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 LD_PRELOAD="$RT" \
  python -m pytest tests -x -q -m "not gpu" -p no:cacheprovider "$@"
