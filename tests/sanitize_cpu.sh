#!/usr/bin/env bash
# CPU-only sanitizer run over the host code: the oracle (gcc, ASan + UBSan) under the oracle
# pins, and the library's host-side argument validation (clang through hipcc, ASan + UBSan on
# the host pass only) under the ABI host tests.  Needs no GPU; nothing here launches a kernel.
#
#   bash tests/sanitize_cpu.sh
#
# The two builds go to a temporary directory, so the in-tree libraries are left alone.  gcc's
# and clang's sanitizer runtimes cannot share a process, hence two pytest runs.
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
OUT="$(mktemp -d /tmp/dsa_sanitize.XXXXXX)"
trap 'rm -rf "$OUT"' EXIT
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer"

echo "[sanitize] oracle with gcc ASan+UBSan"
gcc -O1 -g -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared $SAN -Wall \
    -o "$OUT/libdsa_oracle.so" "$ROOT/oracle/dsa_oracle.c" -lm
(cd "$ROOT" && ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
    DSA_ORACLE_LIB="$OUT/libdsa_oracle.so" \
    python -m pytest -q -m "not gpu" -p no:cacheprovider tests/test_oracle_formats.py tests/test_oracle_layout.py \
        tests/test_oracle_score.py tests/test_oracle_topk_mla.py tests/test_oracle_dcp.py)

echo "[sanitize] library host code with clang ASan+UBSan (device code built as usual)"
FLAGS=(--offload-arch=gfx950 -O1 -g -fPIC -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops
       -I "$ROOT/include" -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined
       -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer)
objs=()
# the library's sources, as the in-tree build lists them
SRCS="$(cd "$ROOT/long_context_sparse_paged_amd" && python -c 'import build; print(" ".join(build.SOURCES))')"
for src in $SRCS; do
    "$HIPCC" -x hip "${FLAGS[@]}" -c "$ROOT/long_context_sparse_paged_amd/csrc/$src" -o "$OUT/${src%.*}.o" 2>&1 \
        | grep -v "is not a recognized feature for this target" || true
    objs+=("$OUT/${src%.*}.o")
done
"$HIPCC" --offload-arch=gfx950 -shared -fPIC -o "$OUT/libdsa.so" "${objs[@]}"
RT="$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
(cd "$ROOT" && ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD="$RT" DSA_LIB="$OUT/libdsa.so" \
    python -m pytest -q -m "not gpu" -p no:cacheprovider tests/test_abi_host.py)
echo "[sanitize] clean"
