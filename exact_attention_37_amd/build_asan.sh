#!/bin/bash
# Host AddressSanitizer build of libmiattn's C ABI, for the CPU-only ABI
# tests: miattn.cpp (argument validation, scratch management, chunk driver)
# is compiled with the sanitizer on its host code only and linked with the
# ordinary kernel objects of the last build (exact_attention_37_amd/_build).
# Output: exact_attention_37_amd/_build/libmiattn_asan.so
set -euo pipefail
PKG=$(cd "$(dirname "$0")" && pwd)
ROOT=$(dirname "$PKG")
B=$PKG/_build
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
mkdir -p "$B"
$HIPCC -O1 -g -fPIC -std=c++20 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops -I"$ROOT/include" -Wno-unused-result -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer -x hip -c "$PKG/csrc/miattn.cpp" -o "$B/miattn_asan.o" 2>&1 | grep -v "is not a recognized feature" || true
$HIPCC --offload-arch=gfx950 -shared -fPIC -shared-libasan -Xarch_host -fsanitize=address -o "$B/libmiattn_asan.so" "$B/miattn_asan.o" "$B/simt.o" "$B/prep.o" "$B/fwd_mfma.o" "$B/bwd_mfma.o" "$B/decode.o"
echo "$B/libmiattn_asan.so"
