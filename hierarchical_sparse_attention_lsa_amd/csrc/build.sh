#!/bin/bash
# Builds liblsa_hip.so for gfx950 next to the Python binding.
set -euo pipefail
here="$(cd "$(dirname "$0")" && pwd)"
out="$here/../liblsa_hip.so"
flags=(--offload-arch=gfx950 -O3 -std=c++17 -fPIC -shared -fvisibility=hidden
       -Xclang -target-feature -Xclang -packed-fp32-ops)
hipcc "${flags[@]}" "$here/lsa_api.hip" "$here/lsa_index.hip" "$here/lsa_select.hip" "$here/lsa_select_fast.hip" \
      "$here/lsa_select_decode.hip" "$here/lsa_attn.hip" "$here/lsa_attn_bwd.hip" "$here/lsa_noalloc.hip" \
      -o "$out.tmp"
mv "$out.tmp" "$out"
echo "built $out"
