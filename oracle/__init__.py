"""CPU oracle for the routed MoE FFN layer and its expert cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The GPU library never calls it and has no CPU fallback; this
package imports nothing from the GPU library either.

Everything here is plain and slow on purpose: float64 NumPy, one function per
step of the layer, each citing the passage it follows.  The pages (FreeToken
linux, quantization, rtx 4090, 290b model and gguf pages) describe the system
around the layer (one LRU over (layer, expert) entries shared by all MoE
layers, hits executed from the GPU copy, misses filled over PCIe from pinned
host memory) but never write the layer's arithmetic.  Where they are silent
the oracle takes the plainest textbook reading; every such reading is listed
in the repository's design notes.

Modules:
  formats -- bfloat16 and OCP MXFP4 (E2M1 codes + E8M0 scales) decoding.
  mx      -- MXFP8 E4M3 activation quantization (native MXFP4 mode).
  moe     -- router logits, top-k, gating, permutation, SwiGLU expert,
             combine, and the whole layer.
  lru     -- the shared (layer, expert) LRU slot-table simulator.
  policy  -- the bandwidth-derived miss split.
"""
from . import formats, mx, moe, lru, policy  # noqa: F401
