"""CPU oracle for the block-quantized MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the timed part of the benchmark) may import, call or link any
module under ``oracle/``.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.

The oracle is a plain, slow, obviously-correct NumPy implementation in float64
of what the GPU path computes:

* ``codecs``  - exact code->value tables for OCP E4M3FN, E2M1 and offset INT4,
  and round-to-nearest-even quantizers onto those grids;
* ``formats`` - the three packed weight formats (INT4 g128, FP8 128x128 block,
  NVFP4 per-16) with their quantizers, packers and dequantizers;
* ``moe``     - router top-k + softmax, stable permutation, the per-expert
  SwiGLU loop and the slot-ordered combine.

It shares no code with the GPU path.  Parity of every function is pinned in
``tests/test_codecs.py`` and ``tests/test_oracle.py`` against values the model
cards print, closed forms, library routines and brute force; the final layer
output against the pages' own systems is "parity unpinned" because the pages
print no layer values.
"""
