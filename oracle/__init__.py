"""Plain, slow fp64 CPU oracle of the JoLT KV-cache codec.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``kv_cache_compression_mode_amd``), and neither imports the other; the
only module both sides consume is the seeded input generator ``kvgen``, which
holds none of the codec's arithmetic.

What the oracle follows
-----------------------
"A JoLT for the KV Cache: Near-Lossless KV Cache Compression via Joint Tucker
and JL-Residual Allocation for LLMs" (arXiv 2607.12550v2), abstract; and the
aimodeling.com news article "JoLT compresses KV cache to one-third with Tucker
residuals", paragraphs 2 and 4.  The pages fix the method only in words:

* the K or V cache of a layer is a third-order tensor (heads x tokens x
  features);
* a partial Tucker decomposition compresses only the token and feature axes;
* the energy that truncation drops is restored by a rotated low-bit residual
  (random orthogonal rotation, then low-bit quantization), which whitens the
  error;
* one Lagrangian dual allocates Tucker ranks and residual bit-widths jointly,
  per layer group, separately for K and V, under one byte budget;
* FlashJoLT replaces the exact factor computation with a randomized SVD.

Every step the pages leave open is taken with a stated reading; each module
lists its readings in its header.  Modules:

``rng``       counter-based SplitMix64 words, uniforms and Box-Muller normals
``bf16``      fp64/fp32 -> bf16 rounding (nearest-even and directed)
``tucker``    Grams, eigen-factors, core, reconstruction (exact path)
``flash``     randomized-SVD factors (FlashJoLT)
``rotation``  the seeded Haar rotation Q
``quant``     group min-max quantizer, bit packing, dequantization
``alloc``     distortion/byte model and the Lagrangian-dual allocation
``codec``     encode / decode / relative Frobenius error, end to end

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, textbook special cases or brute force.  The pages'
printed error figures (0.009 K / 0.006 V at 2x) and the 5-13x FlashJoLT
speed-up were measured on real model caches and unnamed hardware and are not
reproducible here: parity unpinned for those two figures.
"""
