"""Plain fp64 CPU oracle for the DSA hot path (Lightning Indexer + Top-K +
Sparse Flash Attention).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or call anything in this package.
The product path (the C-ABI library and its Python binding) never routes
through it, and this package imports nothing from the product.

What it computes, and where each step comes from:
  * "Deep Dive into Sparse Attention and Engineering Optimizations ..." (page
    1), section 1 "Hybrid Architecture": a lightweight indexer scores every
    historical key for each query, keeps the Top-K positions, and Sparse Flash
    Attention attends only to those positions of an MLA cache.
  * same page, section 2.2 "Memory Optimization": the indexer is fully MXFP8
    quantised with one scale per 32 elements; the SFA KV cache is FP8 with one
    scale per 128-element tile of each token.
  * "Kimi K3.1 Pro Inference Acceleration ..." (page 3), sections "Lightning
    Indexer Three-Stream Coordination" (scoring, head-weight weighting, Top-K
    fused over the paged K cache), "Full MXFP8 Quantization ..." (group 32),
    "FP8 KVCache ..." (tile 128) and "Preserving a Mixed-Precision Path" (bf16
    queries, quantisation only on the index and cache paths).
  * The exact arithmetic the pages leave open is fixed by the benchmark spec
    for this library: I(t,s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]) over s <= t;
    E4M3 elements with an E8M0 scale per 32; KV tiles scaled by amax/448 in
    fp32; Top-K by (higher score, then lower index); SFA softmax scale
    1/sqrt(576) with value = the 512-wide latent.

Readings taken where the pages are silent are listed in the module that
applies them.  Floating point is fp64 from exactly dequantised values.

Parity status: every function here is pinned by tests under tests/ (closed
forms, brute force on tiny inputs, library routines, invariants).  The pages
print no numeric example, so end-to-end values against the pages themselves
are parity unpinned.
"""
from . import formats, quant, pools, indexer, attention  # noqa: F401
