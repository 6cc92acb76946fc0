"""MI355X-native DSA hot path: MXFP8 Lightning Indexer + fused Top-K and
Sparse Flash Attention over paged FP8 caches, as hand-written HIP for gfx950
behind a C ABI (``include/dsa.h``).

The native library is loaded on first use by :mod:`.ops`; importing the
package itself does not touch the GPU.
"""
__all__ = ["ops", "synth"]
