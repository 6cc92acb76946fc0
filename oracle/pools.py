"""Paged cache layouts, written out plainly.

Test infrastructure only (see package docstring).

The pages say the fused indexer reads "paged K-cache directly" ("Deep Dive
into Sparse Attention ...", page 1, section 2.1 "Computation Optimization")
and that SFA reads "paged key-value caches based on indices" ("Adapting and
Optimizing Kimi K3.1 Pro ...", page 2, section 2).  They give no layout.
Readings taken:
  * pages hold 64 tokens; one block table [B, pages] of physical page ids is
    shared by both caches, and token s of sequence b is in page
    block_table[b][s // 64] at offset s % 64;
  * indexer K page (8448 bytes): the 64 tokens' 128 E4M3 codes in four
    tiles of 16 tokens (bytes 2048j .. 2048j + 2047 for tokens 16j .. 16j+15),
    then their 4 E8M0 bytes in four 64-byte tiles.  Inside a code tile, code d
    of the tile's token n sits at 1024*(d // 64) + 256*((d % 64) // 16)
    + 16*n + d % 16: sixteen-byte pieces of the tile's tokens side by side,
    the pieces of dims 0-15 first, then 16-31, 32-47, 48-63 (1 KB), then the
    same for dims 64-127.  Inside a scale tile, byte b of token n sits at
    16*b + n.  (Any byte order inside a page serves the method; this one
    lets a reader take one piece per token and dim range from contiguous
    memory.)
  * SFA KV page (41984 bytes): 64 records of 656 bytes (layout in quant.py),
    i.e. record of slot p*64+o at byte (p*64+o)*656 of the pool.
"""
from __future__ import annotations

import numpy as np

from .quant import RECORD_BYTES

PAGE = 64
D_I = 128
K_PAGE_BYTES = PAGE * D_I + PAGE * (D_I // 32)   # 8448
K_TILE = 16                                      # tokens per K-page tile


def _k_code_offsets() -> np.ndarray:
    """[64, 128]: byte offset in a K page of code d of the token at offset o."""
    off = np.empty((PAGE, D_I), dtype=np.int64)
    for o in range(PAGE):
        tile, n = divmod(o, K_TILE)
        for d in range(D_I):
            half, rest = divmod(d, 64)
            piece, byte = divmod(rest, 16)
            off[o, d] = tile * K_TILE * D_I + half * 1024 + piece * 256 + n * 16 + byte
    return off


def _k_scale_offsets() -> np.ndarray:
    """[64, 4]: byte offset in a K page of E8M0 byte b of the token at offset o."""
    off = np.empty((PAGE, D_I // 32), dtype=np.int64)
    for o in range(PAGE):
        tile, n = divmod(o, K_TILE)
        for b in range(D_I // 32):
            off[o, b] = PAGE * D_I + tile * 64 + b * K_TILE + n
    return off


K_CODE_OFF = _k_code_offsets()
K_SCALE_OFF = _k_scale_offsets()


def k_pool_write(codes: np.ndarray, e8m0: np.ndarray, slots: np.ndarray,
                 n_pages: int, pool: np.ndarray = None) -> np.ndarray:
    """Scatter MXFP8 rows (codes [n,128], e8m0 [n,4]) to their slots."""
    if pool is None:
        pool = np.zeros((n_pages, K_PAGE_BYTES), dtype=np.uint8)
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        p, o = divmod(int(slot), PAGE)
        pool[p, K_CODE_OFF[o]] = codes[i]
        pool[p, K_SCALE_OFF[o]] = e8m0[i]
    return pool


def k_pool_read(pool: np.ndarray, bt_row: np.ndarray, n_tokens: int):
    """Gather the first n_tokens of one sequence -> (codes [n,128], e8m0 [n,4])."""
    codes = np.empty((n_tokens, D_I), dtype=np.uint8)
    e8 = np.empty((n_tokens, 4), dtype=np.uint8)
    for s in range(0, n_tokens, PAGE):
        n = min(PAGE, n_tokens - s)
        page = pool[int(bt_row[s // PAGE])]
        codes[s:s + n] = page[K_CODE_OFF[:n]]
        e8[s:s + n] = page[K_SCALE_OFF[:n]]
    return codes, e8


def kv_pool_write(records: np.ndarray, slots: np.ndarray, n_pages: int,
                  pool: np.ndarray = None) -> np.ndarray:
    """Scatter 656-byte records to their slots; pool shape [n_pages*64, 656]."""
    if pool is None:
        pool = np.zeros((n_pages * PAGE, RECORD_BYTES), dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    pool[slots[keep]] = records[keep]
    return pool


def kv_pool_read(pool: np.ndarray, bt_row: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Records of logical positions of one sequence (positions must be >= 0)."""
    positions = np.asarray(positions, dtype=np.int64)
    slots = bt_row[positions // PAGE].astype(np.int64) * PAGE + positions % PAGE
    return pool[slots]
