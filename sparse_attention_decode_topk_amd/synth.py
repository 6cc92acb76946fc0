"""Seeded synthetic inputs for the DSA decode/prefill hot path.

This module draws random numbers and lays out sequence/page bookkeeping.  It
holds none of the method's arithmetic: no quantisation, no scoring, no
selection, no attention.  Both the HIP path (through the Python binding) and
the fp64 CPU oracle consume what it returns.

Value distributions follow the workloads described for the Lightning Indexer
and Sparse Flash Attention ("Deep Dive into Sparse Attention ...", section 1
"Hybrid Architecture", and "Kimi K3.1 Pro Inference Acceleration", sections
"Full MXFP8 Quantization ..." and "FP8 KVCache ..."): every query, key, latent
and rope value is N(0,1) drawn in float32; tensors the method keeps in bf16
(indexer q/k before MXFP8, SFA q, KV before FP8) are rounded to bf16 with
round-to-nearest-even; head weights are N(0,1)/sqrt(H_I) in float32.

Recipe (per config index c, 1-based):
  * one numpy SeedSequence(1000 + c) spawns 8 independent PCG64 streams, one
    per draw, in this fixed order: 0 ragged lengths, 1 indexer q, 2 indexer k,
    3 head weights, 4 SFA q, 5 KV, 6 needle positions, 7 page permutation;
  * needles (single-query decode config): 16 distinct positions whose
    indexer-k row and 576-wide KV row are multiplied by 4 after bf16 rounding
    (exact in bf16);
  * pages: sequence b owns ceil(L_b / 64) pages taken in order from a
    permutation of all pages (identity when the config says so).  Token s of
    sequence b lives in slot block_table[b][s // 64] * 64 + s % 64.

bf16 tensors are returned as uint16 bit patterns so that both consumers see
identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

PAGE = 64          # tokens per KV page
D_I = 128          # indexer head dim
D_LATENT = 512     # MLA latent dim (also the value dim)
D_ROPE = 64        # MLA rope dim
D_QK = D_LATENT + D_ROPE


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload (sizes only; values come from `make`)."""
    index: int                 # 1-based config number, seeds the generator
    name: str
    batch: int
    h_index: int               # indexer heads H_I
    h_attn: int                # SFA query heads H
    topk: int
    # context lengths: either fixed `ctx` or ragged uniform [lo, hi]
    ctx: int = 0
    ragged: Optional[tuple] = None
    # query rows: "last" = one decode row per sequence at t = L-1,
    # "all" = every position of sequence 0, or an explicit (first, count) range
    rows: object = "last"
    q_per_seq: int = 1         # with rows="last": query rows per sequence, t = L-q .. L-1
    needles: int = 0
    identity_pages: bool = False
    description: str = ""


# Workloads: tiny causal prefill, single-query decode with needles, ragged
# decode batch, long-context decode batch (the throughput headline), and a
# chunked prefill against a long paged cache.
CONFIGS: Dict[str, Config] = {
    "tiny_prefill": Config(1, "tiny_prefill", batch=1, h_index=4, h_attn=8, topk=64,
                           ctx=512, rows="all", identity_pages=True,
                           description="1 seq, L=512, all 512 positions query, H_I=4, H=8, K=64"),
    "decode_8k_needles": Config(2, "decode_8k_needles", batch=1, h_index=64, h_attn=128,
                                topk=2048, ctx=8192, needles=16,
                                description="B=1, L=8192, 16 needle keys x4, permuted pages"),
    "decode_ragged_b32": Config(3, "decode_ragged_b32", batch=32, h_index=64, h_attn=128,
                                topk=2048, ragged=(4096, 65536),
                                description="B=32, L~U[4096,65536], shuffled pages"),
    "decode_128k_b8": Config(4, "decode_128k_b8", batch=8, h_index=64, h_attn=128,
                             topk=2048, ctx=131072,
                             description="B=8, L=131072, shuffled pages"),
    "prefill_chunk_8k_of_128k": Config(5, "prefill_chunk_8k_of_128k", batch=1, h_index=64,
                                       h_attn=128, topk=2048, ctx=131072,
                                       rows=(131072 - 8192, 8192),
                                       description="1 seq, 8192 query rows t=122880..131071 "
                                                   "against a 131072-token cache"),
    # multi-query decode (speculative verification of drafted tokens): the
    # long-context decode batch with 4 query tokens per sequence
    "decode_mtp4_128k_b8": Config(6, "decode_mtp4_128k_b8", batch=8, h_index=64, h_attn=128,
                                  topk=2048, ctx=131072, q_per_seq=4,
                                  description="B=8 x 4 query tokens t=L-4..L-1, L=131072, "
                                              "shuffled pages"),
}
CONFIG_ORDER: List[str] = list(CONFIGS)


def config(name_or_index) -> Config:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index - 1]]
    return CONFIGS[name_or_index]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the uint16 bit pattern.

    Uses torch's CPU cast (torch is only the rounding tool here)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(cfg: Config):
    ss = np.random.SeedSequence(1000 + cfg.index)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8)]


def _normal_bf16(rng, shape, chunk_rows: int = 1 << 16) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, produced in row chunks to bound
    peak memory (the stream is consumed in the same order either way)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    flat = out.reshape(rows, inner)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        flat[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, inner), dtype=np.float32))
    return out


def lengths(cfg: Config) -> np.ndarray:
    rng = _streams(cfg)[0]
    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    return np.full(cfg.batch, cfg.ctx, dtype=np.int32)


def rows_of(cfg: Config, seq_lens: np.ndarray):
    """Query rows as (row_seq, row_pos) with row_pos the causal limit t."""
    if cfg.rows == "last":
        q = cfg.q_per_seq
        row_seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), q)
        row_pos = (seq_lens.astype(np.int64)[:, None] - q + np.arange(q)[None, :]).reshape(-1)
        return row_seq, row_pos.astype(np.int32)
    if cfg.rows == "all":
        L = int(seq_lens[0])
        return np.zeros(L, dtype=np.int32), np.arange(L, dtype=np.int32)
    first, count = cfg.rows
    return np.zeros(count, dtype=np.int32), np.arange(first, first + count, dtype=np.int32)


def page_tables(cfg: Config, seq_lens: np.ndarray, rng=None):
    """Block table [B, max_pages] (unused entries 0), per-token slot mapping,
    sequence token offsets and the page count of the pool."""
    n_pages = [(int(L) + PAGE - 1) // PAGE for L in seq_lens]
    total = int(sum(n_pages))
    if cfg.identity_pages:
        perm = np.arange(total, dtype=np.int64)
    else:
        if rng is None:
            rng = _streams(cfg)[7]
        perm = rng.permutation(total).astype(np.int64)
    max_pages = max(n_pages)
    bt = np.zeros((cfg.batch, max_pages), dtype=np.int32)
    starts = np.zeros(cfg.batch, dtype=np.int64)
    off = 0
    tok = 0
    slots = []
    for b, npg in enumerate(n_pages):
        bt[b, :npg] = perm[off:off + npg]
        starts[b] = tok
        s = np.arange(int(seq_lens[b]), dtype=np.int64)
        slots.append(bt[b, s // PAGE].astype(np.int64) * PAGE + s % PAGE)
        off += npg
        tok += int(seq_lens[b])
    return bt, np.concatenate(slots), starts, total


def make(cfg_or_name, with_sfa: bool = True, with_index: bool = True,
         row_subset: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Draw the full input set of one config.

    `with_sfa` / `with_index` skip drawing the (large) SFA or indexer tensors;
    the streams are independent, so the remaining tensors are unchanged.
    `row_subset` keeps only those query rows of the row-shaped tensors (they
    are still drawn in full so that the values do not depend on the subset).
    """
    cfg = cfg_or_name if isinstance(cfg_or_name, Config) else config(cfg_or_name)
    st = _streams(cfg)
    seq_lens = lengths(cfg)
    row_seq, row_pos = rows_of(cfg, seq_lens)
    R = len(row_seq)
    total_tokens = int(seq_lens.sum())
    bt, slots, starts, total_pages = page_tables(cfg, seq_lens, st[7])
    out: Dict[str, np.ndarray] = dict(
        seq_lens=seq_lens, row_seq=row_seq, row_pos=row_pos, block_table=bt,
        slot_mapping=slots, seq_starts=starts,
        total_pages=np.int64(total_pages), h_index=np.int32(cfg.h_index),
        h_attn=np.int32(cfg.h_attn), topk=np.int32(cfg.topk))
    needle_pos = None
    if cfg.needles:
        needle_pos = np.sort(st[6].choice(total_tokens, size=cfg.needles, replace=False))
        out["needles"] = needle_pos.astype(np.int64)
    if with_index:
        q_idx = _normal_bf16(st[1], (R, cfg.h_index, D_I))
        k_idx = _normal_bf16(st[2], (total_tokens, D_I))
        w = (st[3].standard_normal((R, cfg.h_index), dtype=np.float32)
             * np.float32(1.0 / math.sqrt(cfg.h_index))).astype(np.float32)
        if needle_pos is not None:
            k_idx[needle_pos] = _times4_bf16(k_idx[needle_pos])
        out.update(q_idx=q_idx, k_idx=k_idx, w=w)
    if with_sfa:
        q_sfa = _normal_bf16(st[4], (R, cfg.h_attn, D_QK))
        kv = _normal_bf16(st[5], (total_tokens, D_QK))
        if needle_pos is not None:
            kv[needle_pos] = _times4_bf16(kv[needle_pos])
        out.update(q_sfa=q_sfa, kv=kv)
    if row_subset is not None:
        sel = np.asarray(row_subset, dtype=np.int64)
        for k in ("row_seq", "row_pos", "q_idx", "w", "q_sfa"):
            if k in out:
                out[k] = np.ascontiguousarray(out[k][sel])
    return out


def _times4_bf16(bits: np.ndarray) -> np.ndarray:
    """Multiply bf16 values by 4 (exact: exponent + 2; inputs are far from
    the bf16 overflow threshold)."""
    return f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(4.0))


def rotate_pages(block_table: np.ndarray, seq_lens: np.ndarray, total_pages: int,
                 seed: int) -> np.ndarray:
    """A block table with the same sequences mapped onto a different page
    permutation (used to check that results do not depend on page placement)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    remap = rng.permutation(total_pages).astype(np.int32)
    bt = block_table.copy()
    for b, L in enumerate(seq_lens):
        npg = (int(L) + PAGE - 1) // PAGE
        bt[b, :npg] = remap[block_table[b, :npg]]
    return bt
