"""Device-side state of one synthetic workload, built through the C ABI
(quantisers included), plus the parity rules the GPU tests apply.

Nothing here computes the method: the caches are written by the HIP
quantisers, and expected values come from the oracle in the tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import pools
from sparse_attention_decode_topk_amd import ops, synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class DeviceState:
    """Quantised caches and query tensors of one config on the GPU."""

    def __init__(self, inp, with_sfa: bool = True, device: str = "cuda"):
        dev = torch.device(device)
        self.inp = inp
        self.dev = dev
        self.R, self.H_I = inp["q_idx"].shape[:2]
        self.topk = int(inp["topk"])
        self.pages = int(inp["total_pages"])
        self.block_table = torch.from_numpy(inp["block_table"]).to(dev)
        self.row_seq = torch.from_numpy(inp["row_seq"]).to(dev)
        self.row_pos = torch.from_numpy(inp["row_pos"]).to(dev)
        self.slots = torch.from_numpy(inp["slot_mapping"]).to(dev)
        q = bf16_tensor(inp["q_idx"], dev)
        self.q_fp8, self.q_e8m0 = ops.mxfp8_quant(q)
        self.w = torch.from_numpy(inp["w"]).to(dev)
        self.k_pool = torch.zeros((self.pages, ops.K_PAGE_BYTES), dtype=torch.uint8, device=dev)
        ops.mxfp8_quant_paged(bf16_tensor(inp["k_idx"], dev), self.slots, self.k_pool)
        self.kv_pool = None
        if with_sfa and "kv" in inp:
            self.H = inp["q_sfa"].shape[1]
            self.q_sfa = bf16_tensor(inp["q_sfa"], dev)
            self.kv_pool = torch.zeros((self.pages, ops.KV_PAGE_BYTES), dtype=torch.uint8, device=dev)
            kv = bf16_tensor(inp["kv"], dev)
            ops.kv_fp8_quant_paged_write(kv, self.slots, self.kv_pool)
            del kv
        torch.cuda.synchronize()

    def indexer(self, topk=None, workspace=None):
        topk = self.topk if topk is None else topk
        return ops.dsa_indexer_topk(self.q_fp8, self.q_e8m0, self.w, self.k_pool, self.block_table,
                                    self.row_seq, self.row_pos, topk, workspace=workspace)

    def scores(self):
        ld = int(self.inp["row_pos"].max()) + 1
        return ops.dsa_indexer_scores(self.q_fp8, self.q_e8m0, self.w, self.k_pool,
                                      self.block_table, self.row_seq, self.row_pos, ld)

    def sfa(self, idx: torch.Tensor, workspace=None):
        return ops.dsa_sparse_attn(self.q_sfa, self.kv_pool, self.block_table, self.row_seq, idx,
                                   workspace=workspace)


def stale_caches(st, slots, seed):
    """Copies of the state's caches with the given slots overwritten by
    random bytes (what a cache holds before a step writes its new tokens);
    slots < 0 or past the pool are left alone."""
    rng = np.random.default_rng(seed)
    kp, kvp = st.k_pool.clone(), st.kv_pool.clone()
    for s in slots:
        if s < 0 or s >= st.pages * 64:
            continue
        p, o = divmod(int(s), 64)
        kp[p, torch.from_numpy(pools.K_CODE_OFF[o]).cuda()] = \
            torch.from_numpy(rng.integers(0, 256, 128, dtype=np.uint8)).cuda()
        kp[p, torch.from_numpy(pools.K_SCALE_OFF[o]).cuda()] = \
            torch.from_numpy(rng.integers(100, 140, 4, dtype=np.uint8)).cuda()
        kvp[p, o * 656:(o + 1) * 656] = torch.from_numpy(rng.integers(0, 256, 656, dtype=np.uint8)).cuda()
    return kp, kvp


def check_topk_row(gidx, gsc, ora, K, t, tol_rel=1e-4):
    """Top-K pass rule for one row against the oracle's result dict.

    |S_gpu| = |S_oracle| = min(K, t+1), unique, within [0, t], ascending,
    -1 padding; every position in the symmetric difference has an oracle
    score within tol_rel * max|I| of the oracle's K-th score; the GPU's
    reported scores are within the same tolerance of the oracle's."""
    n = min(K, t + 1)
    g = np.asarray(gidx)
    assert np.all(g[n:] == -1), "padding"
    sel = g[:n]
    assert np.all(sel >= 0) and np.all(sel <= t), "range"
    assert np.all(np.diff(sel) > 0), "ascending and unique"
    I = ora["scores"]
    tol = tol_rel * ora["maxabs"]
    o = ora["idx"][:n]
    diff = np.setxor1d(sel, o)
    if len(diff):
        assert np.all(np.abs(I[diff] - ora["kth"]) <= tol), \
            f"swap outside tolerance: {diff[:8]} {(I[diff] - ora['kth'])[:8]} tol {tol}"
    if gsc is not None:
        gs = np.asarray(gsc)
        assert np.all(np.abs(gs[:n] - I[sel]) <= tol), "reported scores"
        assert np.all(np.isneginf(gs[n:]))
    return len(diff)


def exact_topk_of(scores: np.ndarray, K: int) -> np.ndarray:
    """Reference selection of a score row by (score desc, position asc),
    used to check the kernel's selection against the kernel's own scores."""
    s = np.asarray(scores, dtype=np.float64)
    finite = np.flatnonzero(np.isfinite(s))
    order = finite[np.lexsort((finite, -s[finite]))]
    return np.sort(order[:K])
