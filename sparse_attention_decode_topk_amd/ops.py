"""Thin Python binding of the C ABI in include/dsa.h.

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libdsa_mi355x.so.  Tensors are torch tensors on the current HIP
device; the current torch stream is passed to every call.  If the native
library is missing the first call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_mi355x.so")

DSA_OK = 0
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
          3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}
PAGE = 64
K_PAGE_BYTES = 8448
KV_RECORD_BYTES = 656
KV_PAGE_BYTES = 64 * 656
DEFAULT_SCALE = 1.0 / math.sqrt(576.0)

_lib = None

_c = ctypes
_P = _c.c_void_p
_I32 = _c.c_int32
_I64 = _c.c_int64
_SZ = _c.c_size_t
_F = _c.c_float

SIGNATURES = {
    "dsa_status_str": (_c.c_char_p, [_c.c_int]),
    "dsa_version": (_c.c_int, []),
    "mxfp8_quant": (_c.c_int, [_P, _I64, _I32, _P, _P, _P, _P, _I64, _P]),
    "kv_fp8_quant_paged_write": (_c.c_int, [_P, _I64, _P, _P, _I64, _P]),
    "dsa_decode_prolog": (_c.c_int, [_P, _I64, _I32, _P, _P, _P, _P, _I64, _P, _P, _P, _I64, _P]),
    "dsa_indexer_topk_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "dsa_indexer_topk": (_c.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32,
                                    _P, _P, _P, _SZ, _P]),
    "dsa_indexer_topk_noalloc": (_c.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32,
                                            _I32, _P, _P, _P]),
    "dsa_decode_indexer_topk": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _P,
                                           _I32, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "dsa_indexer_topk_seq_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "dsa_indexer_topk_seq": (_c.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32,
                                        _P, _P, _P, _SZ, _P]),
    "dsa_indexer_topk_mq": (_c.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32,
                                       _I32, _P, _P, _P, _SZ, _P]),
    "dsa_indexer_scores": (_c.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32,
                                      _P, _I64, _P]),
    "dsa_sparse_attn_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "dsa_sparse_attn": (_c.c_int, [_P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _F,
                                   _P, _P, _P, _SZ, _P]),
    "dsa_probe_stream_read": (_c.c_int, [_P, _SZ, _P, _I32, _P]),
}


class DSAError(RuntimeError):
    pass


def lib():
    """The loaded native library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DSAError(f"native library not built: {LIB_PATH} (run __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str):
    if status != DSA_OK:
        raise DSAError(f"{what}: {STATUS.get(status, status)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous tensor")


# ---------------------------------------------------------------- quantisers

def mxfp8_quant(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [..., cols] -> (E4M3 codes uint8 [..., cols], E8M0 uint8 [..., cols/32])."""
    _need(x, torch.bfloat16, "x")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quant(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), None, None, 0,
                             _stream()), "mxfp8_quant")
    return codes, scales


def mxfp8_quant_paged(x: torch.Tensor, slot_mapping: torch.Tensor, k_pool: torch.Tensor):
    """bf16 [n, 128] indexer keys -> written into k_pool (uint8 [pages, 8448])."""
    _need(x, torch.bfloat16, "x"); _need(slot_mapping, torch.int64, "slot_mapping")
    _need(k_pool, torch.uint8, "k_pool")
    _check(lib().mxfp8_quant(_ptr(x), x.shape[0], x.shape[1], None, None, _ptr(k_pool),
                             _ptr(slot_mapping), k_pool.shape[0], _stream()), "mxfp8_quant")


def kv_fp8_quant_paged_write(kv: torch.Tensor, slot_mapping: torch.Tensor, kv_pool: torch.Tensor):
    """bf16 [n, 576] -> 656-byte records in kv_pool (uint8 [pages, 41984])."""
    _need(kv, torch.bfloat16, "kv"); _need(slot_mapping, torch.int64, "slot_mapping")
    _need(kv_pool, torch.uint8, "kv_pool")
    _check(lib().kv_fp8_quant_paged_write(_ptr(kv), kv.shape[0], _ptr(slot_mapping), _ptr(kv_pool),
                                          kv_pool.shape[0], _stream()), "kv_fp8_quant_paged_write")


def decode_prolog(q: torch.Tensor, k_new: torch.Tensor, kv_new: torch.Tensor,
                  slot_mapping: torch.Tensor, k_pool: torch.Tensor, kv_pool: torch.Tensor,
                  q_out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """One launch: mxfp8_quant(q) -> (codes, scales), the new indexer keys into
    k_pool and the new KV rows into kv_pool (pools share page ids)."""
    _need(q, torch.bfloat16, "q"); _need(k_new, torch.bfloat16, "k_new")
    _need(kv_new, torch.bfloat16, "kv_new"); _need(slot_mapping, torch.int64, "slot_mapping")
    _need(k_pool, torch.uint8, "k_pool"); _need(kv_pool, torch.uint8, "kv_pool")
    if k_pool.shape[0] != kv_pool.shape[0]:
        raise ValueError("k_pool and kv_pool must have the same number of pages")
    cols = q.shape[-1]
    rows = q.numel() // cols if cols else 0
    if q_out is None:
        q_out = (torch.empty(q.shape, dtype=torch.uint8, device=q.device),
                 torch.empty(q.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=q.device))
    codes, scales = q_out
    _check(lib().dsa_decode_prolog(_ptr(q), rows, cols, _ptr(codes), _ptr(scales), _ptr(k_new),
                                   _ptr(kv_new), k_new.shape[0], _ptr(slot_mapping), _ptr(k_pool),
                                   _ptr(kv_pool), k_pool.shape[0], _stream()), "dsa_decode_prolog")
    return codes, scales


# ------------------------------------------------------------------- indexer

def indexer_workspace(R: int, bt_stride: int, H_I: int, topk: int, device=None) -> torch.Tensor:
    n = lib().dsa_indexer_topk_workspace_size(R, bt_stride, H_I, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def dsa_indexer_topk(q_fp8, q_e8m0, w, k_pool, block_table, row_seq, row_pos, topk: int,
                     out_idx=None, out_score=None, workspace=None, with_scores: bool = True):
    """Top-K positions per query row (ascending, -1 padded) and their scores."""
    R, H = q_fp8.shape[0], q_fp8.shape[1]
    for t, dt, n in ((q_fp8, torch.uint8, "q_fp8"), (q_e8m0, torch.uint8, "q_e8m0"),
                     (w, torch.float32, "w"), (k_pool, torch.uint8, "k_pool"),
                     (block_table, torch.int32, "block_table"), (row_seq, torch.int32, "row_seq"),
                     (row_pos, torch.int32, "row_pos")):
        _need(t, dt, n)
    dev = q_fp8.device
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=dev)
    if out_score is None and with_scores:
        out_score = torch.empty((R, topk), dtype=torch.float32, device=dev)
    bt_stride = block_table.shape[1]
    if workspace is None:
        workspace = indexer_workspace(R, bt_stride, H, topk, dev)
    _check(lib().dsa_indexer_topk(_ptr(q_fp8), _ptr(q_e8m0), _ptr(w), _ptr(k_pool), k_pool.shape[0],
                                  _ptr(block_table), bt_stride, _ptr(row_seq), _ptr(row_pos), R, H,
                                  topk, _ptr(out_idx), _ptr(out_score), _ptr(workspace),
                                  workspace.numel(), _stream()), "dsa_indexer_topk")
    return out_idx, out_score


def dsa_indexer_topk_noalloc(q_fp8, q_e8m0, w, k_pool, block_table, row_seq, row_pos, topk: int,
                             out_idx=None, out_score=None, with_scores: bool = True):
    """dsa_indexer_topk on the library's own per-GPU scratch array (no
    workspace; calls on one GPU must not overlap)."""
    R, H = q_fp8.shape[0], q_fp8.shape[1]
    for t, dt, n in ((q_fp8, torch.uint8, "q_fp8"), (q_e8m0, torch.uint8, "q_e8m0"),
                     (w, torch.float32, "w"), (k_pool, torch.uint8, "k_pool"),
                     (block_table, torch.int32, "block_table"), (row_seq, torch.int32, "row_seq"),
                     (row_pos, torch.int32, "row_pos")):
        _need(t, dt, n)
    dev = q_fp8.device
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=dev)
    if out_score is None and with_scores:
        out_score = torch.empty((R, topk), dtype=torch.float32, device=dev)
    _check(lib().dsa_indexer_topk_noalloc(_ptr(q_fp8), _ptr(q_e8m0), _ptr(w), _ptr(k_pool),
                                          k_pool.shape[0], _ptr(block_table), block_table.shape[1],
                                          _ptr(row_seq), _ptr(row_pos), R, H, topk, _ptr(out_idx),
                                          _ptr(out_score), _stream()), "dsa_indexer_topk_noalloc")
    return out_idx, out_score


def dsa_decode_indexer_topk(q_bf16, w, k_new, kv_new, slot_mapping, k_pool, kv_pool, block_table,
                            row_seq, row_pos, topk: int, out_idx=None, out_score=None,
                            workspace=None, with_scores: bool = True):
    """The decode prolog (q quantisation, new key / KV record writes) and
    dsa_indexer_topk in the indexer's launches; q_bf16 [R, H_I, 128],
    k_new [R, 128], kv_new [R, 576] bf16, slot_mapping int64 [R]."""
    R, H = q_bf16.shape[0], q_bf16.shape[1]
    for t, dt, n in ((q_bf16, torch.bfloat16, "q_bf16"), (w, torch.float32, "w"),
                     (k_new, torch.bfloat16, "k_new"), (kv_new, torch.bfloat16, "kv_new"),
                     (slot_mapping, torch.int64, "slot_mapping"), (k_pool, torch.uint8, "k_pool"),
                     (kv_pool, torch.uint8, "kv_pool"), (block_table, torch.int32, "block_table"),
                     (row_seq, torch.int32, "row_seq"), (row_pos, torch.int32, "row_pos")):
        _need(t, dt, n)
    if k_pool.shape[0] != kv_pool.shape[0]:
        raise ValueError("k_pool and kv_pool must have the same number of pages")
    dev = q_bf16.device
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=dev)
    if out_score is None and with_scores:
        out_score = torch.empty((R, topk), dtype=torch.float32, device=dev)
    bt_stride = block_table.shape[1]
    if workspace is None:
        workspace = indexer_workspace(R, bt_stride, H, topk, dev)
    _check(lib().dsa_decode_indexer_topk(_ptr(q_bf16), _ptr(w), _ptr(k_new), _ptr(kv_new),
                                         _ptr(slot_mapping), _ptr(k_pool), _ptr(kv_pool),
                                         k_pool.shape[0], _ptr(block_table), bt_stride,
                                         _ptr(row_seq), _ptr(row_pos), R, H, topk, _ptr(out_idx),
                                         _ptr(out_score), _ptr(workspace), workspace.numel(),
                                         _stream()), "dsa_decode_indexer_topk")
    return out_idx, out_score


def indexer_seq_workspace(R: int, n_pages: int, H_I: int, topk: int, device=None) -> torch.Tensor:
    n = lib().dsa_indexer_topk_seq_workspace_size(R, n_pages, H_I, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def dsa_indexer_topk_seq(q_fp8, q_e8m0, w, k_pool, block_table_row, row_pos, topk: int,
                         out_idx=None, out_score=None, workspace=None, with_scores: bool = True):
    """Top-K for query rows that all belong to one sequence (block_table_row:
    int32 [n_pages]); same results as dsa_indexer_topk, K read once per tile
    of rows."""
    R, H = q_fp8.shape[0], q_fp8.shape[1]
    for t, dt, n in ((q_fp8, torch.uint8, "q_fp8"), (q_e8m0, torch.uint8, "q_e8m0"),
                     (w, torch.float32, "w"), (k_pool, torch.uint8, "k_pool"),
                     (block_table_row, torch.int32, "block_table_row"), (row_pos, torch.int32, "row_pos")):
        _need(t, dt, n)
    dev = q_fp8.device
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=dev)
    if out_score is None and with_scores:
        out_score = torch.empty((R, topk), dtype=torch.float32, device=dev)
    n_pages = block_table_row.numel()
    if workspace is None:
        workspace = indexer_seq_workspace(R, n_pages, H, topk, dev)
    _check(lib().dsa_indexer_topk_seq(_ptr(q_fp8), _ptr(q_e8m0), _ptr(w), _ptr(k_pool), k_pool.shape[0],
                                      _ptr(block_table_row), n_pages, _ptr(row_pos), R, H, topk,
                                      _ptr(out_idx), _ptr(out_score), _ptr(workspace),
                                      workspace.numel(), _stream()), "dsa_indexer_topk_seq")
    return out_idx, out_score


def dsa_indexer_topk_mq(q_fp8, q_e8m0, w, k_pool, block_table, row_seq, row_pos, q_per_seq: int,
                        topk: int, out_idx=None, out_score=None, workspace=None,
                        with_scores: bool = True):
    """Multi-query decode: rows come in groups of q_per_seq consecutive rows of
    one sequence whose K pages are read once per group; same results as
    dsa_indexer_topk."""
    R, H = q_fp8.shape[0], q_fp8.shape[1]
    for t, dt, n in ((q_fp8, torch.uint8, "q_fp8"), (q_e8m0, torch.uint8, "q_e8m0"),
                     (w, torch.float32, "w"), (k_pool, torch.uint8, "k_pool"),
                     (block_table, torch.int32, "block_table"), (row_seq, torch.int32, "row_seq"),
                     (row_pos, torch.int32, "row_pos")):
        _need(t, dt, n)
    dev = q_fp8.device
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=dev)
    if out_score is None and with_scores:
        out_score = torch.empty((R, topk), dtype=torch.float32, device=dev)
    bt_stride = block_table.shape[1]
    if workspace is None:
        workspace = indexer_workspace(R, bt_stride, H, topk, dev)
    _check(lib().dsa_indexer_topk_mq(_ptr(q_fp8), _ptr(q_e8m0), _ptr(w), _ptr(k_pool), k_pool.shape[0],
                                     _ptr(block_table), bt_stride, _ptr(row_seq), _ptr(row_pos), R,
                                     q_per_seq, H, topk, _ptr(out_idx), _ptr(out_score),
                                     _ptr(workspace), workspace.numel(), _stream()),
           "dsa_indexer_topk_mq")
    return out_idx, out_score


def dsa_indexer_scores(q_fp8, q_e8m0, w, k_pool, block_table, row_seq, row_pos, ld: int):
    """TEST ONLY: full score rows [R, ld] (-inf beyond each row's t)."""
    R, H = q_fp8.shape[0], q_fp8.shape[1]
    out = torch.empty((R, ld), dtype=torch.float32, device=q_fp8.device)
    _check(lib().dsa_indexer_scores(_ptr(q_fp8), _ptr(q_e8m0), _ptr(w), _ptr(k_pool), k_pool.shape[0],
                                    _ptr(block_table), block_table.shape[1], _ptr(row_seq),
                                    _ptr(row_pos), R, H, _ptr(out), ld, _stream()),
           "dsa_indexer_scores")
    return out


# ---------------------------------------------------------- sparse attention

def sparse_attn_workspace(R: int, H: int, topk: int, device=None) -> torch.Tensor:
    n = lib().dsa_sparse_attn_workspace_size(R, H, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def dsa_sparse_attn(q, kv_pool, block_table, row_seq, idx, softmax_scale: float = DEFAULT_SCALE,
                    out=None, lse=None, workspace=None, with_lse: bool = True):
    """out [R, H, 512] fp32 and lse [R, H] over the listed positions."""
    _need(q, torch.bfloat16, "q"); _need(kv_pool, torch.uint8, "kv_pool")
    _need(block_table, torch.int32, "block_table"); _need(row_seq, torch.int32, "row_seq")
    _need(idx, torch.int32, "idx")
    R, H = q.shape[0], q.shape[1]
    topk = idx.shape[1]
    if out is None:
        out = torch.empty((R, H, 512), dtype=torch.float32, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((R, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = sparse_attn_workspace(R, H, topk, q.device)
    _check(lib().dsa_sparse_attn(_ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(block_table),
                                 block_table.shape[1], _ptr(row_seq), _ptr(idx), R, H, topk,
                                 float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel(), _stream()), "dsa_sparse_attn")
    return out, lse


# ------------------------------------------------------------- measurement

def probe_stream_read(src: torch.Tensor, out: torch.Tensor, grid: int):
    """Streaming read of every byte of `src` (device, contiguous, size a
    multiple of 16); one folded word per work-group into out (int32 [grid])."""
    if not src.is_cuda or not src.is_contiguous():
        raise TypeError("src: expected a contiguous device tensor")
    _need(out, torch.int32, "out")
    if out.numel() < grid:
        raise ValueError("out needs one word per work-group")
    nbytes = src.numel() * src.element_size()
    _check(lib().dsa_probe_stream_read(_ptr(src), nbytes, _ptr(out), grid, _stream()),
           "dsa_probe_stream_read")
