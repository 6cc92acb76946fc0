"""The C-ABI library loads, exports every entry point include/dsa.h declares,
and rejects bad arguments before any device work (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from sparse_attention_decode_topk_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("native library not built; run __graft_entry__.build()")
    return ops.lib()


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("mxfp8_quant", "kv_fp8_quant_paged_write", "dsa_indexer_topk", "dsa_sparse_attn"):
        assert n in names
    assert set(names) == set(ops.SIGNATURES), "binding signatures must cover the header exactly"


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.dsa_status_str(0) == b"DSA_OK"
    assert lib.dsa_status_str(3) == b"DSA_ERR_WORKSPACE"
    assert lib.dsa_status_str(99) == b"DSA_ERR_UNKNOWN"
    assert lib.dsa_version() >= 100


def test_workspace_sizes_are_host_only(lib):
    a = lib.dsa_indexer_topk_workspace_size(8, 2048, 64, 2048)
    b = lib.dsa_indexer_topk_workspace_size(16, 2048, 64, 2048)
    assert 0 < a < b
    # status word + the 1 KB zero record, plus the split partials when the
    # index list is split (8 rows of 128 heads: 8 splits of 256 entries)
    small = lib.dsa_sparse_attn_workspace_size(0, 128, 2048)
    assert small == 256 + 1024
    assert lib.dsa_sparse_attn_workspace_size(8, 128, 2048) >= small + 8 * 128 * 8 * 512 * 4
    # 512 rows of 8 heads need no split: no partials
    assert lib.dsa_sparse_attn_workspace_size(512, 8, 64) == small


def test_chunked_prefill_workspace_is_bounded(lib):
    # the sequence entry point keeps a launch's candidate region (8 bytes
    # per history slot of every row) within 512 MiB by taking fewer rows per
    # launch: 8192 rows of a 2048-page sequence need 512 rows' worth, not
    # 4096 rows' (4 GiB)
    per_row = 2048 * 64 * 8
    big = lib.dsa_indexer_topk_seq_workspace_size(8192, 2048, 64, 2048)
    assert 512 * per_row <= big < 600 * 2**20
    assert lib.dsa_indexer_topk_seq_workspace_size(4096, 2048, 64, 2048) == big
    # short contexts keep up to 4096 rows per launch; a small R needs only its own rows
    short = lib.dsa_indexer_topk_seq_workspace_size(8192, 64, 64, 2048)
    assert short >= 4096 * 64 * 64 * 8
    assert lib.dsa_indexer_topk_seq_workspace_size(16, 2048, 64, 2048) < 17 * per_row
    # the longest sequence (4096 pages) still fits: one tile height of rows at least
    assert lib.dsa_indexer_topk_seq_workspace_size(8192, 4096, 64, 2048) < 600 * 2**20


P = ctypes.c_void_p
FAKE = P(0x1000)   # never dereferenced: every call below fails validation first


def test_quant_argument_errors(lib):
    assert lib.mxfp8_quant(None, 4, 128, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.mxfp8_quant(FAKE, 4, 100, FAKE, FAKE, None, None, 0, None) == 2   # cols % 32
    assert lib.mxfp8_quant(FAKE, 4, 128, None, FAKE, None, None, 0, None) == 1
    assert lib.mxfp8_quant(FAKE, 4, 256, None, None, FAKE, FAKE, 10, None) == 2  # paged needs 128
    assert lib.mxfp8_quant(FAKE, 4, 128, FAKE, None, FAKE, FAKE, 10, None) == 1  # mixed modes
    assert lib.mxfp8_quant(FAKE, 0, 128, FAKE, FAKE, None, None, 0, None) == 0   # empty: no work
    assert lib.kv_fp8_quant_paged_write(None, 4, FAKE, FAKE, 1, None) == 1
    assert lib.kv_fp8_quant_paged_write(FAKE, 4, FAKE, FAKE, 0, None) == 1
    assert lib.kv_fp8_quant_paged_write(FAKE, 0, FAKE, FAKE, 1, None) == 0


def _idx_call(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, kpool=FAKE, pages=100, bt=FAKE, bts=4, rs=FAKE, rp=FAKE,
             R=2, H=64, K=2048, oi=FAKE, osc=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dsa_indexer_topk(a["q"], a["qs"], a["w"], a["kpool"], a["pages"], a["bt"], a["bts"],
                                a["rs"], a["rp"], a["R"], a["H"], a["K"], a["oi"], a["osc"],
                                a["ws"], a["wsb"], None)


def test_indexer_argument_errors(lib):
    assert _idx_call(lib, q=None) == 1
    assert _idx_call(lib, oi=None) == 1
    assert _idx_call(lib, bts=0) == 1
    assert _idx_call(lib, pages=0) == 1
    assert _idx_call(lib, H=65) == 2
    assert _idx_call(lib, H=0) == 2
    assert _idx_call(lib, K=0) == 2
    assert _idx_call(lib, K=2049) == 2
    assert _idx_call(lib, ws=None) == 3
    assert _idx_call(lib, wsb=16) == 3
    assert _idx_call(lib, R=0) == 0
    assert lib.dsa_indexer_scores(FAKE, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, FAKE, 2, 64, None,
                                  100, None) == 1
    assert lib.dsa_indexer_scores(FAKE, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, FAKE, 2, 64, FAKE,
                                  0, None) == 1


def _sfa_call(lib, **kw):
    a = dict(q=FAKE, pool=FAKE, pages=100, bt=FAKE, bts=4, rs=FAKE, idx=FAKE, R=2, H=128, K=2048,
             scale=1 / 24, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dsa_sparse_attn(a["q"], a["pool"], a["pages"], a["bt"], a["bts"], a["rs"], a["idx"],
                               a["R"], a["H"], a["K"], a["scale"], a["out"], a["lse"], a["ws"],
                               a["wsb"], None)


def test_sparse_attn_argument_errors(lib):
    assert _sfa_call(lib, q=None) == 1
    assert _sfa_call(lib, out=None) == 1
    assert _sfa_call(lib, scale=0.0) == 1
    assert _sfa_call(lib, scale=float("nan")) == 1
    assert _sfa_call(lib, H=129) == 2
    assert _sfa_call(lib, K=0) == 2
    assert _sfa_call(lib, ws=None) == 3
    assert _sfa_call(lib, wsb=8) == 3
    assert _sfa_call(lib, R=0) == 0


def _mq_call(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, kpool=FAKE, pages=100, bt=FAKE, bts=4, rs=FAKE, rp=FAKE,
             R=8, qps=4, H=64, K=2048, oi=FAKE, osc=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dsa_indexer_topk_mq(a["q"], a["qs"], a["w"], a["kpool"], a["pages"], a["bt"],
                                   a["bts"], a["rs"], a["rp"], a["R"], a["qps"], a["H"], a["K"],
                                   a["oi"], a["osc"], a["ws"], a["wsb"], None)


def test_multi_query_indexer_argument_errors(lib):
    assert _mq_call(lib, q=None) == 1
    assert _mq_call(lib, rs=None) == 1
    assert _mq_call(lib, oi=None) == 1
    assert _mq_call(lib, qps=0) == 2
    assert _mq_call(lib, qps=9) == 2
    assert _mq_call(lib, R=6) == 1          # not a multiple of q_per_seq
    assert _mq_call(lib, bts=4097) == 2     # tiles hold at most 4096 page ids
    assert _mq_call(lib, H=65) == 2
    assert _mq_call(lib, K=2049) == 2
    assert _mq_call(lib, ws=None) == 3
    assert _mq_call(lib, wsb=16) == 3
    assert _mq_call(lib, R=0) == 0


def _prolog_call(lib, **kw):
    a = dict(q=FAKE, rows=8, cols=128, qf=FAKE, qs=FAKE, k=FAKE, kv=FAKE, n=8, slots=FAKE,
             kpool=FAKE, kvpool=FAKE, pages=100)
    a.update(kw)
    return lib.dsa_decode_prolog(a["q"], a["rows"], a["cols"], a["qf"], a["qs"], a["k"], a["kv"],
                                 a["n"], a["slots"], a["kpool"], a["kvpool"], a["pages"], None)


def test_decode_prolog_argument_errors(lib):
    assert _prolog_call(lib, q=None) == 1
    assert _prolog_call(lib, qf=None) == 1
    assert _prolog_call(lib, qs=None) == 1
    assert _prolog_call(lib, rows=-1) == 1
    assert _prolog_call(lib, cols=0) == 1
    assert _prolog_call(lib, cols=100) == 2      # not a multiple of the 32-element block
    assert _prolog_call(lib, n=-1) == 1
    for name in ("k", "kv", "slots", "kpool", "kvpool"):
        assert _prolog_call(lib, **{name: None}) == 1, name
    assert _prolog_call(lib, pages=0) == 1
    # no new tokens: the cache arguments may be absent
    assert _prolog_call(lib, rows=0, n=0, k=None, kv=None, slots=None, kpool=None, kvpool=None,
                        pages=0) == 0


def test_probe_argument_errors(lib):
    assert lib.dsa_probe_stream_read(None, 1 << 20, FAKE, 256, None) == 1
    assert lib.dsa_probe_stream_read(FAKE, 1 << 20, None, 256, None) == 1
    assert lib.dsa_probe_stream_read(FAKE, 1000, FAKE, 256, None) == 1   # not a multiple of 16
    assert lib.dsa_probe_stream_read(FAKE, 1 << 20, FAKE, 0, None) == 1


def test_concurrent_first_calls_from_host_threads(lib):
    """Many host threads enter the indexer entry points at once, the first
    calls of the process included: the per-device occupancy cache they all
    consult is filled without a lock.  Without a GPU every call gets past
    validation and stops at the device query with DSA_ERR_HIP; every thread
    must see the same status and nothing may crash."""
    import threading
    import torch
    if torch.cuda.is_available():
        pytest.skip("the device query succeeds on a GPU host; covered by the GPU tests")
    results = []
    lock = threading.Lock()

    def worker():
        st = [_idx_call(lib) for _ in range(20)] + [_mq_call(lib) for _ in range(20)]
        with lock:
            results.extend(st)

    threads = [threading.Thread(target=worker) for _ in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert len(results) == 8 * 40 and set(results) == {4}
