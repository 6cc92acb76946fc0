"""GPU parity of the quantisers: bitwise equal to the oracle's codes, scales,
K pages and KV records."""
import numpy as np
import pytest
import torch

from oracle import pools, quant
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import bf16_tensor, say

pytestmark = pytest.mark.gpu


def _spread_bf16(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-40, 40, size=shape[:-1] + (1,)).astype(np.float32)
    # special groups: zeros, +-448 boundaries, tiny values, exact ties
    x[0] = 0.0
    if shape[0] > 4:
        x[1] = 448.0; x[2, ::2] = -448.0; x[3] = 2.0 ** -130
        x[4] = np.float32(1.0625)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 128), (300, 64 * 128 // 64), (1024, 128), (33, 576)])
def test_mxfp8_contiguous_bitwise(need_gpu, rows, cols):
    say(f"[mxfp8 contiguous] rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    xb = _spread_bf16(rng, (rows, cols))
    codes, scales = ops.mxfp8_quant(bf16_tensor(xb, "cuda"))
    c_ref, s_ref = quant.mxfp8_quant(xb)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles"])
def test_mxfp8_queries_of_configs(need_gpu, cfg):
    say(f"[mxfp8 q] {cfg}")
    inp = synth.make(cfg, with_sfa=False)
    codes, scales = ops.mxfp8_quant(bf16_tensor(inp["q_idx"], "cuda"))
    R, H = inp["q_idx"].shape[:2]
    c_ref, s_ref = quant.mxfp8_quant(inp["q_idx"].reshape(R * H, 128))
    assert np.array_equal(codes.cpu().numpy().reshape(R * H, 128), c_ref)
    assert np.array_equal(scales.cpu().numpy().reshape(R * H, 4), s_ref)


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles"])
def test_paged_k_pool_bitwise(need_gpu, cfg):
    say(f"[k pool] {cfg}")
    inp = synth.make(cfg, with_sfa=False)
    npages = int(inp["total_pages"])
    pool = torch.zeros((npages, ops.K_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    slots = inp["slot_mapping"].copy()
    # a few rows are skipped: negative and out-of-pool slots
    slots[3] = -1
    slots[5] = npages * 64 + 10
    ops.mxfp8_quant_paged(bf16_tensor(inp["k_idx"], "cuda"), torch.from_numpy(slots).cuda(), pool)
    codes, e8 = quant.mxfp8_quant(inp["k_idx"])
    ref = pools.k_pool_write(codes, e8, np.where(slots >= npages * 64, -1, slots), npages)
    assert np.array_equal(pool.cpu().numpy(), ref)


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles"])
def test_kv_pool_bitwise(need_gpu, cfg):
    say(f"[kv pool] {cfg}")
    inp = synth.make(cfg, with_index=False)
    npages = int(inp["total_pages"])
    pool = torch.zeros((npages, ops.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    slots = inp["slot_mapping"].copy()
    slots[0] = -5
    ops.kv_fp8_quant_paged_write(bf16_tensor(inp["kv"], "cuda"), torch.from_numpy(slots).cuda(), pool)
    ref = pools.kv_pool_write(quant.kv_quant(inp["kv"]), slots, npages)
    got = pool.cpu().numpy().reshape(npages * 64, 656)
    assert np.array_equal(got, ref)


def test_kv_records_wide_range(need_gpu):
    say("[kv records] wide-range values")
    rng = np.random.default_rng(5)
    kvb = _spread_bf16(rng, (512, 576))
    pool = torch.zeros((8, ops.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    slots = np.arange(512, dtype=np.int64)
    ops.kv_fp8_quant_paged_write(bf16_tensor(kvb, "cuda"), torch.from_numpy(slots).cuda(), pool)
    got = pool.cpu().numpy().reshape(512, 656)
    assert np.array_equal(got, quant.kv_quant(kvb))


@pytest.mark.parametrize("cfg", ["decode_128k_b8"])
def test_big_pools_sampled(need_gpu, cfg):
    """Full-size cache build; sampled tokens compared bitwise."""
    say(f"[big pools] {cfg}")
    inp = synth.make(cfg)
    npages = int(inp["total_pages"])
    slots = torch.from_numpy(inp["slot_mapping"]).cuda()
    kpool = torch.zeros((npages, ops.K_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    kvpool = torch.zeros((npages, ops.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    ops.mxfp8_quant_paged(bf16_tensor(inp["k_idx"], "cuda"), slots, kpool)
    ops.kv_fp8_quant_paged_write(bf16_tensor(inp["kv"], "cuda"), slots, kvpool)
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(len(inp["slot_mapping"]), 4096, replace=False))
    sl = inp["slot_mapping"][tok]
    codes, e8 = quant.mxfp8_quant(inp["k_idx"][tok])
    kp = kpool.cpu().numpy()
    for i, s in enumerate(sl):
        p, o = divmod(int(s), 64)
        assert np.array_equal(kp[p, pools.K_CODE_OFF[o]], codes[i])
        assert np.array_equal(kp[p, pools.K_SCALE_OFF[o]], e8[i])
    rec = quant.kv_quant(inp["kv"][tok])
    kvp = kvpool.view(npages * 64, 656)[torch.from_numpy(sl).cuda()].cpu().numpy()
    assert np.array_equal(kvp, rec)


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles"])
def test_decode_prolog_bitwise(need_gpu, cfg):
    """The one-launch prolog: indexer q codes/scales, K pages and KV records
    bitwise equal to the oracle's (same skipped-slot rules)."""
    say(f"[decode prolog] {cfg}")
    inp = synth.make(cfg)
    npages = int(inp["total_pages"])
    R, H = inp["q_idx"].shape[:2]
    slots = inp["slot_mapping"].copy()
    slots[1] = -1
    slots[2] = npages * 64 + 3
    kpool = torch.zeros((npages, ops.K_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    kvpool = torch.zeros((npages, ops.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    codes, scales = ops.decode_prolog(bf16_tensor(inp["q_idx"], "cuda"), bf16_tensor(inp["k_idx"], "cuda"),
                                      bf16_tensor(inp["kv"], "cuda"), torch.from_numpy(slots).cuda(),
                                      kpool, kvpool)
    c_ref, s_ref = quant.mxfp8_quant(inp["q_idx"].reshape(R * H, 128))
    assert np.array_equal(codes.cpu().numpy().reshape(R * H, 128), c_ref)
    assert np.array_equal(scales.cpu().numpy().reshape(R * H, 4), s_ref)
    skip = np.where(slots >= npages * 64, -1, slots)
    kc, ke = quant.mxfp8_quant(inp["k_idx"])
    assert np.array_equal(kpool.cpu().numpy(), pools.k_pool_write(kc, ke, skip, npages))
    kv_ref = pools.kv_pool_write(quant.kv_quant(inp["kv"]), skip, npages)
    assert np.array_equal(kvpool.cpu().numpy().reshape(npages * 64, 656), kv_ref)


def test_decode_prolog_no_new_tokens(need_gpu):
    say("[decode prolog] queries only")
    rng = np.random.default_rng(3)
    xb = _spread_bf16(rng, (8, 64 * 128))
    kpool = torch.zeros((1, ops.K_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    kvpool = torch.zeros((1, ops.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    empty = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    codes, scales = ops.decode_prolog(bf16_tensor(xb, "cuda"), empty,
                                      torch.zeros((0, 576), dtype=torch.bfloat16, device="cuda"),
                                      torch.zeros((0,), dtype=torch.int64, device="cuda"), kpool, kvpool)
    c_ref, s_ref = quant.mxfp8_quant(xb)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert int(kpool.sum()) == 0 and int(kvpool.sum()) == 0


def test_mxfp8_every_in_range_bf16_value(need_gpu):
    """Every finite bf16 value v with |v| <= 448 is quantised in a group whose
    scale is 2^0 (each group of 32 holds 448 in its first element), so its
    E4M3 code is the code of v itself: all of them against the oracle's
    encoder.  This covers the whole input domain of the element conversion
    of MXFP8 (a bf16 value times a power of two is a bf16 value, and the
    scale rule keeps it within 448)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    dom = bits[keep]
    per = 31
    n_groups = (len(dom) + per - 1) // per
    grid = np.zeros((n_groups, 32), dtype=np.uint16)
    grid[:, 0] = synth.f32_to_bf16_bits(np.array([448.0], dtype=np.float32))[0]
    flat = np.zeros(n_groups * per, dtype=np.uint16)
    flat[:len(dom)] = dom
    grid[:, 1:] = flat.reshape(n_groups, per)
    x = grid.reshape(-1, 128) if (n_groups % 4 == 0) else np.concatenate(
        [grid, np.zeros((4 - n_groups % 4, 32), dtype=np.uint16)]).reshape(-1, 128)
    codes, e8 = ops.mxfp8_quant(bf16_tensor(x, "cuda"))
    torch.cuda.synchronize()
    ref_c, ref_e = quant.mxfp8_quant(x)
    assert np.array_equal(e8.cpu().numpy(), ref_e)
    assert np.all(ref_e.reshape(-1)[:n_groups] == 127)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    say(f"[quant] {len(dom)} in-range bf16 values: codes equal to the oracle's")
