"""Pins of the oracle's MXFP8 and FP8-KV quantisers: hand-worked examples,
the scale rule's defining inequalities, half-step error bounds, power-of-two
invariance, and the record / page layouts."""
import os

import numpy as np
import pytest

from oracle import formats, pools, quant
from sparse_attention_decode_topk_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _golden(kind):
    """Data lines of tests/golden/quant_examples.txt: name -> {key: int}."""
    out = {}
    with open(os.path.join(GOLDEN, "quant_examples.txt")) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#") or parts[0] != kind:
                continue
            out[parts[1]] = {k: int(v, 0) for k, v in (p.split("=") for p in parts[2:])}
    return out


# the input group / tile each golden line describes (its comment block)
def _mx_input(name):
    g = np.ones(32, dtype=np.float32)
    if name == "ones_with_3_at_5":
        g[5] = 3.0
    elif name == "zeros":
        g[:] = 0.0
    elif name == "all_448":
        g[:] = 448.0
    elif name == "all_0.875":
        g[:] = 0.875
    else:
        raise KeyError(name)
    return g


def _kv_input(name):
    t = np.full(576, 0.25, dtype=np.float32)
    if name == "half_with_minus7_at_9":
        t[:128] = 0.5
        t[9] = -7.0
    elif name == "zeros":
        t[:] = 0.0
    else:
        raise KeyError(name)
    return t


def test_mx_golden_examples():
    gold = _golden("mx_group")
    assert set(gold) == {"ones_with_3_at_5", "zeros", "all_448", "all_0.875"}
    for name, exp in gold.items():
        codes, e8 = quant.mxfp8_quant(bf16(_mx_input(name))[None])
        assert e8[0, 0] == exp["e8m0"], name
        if name == "ones_with_3_at_5":
            assert codes[0, 5] == exp["code_three"]
            assert np.all(np.delete(codes[0], 5) == exp["code_one"])
        else:
            assert np.all(codes == exp["code"]), name


def test_kv_golden_examples():
    gold = _golden("kv_tile")
    assert set(gold) == {"half_with_minus7_at_9", "zeros"}
    for name, exp in gold.items():
        rec = quant.kv_quant(bf16(_kv_input(name))[None])[0]
        scale_bits = int(np.frombuffer(rec[512:516].tobytes(), dtype="<u4")[0])
        assert scale_bits == exp["scale_bits"], name
        if name == "half_with_minus7_at_9":
            assert rec[9] == exp["code_m7"]
            assert np.all(np.delete(rec[:128], 9) == exp["code_half"])
        else:
            assert np.all(rec[:512] == exp["code"])


def _random_bf16(rng, shape, spread=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if spread:   # per-row magnitudes spanning many binades
        x *= np.float32(2.0) ** rng.integers(-30, 30, size=shape[:-1] + (1,)).astype(np.float32)
    return bf16(x)


def test_mx_scale_rule_and_error_bound():
    rng = np.random.default_rng(1)
    xb = _random_bf16(rng, (2000, 128))
    codes, e8 = quant.mxfp8_quant(xb)
    x = formats.bf16_decode(xb).reshape(2000, 4, 32)
    amax = np.abs(x).max(axis=2)
    e = e8.astype(np.int64) - 127
    X = np.ldexp(1.0, e)
    # defining inequalities of the scale: in range, and minimal
    assert np.all(amax <= 448 * X)
    assert np.all(amax > 448 * X / 2)
    # no saturation, and every element within half an E4M3 step
    y = x / X[:, :, None]
    deq = quant.mxfp8_dequant(codes, e8).reshape(2000, 4, 32)
    assert np.all(np.abs(deq - x) <= formats.e4m3_half_ulp(np.abs(y)) * X[:, :, None])


def test_mx_power_of_two_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 128)).astype(np.float32)
    xb = bf16(x)
    c0, e0 = quant.mxfp8_quant(xb)
    for k in (-5, 2, 9):
        ck, ek = quant.mxfp8_quant(bf16(x * np.float32(2.0 ** k)))
        assert np.array_equal(ck, c0)
        assert np.array_equal(ek.astype(int), e0.astype(int) + k)


def test_mx_clamp_low():
    # amax below 448 * 2^-127: e clamps at -127 (E8M0 0), elements still in range
    tiny = np.full((1, 32), 2.0 ** -130, dtype=np.float32)
    codes, e8 = quant.mxfp8_quant(bf16(tiny))
    assert e8[0, 0] == 0
    assert np.all(formats.e4m3_decode(codes) * 2.0 ** -127 == 2.0 ** -130)


def test_kv_error_bound_and_saturation_free_max():
    rng = np.random.default_rng(4)
    kvb = _random_bf16(rng, (3000, 576))
    rec = quant.kv_quant(kvb)
    lat, rope = quant.kv_dequant(rec)
    x = formats.bf16_decode(kvb[:, :512]).reshape(3000, 4, 128)
    s = quant.kv_record_scales(rec).astype(np.float64)
    # the scale is the IEEE float32 quotient amax / 448
    amax = np.abs(x).max(axis=2).astype(np.float32)
    assert np.array_equal(quant.kv_record_scales(rec), (amax / np.float32(448)).astype(np.float32))
    # element error: half an E4M3 step at x/s (times s) plus the f32 division
    y = np.abs(x) / s[:, :, None]
    bound = formats.e4m3_half_ulp(np.minimum(y, 448)) * s[:, :, None] + np.abs(x) * 2.0 ** -22
    assert np.all(np.abs(lat.reshape(3000, 4, 128) - x) <= bound)
    # the element holding amax encodes as +-448
    codes = rec[:, :512].reshape(3000, 4, 128)
    am = np.abs(x).argmax(axis=2)
    top = np.take_along_axis(codes, am[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    # rope copied bit-exactly
    assert np.array_equal(rope, formats.bf16_decode(kvb[:, 512:]))


def test_kv_power_of_two_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((400, 576)).astype(np.float32)
    r0 = quant.kv_quant(bf16(x))
    for k in (-7, 3):
        xk = x.copy(); xk[:, :512] *= np.float32(2.0 ** k)
        rk = quant.kv_quant(bf16(xk))
        assert np.array_equal(rk[:, :512], r0[:, :512])
        assert np.array_equal(quant.kv_record_scales(rk),
                              quant.kv_record_scales(r0) * np.float32(2.0 ** k))


def test_record_and_page_sizes():
    assert quant.RECORD_BYTES == 656 and pools.K_PAGE_BYTES == 8448
    assert (64 * 656) % 256 == 0 and 8448 % 256 == 0
    # closed-form memory claims of the page-3 quantisation sections:
    # index data 132 B/token vs 256 B bf16 (-48.4%), KV 656 vs 1152 B (-43.1%)
    assert round(1 - 132 / 256, 3) == 0.484 and round(1 - 656 / 1152, 3) == 0.431


def test_k_pool_roundtrip_permuted():
    rng = np.random.default_rng(6)
    cfg = synth.Config(99, "t", batch=3, h_index=4, h_attn=8, topk=16, ragged=(70, 200))
    lens = np.array([70, 200, 129], dtype=np.int32)
    bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
    kb = _random_bf16(rng, (int(lens.sum()), 128), spread=False)
    codes, e8 = quant.mxfp8_quant(kb)
    pool = pools.k_pool_write(codes, e8, slots, npages)
    for b in range(3):
        c, e = pools.k_pool_read(pool, bt[b], int(lens[b]))
        st = int(starts[b])
        assert np.array_equal(c, codes[st:st + lens[b]]) and np.array_equal(e, e8[st:st + lens[b]])
    # byte placement: token 65 of sequence 1 -> page bt[1][1], offset 1
    # (tile 0, token 1): code pieces at 16 + 256q and 1040 + 256q, scale
    # bytes at 8193 + 16b
    p = bt[1][1]
    st = int(starts[1])
    for q in range(4):
        assert np.array_equal(pool[p, 16 + 256 * q:32 + 256 * q], codes[st + 65][16 * q:16 * q + 16])
        assert np.array_equal(pool[p, 1040 + 256 * q:1056 + 256 * q], codes[st + 65][64 + 16 * q:80 + 16 * q])
    assert np.array_equal(pool[p, [8193, 8209, 8225, 8241]], e8[st + 65])


def test_kv_pool_roundtrip_and_skip():
    rng = np.random.default_rng(8)
    kvb = _random_bf16(rng, (130, 576), spread=False)
    rec = quant.kv_quant(kvb)
    slots = rng.permutation(3 * 64)[:130].astype(np.int64)
    slots[7] = -1
    pool = pools.kv_pool_write(rec, slots, 3)
    assert np.array_equal(pool[slots[8]], rec[8])
    assert not np.any(pool[np.setdiff1d(np.arange(192), slots)])
