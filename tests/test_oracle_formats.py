"""Pins of the oracle's number formats (E4M3, E8M0, bf16) against the OCP
definitions, exhaustive search and torch's float8_e4m3fn cast."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def test_e4m3_table_closed_form():
    t = formats.E4M3_TABLE
    finite = np.isfinite(t)
    assert finite.sum() == 254                       # 256 codes minus 0x7f, 0xff
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # strictly monotone magnitudes
    # negative half mirrors the positive half
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])
    assert math.copysign(1.0, t[0x80]) == -1.0
    # every finite value has at most 4 significant bits
    for v in pos[1:]:
        m, e = math.frexp(v)
        assert (m * 16) == int(m * 16)


def test_e4m3_golden():
    for parts in _golden_lines("e4m3_codes.txt"):
        if parts[0] == "decode":
            code, val = int(parts[1], 16), float(parts[2])
            got = formats.e4m3_decode(np.array([code]))[0]
            if math.isnan(val):
                assert math.isnan(got)
            else:
                assert got == val and math.copysign(1, got) == math.copysign(1, val), parts
        else:
            val, code = float(parts[1]), int(parts[2], 16)
            assert int(formats.e4m3_encode(np.array([val]))[0]) == code, parts
            assert int(formats.e4m3_encode_nearest(np.array([val]))[0]) == code, parts


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    return v[np.isfinite(v)]


def test_e4m3_encode_matches_exhaustive_search():
    vals = _all_bf16_finite()
    # bring bf16 values into and around the E4M3 range at several offsets
    rng = np.random.default_rng(7)
    pieces = [vals[np.abs(vals) < 1e4]]
    for k in (-12, -6, 0, 5):
        pieces.append(vals[(np.abs(vals) > 2.0 ** -20) & (np.abs(vals) < 2.0 ** 12)] * 2.0 ** k)
    # exact midpoints between neighbouring codes (tie cases) and their negatives
    mids = (formats.E4M3_POS[1:] + formats.E4M3_POS[:-1]) / 2
    pieces += [mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)]
    pieces.append(rng.standard_normal(200000) * rng.choice([1e-3, 1, 30, 300], 200000))
    y = np.concatenate(pieces)
    for chunk in np.array_split(y, 40):
        assert np.array_equal(formats.e4m3_encode(chunk), formats.e4m3_encode_nearest(chunk))


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        rng.standard_normal(300000).astype(np.float32) * np.float32(40),
        rng.uniform(-448, 448, 300000).astype(np.float32),
        (rng.standard_normal(100000) * 1e-3).astype(np.float32),
    ])
    y = y[np.abs(y) <= 448]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3_encode(y.astype(np.float64)), ref)


def test_e4m3_roundtrip_and_half_ulp():
    # decode(encode(v)) == v for every finite code; the error of any input in
    # range is at most half a step of its binade
    pos = formats.E4M3_POS
    assert np.array_equal(formats.e4m3_decode(formats.e4m3_encode(pos)), pos)
    rng = np.random.default_rng(3)
    y = rng.uniform(-448, 448, 100000)
    err = np.abs(formats.e4m3_decode(formats.e4m3_encode(y)) - y)
    assert np.all(err <= formats.e4m3_half_ulp(np.abs(y)))


def test_e8m0_and_bf16():
    assert formats.e8m0_decode(np.array([127]))[0] == 1.0
    assert formats.e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert formats.e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert np.isnan(formats.e8m0_decode(np.array([255]))[0])
    # bf16 widening: 0x3f80 = 1.0, 0xc000 = -2.0, 0x0001 = smallest subnormal 2^-133
    got = formats.bf16_decode(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], dtype=np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert got[3] == (2 - 2 ** -7) * 2.0 ** 127
    # agrees with torch's bf16 -> fp64 widening on all patterns
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = formats.bf16_decode(bits)
    both = np.isfinite(ref)
    assert np.array_equal(got[both], ref[both])
