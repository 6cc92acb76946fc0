"""Quantisers of the two caches, written from their definitions.

Test infrastructure only (see package docstring).

MXFP8 (indexer q and k): "Deep Dive into Sparse Attention ..." (page 1),
section 2.2 "Memory Optimization", and "Kimi K3.1 Pro Inference Acceleration"
(page 3), section "Full MXFP8 Quantization with Per-Group Dynamic Scaling for
LI": every 32 consecutive elements share one dynamic scale.  Reading taken for
the scale (the pages do not give the rule): X = 2^e with e the smallest
integer such that amax <= 448 * 2^e, clamped to [-127, 127]; a group whose
amax is 0 gets e = 0.  This is the smallest power-of-two scale that keeps every
element in range, so no element saturates and every element lies within half
an E4M3 step of its input.  Elements are RNE-satfinite E4M3 of x / X (exact
division by a power of two).

FP8 KV tile (SFA cache): page 1 section 2.2 and page 3 section "FP8 KVCache
with Per-Token-Head-Tile Quantization for SFA": one independent scale per 128
elements of each token.  The scale is fp32(amax) / 448 computed as an IEEE
float32 division (correctly rounded); a tile whose amax is 0 gets scale 1.
Elements are RNE-satfinite E4M3 of the float32 quotient fp32(x / scale).  The
64-wide rope part stays bf16 ("Preserving a Mixed-Precision Path", page 3).

Record layout of one token of the SFA cache (656 bytes):
  [0, 512)   512 E4M3 latent codes
  [512, 528) 4 float32 tile scales, little-endian
  [528, 656) 64 bf16 rope values, little-endian
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, bf16_decode, e4m3_decode, e4m3_encode, e8m0_decode

GROUP = 32
TILE = 128
D_LATENT = 512
D_ROPE = 64
RECORD_BYTES = D_LATENT + 4 * 4 + 2 * D_ROPE     # 656


def mx_scale_exponent(amax) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 if amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # exact corrections of the floating-point estimate
    e = np.where(safe > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(safe <= E4M3_MAX * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.clip(e, -127, 127)
    return np.where(amax > 0, e, 0)


def mxfp8_quant(x_bf16_bits: np.ndarray):
    """bf16 [rows, cols] (cols % 32 == 0) -> (E4M3 codes [rows, cols] uint8,
    E8M0 bytes [rows, cols/32] uint8)."""
    x = bf16_decode(x_bf16_bits)
    rows, cols = x.shape
    assert cols % GROUP == 0
    g = x.reshape(rows, cols // GROUP, GROUP)
    e = mx_scale_exponent(np.abs(g).max(axis=2))
    y = g / np.ldexp(1.0, e)[:, :, None]
    codes = e4m3_encode(y).reshape(rows, cols)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequant(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    rows, cols = codes.shape
    v = e4m3_decode(codes).reshape(rows, cols // GROUP, GROUP)
    return (v * e8m0_decode(e8m0)[:, :, None]).reshape(rows, cols)


def kv_tile_scales(latent_bf16_bits: np.ndarray) -> np.ndarray:
    """float32 [n, 4]: fp32(amax) / 448 per 128-element tile (1 when amax is 0)."""
    x = bf16_decode(latent_bf16_bits).reshape(-1, D_LATENT // TILE, TILE)
    amax = np.abs(x).max(axis=2).astype(np.float32)        # exact: bf16 values
    scale = amax / np.float32(E4M3_MAX)                     # IEEE float32 division
    return np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)


def kv_quant(kv_bf16_bits: np.ndarray) -> np.ndarray:
    """bf16 [n, 576] (latent 512 | rope 64) -> uint8 records [n, 656]."""
    kv_bf16_bits = np.asarray(kv_bf16_bits, dtype=np.uint16)
    n = kv_bf16_bits.shape[0]
    lat_bits = kv_bf16_bits[:, :D_LATENT]
    rope_bits = np.ascontiguousarray(kv_bf16_bits[:, D_LATENT:])
    scale = kv_tile_scales(lat_bits)                                   # [n, 4] f32
    x32 = bf16_decode(lat_bits).astype(np.float32).reshape(n, 4, TILE)  # exact
    y32 = (x32 / scale[:, :, None]).astype(np.float32)                  # IEEE f32 division
    codes = e4m3_encode(y32.astype(np.float64)).reshape(n, D_LATENT)
    rec = np.empty((n, RECORD_BYTES), dtype=np.uint8)
    rec[:, :D_LATENT] = codes
    rec[:, D_LATENT:D_LATENT + 16] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, D_LATENT + 16:] = rope_bits.astype("<u2").view(np.uint8).reshape(n, 2 * D_ROPE)
    return rec


def kv_record_scales(rec: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(rec[:, D_LATENT:D_LATENT + 16]).view("<f4").reshape(-1, 4)


def kv_dequant(rec: np.ndarray):
    """uint8 records [n, 656] -> (latent fp64 [n, 512], rope fp64 [n, 64])."""
    rec = np.asarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    codes = rec[:, :D_LATENT]
    scale = kv_record_scales(rec).astype(np.float64)
    lat = (e4m3_decode(codes).reshape(n, 4, TILE) * scale[:, :, None]).reshape(n, D_LATENT)
    rope_bits = np.ascontiguousarray(rec[:, D_LATENT + 16:]).view("<u2").reshape(n, D_ROPE)
    return lat, bf16_decode(rope_bits)
