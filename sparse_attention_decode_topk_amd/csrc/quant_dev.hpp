// Quantiser device routines shared by the quantisation kernels and the
// indexer launch that folds the decode prolog in: one implementation, so
// both produce the same bytes.
//
// MXFP8: one E8M0 scale per 32 elements ("Full MXFP8 Quantization with
// Per-Group Dynamic Scaling for LI", Kimi K3.1 Pro Day0 page).  KV: one fp32
// scale amax/448 per 128-element tile of each token's latent, rope kept in
// bf16 ("FP8 KVCache with Per-Token-Head-Tile Quantization for SFA" and
// "Preserving a Mixed-Precision Path", same page).
#pragma once

#include "common.hpp"

namespace dsa {

// Four consecutive threads own one 32-element group; each thread converts 8
// elements (one 16-byte load, one 8-byte store).  Thread `first` of
// `nthreads` (multiples of 64) walks the element groups with that stride.
__device__ __forceinline__ void mxfp8_quant_range(
    int64_t first, int64_t nthreads, const uint16_t* __restrict__ x, int64_t rows, int cols,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_scale, uint8_t* __restrict__ kpool,
    const int64_t* __restrict__ slots, int64_t pool_slots) {
  const int64_t per_row = cols / 8;
  const int64_t total = rows * per_row;
  for (int64_t i = first; i < total; i += nthreads) {
    // the slot (paged mode) is loaded together with the data, not after the
    // conversion, so the two loads' latencies overlap
    const int64_t row = i / per_row;
    const int64_t slot = kpool != nullptr ? slots[row] : 0;
    const uint4 raw = *reinterpret_cast<const uint4*>(x + i * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
    // group of 4 consecutive lanes (groups never straddle the loop bound)
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int e = mx_exponent(amax);
    const float inv = pow2f(-e);  // exact: -e in [-120, 127] for bf16 input
    // |v * inv| <= 448 by the scale rule: the hardware conversion applies
    const uint32_t lo = e4m3x4_in_range(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = e4m3x4_in_range(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    const uint8_t sbyte = (uint8_t)(e + 127);
    if (kpool == nullptr) {
      *reinterpret_cast<uint2*>(out + i * 8) = make_uint2(lo, hi);
      if ((i & 3) == 0) out_scale[i >> 2] = sbyte;
    } else {
      const int c8 = (int)(i - row * per_row);  // 0..15
      if (slot < 0 || slot >= pool_slots) continue;
      uint8_t* page = kpool + (slot >> 6) * (int64_t)kKPageBytes;
      const int off = (int)(slot & 63);
      *reinterpret_cast<uint2*>(page + k_code_off(off, c8 * 8)) = make_uint2(lo, hi);
      if ((c8 & 3) == 0) page[k_scale_off(off, c8 >> 2)] = sbyte;
    }
  }
}

// One wave per token: lane j quantises latent elements [8j, 8j+8) (tile
// j/16); lanes 0..7 copy the rope part.  Wave `first` of `nwaves` walks the
// tokens with that stride.
__device__ __forceinline__ void kv_quant_range(
    int64_t first, int64_t waves, const uint16_t* __restrict__ kv, int64_t n,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ pool, int64_t pool_slots) {
  const int lane = threadIdx.x & 63;
  for (int64_t tok = first; tok < n; tok += waves) {
    // the token's data is loaded together with its slot (its address does
    // not depend on the slot), so the two loads' latencies overlap
    const int64_t slot = slots[tok];
    const uint16_t* src = kv + tok * kQK;
    const uint4 raw = *reinterpret_cast<const uint4*>(src + lane * 8);
    const uint4 rope = *reinterpret_cast<const uint4*>(src + kLatent + (lane & 7) * 8);
    if (slot < 0 || slot >= pool_slots) continue;  // uniform across the wave
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float scale = amax == 0.f ? 1.0f : __fdiv_rn(amax, 448.0f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo |= e4m3_rne_sat(__fdiv_rn(v[j], scale)) << (8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi |= e4m3_rne_sat(__fdiv_rn(v[4 + j], scale)) << (8 * j);
    uint8_t* rec = pool + slot * (int64_t)kRec;
    *reinterpret_cast<uint2*>(rec + lane * 8) = make_uint2(lo, hi);
    if ((lane & 15) == 0) *reinterpret_cast<float*>(rec + kRecScaleOff + (lane >> 4) * 4) = scale;
    if (lane < 8) *reinterpret_cast<uint4*>(rec + kRecRopeOff + lane * 16) = rope;
  }
}

}  // namespace dsa
