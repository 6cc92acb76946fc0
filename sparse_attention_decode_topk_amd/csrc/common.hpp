// Device and host helpers shared by the DSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr int kPage = DSA_PAGE_TOKENS;          // tokens per page
constexpr int kIdxDim = DSA_INDEX_DIM;          // indexer head dim
constexpr int kKPageBytes = DSA_K_PAGE_BYTES;   // 64*128 codes + 64*4 scales
constexpr int kKScaleOff = kPage * kIdxDim;     // scale bytes start in a K page
constexpr int kKTileTok = 16;                   // tokens per K-page tile
constexpr int kKTileBytes = kKTileTok * kIdxDim;   // 2048 code bytes per tile

// K page byte of code d (0..127) of the token at page offset o: tile j = o/16
// holds its tokens' codes as [d/64][(d%64)/16][o%16][d%16], so the 16-byte
// chunk that lane n + 16g of a token-tile MFMA operand holds (dims 16g..+15,
// or 64+16g..+15) sits at 16 * lane of a contiguous kilobyte.
__host__ __device__ constexpr int k_code_off(int o, int d) {
  return kKTileBytes * (o / kKTileTok) + 1024 * (d / 64) + 256 * ((d % 64) / 16) +
         16 * (o % kKTileTok) + d % 16;
}
// K page byte of E8M0 scale b (dims 32b..32b+31) of the token at offset o:
// [tile][b][o%16] after the codes.
__host__ __device__ constexpr int k_scale_off(int o, int b) {
  return kKScaleOff + 64 * (o / kKTileTok) + kKTileTok * b + o % kKTileTok;
}
static_assert(k_code_off(63, 127) == kKScaleOff - 1 && k_scale_off(63, 3) == kKPageBytes - 1,
              "the K page layout fills the page");
constexpr int kLatent = DSA_LATENT_DIM;
constexpr int kRope = DSA_ROPE_DIM;
constexpr int kQK = kLatent + kRope;            // 576
constexpr int kRec = DSA_KV_RECORD_BYTES;       // 656
constexpr int kRecScaleOff = kLatent;           // 4 fp32 tile scales
constexpr int kRecRopeOff = kLatent + 16;       // 64 bf16 rope values

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// 2^e as fp32 for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// OCP E4M3 ("FN": max 448, no infinities) encoder: round to nearest, ties to
// even mantissa, saturate to +-448, keep the sign (a negative value that
// rounds to zero gives 0x80).  Integer rounding on the fp32 bit pattern for
// the normal range; the subnormal grid (step 2^-9) via round-half-even rint.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
  uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  uint32_t code;
  if (u >= 0x43E80000u) {              // |y| >= 464 (midpoint 448|480) or non-finite
    code = 0x7Eu;
  } else if (u >= 0x3C800000u) {       // |y| >= 2^-6: normal E4M3
    uint32_t v = u - (120u << 23);     // exponent bias 127 -> 7
    v += 0x7FFFFu + ((v >> 20) & 1u);  // keep 3 mantissa bits, ties to even
    code = v >> 20;
    if (code > 0x7Eu) code = 0x7Eu;    // 480 is not a finite E4M3 value
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(u) * 512.0f);  // 0..8
  }
  return code | sign;
}

// Four E4M3 codes of values already inside [-448, 448], packed little-end
// first, by the hardware conversion v_cvt_pk_fp8_f32 (gfx950: OCP E4M3FN,
// round to nearest even under the default mode).  On that domain it returns
// exactly e4m3_rne_sat's code: an exhaustive run over every bf16 value with
// |v| <= 448 found no difference (bf16 inputs scaled by a power of two, as
// MXFP8 produces them, are bf16 values).  Above 464 it returns NaN instead
// of saturating, so callers whose values may exceed 448 use e4m3_rne_sat.
__device__ __forceinline__ uint32_t e4m3x4_in_range(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// MXFP8 scale exponent of a group: smallest e with amax <= 448 * 2^e,
// clamped to [-127, 127]; 0 for an all-zero group.  amax is a bf16 value.
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0) return 0;
  const uint32_t ef = u >> 23;
  if (ef == 0) return -127;            // below 2^-126: far under 448 * 2^-127
  int e = (int)ef - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Order-preserving 32-bit key of a finite score: larger score <=> larger
// key; -0 and +0 map to the same key.  Key 0 is never produced for a finite
// score and marks "no candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Agent-scope (whole GPU) atomics and loads for data shared between
// workgroups of one launch.
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dsa

// Host-side helpers (validation and launch bookkeeping).
namespace dsa_host {
inline int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
}  // namespace dsa_host
