// Lightning Indexer: scoring, head weighting and Top-K over the paged MXFP8
// K cache with no score matrix written to HBM ("Deep Dive into Sparse
// Attention ...", section "1. Computation Optimization ... DSA Fused Kernel";
// Kimi K3.1 Pro Day0 page, "Lightning Indexer Three-Stream Coordination":
// scoring, head weighting and Top-K selection fused, selection pipelined with
// the paged K-cache reads).
//
//   I(t,s) = sum_h w[r,h] * max(0, q[r,h] . k[s]),  s <= t = row_pos[r]
//
// Two launches on the caller's stream:
//  1. scan: every row's causal history is cut into units of 16 pages (1024
//     positions); workgroups take units in row-major order.  For a unit, each
//     wave streams eight half pages through a four-deep register ring and
//     runs v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 codes of both operands,
//     their E8M0 block scales applied by the instruction, fp32 accumulation)
//     against the resident query heads, applies ReLU and the head weights in
//     fp32 and keeps the unit's
//     scores as order-preserving 32-bit keys in LDS.  A local filter (a
//     bitwise search with ballot counts over each lane's largest keys) finds
//     an edge e_u with zero low 16 bits that at least the unit's quota of
//     keys reach (quota: about the unit's expected share of the Top-K plus
//     four standard deviations), so e_u never exceeds the unit's quota-th
//     largest key; the unit writes every key >= e_u with its position, in
//     position order, to its slice of the candidate workspace and records
//     e_u.
//  2. select: one workgroup per row holds the row's candidates in registers
//     (eight per lane in position order, in one of five layouts by the
//     size of the row's largest unit; rows that fit none are gathered into
//     LDS), finds the exact K-th key T among those >= max_u e_u with radix
//     passes over the occupied key range, and writes the kept
//     positions in ascending order.  Every key a unit left out is below its
//     e_u <= T, so the result is the exact Top-K.  When fewer than K
//     candidates reach max_u e_u, the units whose edge could hide a Top-K key
//     are rescored in full and the selection is repeated (exact, rarely
//     taken).  Ties are broken by the lower position.
// No floating-point atomics are used, so results are deterministic.
#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>

#include "quant_dev.hpp"

namespace {

using namespace dsa;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnitPages = 16;
constexpr int kUnitTok = kUnitPages * kPage;           // 1024 keys per unit
constexpr int kHalvesPerWave = 2 * kUnitPages / kWaves;  // 8 half pages per wave (unit rescoring)
// The per-row scan: two work-groups of four waves per CU (measured faster
// than one of eight).
constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanHalves = 2 * kUnitPages / kScanWaves;  // 8 half pages per wave and unit
constexpr int kRing = 4;                               // half pages in flight per wave
constexpr int kBins = 4096;                            // select histogram (12-bit passes)
constexpr int kCandPer = 24;                           // select: candidates per thread
constexpr int kChunk = kCandPer * kThreads;            // candidates held in registers at once
constexpr int kMaxRows = 1024;                         // rows per launch
constexpr int kMaxBtStride = 16384;                    // pages per row (1M tokens)
constexpr int kMaxUnitsPerRow = kMaxBtStride / kUnitPages;
constexpr int kSelThreads = 1024;                      // select workgroup
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kFastUnits = 128;                        // select fast path: units per row
constexpr int kFastPer = kFastUnits / kSelWaves;       // units per wave
static_assert(kHalvesPerWave % kRing == 0, "the ring wraps at unit boundaries");
static_assert(kScanHalves % kRing == 0, "the scan ring wraps at unit boundaries");

// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-class
// GPUs: 32-bit data format, no swizzle.
constexpr int kRawBufferWord3 = 0x00020000;

enum : uint32_t { kErrBadPage = 4u, kErrFallback = 8u, kErrMixedTile = 16u };

struct Params {
  const uint8_t* q;      // [R, H, 128] E4M3
  const uint8_t* qs;     // [R, H, 4]  E8M0
  const float* w;        // [R, H]
  const uint8_t* kpool;
  int64_t pool_pages;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* row_seq;  // null: every row reads block-table row 0
  const int32_t* row_pos;
  int32_t R;
  int32_t H;
  int32_t topk;
  int32_t upr;           // units-per-row stride of ucount / uedge
  int32_t tile_rows;     // tiled paths: rows per tile (<= kTileRows), all of one sequence
  int32_t j_start;       // select: the first layout tried (slots per unit / 64)
  int32_t* out_idx;
  float* out_score;
  float* dump;           // score rows (test entry point only)
  int64_t ld;
  uint32_t* hdr;         // [2] sticky status bits (may be null)
  uint32_t* ucount;      // [R][upr] candidates emitted per unit
  uint32_t* uedge;       // [R][upr] every key a unit left out is below this
  uint2* cand;           // [R][bt_stride * 64] (key, position)
  // decode prolog folded into the scan (dsa_decode_indexer_topk only)
  const uint16_t* q_bf16;  // [R, H, 128] bf16 queries (quantised in LDS; q / qs unused)
  const uint16_t* k_new;   // [R, 128] bf16 new indexer key of each row
  const uint16_t* kv_new;  // [R, 576] bf16 new KV row of each row
  const int64_t* new_slot; // [R] slot of each row's new token (< 0: none)
  uint8_t* kpool_w;        // the K pool, written with the new keys
  uint8_t* kvpool_w;       // the KV pool, written with the new records
  uint8_t* q_ws;           // [R, H, 128] the quantised queries, written for the select (== q)
  uint8_t* qs_ws;          // [R, H, 4] their scales (== qs)
  int32_t extra_wgs;       // work-groups after the scan's that write the new tokens
};

struct ScanSmem {
  uint32_t keys[kUnitTok];            // scores of the current unit as keys
  uint32_t rowpre[kMaxRows + 1];      // exclusive prefix of units per row
  int32_t rowt[kMaxRows];             // row_pos of every row
  int32_t rowseq[kMaxRows];           // row_seq of every row
  uint32_t red[2 * kScanWaves + 2];
};

struct SelSmem {
  uint32_t keys[kUnitTok];            // rescoring a unit
  uint32_t hist[2 * kBins];           // general path: the first kBins
  uint32_t cpre[kMaxUnitsPerRow + 1]; // candidate prefix per unit
  alignas(16) uint32_t wred[kSelWaves][4];  // fast path: per-wave sums and maxima
  alignas(16) uint32_t wsum[2][kSelWaves];  // fast path: per-wave histogram sums
  alignas(16) uint32_t wtot[kSelWaves];     // fast path: per-wave (equal, greater) counts
  uint32_t red[2 * kWaves + 2];
  uint32_t misc[16];
  uint32_t rcount;                    // fast path: keys of a small bin collected so far
  uint32_t rlist[64];                 // fast path: the keys of a small bin (any order)
};

__device__ __forceinline__ void flag_error(uint32_t* hdr, uint32_t bits) {
  // through a global-address-space pointer: a flat atomic here would need an
  // aperture check
  typedef __attribute__((address_space(1))) uint32_t guint32;
  if (hdr) __hip_atomic_fetch_or((guint32*)hdr + 2, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- block primitives (256 threads) -------------------------------------

// Inclusive prefix sum / max across the 64 lanes of a wave with DPP row
// shifts (within rows of 16 lanes) and row broadcasts (across rows).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return x;
}

// Exclusive prefix of v over the block of NT threads; *total receives the
// block sum.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t* total) {
  const int wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) red[wv] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = red[i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  const int wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_max(v);
  if ((threadIdx.x & 63) == 63) red[wv] = x;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) m = max(m, red[i]);
  __syncthreads();
  return m;
}

// ---- units ------------------------------------------------------------------

struct Unit {
  int row, uir, units_r, pg0, pg1, t;
};

// Pages a row scans: positions 0..t, bounded by the block table width.
__device__ __forceinline__ int row_pages(int t, int bt_stride) {
  return t < 0 ? 1 : min(t / kPage + 1, bt_stride);
}
__device__ __forceinline__ int row_units(int t, int bt_stride) {
  return (row_pages(t, bt_stride) + kUnitPages - 1) / kUnitPages;
}

template <int NT>
__device__ __forceinline__ void plan_rows(const Params& P, ScanSmem& S) {
  uint32_t* rowpre = S.rowpre;
  uint32_t* red = S.red;
  constexpr int kPerMax = (kMaxRows + NT - 1) / NT;
  const int per = (P.R + NT - 1) / NT;
  const int r0 = threadIdx.x * per;
  // every load is issued before the first store to LDS (a store through a
  // generic pointer would otherwise keep the next load behind it)
  int tv[kPerMax], sv[kPerMax];
#pragma unroll
  for (int i = 0; i < kPerMax; ++i) {
    const bool in = i < per && r0 + i < P.R;
    tv[i] = in ? P.row_pos[r0 + i] : 0;
    sv[i] = in && P.row_seq ? P.row_seq[r0 + i] : 0;
  }
  uint32_t lu = 0;
#pragma unroll
  for (int i = 0; i < kPerMax; ++i) {
    if (i < per && r0 + i < P.R) {
      S.rowt[r0 + i] = tv[i];
      S.rowseq[r0 + i] = sv[i];
      lu += (uint32_t)row_units(tv[i], P.bt_stride);
    }
  }
  uint32_t total;
  uint32_t run = block_excl_scan<NT>(lu, red, &total);
  for (int i = 0; i < per; ++i) {
    if (r0 + i < P.R) {
      rowpre[r0 + i] = run;
      run += (uint32_t)row_units(S.rowt[r0 + i], P.bt_stride);
    }
  }
  if (threadIdx.x == 0) rowpre[P.R] = total;
  __syncthreads();
}

__device__ __forceinline__ Unit decode_unit(const Params& P, const ScanSmem& S, uint32_t u) {
  const uint32_t* rowpre = S.rowpre;
  int lo = 0, hi = P.R - 1;     // row r with rowpre[r] <= u < rowpre[r+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rowpre[mid] <= u) lo = mid; else hi = mid - 1;
  }
  Unit U;
  U.row = lo;
  U.uir = (int)(u - rowpre[lo]);
  U.units_r = (int)(rowpre[lo + 1] - rowpre[lo]);
  U.t = S.rowt[lo];
  const int pr = row_pages(U.t, P.bt_stride);
  U.pg0 = U.uir * kUnitPages;
  U.pg1 = min(pr, U.pg0 + kUnitPages);
  // identical in every lane: keep the fields in scalar registers
  U.row = __builtin_amdgcn_readfirstlane(U.row);
  U.uir = __builtin_amdgcn_readfirstlane(U.uir);
  U.units_r = __builtin_amdgcn_readfirstlane(U.units_r);
  U.t = __builtin_amdgcn_readfirstlane(U.t);
  U.pg0 = __builtin_amdgcn_readfirstlane(U.pg0);
  U.pg1 = __builtin_amdgcn_readfirstlane(U.pg1);
  return U;
}

// Unit uir of a row whose last position is t (used by the rescoring path).
__device__ __forceinline__ Unit row_unit(const Params& P, int row, int t, int uir) {
  Unit U;
  U.row = row;
  U.uir = uir;
  U.units_r = row_units(t, P.bt_stride);
  U.t = t;
  U.pg0 = uir * kUnitPages;
  U.pg1 = min(row_pages(t, P.bt_stride), U.pg0 + kUnitPages);
  return U;
}

// ---- scoring ---------------------------------------------------------------

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

template <int NHT>
struct QOperand {
  v8i a[NHT];       // A operand per head tile: 32 E4M3 codes
  int s[NHT];       // E8M0 scale of the lane's 32-dim block
  float w[NHT][4];  // weights of heads 16i + 4g + c
};

// Query heads as the A operand of v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3
// times E4M3, one E8M0 scale per operand row and 32-wide k block): lane
// (head 16i + lane%16, group g = lane/16) holds dims 16g .. 16g+15 and
// 64+16g .. 64+16g+15 of its head, and supplies the scale of dims
// 32g .. 32g+31 (the instruction's k order and scale ownership; the key
// operand uses the same ones).  No dequantisation: the instruction applies
// both scales.
template <int NHT>
__device__ __forceinline__ void load_q(const Params& P, int row, QOperand<NHT>& Q) {
  const int lane = threadIdx.x & 63, hr = lane & 15, g = lane >> 4;
  // Buffer loads over the row's q codes, scales and weights: a head beyond H
  // reads out of range, which returns zeros.  No value is selected after
  // its load, so nothing here waits for the loads; every path issues the
  // same loads, so the compiler's wait counting sees a fixed number.
  row = __builtin_amdgcn_readfirstlane(row);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.q + (int64_t)row * P.H * kIdxDim), (short)0, P.H * kIdxDim, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.qs + (int64_t)row * P.H * 4), (short)0, P.H * 4, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(P.w + (int64_t)row * P.H), (short)0, P.H * 4, kRawBufferWord3);
  constexpr uint32_t kOut = 0x7FFFFFF0u;
#pragma unroll
  for (int i = 0; i < NHT; ++i) {
    const int h = 16 * i + hr;
    const bool live = h < P.H;
    const uint32_t oq = live ? (uint32_t)(h * kIdxDim + 16 * g) : kOut;
    const v4u a = __builtin_amdgcn_raw_buffer_load_b128(rq, oq, 0, 0);
    const v4u b = __builtin_amdgcn_raw_buffer_load_b128(rq, live ? oq + 64u : kOut, 0, 0);
    Q.a[i] = v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    Q.s[i] = (int)__builtin_amdgcn_raw_buffer_load_b8(rs, live ? (uint32_t)(h * 4 + g) : kOut, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int hh = 16 * i + 4 * g + c;
      Q.w[i][c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, hh < P.H ? (uint32_t)hh * 4u : kOut, 0, 0));
    }
  }
}

// Half a page (two token tiles of 16) as held by one lane: for tile
// j = 2*half + jj, d[2jj], d[2jj+1] are this lane's 32 code bytes of token
// 16j + lane%16 (dims 16g..16g+15 and 64+16g..64+16g+15, g = lane/16) and
// s[jj] the E8M0 byte of its dims 32g..32g+31.
struct HalfRegs {
  uint4 d[4];
  uint32_t s[2];
};

// Loads half `half` of the page behind `rsrc` (a raw buffer descriptor
// covering the page, or with zero records when the half is absent: then
// every load is out of range, reads nothing and returns 0).  The page's
// tile layout makes each of the four code loads one contiguous kilobyte
// (16 bytes at 16 * lane) and each scale load 64 contiguous bytes.
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t rsrc, int half, HalfRegs& hr) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int o = 32 * half + 16 * jj + r;   // the lane's token in the page
    const v4u a = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)k_code_off(o, 16 * g), 0, 0);
    const v4u b = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)k_code_off(o, 64 + 16 * g), 0, 0);
    hr.d[2 * jj] = make_uint4(a[0], a[1], a[2], a[3]);
    hr.d[2 * jj + 1] = make_uint4(b[0], b[1], b[2], b[3]);
    hr.s[jj] = __builtin_amdgcn_raw_buffer_load_b8(rsrc, (uint32_t)k_scale_off(o, g), 0, 0);
  }
}

// ReLU in one instruction (v_maximum3_f32, the NaN-propagating maximum;
// fmaxf would add a canonicalising max per element for signalling NaNs).
// maximum(-0, +0) is +0.
__device__ __forceinline__ float relu(float x) {
  return __builtin_elementwise_maximum(x, 0.f);
}

// Sum over the four 16-lane rows of a wave, every lane receiving the total,
// associated as (row0 + row1) + (row2 + row3); cross-row moves with
// v_permlane16_swap / v_permlane32_swap.
__device__ __forceinline__ float rows_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);   // rows 0,0,2,2 | 1,1,3,3
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // pairs 01 | 23
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Four per-lane partial sums p[j] (row g holds its share of item j): row g
// returns item g's total over the four rows, associated exactly as rows_sum.
__device__ __forceinline__ float rows_sum_scatter(const float (&p)[4]) {
  const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[2]), __float_as_uint(p[3]), false, false);
  // rows 0..3: items 0,1,0,1 (x) and 2,3,2,3 (y), each summed over its row pair
  const float sa = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const float sb = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(sa), __float_as_uint(sb), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// One head tile's terms of a lane's weighted ReLU sum: for the lane's four
// heads c of head tile i, p += w * ReLU(S), a chain of FMAs (head tile 0
// starts the chain with a product).
template <int NHT>
__device__ __forceinline__ float head_acc(const QOperand<NHT>& Q, int i, const v4f& acc, float p) {
  p = i == 0 ? Q.w[0][0] * relu(acc[0]) : __builtin_fmaf(Q.w[i][0], relu(acc[0]), p);
#pragma unroll
  for (int c = 1; c < 4; ++c) p = __builtin_fmaf(Q.w[i][c], relu(acc[c]), p);
  return p;
}

// One scaled FP8 MFMA: head tile i of Q against a token tile (formats 0 / 0:
// E4M3 for both operands; scale byte 0 of each lane).
template <int NHT>
__device__ __forceinline__ v4f head_mfma(const QOperand<NHT>& Q, int i, const v8i& kb, int ks) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[i], kb, zero, 0, 0, 0, Q.s[i], 0, ks);
}

// A lane's share of the weighted ReLU sum over the heads of one token tile:
// one chain over head tiles i = 0..NHT-1 and heads c = 0..3.  Every scoring
// path takes these operations in this order, so all produce the same bits.
template <int NHT>
__device__ __forceinline__ float head_part(const QOperand<NHT>& Q, const v8i& kb, int ks) {
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < NHT; ++i) p = head_acc(Q, i, head_mfma(Q, i, kb, ks), p);
  return p;
}

// Scores of the 32 tokens of one half page; lanes 0..15 end with token
// 16jj + lane of the half in out[jj].  One scaled FP8 MFMA per head tile
// and token tile covers all 128 dims.  Head sum: in-lane over the lane's
// heads, then across the four lane groups, in a fixed order.
template <int NHT>
__device__ __forceinline__ void score_half(const QOperand<NHT>& Q, const HalfRegs& hr,
                                           float out[2]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const uint4 lo = hr.d[2 * jj], hi = hr.d[2 * jj + 1];
    const v8i kb = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const int ks = (int)hr.s[jj];
    out[jj] = rows_sum(head_part<NHT>(Q, kb, ks));
  }
}

// Block-table entries of unit U of a row mapped to block-table row `seq`,
// one per lane (lanes < the unit's page count; other lanes read out of range,
// which moves nothing).  The value is not examined here: its first use is
// when the unit's half pages are requested, so waiting for it never waits
// for ring loads issued after it.
__device__ __forceinline__ int32_t unit_pages(const Params& P, const Unit& U, int seq) {
  const int lane = threadIdx.x & 63;
  seq = __builtin_amdgcn_readfirstlane(seq);   // uniform: the descriptor lives in scalar registers
  const bool want = lane < U.pg1 - U.pg0;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(P.bt + (int64_t)seq * P.bt_stride), (short)0, P.bt_stride * 4, kRawBufferWord3);
  return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      rsrc, want ? (uint32_t)(U.pg0 + lane) * 4u : (uint32_t)P.bt_stride * 4u, 0, 0);
}

// Issues the loads of half page h of unit U (block-table entries `pid` as
// returned by unit_pages).  Every call issues the same loads: an absent half
// (past the unit, a row with t < 0, or a page id out of the pool, which sets
// *bad) gets a zero-record descriptor, so the loads retire in issue order
// and the compiler's wait counting never has to drain the ring.  Returns
// whether the half exists.
__device__ __forceinline__ bool fetch_half(const Params& P, const Unit& U, int32_t pid, int h,
                                           HalfRegs& b, bool* bad) {
  const bool want = h < 2 * (U.pg1 - U.pg0) && U.t >= 0;
  const int32_t raw = __builtin_amdgcn_readlane(pid, (h >> 1) & 63);
  const bool inpool = raw >= 0 && (int64_t)raw < P.pool_pages;
  *bad |= want && !inpool;
  const int32_t id = want && inpool ? raw : -1;
  const bool ok = id >= 0;
  const uint8_t* page = P.kpool + (int64_t)(ok ? id : 0) * kKPageBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(page), (short)0, ok ? kKPageBytes : 0, kRawBufferWord3);
  load_half(rsrc, h & 1, b);
  return ok;
}

// Scores half page h of unit U: keys of its 32 positions into keys[] (key 0
// for positions past t or on an absent page), or, for the dump, the scores.
template <int NHT, bool DUMP>
__device__ __forceinline__ void consume_half(const Params& P, const Unit& U, const QOperand<NHT>& Q,
                                             int h, const HalfRegs& b, bool ok, uint32_t* keys) {
  const int lane = threadIdx.x & 63;
  float sc[2] = {0.f, 0.f};
  if (ok) score_half<NHT>(Q, b, sc);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tok = 32 * h + 16 * jj + lane;      // unit-local, lanes 0..15
    const int pos = U.pg0 * kPage + tok;
    const bool valid = ok && pos <= U.t;
    if (lane < 16) {
      if (DUMP) {
        if (valid && pos < P.ld) P.dump[(int64_t)U.row * P.ld + pos] = sc[jj] == 0.f ? 0.f : sc[jj];
      } else {
        keys[tok] = valid ? score_key(sc[jj]) : 0u;
      }
    }
  }
}

// Score one unit on its own (the dump and the rescoring of the select):
// wave w takes half pages w, w+4, ..., w+28 of the unit, fully unrolled,
// with kRing of them in flight.
template <int NHT, bool DUMP>
__device__ __forceinline__ void score_unit(const Params& P, const Unit& U, uint32_t* keys) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bool bad = false;
  const int32_t pid = unit_pages(P, U, P.row_seq ? P.row_seq[U.row] : 0);
  // the query loads go before the ring: they are then older than every
  // ring load
  QOperand<NHT> Q;
  load_q<NHT>(P, U.row, Q);
  HalfRegs b[kRing];
  bool ok[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) ok[k] = fetch_half(P, U, pid, wv + kWaves * k, b[k], &bad);
#pragma unroll
  for (int k = 0; k < kHalvesPerWave; ++k) {
    consume_half<NHT, DUMP>(P, U, Q, wv + kWaves * k, b[k % kRing], ok[k % kRing], keys);
    if (k + kRing < kHalvesPerWave)
      ok[k % kRing] = fetch_half(P, U, pid, wv + kWaves * (k + kRing), b[k % kRing], &bad);
  }
  if (bad && (threadIdx.x & 63) == 0) flag_error(P.hdr, kErrBadPage);
}

// ---- scan kernel: local filter ------------------------------------------------

// Keys a unit keeps: its expected share E of the Top-K (about
// topk * 1024 / (t+1)) plus four standard deviations and a margin; every key
// when the row has no more than topk positions.
__host__ __device__ __forceinline__ uint32_t unit_quota(int t, int topk) {
  const int64_t n = (int64_t)t + 1;
  if (n <= topk) return 0xFFFFFFFFu;
  const float e = (float)topk * (float)kUnitTok / (float)n;
  float m = e + 4.0f * sqrtf(e) + 8.0f;
  // A row of more than 64 units can only take the select's first layout (64
  // slots per unit): keep the quota, and so the edge's few surplus keys,
  // below that.  There e < 32 (topk <= 2048), so 56 is still more than four
  // standard deviations above the unit's expected share.
  if (n > (int64_t)64 * kUnitTok) m = fminf(m, 56.0f);
  return (uint32_t)fminf(ceilf(m), (float)kUnitTok);
}

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));   // one v_med3_u32
}

// The N largest of a lane's keys, m[0] >= ... >= m[N-1] (0 = none): each
// key is inserted by clamping it between neighbours, from the bottom up.
template <int N>
__device__ __forceinline__ void lane_top(const uint32_t (&k)[kUnitPages], uint32_t (&m)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) m[j] = 0u;
#pragma unroll
  for (int i = 0; i < kUnitPages; ++i) {
#pragma unroll
    for (int j = N - 1; j > 0; --j) m[j] = umed3(m[j - 1], m[j], k[i]);
    m[0] = max(m[0], k[i]);
  }
}

// A unit's edge (values v: D per lane over the wave): the largest key T
// with zero low 16 bits such that at least `need` of the values are >= T,
// found bit by bit from the top with ballot counts (no memory traffic, no
// atomics); 0 when fewer than `need` values reach 2^16.  The values are the
// unit's keys or a subset of them, so at least `need` of the unit's keys are
// >= T: T never exceeds the unit's need-th largest key.
template <int D>
__device__ __forceinline__ uint32_t key_floor(const uint32_t (&v)[D], uint32_t need) {
  uint32_t a = 0u;
#pragma unroll
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t ca = a | (1u << bit);
    uint32_t sa = 0u;
#pragma unroll
    for (int i = 0; i < D; ++i) sa += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v[i] >= ca));
    if (sa >= need) a = ca;
  }
  return a;
}

// The edge search runs over each lane's three largest keys when the quota
// is at most 64 (one key per lane on average), over its five largest up to
// 320, and over all keys above.  The subset must hold about the quota
// largest keys: a lane that holds more of them than the subset keeps makes
// the edge lower and the unit keeps more candidates (a Binomial(16, q/1024)
// count per lane exceeds 3 for q = 192 often enough to add a hundred
// candidates; 5 rarely).
constexpr uint32_t kTop3Quota = 64;
constexpr uint32_t kTop5Quota = 5 * 64;

// Local filter of a scored unit (keys of unit-local position 64i + lane in
// S.keys).  Every wave reads all 1024 keys and finds the same edge: the
// largest 16-bit-prefix key that at least `quota` keys reach, searched over
// each lane's three or five largest keys (a subset, so the edge never
// exceeds the unit's quota-th largest key), or over all keys for quotas
// above 320.
// Keys at or above the edge are emitted in position order: wave w writes
// its share of the pages (16 / waves), at offsets from the per-page ballot counts that every
// wave holds.  No atomics; one barrier, once every wave holds the keys in
// registers, so the next unit may overwrite them.
__device__ __forceinline__ void filter_unit(const Params& P, ScanSmem& S, const Unit& U) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t k[kUnitPages];
#pragma unroll
  for (int i = 0; i < kUnitPages; ++i) k[i] = S.keys[kPage * i + lane];
  __syncthreads();
  const int ntok = (U.pg1 - U.pg0) * kPage;
  const uint32_t quota = unit_quota(U.t, P.topk);
  uint32_t edge = 0;
  if (quota < (uint32_t)ntok) {
    if (quota <= kTop3Quota) {
      uint32_t m[3];
      lane_top<3>(k, m);
      edge = key_floor<3>(m, quota);
    } else if (quota <= kTop5Quota) {
      uint32_t m[5];
      lane_top<5>(k, m);
      edge = key_floor<5>(m, quota);
    } else {
      edge = key_floor<kUnitPages>(k, quota);
    }
  }
  const uint32_t thr = max(edge, 1u);   // key 0 (no candidate) is never kept
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kUnitPages; ++i) {
    const uint32_t c = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k[i] >= thr));
    before += i < kUnitPages / kScanWaves * wv ? c : 0u;
    total += c;
  }
  const int64_t slice = ((int64_t)U.row * P.bt_stride + U.pg0) * kPage;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(P.cand + slice, (short)0, kUnitTok * 8, kRawBufferWord3);
#pragma unroll
  for (int i = 0; i < kUnitPages; ++i) {
    if (i / (kUnitPages / kScanWaves) != wv) continue;   // uniform
    const bool kept = k[i] >= thr;
    const uint64_t m = __builtin_amdgcn_ballot_w64(kept);
    const uint32_t off = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, before));
    const v2u v = {k[i], (uint32_t)(U.pg0 * kPage + kPage * i + lane)};
    __builtin_amdgcn_raw_buffer_store_b64(v, rc, kept ? off * 8u : 0x7FFFFFF0u, 0, 0);
    before += (uint32_t)__builtin_popcountll(m);
  }
  if (threadIdx.x == 0) {
    const int64_t slot = (int64_t)U.row * P.upr + U.uir;
    P.ucount[slot] = total;
    P.uedge[slot] = edge;
  }
}

// ---- the decode prolog folded into the scan ----------------------------------
//
// dsa_decode_indexer_topk hands the scan bf16 queries and each row's new
// token (indexer key, KV row, slot).  A work-group quantises its current
// row's queries and new key into LDS with the quantisers' own arithmetic
// (so the codes are the bytes mxfp8_quant writes) and takes its query operand
// from there.  The new token's own score is computed from the LDS copy of its
// key with the same instruction and operand layout as a key read from the
// cache, and replaces the score of position t, whose cache slot this launch
// writes concurrently (so the page read may hold either bytes).  The cache
// writes themselves (the new keys and KV records) are spread over the grid;
// later launches read them.

struct FusedSmem {
  alignas(16) uint8_t qc[DSA_MAX_INDEX_HEADS * kIdxDim];   // query codes [h][128]
  uint8_t qsc[DSA_MAX_INDEX_HEADS * 4];                     // query scales [h][4]
  alignas(16) uint8_t kc[kIdxDim];                          // new key codes
  uint8_t ksc[4];                                           // new key scales
};
struct NoSmem {};

// Whether row `row` brings a new token this launch writes (slot in the pool).
__device__ __forceinline__ bool has_new_token(const Params& P, int row) {
  const int64_t sl = P.new_slot[row];
  return sl >= 0 && sl < P.pool_pages * kPage;
}

// MXFP8 codes of 32 consecutive bf16 values (one E8M0 group, as 16 packed
// words): the same amax, exponent and rounding as mxfp8_quant_range.
__device__ __forceinline__ uint32_t quant_group32(const uint32_t (&w)[16], uint32_t (&codes)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[j] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[j] >> 16))));
  const int e = mx_exponent(amax);
  const float inv = pow2f(-e);
  // |x * inv| <= 448 by the scale rule: the hardware conversion applies
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t a = w[2 * d], b = w[2 * d + 1];
    codes[d] = e4m3x4_in_range(bf16_bits_to_f32(a & 0xFFFFu) * inv, bf16_bits_to_f32(a >> 16) * inv,
                               bf16_bits_to_f32(b & 0xFFFFu) * inv, bf16_bits_to_f32(b >> 16) * inv);
  }
  return (uint32_t)(e + 127);
}

// A thread's raw bf16 inputs of a row: its query group (head t/4, dims
// 32(t%4)..+31) and, for threads 0..3, a group of the row's new key.  Loaded
// before the ring's first loads so that waiting for them never waits for the
// ring; quantised while the ring is in flight.
struct RowIn {
  uint32_t q[16];
  uint32_t k[16];
  int64_t slot;        // the row's new-token slot
  bool qlive, knew;
};

__device__ __forceinline__ void load_words32(const uint16_t* src, uint32_t (&w)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * j);
    w[4 * j] = raw.x; w[4 * j + 1] = raw.y; w[4 * j + 2] = raw.z; w[4 * j + 3] = raw.w;
  }
}

// Every load is unconditional (threads without a query group or key group
// address past a buffer descriptor's end and read zeros), so the compiler's
// wait counting stays exact and waiting for these never waits for younger
// loads.
__device__ __forceinline__ void row_in_load(const Params& P, int row, RowIn& in) {
  const int t = threadIdx.x, h = t >> 2, grp = t & 3;
  row = __builtin_amdgcn_readfirstlane(row);
  in.qlive = h < P.H;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.q_bf16 + (int64_t)row * P.H * kIdxDim), (short)0, P.H * kIdxDim * 2, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.k_new + (int64_t)row * kIdxDim), (short)0, kIdxDim * 2, kRawBufferWord3);
  const uint32_t oq = in.qlive ? (uint32_t)((h * kIdxDim + 32 * grp) * 2) : 0x7FFFF000u;
  const uint32_t ok = t < 4 ? (uint32_t)(64 * t) : 0x7FFFF000u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v4u a = __builtin_amdgcn_raw_buffer_load_b128(rq, oq + 16 * j, 0, 0);
    const v4u b = __builtin_amdgcn_raw_buffer_load_b128(rk, ok + 16 * j, 0, 0);
    in.q[4 * j] = a[0]; in.q[4 * j + 1] = a[1]; in.q[4 * j + 2] = a[2]; in.q[4 * j + 3] = a[3];
    in.k[4 * j] = b[0]; in.k[4 * j + 1] = b[1]; in.k[4 * j + 2] = b[2]; in.k[4 * j + 3] = b[3];
  }
  in.slot = P.new_slot[row];
  in.knew = t < 4 && in.slot >= 0 && in.slot < P.pool_pages * kPage;
}

// The row's query codes and scales (heads >= H: zeros, as the out-of-range
// loads of load_q return) and new key into LDS.  No barrier.
__device__ __forceinline__ void row_in_store(const RowIn& in, FusedSmem& F) {
  const int t = threadIdx.x, h = t >> 2, grp = t & 3;
  uint32_t codes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint32_t sb = in.qlive ? quant_group32(in.q, codes) : 0u;
  uint4* dst = reinterpret_cast<uint4*>(F.qc + h * kIdxDim + 32 * grp);
  dst[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  dst[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
  F.qsc[h * 4 + grp] = (uint8_t)sb;
  if (in.knew) {
    uint32_t kc[8];
    const uint32_t ks = quant_group32(in.k, kc);
    uint4* kd = reinterpret_cast<uint4*>(F.kc + 32 * t);
    kd[0] = make_uint4(kc[0], kc[1], kc[2], kc[3]);
    kd[1] = make_uint4(kc[4], kc[5], kc[6], kc[7]);
    F.ksc[t] = (uint8_t)ks;
  }
}

// The head weights of the query operand (global loads, issued early).
template <int NHT>
__device__ __forceinline__ void load_w(const Params& P, int row, QOperand<NHT>& Q) {
  const int g = (threadIdx.x & 63) >> 4;
  row = __builtin_amdgcn_readfirstlane(row);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(P.w + (int64_t)row * P.H), (short)0, P.H * 4, kRawBufferWord3);
  constexpr uint32_t kOut = 0x7FFFFFF0u;
#pragma unroll
  for (int i = 0; i < NHT; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int hh = 16 * i + 4 * g + c;
      Q.w[i][c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, hh < P.H ? (uint32_t)hh * 4u : kOut, 0, 0));
    }
}

// The query codes and scales of the operand from LDS (load_q's layout).
template <int NHT>
__device__ __forceinline__ void load_q_codes_lds(const FusedSmem& F, QOperand<NHT>& Q) {
  const int lane = threadIdx.x & 63, hr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < NHT; ++i) {
    const int h = 16 * i + hr;
    const uint4 a = *reinterpret_cast<const uint4*>(F.qc + h * kIdxDim + 16 * g);
    const uint4 b = *reinterpret_cast<const uint4*>(F.qc + h * kIdxDim + 64 + 16 * g);
    Q.a[i] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    Q.s[i] = (int)F.qsc[h * 4 + g];
  }
}

// Score of the row's new key (every lane holds it): the key operand of a
// token tile whose 16 columns all carry the new key, through head_part and
// rows_sum as in score_half, so the bits equal the score of that key read
// from the cache.
template <int NHT>
__device__ __forceinline__ float new_token_score(const QOperand<NHT>& Q, const FusedSmem& F) {
  const int g = (threadIdx.x & 63) >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(F.kc + 16 * g);
  const uint4 hi = *reinterpret_cast<const uint4*>(F.kc + 64 + 16 * g);
  const v8i kb = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return rows_sum(head_part<NHT>(Q, kb, (int)F.ksc[g]));
}

// Fused path, at the first unit of a row (its inputs loaded by row_in_load
// and the head weights by load_w): the row's queries and new key into LDS,
// then the query operand; the work-group that holds the row's first unit
// also writes the row's query codes and scales to the workspace for the
// select's rescoring path.  Ends after a barrier.
template <int NHT>
__device__ __forceinline__ void fused_row(const Params& P, int row, int uir, const RowIn& in,
                                          FusedSmem& F, QOperand<NHT>& Q) {
  row_in_store(in, F);
  __syncthreads();
  load_q_codes_lds<NHT>(F, Q);
  if (uir == 0) {
    const int t = threadIdx.x;
    if (t * 32 < P.H * kIdxDim) {
      uint4* dst = reinterpret_cast<uint4*>(P.q_ws + (int64_t)row * P.H * kIdxDim + t * 32);
      const uint4* src = reinterpret_cast<const uint4*>(F.qc + t * 32);
      dst[0] = src[0];
      dst[1] = src[1];
    }
    if (t < P.H * 4) P.qs_ws[(int64_t)row * P.H * 4 + t] = F.qsc[t];
  }
}

// A workgroup takes a contiguous run of units (usually of one row, so the
// query operand stays resident).  The half-page ring runs across the units:
// while a unit's last half pages are scored, the first kRing half pages of
// the next unit are already requested, so they are in flight during the
// local filter and the memory system never idles at a unit boundary.
//
// FUSED (dsa_decode_indexer_topk): the decode prolog is folded in.  The new
// tokens' cache writes are spread over the grid; the queries come from bf16
// and are quantised per row into LDS (after the first ring loads are
// issued); the work-group holding a row's first unit also writes the row's
// quantised queries to the workspace for the select's rescoring path; and
// the new token's score is computed from its LDS copy.
// Fused launches: the last P.extra_wgs work-groups write the step's new
// indexer keys and KV records into the caches, one token per wave (later
// launches read them; the scan scores each new key from its own copy).  They
// come last in the grid, so they never hold a slot a scan work-group waits
// for at the start.
__device__ __forceinline__ void write_new_tokens(const Params& P, int scan_wgs) {
  const int lane = threadIdx.x & 63;
  const int r = ((int)blockIdx.x - scan_wgs) * kScanWaves + (int)(threadIdx.x >> 6);
  if (r < P.R) {
    const int64_t pool_slots = P.pool_pages * kPage;
    mxfp8_quant_range(lane < 16 ? lane : 16, 16, P.k_new + (int64_t)r * kIdxDim, 1, kIdxDim,
                      nullptr, nullptr, P.kpool_w, P.new_slot + r, pool_slots);
    kv_quant_range(0, 1, P.kv_new + (int64_t)r * kQK, 1, P.new_slot + r, P.kvpool_w, pool_slots);
  }
}

template <int NHT, bool FUSED>
__global__ __launch_bounds__(kScanThreads, 2) void indexer_scan_kernel(Params P) {
  __shared__ ScanSmem S;
  __shared__ typename std::conditional<FUSED, FusedSmem, NoSmem>::type F;
  const int scan_wgs = (int)gridDim.x - (FUSED ? P.extra_wgs : 0);
  if constexpr (FUSED) {
    if ((int)blockIdx.x >= scan_wgs) {
      write_new_tokens(P, scan_wgs);
      return;
    }
  }
  plan_rows<kScanThreads>(P, S);   // ends with a barrier
  const uint32_t U_total = S.rowpre[P.R];
  const uint32_t per = (U_total + scan_wgs - 1) / scan_wgs;
  uint32_t u = blockIdx.x * per;
  const uint32_t uend = min(U_total, u + per);
  if (u >= uend) return;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bool bad = false;   // a page id out of the pool (flagged once at the end)
  Unit U = decode_unit(P, S, u);
  int32_t pid = unit_pages(P, U, S.rowseq[U.row]);
  QOperand<NHT> Q;
  RowIn in;
  if constexpr (FUSED) {
    row_in_load(P, U.row, in);
    load_w<NHT>(P, U.row, Q);
  } else {
    load_q<NHT>(P, U.row, Q);
  }
  int qrow = U.row;
  HalfRegs b[kRing];
  bool ok[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) ok[k] = fetch_half(P, U, pid, wv + kScanWaves * k, b[k], &bad);
  if constexpr (FUSED) fused_row<NHT>(P, U.row, U.uir, in, F, Q);
  for (;;) {
    const bool more = u + 1 < uend;
    // the next unit (the current one again when there is none: its ring
    // loads then get page id -1 and move nothing)
    const Unit V = decode_unit(P, S, more ? u + 1 : u);
    const int32_t pidn = unit_pages(P, V, S.rowseq[V.row]);
    Unit Vf = V;          // the ring's view of the next unit: no pages when there is none
    if (!more) Vf.t = -1;
#pragma unroll
    for (int k = 0; k < kScanHalves; ++k) {
      consume_half<NHT, false>(P, U, Q, wv + kScanWaves * k, b[k % kRing], ok[k % kRing], S.keys);
      const int kn = k + kRing;
      if (kn < kScanHalves)
        ok[k % kRing] = fetch_half(P, U, pid, wv + kScanWaves * kn, b[k % kRing], &bad);
      else
        ok[k % kRing] = fetch_half(P, Vf, pidn, wv + kScanWaves * (kn - kScanHalves), b[k % kRing], &bad);
    }
    if constexpr (FUSED) {
      // the new token's key, when it lies in this unit, from its LDS copy:
      // written by the lane that wrote the cache-read key (half h of wave
      // h % 4, lane tok % 16), so program order puts it last; a key of 0
      // (the page is absent) stays 0
      const int tl = U.t - U.pg0 * kPage;
      if (tl >= 0 && U.t < U.pg1 * kPage && in.slot >= 0 && in.slot < P.pool_pages * kPage) {
        const float ns = new_token_score<NHT>(Q, F);
        if (wv == ((tl >> 5) & (kScanWaves - 1)) && (threadIdx.x & 63) == (tl & 15) &&
            S.keys[tl] != 0u)
          S.keys[tl] = score_key(ns);
      }
    }
    __syncthreads();
    filter_unit(P, S, U);   // its barrier orders the key reads before the next unit's writes
    if (!more) break;
    if (V.row != qrow) {
      if constexpr (FUSED) {
        row_in_load(P, V.row, in);
        load_w<NHT>(P, V.row, Q);
        __syncthreads();   // every wave has read the previous row's LDS operands
        fused_row<NHT>(P, V.row, V.uir, in, F, Q);
      } else {
        load_q<NHT>(P, V.row, Q);
      }
      qrow = V.row;
    }
    U = V;
    pid = pidn;
    ++u;
  }
  if (bad && (threadIdx.x & 63) == 0) flag_error(P.hdr, kErrBadPage);
}

// Test entry: write every score of every row.
template <int NHT>
__global__ __launch_bounds__(kThreads, 2) void indexer_dump_kernel(Params P) {
  __shared__ ScanSmem S;
  plan_rows<kThreads>(P, S);
  const uint32_t U_total = S.rowpre[P.R];
  for (uint32_t u = blockIdx.x; u < U_total; u += gridDim.x) {
    const Unit U = decode_unit(P, S, u);
    score_unit<NHT, true>(P, U, S.keys);
  }
}

// ---- select kernel ---------------------------------------------------------------
//
// Radix passes keep the histogram in LDS and the keys in registers; every
// pass alternates between two sets of reduction slots (par = pass parity),
// so four barriers per pass suffice.

// Candidate prefix per unit (S.cpre, S.cpre[units_r] = total); *emax
// receives the largest unit edge and *cmax the largest unit count.
__device__ __forceinline__ void load_counts(const Params& P, SelSmem& S, int row, int units_r,
                                            uint32_t* emax_out, uint32_t* cmax_out) {
  constexpr int kPer = kMaxUnitsPerRow / kThreads;   // 4
  const int u0 = threadIdx.x * kPer;
  const int64_t base = (int64_t)row * P.upr;
  uint32_t c[kPer];
  uint32_t local = 0, emax = 0, cmax = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool in = u0 + i < units_r;
    c[i] = in ? load_agent(&P.ucount[base + u0 + i]) : 0u;
    emax = max(emax, in ? load_agent(&P.uedge[base + u0 + i]) : 0u);
    cmax = max(cmax, c[i]);
    local += c[i];
  }
  uint32_t total;
  uint32_t run = block_excl_scan(local, S.red, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (u0 + i < units_r) S.cpre[u0 + i] = run;
    run += c[i];
  }
  if (threadIdx.x == 0) S.cpre[units_r] = total;
  // (block_max's first barrier publishes cpre)
  *emax_out = block_max(emax, S.red);
  *cmax_out = block_max(cmax, S.red);
}

// Clears the histogram and the pass's result flag (no barrier).
__device__ __forceinline__ void hist_clear(SelSmem& S, int par) {
  uint4* h4 = reinterpret_cast<uint4*>(S.hist);
#pragma unroll
  for (int i = 0; i < kBins / 4 / kThreads; ++i) h4[threadIdx.x + i * kThreads] = make_uint4(0, 0, 0, 0);
  if (threadIdx.x == 0) S.misc[4 * par + 2] = 0;
}

// Adds the keys in [base, base + span) of an array held in registers.
template <int N>
__device__ __forceinline__ void hist_add(SelSmem& S, const uint32_t (&k)[N], uint32_t base,
                                         uint32_t shift, uint64_t span) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (k[j] >= base && (uint64_t)(k[j] - base) < span) atomicAdd(&S.hist[(k[j] - base) >> shift], 1u);
}

// With the histogram complete (a barrier after the last add): the bin b
// holding the key of rank `need` from the top, and the count of keys in
// bins above it.  Returns false if the histogram holds fewer than `need`
// keys.  Two barriers; the histogram is left unchanged.
__device__ __forceinline__ bool hist_find(SelSmem& S, uint32_t need, int par, uint32_t* bin,
                                          uint32_t* above) {
  constexpr int kPer = kBins / kThreads;   // 16 bins per thread, thread 0 holds the top ones
  const int top = kBins - 1 - kPer * threadIdx.x;
  const int wv = threadIdx.x >> 6;
  uint32_t c[kPer];
#pragma unroll
  for (int i = 0; i < kPer / 4; ++i) {
    const uint4 q = reinterpret_cast<const uint4*>(S.hist)[(top - 4 * i - 3) / 4];
    c[4 * i] = q.w;
    c[4 * i + 1] = q.z;
    c[4 * i + 2] = q.y;
    c[4 * i + 3] = q.x;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += c[i];
  const uint32_t x = wave_incl_scan(mine);
  uint32_t* red = S.red + 4 * par;
  if ((threadIdx.x & 63) == 63) red[wv] = x;
  __syncthreads();
  uint32_t run = x - mine;    // keys in higher bins of this wave
#pragma unroll
  for (int i = 0; i < kWaves; ++i) run += i < wv ? red[i] : 0u;
  uint32_t* misc = S.misc + 4 * par;
  if (run < need && run + mine >= need) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (run < need && run + c[i] >= need) {
        misc[0] = (uint32_t)(top - i);
        misc[1] = run;
        misc[2] = 1;
      }
      run += c[i];
    }
  }
  __syncthreads();
  *bin = misc[0];
  *above = misc[1];
  return misc[2] != 0;
}

// Number of bits to drop so that keys in [lo, lo + range] map to 4096 bins.
__device__ __forceinline__ int range_shift(uint32_t range) {
  return range == 0 ? 0 : max(0, 32 - __builtin_clz(range) - 12);
}

// ---- general path: contiguous segments, any number of candidates --------------

// This thread's contiguous segment of chunk ch of the row's candidates
// (flat order = position order): elements f0 .. f0 + kCandPer - 1 with
// f0 = ch*kChunk + tid*kCandPer, key 0 past the end.  The unit of f0 comes
// from a binary search over the count prefix, later elements walk forward;
// every load is issued before any is used.
struct Seg {
  uint32_t k[kCandPer];
  uint32_t p[kCandPer];
};

__device__ __forceinline__ void load_segment(const Params& P, const SelSmem& S, int row, int units_r,
                                             uint32_t n_c, uint32_t ch, Seg& sg) {
  const uint32_t f0 = ch * kChunk + threadIdx.x * kCandPer;
  const uint2* rowc = P.cand + (int64_t)row * P.bt_stride * kPage;
  int lo = 0, hi = units_r - 1;    // last unit with cpre[u] <= f0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.cpre[mid] <= f0) lo = mid; else hi = mid - 1;
  }
  int u = lo;
  uint32_t base = S.cpre[u], next = S.cpre[u + 1];
  int32_t off[kCandPer];
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint32_t f = f0 + j;
    off[j] = -1;
    if (f < n_c) {
      while (f >= next) {
        ++u;
        base = next;
        next = S.cpre[u + 1];
      }
      off[j] = u * kUnitTok + (int32_t)(f - base);
    }
  }
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint2 v = off[j] >= 0 ? rowc[off[j]] : make_uint2(0u, 0u);
    sg.k[j] = v.x;
    sg.p[j] = v.y;
  }
}

// Exact key T of rank K among the candidates with key >= lo (keys in
// [lo, hi] are binned over the occupied range, at most three passes), and
// the number of keys equal to T to keep.  Returns false if fewer than K
// candidates are >= lo.  With one chunk the segment is already in
// registers; otherwise every pass loads every chunk again.
__device__ __forceinline__ bool seg_threshold(const Params& P, SelSmem& S, int row, int units_r,
                                              uint32_t n_c, Seg& sg, uint32_t lo, uint32_t hi,
                                              uint32_t K, uint32_t* T_out, uint32_t* ties_out) {
  if (hi < lo) return false;
  const uint32_t nch = (n_c + kChunk - 1) / kChunk;
  const uint32_t range = hi - lo;
  int shift = range_shift(range);
  uint64_t span = (uint64_t)range + 1;
  uint32_t base = lo, need = K;
  for (int pass = 0;; ++pass) {
    hist_clear(S, pass & 1);
    __syncthreads();
    for (uint32_t ch = 0; ch < nch; ++ch) {
      if (nch > 1) load_segment(P, S, row, units_r, n_c, ch, sg);
      hist_add(S, sg.k, base, (uint32_t)shift, span);
    }
    __syncthreads();
    uint32_t bin, above;
    if (!hist_find(S, need, pass & 1, &bin, &above)) return false;
    base += bin << shift;
    need -= above;
    if (shift == 0) break;
    span = 1ull << shift;            // the keys of the chosen bin
    shift = max(0, shift - 12);
  }
  *T_out = base;
  *ties_out = need;
  return true;
}

// Ordered emission of keys > T and the first `ties` keys equal to T: one
// block scan of the packed (equal, greater) counts of every segment places
// every kept key.
__device__ __forceinline__ void seg_emit(const Params& P, SelSmem& S, int row, int units_r,
                                         uint32_t n_c, Seg& sg, uint32_t T, uint32_t ties) {
  const int K = P.topk;
  int32_t* oidx = P.out_idx + (int64_t)row * K;
  float* osc = P.out_score ? P.out_score + (int64_t)row * K : nullptr;
  const uint32_t nch = (n_c + kChunk - 1) / kChunk;
  uint32_t run_gt = 0, run_eq = 0;
  for (uint32_t ch = 0; ch < nch; ++ch) {
    if (nch > 1) load_segment(P, S, row, units_r, n_c, ch, sg);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) {
      gt += sg.k[j] > T ? 1u : 0u;
      eq += sg.k[j] == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan((eq << 16) | gt, S.red, &tot);
    uint32_t er = run_eq + (pre >> 16);                       // equal keys before mine
    uint32_t opos = run_gt + (pre & 0xFFFFu) + min(er, ties); // kept keys before mine
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) {
      const uint32_t k = sg.k[j];
      bool kp = k > T;
      if (k == T) {
        kp = er < ties;
        ++er;
      }
      if (kp && opos < (uint32_t)K) {
        oidx[opos] = (int32_t)sg.p[j];
        if (osc) osc[opos] = key_score(k);
        ++opos;
      }
    }
    run_gt += tot & 0xFFFFu;
    run_eq += tot >> 16;
  }
}

// All candidates (n_c <= K, one chunk, already loaded) in position order,
// then -1 padding.
__device__ __forceinline__ void seg_emit_all(const Params& P, const Seg& sg, int row, uint32_t n_c) {
  const int K = P.topk;
  int32_t* oidx = P.out_idx + (int64_t)row * K;
  float* osc = P.out_score ? P.out_score + (int64_t)row * K : nullptr;
  const uint32_t f0 = threadIdx.x * kCandPer;
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint32_t f = f0 + j;
    if (f < n_c && f < (uint32_t)K) {
      oidx[f] = (int32_t)sg.p[j];
      if (osc) osc[f] = key_score(sg.k[j]);
    }
  }
  for (uint32_t f = n_c + threadIdx.x; f < (uint32_t)K; f += kThreads) {
    oidx[f] = -1;
    if (osc) osc[f] = -__builtin_huge_valf();
  }
}

// ---- fast path: at most 128 units of at most 64 candidates each --------------
//
// The select workgroup has 16 waves; wave w owns units 8w .. 8w+7 of the row
// and holds, in registers, slot `lane` of each unit's slice (a unit's
// candidates are slots 0 .. count-1 of its slice, in position order).  Every
// load (row position, counts, edges, candidate slots) is issued at entry,
// before the row's length is known: loads go through buffer descriptors
// that cover the row's part of the workspace, and units past the row's end
// are masked afterwards.  The threshold comes from 12-bit radix passes over
// the occupied key range with the histograms in LDS; each pass locates the
// bin of rank `need` in two levels (per-wave bin sums, then the bins of the
// wave that holds it, scanned again by every wave), so that every wave knows
// the result without another barrier.  Outputs are written through
// global-address-space pointers, which cannot alias LDS.
typedef __attribute__((address_space(1))) int32_t gint32;
typedef __attribute__((address_space(1))) float gfloat;

// Bin of rank `need` from the top of histogram H (kBins bins) and the count
// of keys in the bins above it; false when H holds fewer than `need` keys.
// Called by every wave after the barrier that completes H; `wsum` (16 slots)
// must not be read by any other pass in flight.
__device__ __forceinline__ bool fast_find(SelSmem& S, const uint32_t* H, uint32_t* wsum,
                                          uint32_t need, uint32_t* bin, uint32_t* above) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // level 1: this wave's 256 bins, the highest ones in wave 0
  {
    const int hb = kBins - 1 - 256 * wv - 4 * lane;
    const uint4 q = reinterpret_cast<const uint4*>(H)[(hb - 3) / 4];
    const uint32_t incl = wave_incl_scan(q.x + q.y + q.z + q.w);
    if (lane == 63) wsum[wv] = incl;
  }
  __syncthreads();
  // level 2: the wave that holds rank `need`, then its bins
  const uint32_t v = lane < kSelWaves ? wsum[lane] : 0u;
  const uint32_t vin = wave_incl_scan(v);
  const uint64_t wh = __builtin_amdgcn_ballot_w64(lane < kSelWaves && vin - v < need && vin >= need);
  if (wh == 0) return false;
  const int ws = __builtin_ctzll(wh);
  const uint32_t wabove = (uint32_t)__builtin_amdgcn_readlane((int)(vin - v), ws);
  const int hb = kBins - 1 - 256 * ws - 4 * lane;
  const uint4 q = reinterpret_cast<const uint4*>(H)[(hb - 3) / 4];
  const uint32_t c[4] = {q.w, q.z, q.y, q.x};   // bins hb, hb-1, hb-2, hb-3
  const uint32_t mine = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_incl_scan(mine) + wabove;
  const uint32_t excl = incl - mine;
  const uint64_t lh = __builtin_amdgcn_ballot_w64(excl < need && incl >= need);
  const int src = __builtin_ctzll(lh);
  uint32_t b = (uint32_t)(hb - 3), run = excl;
  bool done = false;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (!done && run + c[i] >= need) {
      b = (uint32_t)(hb - i);
      done = true;
    }
    if (!done) run += c[i];
  }
  *bin = (uint32_t)__builtin_amdgcn_readlane((int)b, src);
  *above = (uint32_t)__builtin_amdgcn_readlane((int)run, src);
  return true;
}

// Candidate slots of a row's first nu units that lie inside the row's region
// of the workspace (bt_stride * 64 slots): the last unit of a block table
// whose width is not a multiple of 16 pages has a shorter slice, and a
// layout's loads past it must read nothing (out-of-range buffer loads return
// 0) rather than the next row's region or memory past the workspace.
__device__ __forceinline__ int row_slots(const Params& P, int nu) {
  return min(nu * kUnitTok, P.bt_stride * kPage);
}

// A radix bin holding at most kSmallBin keys: instead of a further radix
// pass, its keys are collected in LDS (in any order) and every wave ranks
// them directly.  Returns the key T of rank `need` from the top within the
// bin and the number of keys equal to T that are kept (need minus the keys
// above T), the same result the remaining passes give.  One barrier.
// S.rcount must be zero (cleared with the histograms).
constexpr uint32_t kSmallBin = 64;

template <int NK>
__device__ __forceinline__ void small_bin_resolve(SelSmem& S, const uint32_t (&k)[NK], uint32_t lo,
                                                  uint64_t span, uint32_t need, uint32_t* T,
                                                  uint32_t* ties) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NK; ++i)
    if (k[i] >= lo && (uint64_t)(k[i] - lo) < span) S.rlist[atomicAdd(&S.rcount, 1u)] = k[i];
  __syncthreads();
  const uint32_t c = __builtin_amdgcn_readfirstlane(S.rcount);
  const uint32_t v = (uint32_t)lane < c ? S.rlist[lane] : 0u;
  uint32_t gt = 0, eq = 0;
  for (uint32_t j = 0; j < c; ++j) {
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)j);
    gt += kj > v ? 1u : 0u;
    eq += kj == v ? 1u : 0u;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64((uint32_t)lane < c && gt < need && gt + eq >= need);
  const int src = __builtin_ctzll(hit);
  *T = (uint32_t)__builtin_amdgcn_readlane((int)v, src);
  *ties = need - (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
}

// Layout J (1, 2, 4, 8 or 16): for J <= 8 wave w owns units (8/J)w ..
// (8/J)w + 8/J - 1 and holds slots lane, lane + 64, ..., lane + 64(J-1) of
// each; for J = 16 waves 2u and 2u+1 share unit u, slots lane + 64j and
// 512 + lane + 64j (j < 8).  Eight keys per lane in position order (unit,
// then slot); the path takes rows of up to 128/J units of up to 64J
// candidates.
// Returns 1 when the row is done.  Otherwise nothing was written and it
// returns the layout that would fit the row (2, 4 or 8, only from layout 1:
// the row has a unit with more than 64J candidates but few enough units),
// or 0: the row fits no layout, or fewer than K candidates reach the
// largest unit edge; the caller then takes the general path.  Block-uniform.
template <int J>
__device__ __forceinline__ int select_fast(const Params& P, SelSmem& S, int row) {
  constexpr int WPU = J > kFastPer ? J / kFastPer : 1;   // waves per unit
  constexpr int UPW = J > kFastPer ? 1 : kFastPer / J;   // units per wave
  constexpr int JW = J / WPU;                            // 64-slot groups a wave holds per unit
  constexpr int kUnits = kFastUnits / J;                 // units per row
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = UPW * (wv / WPU);
  const uint32_t sbase = (uint32_t)(64 * JW * (wv % WPU));   // first slot this wave holds
  const int K = P.topk;
  const int nu = min(P.upr, kUnits);   // units whose slices exist in the workspace
  // loads: row position; count and edge of unit u0 + lane (lanes < UPW);
  // slot lane + 64j of each of the wave's units
  const int t = P.row_pos[row];
  const int64_t ub = (int64_t)row * P.upr;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(P.ucount + ub, (short)0, nu * 4, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(P.uedge + ub, (short)0, nu * 4, kRawBufferWord3);
  const uint32_t uoff = lane < UPW ? (uint32_t)(u0 + lane) * 4u : (uint32_t)nu * 4u;
  uint32_t cnt_l = __builtin_amdgcn_raw_buffer_load_b32(rc, uoff, 0, 0);
  uint32_t edge_l = __builtin_amdgcn_raw_buffer_load_b32(re, uoff, 0, 0);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      P.cand + (int64_t)row * P.bt_stride * kPage, (short)0, row_slots(P, nu) * 8, kRawBufferWord3);
  uint32_t k[kFastPer], p[kFastPer];
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    const int a = i / JW, jj = i % JW;
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(
        rk, (uint32_t)(((u0 + a) * kUnitTok + sbase + lane + 64 * jj) * 8), 0, 0);
    k[i] = v[0];
    p[i] = v[1];
  }
  // clear both radix histograms (ordered before any add by the first barrier)
  {
    uint4* h4 = reinterpret_cast<uint4*>(S.hist);
#pragma unroll
    for (int i = 0; i < 2 * kBins / 4 / kSelThreads; ++i) h4[threadIdx.x + i * kSelThreads] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) S.rcount = 0;
  }
  const int units_r = row_units(t, P.bt_stride);
  if (units_r > kUnits) return 0;
  const bool take_all = t < 0 || unit_quota(t, K) == 0xFFFFFFFFu;   // at most K positions
  const bool uin = lane < UPW && u0 + lane < units_r;
  cnt_l = uin ? cnt_l : 0u;
  edge_l = uin ? edge_l : 0u;
  // candidates of unit u0+a (vis) and of the wave's units before it (vpre)
  const uint32_t csum_l = wave_incl_scan(cnt_l);   // lane i: candidates of units u0 .. u0+i
  uint32_t vis[UPW], vpre[UPW];
#pragma unroll
  for (int a = 0; a < UPW; ++a) {
    vis[a] = (uint32_t)__builtin_amdgcn_readlane((int)cnt_l, a);
    vpre[a] = (uint32_t)__builtin_amdgcn_readlane((int)csum_l, a) - vis[a];
  }
  const uint32_t tot_w = (uint32_t)__builtin_amdgcn_readlane((int)csum_l, 63);
  uint32_t km = 0;
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    if ((uint32_t)(lane + 64 * (i % JW)) >= vis[i / JW]) k[i] = 0u;
    km = max(km, k[i]);
  }
  const uint32_t cmax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(cnt_l), 63);
  const uint32_t emax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(edge_l), 63);
  const uint32_t kmax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(km), 63);
  if (lane == 0) *reinterpret_cast<uint4*>(S.wred[wv]) = make_uint4(tot_w, cmax_w, emax_w, kmax_w);
  __syncthreads();
  uint32_t n_c = 0, cmax = 0, emax = 0, kmax = 0, wbase = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint4 x = *reinterpret_cast<const uint4*>(S.wred[w]);
    wbase += w < wv ? x.x : 0u;
    n_c += x.x;
    cmax = max(cmax, x.y);
    emax = max(emax, x.z);
    kmax = max(kmax, x.w);
  }
  if (cmax > 64u * J) {
    // a layout with more slots per unit, if the row has few enough units
    if (J > 1) return 0;
    for (int jn = 2; jn <= 2 * kFastPer; jn *= 2)
      if (cmax <= 64u * jn && units_r <= kFastUnits / jn) return jn;
    return 0;
  }
  gint32* oidx = (gint32*)(P.out_idx + (int64_t)row * K);
  gfloat* osc = P.out_score ? (gfloat*)(P.out_score + (int64_t)row * K) : nullptr;
  if (take_all) {
    // every candidate is kept: unit u0+i's slot j goes to its flat index
#pragma unroll
    for (int i = 0; i < kFastPer; ++i) {
      const uint32_t sl = (uint32_t)(lane + 64 * (i % JW));   // relative to sbase
      const uint32_t f = wbase + vpre[i / JW] + sl;
      if (sl < vis[i / JW] && f < (uint32_t)K) {
        oidx[f] = (int32_t)p[i];
        if (osc) osc[f] = key_score(k[i]);
      }
    }
    for (uint32_t f = n_c + threadIdx.x; f < (uint32_t)K; f += kSelThreads) {
      oidx[f] = -1;
      if (osc) osc[f] = -__builtin_huge_valf();
    }
    return 1;
  }
  // radix passes over [lo, kmax]: pass p bins the keys of [base, base + span)
  // by (key - base) >> shift into histogram p & 1
  const uint32_t lo = max(emax, 1u);
  if (kmax < lo) return 0;
  int shift = range_shift(kmax - lo);
  uint64_t span = (uint64_t)(kmax - lo) + 1;
  uint32_t base = lo, need = (uint32_t)K;
  for (int pass = 0;; ++pass) {
    uint32_t* H = S.hist + (pass & 1) * kBins;
    if (pass >= 2) {
      // every wave finished reading this histogram before the last barrier
      reinterpret_cast<uint4*>(H)[threadIdx.x] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kFastPer; ++i)
      if (k[i] >= base && (uint64_t)(k[i] - base) < span) atomicAdd(&H[(k[i] - base) >> shift], 1u);
    __syncthreads();
    uint32_t bin, above;
    if (!fast_find(S, H, S.wsum[pass & 1], need, &bin, &above)) return 0;   // pass 0 only
    base += bin << shift;
    need -= above;
    if (shift == 0) break;
    span = 1ull << shift;   // the keys of the chosen bin
    if (H[bin] <= kSmallBin) {   // uniform: every wave reads the complete histogram
      uint32_t T0, t0;
      small_bin_resolve(S, k, base, span, need, &T0, &t0);
      base = T0;
      need = t0;
      break;
    }
    shift = max(0, shift - 12);
  }
  const uint32_t T = base, ties = need;   // T >= lo >= 1, so empty slots never equal it
  // emission: per-wave (greater, equal) totals, then every kept key's
  // position from the units' running sums and ballots
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    gt_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k[i] > T));
    eq_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k[i] == T));
  }
  if (lane == 0) S.wtot[wv] = (eq_w << 16) | gt_w;
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w4 = 0; w4 < kSelWaves / 4; ++w4) {
    const uint4 x = *reinterpret_cast<const uint4*>(&S.wtot[4 * w4]);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = 4 * w4 + j < wv ? xs[j] : 0u;
      gt_before += v & 0xFFFFu;
      eq_before += v >> 16;
    }
  }
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    const bool gt = k[i] > T, eq = k[i] == T;
    const uint64_t gb = __builtin_amdgcn_ballot_w64(gt);
    const uint64_t eb = __builtin_amdgcn_ballot_w64(eq);
    const uint32_t erank = eq_before + (uint32_t)__builtin_popcountll(eb & below);
    const bool kept = gt || (eq && erank < ties);
    const uint64_t kb = __builtin_amdgcn_ballot_w64(kept);
    const uint32_t opos = gt_before + min(eq_before, ties) + (uint32_t)__builtin_popcountll(kb & below);
    if (kept && opos < (uint32_t)K) {
      oidx[opos] = (int32_t)p[i];
      if (osc) osc[opos] = key_score(k[i]);
    }
    gt_before += (uint32_t)__builtin_popcountll(gb);
    eq_before += (uint32_t)__builtin_popcountll(eb);
  }
  return 1;
}

// select_fast with the layout J (2, 4, 8 or 16) a runtime value: one copy of
// the code for all wide layouts.  With RETRY, a layout too small for the row
// returns the larger one to try instead of giving up.
template <bool RETRY>
__device__ __forceinline__ int select_fast_rt(const Params& P, SelSmem& S, int row, int J) {
  J = __builtin_amdgcn_readfirstlane(J);
  const int WPU = J > kFastPer ? J / kFastPer : 1;       // waves per unit
  const int UPW = J > kFastPer ? 1 : kFastPer / J;       // units per wave
  const int JW = J / WPU;                                // 64-slot groups a wave holds per unit
  const int lgJW = 31 - __builtin_clz(JW);
  const int kUnits = kFastUnits / J;                     // units per row
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = UPW * (wv / WPU);
  const uint32_t sbase = (uint32_t)(64 * JW * (wv % WPU));   // first slot this wave holds
  const int K = P.topk;
  const int nu = min(P.upr, kUnits);   // units whose slices exist in the workspace
  // loads: row position; count and edge of unit u0 + lane (lanes < UPW);
  // slot lane + 64j of each of the wave's units
  const int t = P.row_pos[row];
  const int64_t ub = (int64_t)row * P.upr;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(P.ucount + ub, (short)0, nu * 4, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(P.uedge + ub, (short)0, nu * 4, kRawBufferWord3);
  const uint32_t uoff = lane < UPW ? (uint32_t)(u0 + lane) * 4u : (uint32_t)nu * 4u;
  uint32_t cnt_l = __builtin_amdgcn_raw_buffer_load_b32(rc, uoff, 0, 0);
  uint32_t edge_l = __builtin_amdgcn_raw_buffer_load_b32(re, uoff, 0, 0);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      P.cand + (int64_t)row * P.bt_stride * kPage, (short)0, row_slots(P, nu) * 8, kRawBufferWord3);
  uint32_t k[kFastPer], p[kFastPer];
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    const int a = i >> lgJW, jj = i & (JW - 1);
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(
        rk, (uint32_t)(((u0 + a) * kUnitTok + sbase + lane + 64 * jj) * 8), 0, 0);
    k[i] = v[0];
    p[i] = v[1];
  }
  // clear both radix histograms (ordered before any add by the first barrier)
  {
    uint4* h4 = reinterpret_cast<uint4*>(S.hist);
#pragma unroll
    for (int i = 0; i < 2 * kBins / 4 / kSelThreads; ++i) h4[threadIdx.x + i * kSelThreads] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) S.rcount = 0;
  }
  const int units_r = row_units(t, P.bt_stride);
  if (units_r > kUnits) return 0;
  const bool take_all = t < 0 || unit_quota(t, K) == 0xFFFFFFFFu;   // at most K positions
  const bool uin = lane < UPW && u0 + lane < units_r;
  cnt_l = uin ? cnt_l : 0u;
  edge_l = uin ? edge_l : 0u;
  // candidates of unit u0+a in this wave's slots: vis_l in lane a, their
  // prefix within the wave in vsc_l
  const uint32_t vis_l = min(cnt_l > sbase ? cnt_l - sbase : 0u, (uint32_t)(64 * JW));
  const uint32_t vsc_l = wave_incl_scan(vis_l);
  const uint32_t tot_w = (uint32_t)__builtin_amdgcn_readlane((int)vsc_l, 63);
  uint32_t km = 0;
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    const uint32_t vis = (uint32_t)__builtin_amdgcn_readlane((int)vis_l, i >> lgJW);
    if ((uint32_t)(lane + 64 * (i & (JW - 1))) >= vis) k[i] = 0u;
    km = max(km, k[i]);
  }
  const uint32_t cmax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(cnt_l), 63);
  const uint32_t emax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(edge_l), 63);
  const uint32_t kmax_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(km), 63);
  if (lane == 0) *reinterpret_cast<uint4*>(S.wred[wv]) = make_uint4(tot_w, cmax_w, emax_w, kmax_w);
  __syncthreads();
  uint32_t n_c = 0, cmax = 0, emax = 0, kmax = 0, wbase = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint4 x = *reinterpret_cast<const uint4*>(S.wred[w]);
    wbase += w < wv ? x.x : 0u;
    n_c += x.x;
    cmax = max(cmax, x.y);
    emax = max(emax, x.z);
    kmax = max(kmax, x.w);
  }
  if (cmax > 64u * J) {
    // a layout with more slots per unit, if the row has few enough units
    if (RETRY)
      for (int jn = 2 * J; jn <= 2 * kFastPer; jn *= 2)
        if (cmax <= 64u * jn && units_r <= kFastUnits / jn) return jn;
    return 0;
  }
  gint32* oidx = (gint32*)(P.out_idx + (int64_t)row * K);
  gfloat* osc = P.out_score ? (gfloat*)(P.out_score + (int64_t)row * K) : nullptr;
  if (take_all) {
    // every candidate is kept: unit u0+i's slot j goes to its flat index
#pragma unroll
    for (int i = 0; i < kFastPer; ++i) {
      const int a = i >> lgJW;
      const uint32_t sl = (uint32_t)(lane + 64 * (i & (JW - 1)));   // relative to sbase
      const uint32_t vis = (uint32_t)__builtin_amdgcn_readlane((int)vis_l, a);
      const uint32_t f = wbase + (uint32_t)__builtin_amdgcn_readlane((int)vsc_l, a) - vis + sl;
      if (sl < vis && f < (uint32_t)K) {
        oidx[f] = (int32_t)p[i];
        if (osc) osc[f] = key_score(k[i]);
      }
    }
    for (uint32_t f = n_c + threadIdx.x; f < (uint32_t)K; f += kSelThreads) {
      oidx[f] = -1;
      if (osc) osc[f] = -__builtin_huge_valf();
    }
    return 1;
  }
  // radix passes over [lo, kmax]: pass p bins the keys of [base, base + span)
  // by (key - base) >> shift into histogram p & 1
  const uint32_t lo = max(emax, 1u);
  if (kmax < lo) return 0;
  int shift = range_shift(kmax - lo);
  uint64_t span = (uint64_t)(kmax - lo) + 1;
  uint32_t base = lo, need = (uint32_t)K;
  for (int pass = 0;; ++pass) {
    uint32_t* H = S.hist + (pass & 1) * kBins;
    if (pass >= 2) {
      // every wave finished reading this histogram before the last barrier
      reinterpret_cast<uint4*>(H)[threadIdx.x] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kFastPer; ++i)
      if (k[i] >= base && (uint64_t)(k[i] - base) < span) atomicAdd(&H[(k[i] - base) >> shift], 1u);
    __syncthreads();
    uint32_t bin, above;
    if (!fast_find(S, H, S.wsum[pass & 1], need, &bin, &above)) return 0;   // pass 0 only
    base += bin << shift;
    need -= above;
    if (shift == 0) break;
    span = 1ull << shift;   // the keys of the chosen bin
    if (H[bin] <= kSmallBin) {   // uniform: every wave reads the complete histogram
      uint32_t T0, t0;
      small_bin_resolve(S, k, base, span, need, &T0, &t0);
      base = T0;
      need = t0;
      break;
    }
    shift = max(0, shift - 12);
  }
  const uint32_t T = base, ties = need;   // T >= lo >= 1, so empty slots never equal it
  // emission: per-wave (greater, equal) totals, then every kept key's
  // position from the units' running sums and ballots
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    gt_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k[i] > T));
    eq_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(k[i] == T));
  }
  if (lane == 0) S.wtot[wv] = (eq_w << 16) | gt_w;
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w4 = 0; w4 < kSelWaves / 4; ++w4) {
    const uint4 x = *reinterpret_cast<const uint4*>(&S.wtot[4 * w4]);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = 4 * w4 + j < wv ? xs[j] : 0u;
      gt_before += v & 0xFFFFu;
      eq_before += v >> 16;
    }
  }
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kFastPer; ++i) {
    const bool gt = k[i] > T, eq = k[i] == T;
    const uint64_t gb = __builtin_amdgcn_ballot_w64(gt);
    const uint64_t eb = __builtin_amdgcn_ballot_w64(eq);
    const uint32_t erank = eq_before + (uint32_t)__builtin_popcountll(eb & below);
    const bool kept = gt || (eq && erank < ties);
    const uint64_t kb = __builtin_amdgcn_ballot_w64(kept);
    const uint32_t opos = gt_before + min(eq_before, ties) + (uint32_t)__builtin_popcountll(kb & below);
    if (kept && opos < (uint32_t)K) {
      oidx[opos] = (int32_t)p[i];
      if (osc) osc[opos] = key_score(k[i]);
    }
    gt_before += (uint32_t)__builtin_popcountll(gb);
    eq_before += (uint32_t)__builtin_popcountll(eb);
  }
  return 1;
}

// Rescore unit u of the row in full and publish all of its keys.
template <int NHT>
__device__ __forceinline__ void rescore_unit(const Params& P, SelSmem& S, int row, int t, int u) {
  const Unit V = row_unit(P, row, t, u);
  __syncthreads();
  score_unit<NHT, false>(P, V, S.keys);
  __syncthreads();
  const uint4 kv = *reinterpret_cast<const uint4*>(&S.keys[4 * threadIdx.x]);
  const uint32_t k[4] = {kv.x, kv.y, kv.z, kv.w};
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) cnt += k[j] != 0u ? 1u : 0u;
  uint32_t total;
  uint32_t off = block_excl_scan(cnt, S.red, &total);
  uint2* dst = P.cand + ((int64_t)row * P.bt_stride + V.pg0) * kPage;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (k[j] != 0u) dst[off++] = make_uint2(k[j], (uint32_t)(V.pg0 * kPage + 4 * threadIdx.x + j));
  if (threadIdx.x == 0) {
    __hip_atomic_store(&P.ucount[(int64_t)row * P.upr + u], total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&P.uedge[(int64_t)row * P.upr + u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NHT, bool SHORT>
__global__ __launch_bounds__(kSelThreads, 1) void indexer_select_kernel(Params P) {
  __shared__ SelSmem S;
  const int row = blockIdx.x;
  int fast;
  if (SHORT) {
    // every row of the launch is short enough to need a layout with more
    // slots per unit (chosen on the host); one too small for a row names a
    // larger one, tried next
    fast = P.j_start;
    bool tried = false;
    while (fast > 1) {
      if (tried) __syncthreads();   // every wave has read the last attempt's LDS results
      tried = true;
      fast = select_fast_rt<true>(P, S, row, fast);
    }
  } else {
    fast = select_fast<1>(P, S, row);
    if (fast > 1) {
      __syncthreads();   // every wave has read the first attempt's LDS results
      fast = select_fast_rt<false>(P, S, row, fast);
    }
  }
  if (fast == 1) return;
  // general path: waves 0..3 (a barrier first, so that no wave still reads
  // what the fast path left in LDS; waves that have ended no longer count
  // at a barrier)
  __syncthreads();
  if (threadIdx.x >= kThreads) return;
  const int K = P.topk;
  const int t = P.row_pos[row];
  const int units_r = row_units(t, P.bt_stride);
  const bool take_all = t < 0 || unit_quota(t, K) == 0xFFFFFFFFu;   // at most K positions
  uint32_t emax, cmax;
  load_counts(P, S, row, units_r, &emax, &cmax);
  uint32_t n_c = S.cpre[units_r];
  Seg sg;
  uint32_t kmax = 0xFFFFFFFFu;
  if (n_c <= (uint32_t)kChunk) {
    load_segment(P, S, row, units_r, n_c, 0, sg);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) m = max(m, sg.k[j]);
    kmax = block_max(m, S.red);
  }
  if (take_all) {
    seg_emit_all(P, sg, row, n_c);
    return;
  }
  uint32_t T = 0, ties = 0;
  bool ok = seg_threshold(P, S, row, units_r, n_c, sg, max(emax, 1u), kmax, (uint32_t)K, &T, &ties);
  if (!ok) {
    // Fewer than K candidates reach the largest unit edge: a unit may have
    // left out a Top-K key.  Take the K-th key T0 of the current candidates
    // (none: every unit with a non-zero edge), rescore every unit whose edge
    // exceeds it in full, and select again.  Keys of the remaining units are
    // below their edge <= T0 <= the new K-th key, so the result is exact.
    if (threadIdx.x == 0) flag_error(P.hdr, kErrFallback);
    uint32_t T0 = 0, ties0 = 0;
    const bool ok0 = seg_threshold(P, S, row, units_r, n_c, sg, 1u, kmax, (uint32_t)K, &T0, &ties0);
    for (int u = 0; u < units_r; ++u) {
      const uint32_t e = load_agent(&P.uedge[(int64_t)row * P.upr + u]);
      if (e > (ok0 ? T0 : 0u)) rescore_unit<NHT>(P, S, row, t, u);
    }
    __threadfence();
    __syncthreads();
    load_counts(P, S, row, units_r, &emax, &cmax);
    n_c = S.cpre[units_r];
    kmax = 0xFFFFFFFFu;
    if (n_c <= (uint32_t)kChunk) {
      load_segment(P, S, row, units_r, n_c, 0, sg);
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) m = max(m, sg.k[j]);
      kmax = block_max(m, S.red);
    }
    ok = seg_threshold(P, S, row, units_r, n_c, sg, 1u, kmax, (uint32_t)K, &T, &ties);
    if (!ok) {   // fewer than K valid positions in the row (n_c < K <= kChunk)
      seg_emit_all(P, sg, row, n_c);
      return;
    }
  }
  seg_emit(P, S, row, units_r, n_c, sg, T, ties);
}

// ---- rows of one sequence in tiles ------------------------------------------------
//
// Multi-query decode and chunked prefill bring many query rows of one
// sequence.  Both take them in tiles of consecutive rows of one sequence,
// scored by the pair-per-wave kernel further below (two rows per wave, each
// unit's pages streamed once per pair, the pairs of a unit side by side in
// one work-group).

constexpr int kTileRows = 8;          // rows per tile of a prefill chunk; the multi-query maximum
constexpr int kTileMaxPages = 4096;   // block-table width the tiled entry points accept
constexpr int kSeqChunkRows = 4096;   // rows per launch of the sequence path (most)
// The candidate region of a launch holds 8 bytes per history slot of every
// row (a unit's slice has room for all 1024 of its keys, which the exact
// rescoring path may write).  A chunked prefill over a long context takes
// fewer rows per launch so that the region stays within this size (at 2048
// pages: 512 rows, 512 MiB, instead of 4 GiB for 4096 rows).
constexpr int64_t kSeqCandBytes = int64_t(512) << 20;
static_assert(kUnitPages == 16, "16 pages per unit: one key per lane and page");

// Candidates of unit u of one row: keys >= edge, in position order, then
// the unit's count and edge.  Every call issues the same buffer stores
// (lanes with nothing to write address out of range).
__device__ __forceinline__ void emit_wave(const Params& P, int row, bool live_row, int np_row, int u,
                                          const uint32_t (&k)[kUnitPages], uint32_t edge) {
  const int lane = threadIdx.x & 63;
  const int pg0 = kUnitPages * u;
  const bool live = live_row && np_row > pg0;
  const int64_t slice = ((int64_t)(live ? row : 0) * P.bt_stride + pg0) * kPage;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      P.cand + slice, (short)0, live ? kUnitTok * 8 : 0, kRawBufferWord3);
  // one compare per key: key 0 (no candidate) is below every threshold >= 1,
  // and no finite score's key reaches 0xFFFFFFFF
  const uint32_t thr = live ? max(edge, 1u) : 0xFFFFFFFFu;
  const uint32_t pos0 = (uint32_t)(pg0 * kPage + lane);
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < kUnitPages; ++i) {
    const bool kept = k[i] >= thr;
    const uint64_t m = __builtin_amdgcn_ballot_w64(kept);
    // cnt + the number of kept lanes below this one
    const uint32_t off = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, cnt));
    const v2u v = {k[i], pos0 + (uint32_t)(i * kPage)};
    __builtin_amdgcn_raw_buffer_store_b64(v, rc, kept ? off * 8u : 0x7FFFFFF0u, 0, 0);
    cnt += (uint32_t)__builtin_popcountll(m);
  }
  const int64_t us = (int64_t)(live ? row : 0) * P.upr;
  // descriptors stay wave-uniform (a per-lane one would be split into a loop)
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(P.ucount + us, (short)0, live ? P.upr * 4 : 0, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(P.uedge + us, (short)0, live ? P.upr * 4 : 0, kRawBufferWord3);
  const uint32_t uoff = lane == 0 ? (uint32_t)u * 4u : 0x7FFFFFF0u;
  __builtin_amdgcn_raw_buffer_store_b32(cnt, rn, uoff, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(edge, re, uoff, 0, 0);
}

// ---- per-row scan, one wave per unit ---------------------------------------------
//
// The launch form for many units (long contexts or large batches: more units
// than the work-group scan above has resident work-groups).  Every wave takes
// its own contiguous run of units and scores all 16 pages of a unit by itself
// through a four-deep register ring of half pages that runs across unit
// boundaries.  Per page, the partial head sums of its four token tiles are
// combined by rows_sum_scatter (associated as rows_sum, so the keys are the
// work-group scan's bits) so that lane l ends with the key of position
// 64p + l; after the unit's 16 pages the wave runs the local filter on its
// registers (wave_edge) and writes the candidates, count and edge
// (emit_wave).  No LDS and no work-group barrier after the row plan, and each
// unit's filter runs once, on the wave that scored it.
//
// FUSED: each wave quantises the queries of its row and the row's new key in
// registers.  A lane holds, per operand row, the 16-dim pieces 16g..16g+15 and
// 64+16g..64+16g+15; the other half of each 32-dim group lies 16 lanes away
// and the group whose scale the lane supplies to the MFMA (dims 32g..32g+31)
// was reduced 32 lanes away for g = 1, 2.  Exponent and conversion are the
// quantisers', so the codes are the bytes mxfp8_quant writes.

// The unit's edge: the work-group scan's filter_unit search on a wave's keys.
__device__ __forceinline__ uint32_t wave_edge(const Params& P, const Unit& U,
                                              const uint32_t (&k)[kUnitPages]) {
  const int ntok = (U.pg1 - U.pg0) * kPage;
  const uint32_t quota = unit_quota(U.t, P.topk);
  if (quota >= (uint32_t)ntok) return 0u;
  if (quota <= kTop3Quota) {
    uint32_t m[3];
    lane_top<3>(k, m);
    return key_floor<3>(m, quota);
  }
  if (quota <= kTop5Quota) {
    uint32_t m[5];
    lane_top<5>(k, m);
    return key_floor<5>(m, quota);
  }
  return key_floor<kUnitPages>(k, quota);
}

// MXFP8 codes (MFMA operand order) and the E8M0 byte of dims 32g..32g+31 of
// one operand row whose 32 bf16 values this lane holds as pieces: w[0..7]
// dims 16g..16g+15, w[8..15] dims 64+16g..64+16g+15 (g = lane/16).  Every
// lane of the wave must take part.  A row that is not live gets zero codes
// and scale byte 0.
__device__ __forceinline__ void quant_operand_row(const uint32_t (&w)[16], bool live, v8i& codes,
                                                  int& sbyte) {
  const int g = (threadIdx.x & 63) >> 4;
  int e[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[8 * p + j] & 0xFFFFu)),
                               fabsf(bf16_bits_to_f32(w[8 * p + j] >> 16))));
    // piece p is half of group p ? 2 + g/2 : g/2; the other half is 16 lanes away
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    e[p] = mx_exponent(amax);
  }
  // the lane supplies group g: lanes g = 0 and 3 reduced it themselves
  // (piece 0 and piece 1); g = 1 takes group 1 from g = 3 (its piece 0) and
  // g = 2 takes group 2 from g = 0 (its piece 1), 32 lanes away
  const int send = g < 2 ? e[1] : e[0];
  const int recv = __shfl_xor(send, 32);
  const int eg = g == 0 ? e[0] : (g == 3 ? e[1] : recv);
  sbyte = live ? eg + 127 : 0;
  int c[8];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float inv = pow2f(-e[p]);
    // |v * inv| <= 448 by the scale rule: the hardware conversion applies
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = w[8 * p + 2 * d], b = w[8 * p + 2 * d + 1];
      const uint32_t q = e4m3x4_in_range(bf16_bits_to_f32(a & 0xFFFFu) * inv, bf16_bits_to_f32(a >> 16) * inv,
                                         bf16_bits_to_f32(b & 0xFFFFu) * inv, bf16_bits_to_f32(b >> 16) * inv);
      c[4 * p + d] = live ? (int)q : 0;
    }
  }
  codes = v8i{c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]};
}

// The lane's two 16-dim pieces of a 128-dim bf16 row at byte offset `off` of
// the buffer behind `rsrc` (out of range: zeros).
__device__ __forceinline__ void load_pieces(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, uint32_t (&w)[16]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + (uint32_t)(2 * (64 * p + 16 * g) + 16 * j), 0, 0);
      w[8 * p + 4 * j] = v[0]; w[8 * p + 4 * j + 1] = v[1];
      w[8 * p + 4 * j + 2] = v[2]; w[8 * p + 4 * j + 3] = v[3];
    }
}

// Fused path, at the first unit of a row: the row's query operand from its
// bf16 queries, the head weights, and the row's new key as the key operand of
// a token tile whose 16 columns all carry it.  The wave holding the row's
// first unit writes the quantised queries to the workspace for the select's
// rescoring path.  Returns whether the row brings a new token.
template <int NHT>
__device__ __forceinline__ bool fused_row_regs(const Params& P, int row, int uir, QOperand<NHT>& Q,
                                               v8i& kn, int& ksn) {
  const int lane = threadIdx.x & 63, hr = lane & 15, g = lane >> 4;
  row = __builtin_amdgcn_readfirstlane(row);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.q_bf16 + (int64_t)row * P.H * kIdxDim), (short)0, P.H * kIdxDim * 2, kRawBufferWord3);
  const bool knew = has_new_token(P, row);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.k_new + (int64_t)row * kIdxDim), (short)0, knew ? kIdxDim * 2 : 0, kRawBufferWord3);
  uint32_t wq[NHT][16], wk[16];
#pragma unroll
  for (int i = 0; i < NHT; ++i) {
    const int h = 16 * i + hr;
    load_pieces(rq, h < P.H ? (uint32_t)(h * kIdxDim * 2) : 0x7FFFF000u, wq[i]);
  }
  load_pieces(rk, 0u, wk);
  quant_operand_row(wk, true, kn, ksn);
#pragma unroll
  for (int i = 0; i < NHT; ++i) quant_operand_row(wq[i], 16 * i + hr < P.H, Q.a[i], Q.s[i]);
  // the head weights after the raw queries are consumed (fewer live registers)
  load_w<NHT>(P, row, Q);
  if (uir == 0) {
#pragma unroll
    for (int i = 0; i < NHT; ++i) {
      const int h = 16 * i + hr;
      if (h < P.H) {
        uint8_t* dst = P.q_ws + ((int64_t)row * P.H + h) * kIdxDim;
        *reinterpret_cast<uint4*>(dst + 16 * g) =
            make_uint4((uint32_t)Q.a[i][0], (uint32_t)Q.a[i][1], (uint32_t)Q.a[i][2], (uint32_t)Q.a[i][3]);
        *reinterpret_cast<uint4*>(dst + 64 + 16 * g) =
            make_uint4((uint32_t)Q.a[i][4], (uint32_t)Q.a[i][5], (uint32_t)Q.a[i][6], (uint32_t)Q.a[i][7]);
        P.qs_ws[((int64_t)row * P.H + h) * 4 + g] = (uint8_t)Q.s[i];
      }
    }
  }
  return knew;
}

// ONE: the launch guarantees at most one unit per wave (the unit bound is
// within four per work-group), so there is no next unit to prefetch and no
// row change: fewer live registers through the scoring loop.
template <int NHT, bool FUSED, bool ONE>
__global__ __launch_bounds__(kScanThreads, 2) void indexer_wave_kernel(Params P) {
  __shared__ ScanSmem S;
  __shared__ typename std::conditional<FUSED, FusedSmem, NoSmem>::type F;
  const int scan_wgs = (int)gridDim.x - (FUSED ? P.extra_wgs : 0);
  if constexpr (FUSED) {
    if ((int)blockIdx.x >= scan_wgs) {
      write_new_tokens(P, scan_wgs);
      return;
    }
  }
  plan_rows<kScanThreads>(P, S);   // ends with a barrier
  const uint32_t U_total = S.rowpre[P.R];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nw = (uint32_t)scan_wgs * kScanWaves;
  const uint32_t per = (U_total + nw - 1) / nw;
  const uint32_t u_wg = (uint32_t)blockIdx.x * kScanWaves * per;   // wave 0's first unit
  if (u_wg >= U_total) return;   // no wave of the work-group has a unit (uniform)
  uint32_t u = u_wg + (uint32_t)wv * per;
  const uint32_t uend = min(U_total, u + per);
  const bool has = u < uend;
  bool bad = false;        // a page id out of the pool (flagged once at the end)
  Unit U = decode_unit(P, S, has ? u : u_wg);
  // fused: the slot of the wave's row's new token, requested first
  const int64_t nslot = FUSED ? P.new_slot[U.row] : -1;
  int32_t pid = unit_pages(P, U, S.rowseq[U.row]);
  QOperand<NHT> Q;
  v8i kn = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  int ksn = 0;
  // key of the row's new token, scored once per row; 0 when the row brings
  // none (no finite score has key 0).  One scalar through the loop.
  uint32_t nkey = 0u;
  HalfRegs b[kRing];
  bool ok[kRing];
  if constexpr (FUSED) {
    // The work-group quantises the rows of its waves' first units into LDS,
    // one row at a time (one 32-value group per thread; usually all four
    // waves start in one row), while the waves' rings are in flight; each
    // wave takes its operands from the copy of its row.  The work-group that
    // holds a row's first unit writes the row's quantised queries to the
    // workspace for the select.
    // The first row's inputs and the head weights are requested before the
    // ring, so waiting for them never waits for the ring.
    // Issued by every wave (one without a unit gets page id -1 loads that
    // move nothing): conditional loads would leave the compiler's wait
    // counts inexact, and the waits below would then wait for the ring.
    RowIn in;
    row_in_load(P, decode_unit(P, S, u_wg).row, in);
    load_w<NHT>(P, U.row, Q);
    __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the ring's
    {
      Unit Ur = U;
      if (!has) Ur.t = -1;
#pragma unroll
      for (int k = 0; k < kRing; ++k) ok[k] = fetch_half(P, Ur, pid, k, b[k], &bad);
    }
    for (int w = 0; w < kScanWaves; ++w) {   // uniform over the work-group
      const uint32_t uw = u_wg + (uint32_t)w * per;
      if (uw >= U_total) break;
      const Unit Uw = decode_unit(P, S, uw);
      bool seen = false;                     // an earlier wave starts in this row
      for (int w2 = 0; w2 < w; ++w2) seen |= decode_unit(P, S, u_wg + (uint32_t)w2 * per).row == Uw.row;
      if (seen) continue;
      if (w > 0) row_in_load(P, Uw.row, in);
      row_in_store(in, F);
      __syncthreads();
      if (Uw.uir == 0) {
        const int t = threadIdx.x;
        if (t * 32 < P.H * kIdxDim) {
          uint4* dst = reinterpret_cast<uint4*>(P.q_ws + (int64_t)Uw.row * P.H * kIdxDim + t * 32);
          const uint4* src = reinterpret_cast<const uint4*>(F.qc + t * 32);
          dst[0] = src[0];
          dst[1] = src[1];
        }
        if (t < P.H * 4) P.qs_ws[(int64_t)Uw.row * P.H * 4 + t] = F.qsc[t];
      }
      if (has && U.row == Uw.row) {
        load_q_codes_lds<NHT>(F, Q);
        const int g = lane >> 4;
        const uint4 lo = *reinterpret_cast<const uint4*>(F.kc + 16 * g);
        const uint4 hi = *reinterpret_cast<const uint4*>(F.kc + 64 + 16 * g);
        kn = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        ksn = (int)F.ksc[g];
      }
      __syncthreads();   // every wave has its copy before the next row overwrites it
    }
    if (!has) return;    // no barrier follows
    if (nslot >= 0 && nslot < P.pool_pages * kPage)
      nkey = __builtin_amdgcn_readfirstlane(score_key(rows_sum(head_part<NHT>(Q, kn, ksn))));
  } else {
    if (!has) return;
#pragma unroll
    for (int k = 0; k < kRing; ++k) ok[k] = fetch_half(P, U, pid, k, b[k], &bad);
    load_q<NHT>(P, U.row, Q);
  }
  int qrow = U.row;
  for (;;) {
    const bool more = !ONE && u + 1 < uend;
    // the next unit (the current one again when there is none: its ring
    // loads then get page id -1 and move nothing).  Fused: a next unit of
    // another row is not prefetched either; its ring is issued after that
    // row's quantisation.
    const Unit V = ONE ? U : decode_unit(P, S, more ? u + 1 : u);
    const int32_t pidn = ONE ? pid : unit_pages(P, V, S.rowseq[V.row]);
    Unit Vf = V;
    if (!more || (FUSED && V.row != U.row)) Vf.t = -1;
    uint32_t key[kUnitPages];
#pragma unroll
    for (int pi = 0; pi < kUnitPages; ++pi) {
      float part[4];
      bool pok = false;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * pi + hh, sl = h % kRing;
        pok = ok[sl];   // both halves of a page are present or absent together
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint4 lo = b[sl].d[2 * jj], hi = b[sl].d[2 * jj + 1];
          const v8i kb = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          part[2 * hh + jj] = head_part<NHT>(Q, kb, (int)b[sl].s[jj]);
        }
        const int hn = h + kRing;
        if (hn < 2 * kUnitPages)
          ok[sl] = fetch_half(P, U, pid, hn, b[sl], &bad);
        else if (!ONE)
          ok[sl] = fetch_half(P, Vf, pidn, hn - 2 * kUnitPages, b[sl], &bad);
      }
      // lane group j receives token tile j: lane l holds position 64p + l
      const float sc = rows_sum_scatter(part);
      const int pos = (U.pg0 + pi) * kPage + lane;
      key[pi] = pok && pos <= U.t ? score_key(sc) : 0u;
    }
    if constexpr (FUSED) {
      // the new token's key, when it lies in this unit, from the wave's own
      // quantisation (the cache slot at t is written by this launch); a key
      // of 0 (the page is absent) stays 0
      const int tl = U.t - U.pg0 * kPage;
      if (nkey != 0u && tl >= 0 && U.t < U.pg1 * kPage) {
#pragma unroll
        for (int pi = 0; pi < kUnitPages; ++pi)
          if (pi == (tl >> 6) && lane == (tl & 63) && key[pi] != 0u) key[pi] = nkey;
      }
    }
    emit_wave(P, U.row, true, row_pages(U.t, P.bt_stride), U.uir, key, wave_edge(P, U, key));
    if (ONE || !more) break;
    if (V.row != qrow) {
      if constexpr (FUSED) {
        const bool knew = fused_row_regs<NHT>(P, V.row, V.uir, Q, kn, ksn);
        nkey = knew ? __builtin_amdgcn_readfirstlane(score_key(rows_sum(head_part<NHT>(Q, kn, ksn)))) : 0u;
#pragma unroll
        for (int k = 0; k < kRing; ++k) ok[k] = fetch_half(P, V, pidn, k, b[k], &bad);
      } else {
        load_q<NHT>(P, V.row, Q);
      }
      qrow = V.row;
    }
    U = V;
    pid = pidn;
    ++u;
  }
  if (bad && lane == 0) flag_error(P.hdr, kErrBadPage);
}

// ---- multi-query decode, one wave per (row group, unit) --------------------------
//
// A tile is the P.tile_rows consecutive rows of one sequence; it is cut into
// groups of up to kMqRows rows.  A wave
// takes one unit of one group: it streams the unit's 16 pages once through
// the per-row scan's register ring (the pages of the group's longest row)
// and scores every page for each row of the group with that row's query
// operand.  Every row's keys come from the per-row scan's operations in the
// same order (head_part, rows_sum_scatter), with the row's own causal limit;
// the row's filter and candidate stores follow the unit, for units within
// the row's own length.  The group reads the pages of its tile's first row's
// sequence; a group whose rows name another sequence sets kErrMixedTile.
// Two rows per wave fit two waves per SIMD (four rows per wave need one
// wave per SIMD, whose scoring chains then go unhidden: 43% slower), with
// three half pages in flight (a fourth does not fit beside the pipelined
// scoring's operands without spilling).
constexpr int kMqRows = 2;
constexpr int kMqRing = 3;
template <int NHT>
__global__ __launch_bounds__(kScanThreads, 2) void indexer_mq_wave_kernel(Params P) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int TR = P.tile_rows;
  const int gpt = (TR + kMqRows - 1) / kMqRows;         // groups per tile
  const int ntiles = (P.R + TR - 1) / TR;
  const uint32_t item = (uint32_t)blockIdx.x * kScanWaves + (uint32_t)wv;
  if (item >= (uint32_t)(ntiles * gpt) * (uint32_t)P.upr) return;
  // the groups of one unit are neighbouring waves (one work-group when the
  // tile has four groups or fewer), so they request the same pages together
  const int sub = (int)(item % (uint32_t)gpt);
  const uint32_t tu = item / (uint32_t)gpt;
  const int tile = (int)(tu / (uint32_t)P.upr), uir = (int)(tu % (uint32_t)P.upr);
  const int rt = tile * TR;                              // the tile's first row
  const int r0 = rt + sub * kMqRows;                     // the group's rows r0, r0 + 1
  const int nr = min(min(kMqRows, TR - sub * kMqRows), P.R - r0);   // 1 or 2
  if (nr <= 0) return;   // past the rows of a partial last tile (uniform)
  // lane j < nr: row r0 + j's position and sequence
  const int t_l = lane < nr ? P.row_pos[r0 + lane] : -1;
  int seq = 0;
  bool mixed = false;
  if (P.row_seq) {
    seq = __builtin_amdgcn_readfirstlane(P.row_seq[rt]);
    const int s_l = lane < nr ? P.row_seq[r0 + lane] : seq;
    mixed = __builtin_amdgcn_ballot_w64(s_l != seq) != 0;
  }
  const int ta = __builtin_amdgcn_readlane(t_l, 0);
  const int tb = nr > 1 ? __builtin_amdgcn_readlane(t_l, 1) : -1;
  const Unit U = row_unit(P, r0, max(ta, tb), uir);   // the pages of the group's longer row
  if (uir >= U.units_r) return;                       // past the group's pages (uniform)
  bool bad = false;
  const int32_t pid = unit_pages(P, U, seq);
  HalfRegs b[kMqRing];
  bool ok[kMqRing];
#pragma unroll
  for (int k = 0; k < kMqRing; ++k) ok[k] = fetch_half(P, U, pid, k, b[k], &bad);
  // a group of one row scores that row twice (the second copy is not kept):
  // every load and MFMA is issued on every path
  QOperand<NHT> Qa, Qb;
  load_q<NHT>(P, r0, Qa);
  load_q<NHT>(P, r0 + nr - 1, Qb);
  uint32_t ka[kUnitPages], kb[kUnitPages];
#pragma unroll
  for (int pi = 0; pi < kUnitPages; ++pi) {
    const bool pok = ok[(2 * pi) % kMqRing];   // both halves of a page are present or absent together
    // token tile j of the page: half j/2 (ring slot (2pi + j/2) % kMqRing), tile j%2
    auto operand = [&](int j, v8i& kv, int& ks) {
      const int sl = (2 * pi + (j >> 1)) % kMqRing, jj = j & 1;
      const uint4 lo = b[sl].d[2 * jj], hi = b[sl].d[2 * jj + 1];
      kv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      ks = (int)b[sl].s[jj];
    };
    // 2*NHT MFMAs per token tile (m < NHT: row a's head tile m, else row b's
    // head tile m - NHT), software-pipelined:
    // MFMA m+1, or the next token tile's first, is issued before the FMA
    // chain reads MFMA m.  Per row and token tile the chain is head_part's.
    constexpr int kM = 2 * NHT;
    float pa[4], pb[4];
    v8i kc, kn;
    int sc, sn = 0;
    operand(0, kc, sc);
    v4f cur = head_mfma(Qa, 0, kc, sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pa[j] = pb[j] = 0.f;
      if (j + 1 < 4) operand(j + 1, kn, sn);
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        v4f nxt = cur;
        if (m + 1 < NHT) nxt = head_mfma(Qa, m + 1, kc, sc);
        else if (m + 1 < kM) nxt = head_mfma(Qb, m + 1 - NHT, kc, sc);
        else if (j + 1 < 4) nxt = head_mfma(Qa, 0, kn, sn);
        if (m < NHT) pa[j] = head_acc(Qa, m, cur, pa[j]);
        else pb[j] = head_acc(Qb, m - NHT, cur, pb[j]);
        cur = nxt;
      }
      kc = kn;
      sc = sn;
      if (j & 1) {
        // both token tiles of half j/2 are taken: its slot takes the half
        // kMqRing ahead
        const int h = 2 * pi + (j >> 1), hn = h + kMqRing;
        if (hn < 2 * kUnitPages) ok[h % kMqRing] = fetch_half(P, U, pid, hn, b[h % kMqRing], &bad);
      }
    }
    // lane group g receives token tile g: lane l holds position 64p + l
    const float sa = rows_sum_scatter(pa), sb = rows_sum_scatter(pb);
    const int pos = (U.pg0 + pi) * kPage + lane;
    ka[pi] = pok && pos <= ta ? score_key(sa) : 0u;
    kb[pi] = pok && pos <= tb ? score_key(sb) : 0u;
  }
  {
    const Unit Ua = row_unit(P, r0, ta, uir);
    emit_wave(P, r0, true, row_pages(ta, P.bt_stride), uir, ka, uir < Ua.units_r ? wave_edge(P, Ua, ka) : 0u);
  }
  if (nr > 1) {   // uniform
    const Unit Ub = row_unit(P, r0 + 1, tb, uir);
    emit_wave(P, r0 + 1, true, row_pages(tb, P.bt_stride), uir, kb, uir < Ub.units_r ? wave_edge(P, Ub, kb) : 0u);
  }
  if (lane == 0) {
    if (bad) flag_error(P.hdr, kErrBadPage);
    if (mixed) flag_error(P.hdr, kErrMixedTile);
  }
}

// ---- host side ----------------------------------------------------------------

struct Layout {
  size_t hdr, ucount, uedge, cand, qcodes, qscales, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int units_stride(int64_t bt_stride) { return (int)((bt_stride + kUnitPages - 1) / kUnitPages); }

Layout layout_for(int64_t rows, int64_t bt_stride) {
  Layout L;
  const int64_t upr = units_stride(bt_stride);
  size_t off = 0;
  L.hdr = off; off += 256;
  L.ucount = off; off += align256((size_t)rows * upr * 4);
  L.uedge = off; off += align256((size_t)rows * upr * 4);
  L.cand = off; off += align256((size_t)rows * bt_stride * kPage * 8);
  // the quantised queries of the fused-prolog entry point (for the select's
  // rescoring path), sized for the largest head count
  L.qcodes = off; off += align256((size_t)rows * DSA_MAX_INDEX_HEADS * kIdxDim);
  L.qscales = off; off += align256((size_t)rows * DSA_MAX_INDEX_HEADS * 4);
  L.total = off;
  return L;
}

enum KernelKind { kScan = 0, kSelect = 1, kDump = 2, kSelectShort = 3, kScanFused = 4, kWave = 5,
                  kWaveFused = 6, kWaveOne = 7, kWaveOneFused = 8 };

template <int NHT>
void* pick_kernel_t(KernelKind kind) {
  switch (kind) {
    case kScan: return (void*)&indexer_scan_kernel<NHT, false>;
    case kScanFused: return (void*)&indexer_scan_kernel<NHT, true>;
    case kWave: return (void*)&indexer_wave_kernel<NHT, false, false>;
    case kWaveFused: return (void*)&indexer_wave_kernel<NHT, true, false>;
    case kWaveOne: return (void*)&indexer_wave_kernel<NHT, false, true>;
    case kWaveOneFused: return (void*)&indexer_wave_kernel<NHT, true, true>;
    case kSelect: return (void*)&indexer_select_kernel<NHT, false>;
    case kSelectShort: return (void*)&indexer_select_kernel<NHT, true>;
    default: return (void*)&indexer_dump_kernel<NHT>;
  }
}

void* pick_kernel(int nht, KernelKind kind) {
  switch (nht) {
    case 1: return pick_kernel_t<1>(kind);
    case 2: return pick_kernel_t<2>(kind);
    case 3: return pick_kernel_t<3>(kind);
    default: return pick_kernel_t<4>(kind);
  }
}

void* pick_mq_wave_kernel(int nht) {
  switch (nht) {
    case 1: return (void*)&indexer_mq_wave_kernel<1>;
    case 2: return (void*)&indexer_mq_wave_kernel<2>;
    case 3: return (void*)&indexer_mq_wave_kernel<3>;
    default: return (void*)&indexer_mq_wave_kernel<4>;
  }
}

// resident workgroups of a kernel on the current device, cached per device
// and kernel slot.  Entries are atomics: two host threads that miss at the
// same time both compute the same value and store it, so no lock is needed
// and a reader never sees a torn value (0 = not computed yet).
constexpr int kCapDevices = 64;
constexpr int kCapSlots = 40;
std::atomic<int> g_capacity[kCapDevices][kCapSlots];

int resident_capacity(void* fn, int slot, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cache = dev >= 0 && dev < kCapDevices && slot >= 0 && slot < kCapSlots;
  if (cache) {
    const int c = g_capacity[dev][slot].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                   threads, 0) != hipSuccess)
    return -1;
  const int cap = std::max(1, per_cu) * prop.multiProcessorCount;
  if (cache) g_capacity[dev][slot].store(cap, std::memory_order_relaxed);
  return cap;
}

int validate(const void* q, const void* qs, const float* w, const void* kpool, int64_t pool_pages,
             const int32_t* bt, int32_t bt_stride, const int32_t* row_seq, const int32_t* row_pos,
             int32_t R, int32_t H) {
  if (!q || !qs || !w || !kpool || !bt || !row_seq || !row_pos) return DSA_ERR_INVALID_ARG;
  if (R < 0 || bt_stride <= 0 || pool_pages <= 0) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > DSA_MAX_INDEX_HEADS) return DSA_ERR_UNSUPPORTED;
  if (bt_stride > kMaxBtStride) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

int run(Params P, bool dump, hipStream_t stream, bool fused = false) {
  const int nht = (P.H + 15) / 16;
  const KernelKind kind = dump ? kDump : fused ? kScanFused : kScan;
  void* scan = pick_kernel(nht, kind);
  void* sel = pick_kernel(nht, P.j_start > 1 ? kSelectShort : kSelect);
  const int scan_threads = dump ? kThreads : kScanThreads;
  const int cap = resident_capacity(scan, fused ? 20 + nht - 1 : (nht - 1) * 3 + (int)kind,
                                    scan_threads);
  if (cap <= 0) return DSA_ERR_HIP;
  const int R = P.R;
  const int upr = units_stride(P.bt_stride);
  // Launches with more units than the work-group scan has resident
  // work-groups (bounded by rows x the block table's units) take the
  // one-wave-per-unit scan; smaller ones keep four waves on every unit.
  void* wave = pick_kernel(nht, fused ? kWaveFused : kWave);
  void* wave1 = pick_kernel(nht, fused ? kWaveOneFused : kWaveOne);
  const int wave_cap = dump ? 0 : resident_capacity(wave, (fused ? 28 : 24) + nht - 1, kScanThreads);
  const int wave1_cap = dump ? 0 : resident_capacity(wave1, (fused ? 36 : 32) + nht - 1, kScanThreads);
  if (!dump && (wave_cap <= 0 || wave1_cap <= 0)) return DSA_ERR_HIP;
  for (int r0 = 0; r0 < R; r0 += kMaxRows) {
    Params Q = P;
    const int rn = std::min(kMaxRows, R - r0);
    Q.R = rn;
    Q.w = P.w + (int64_t)r0 * P.H;
    Q.row_seq = P.row_seq + r0;
    Q.row_pos = P.row_pos + r0;
    if (fused) {
      // the quantised queries live in the workspace, sized for one launch's
      // rows: every launch uses it from its start (launches are stream-ordered)
      Q.q_bf16 = P.q_bf16 + (int64_t)r0 * P.H * kIdxDim;
      Q.k_new = P.k_new + (int64_t)r0 * kIdxDim;
      Q.kv_new = P.kv_new + (int64_t)r0 * kQK;
      Q.new_slot = P.new_slot + r0;
    } else {
      Q.q = P.q + (int64_t)r0 * P.H * kIdxDim;
      Q.qs = P.qs + (int64_t)r0 * P.H * 4;
    }
    if (dump) {
      Q.dump = P.dump + (int64_t)r0 * P.ld;
    } else {
      Q.out_idx = P.out_idx + (int64_t)r0 * P.topk;
      Q.out_score = P.out_score ? P.out_score + (int64_t)r0 * P.topk : nullptr;
    }
    const int64_t units = (int64_t)rn * upr;
    const bool by_wave = !dump && units > cap;
    // a unit per wave at most: the grid has a wave for every unit the block
    // table allows
    const bool one = by_wave && units <= (int64_t)kScanWaves * wave1_cap;
    const int64_t G = one ? (units + kScanWaves - 1) / kScanWaves
                    : by_wave ? std::min<int64_t>((int64_t)wave_cap, (units + kScanWaves - 1) / kScanWaves)
                              : std::min<int64_t>((int64_t)cap, units);
    Q.extra_wgs = fused ? (rn + kScanWaves - 1) / kScanWaves : 0;
    void* args[] = {&Q};
    if (hipLaunchKernel(one ? wave1 : by_wave ? wave : scan, dim3((unsigned)(G + Q.extra_wgs)),
                        dim3(scan_threads), args, 0, stream) != hipSuccess)
      return DSA_ERR_HIP;
    if (!dump && hipLaunchKernel(sel, dim3((unsigned)rn), dim3(kSelThreads), args, 0, stream) != hipSuccess)
      return DSA_ERR_HIP;
  }
  return DSA_OK;
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

Params base_params(const void* q_fp8, const void* q_e8m0, const float* w, const void* k_pool,
                   int64_t pool_pages, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* row_seq, const int32_t* row_pos, int32_t R, int32_t H_I) {
  Params P{};
  P.q = static_cast<const uint8_t*>(q_fp8);
  P.qs = static_cast<const uint8_t*>(q_e8m0);
  P.w = w;
  P.kpool = static_cast<const uint8_t*>(k_pool);
  P.pool_pages = pool_pages;
  P.bt = block_table;
  P.bt_stride = bt_stride;
  P.row_seq = row_seq;
  P.row_pos = row_pos;
  P.R = R;
  P.H = H_I;
  P.upr = units_stride(bt_stride);
  P.tile_rows = kTileRows;
  P.j_start = 1;
  return P;
}

// The select's first layout for rows of up to bt_stride pages: every such
// row keeps at least min(quota, unit size) candidates in its fullest unit,
// and the quota only grows as rows get shorter, so the longest possible
// row's quota is a lower bound for all of them; smaller layouts would be
// tried and abandoned.  Taken only when that bound already asks for 8 or
// more 64-slot groups per unit (rows of up to about 10K positions at
// K = 2048: decode 8K, batch 1, 25.4 -> 23.8 us per call).  With a looser
// bound most rows still need a larger layout than the first one tried, and
// a failed runtime-layout attempt costs more than a failed first-layout one
// (ragged decode of 4K-64K rows, bound 2: 47.2 -> 47.7 us), so those
// launches keep the regular order (returns 1).
int select_j_start(int32_t bt_stride, int32_t topk) {
  const int64_t n_max = (int64_t)bt_stride * kPage;
  if (n_max <= topk) return 1;
  const uint32_t q = unit_quota((int)(n_max - 1), topk);
  int J = 1;
  while (64u * (uint32_t)J < q && J < 2 * kFastPer) J *= 2;
  const int64_t units = (n_max + kUnitTok - 1) / kUnitTok;
  return (J >= 8 && 64u * (uint32_t)J >= q && units <= kFastUnits / J) ? J : 1;
}

}  // namespace

extern "C" size_t dsa_indexer_topk_workspace_size(int32_t R, int32_t bt_stride, int32_t H_I,
                                                  int32_t topk) {
  (void)H_I;
  (void)topk;
  if (R <= 0 || bt_stride <= 0) return 256;
  const int64_t rows = std::min<int64_t>(R, kMaxRows);
  return layout_for(rows, bt_stride).total;
}

namespace {

// dsa_indexer_topk after argument validation, on a workspace of `ws_bytes`
// bytes (from the caller, or the library's static scratch array).
int indexer_topk_on(const void* q_fp8, const void* q_e8m0, const float* w, const void* k_pool,
                    int64_t pool_pages, const int32_t* block_table, int32_t bt_stride,
                    const int32_t* row_seq, const int32_t* row_pos, int32_t R, int32_t H_I,
                    int32_t topk, int32_t* out_idx, float* out_score, uint8_t* ws,
                    const Layout& L, void* stream) {
  Params P = base_params(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                         row_pos, R, H_I);
  P.topk = topk;
  P.out_idx = out_idx;
  P.out_score = out_score;
  P.hdr = reinterpret_cast<uint32_t*>(ws + L.hdr);
  P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
  P.uedge = reinterpret_cast<uint32_t*>(ws + L.uedge);
  P.cand = reinterpret_cast<uint2*>(ws + L.cand);
  P.j_start = select_j_start(bt_stride, topk);
  return run(P, false, dsa_host::as_stream(stream));
}

int indexer_topk_checks(const void* q_fp8, const void* q_e8m0, const float* w, const void* k_pool,
                        int64_t pool_pages, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* row_seq, const int32_t* row_pos, int32_t R, int32_t H_I,
                        int32_t topk, const int32_t* out_idx) {
  const int st = validate(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                          row_pos, R, H_I);
  if (st != DSA_OK) return st;
  if (out_idx == nullptr) return DSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// ---- the allocation-free variant's workspace ---------------------------------
//
// A file-scope device array holds the workspace of dsa_indexer_topk_noalloc:
// each GPU the library runs on holds its own copy until the process ends.
// Host code must not use the array's name as a device address (it is a
// host-side stand-in); the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and is kept per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];

// Device address of this device's scratch array (nullptr if the lookup
// failed or the device index is out of range).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int dsa_indexer_topk(const void* q_fp8, const void* q_e8m0, const float* w,
                                const void* k_pool, int64_t pool_pages, const int32_t* block_table,
                                int32_t bt_stride, const int32_t* row_seq, const int32_t* row_pos,
                                int32_t R, int32_t H_I, int32_t topk, int32_t* out_idx,
                                float* out_score, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const int st = indexer_topk_checks(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride,
                                     row_seq, row_pos, R, H_I, topk, out_idx);
  if (st != DSA_OK) return st;
  if (R == 0) return DSA_OK;
  const Layout L = layout_for(std::min<int64_t>(R, kMaxRows), bt_stride);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  return indexer_topk_on(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                         row_pos, R, H_I, topk, out_idx, out_score, static_cast<uint8_t*>(workspace),
                         L, stream);
}

extern "C" int dsa_indexer_topk_noalloc(const void* q_fp8, const void* q_e8m0, const float* w,
                                        const void* k_pool, int64_t pool_pages,
                                        const int32_t* block_table, int32_t bt_stride,
                                        const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                                        int32_t H_I, int32_t topk, int32_t* out_idx,
                                        float* out_score, void* stream) {
  const int st = indexer_topk_checks(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride,
                                     row_seq, row_pos, R, H_I, topk, out_idx);
  if (st != DSA_OK) return st;
  if (R == 0) return DSA_OK;
  const Layout L = layout_for(std::min<int64_t>(R, kMaxRows), bt_stride);
  if (L.total > kNoAllocScratchBytes) return DSA_ERR_WORKSPACE;
  void* ptr = scratch_on_current_device();
  if (ptr == nullptr) return DSA_ERR_HIP;
  return indexer_topk_on(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                         row_pos, R, H_I, topk, out_idx, out_score, static_cast<uint8_t*>(ptr), L,
                         stream);
}

extern "C" int dsa_decode_indexer_topk(const void* q_bf16, const float* w, const void* k_new_bf16,
                                       const void* kv_new_bf16, const int64_t* slot_mapping,
                                       void* k_pool, void* kv_pool, int64_t pool_pages,
                                       const int32_t* block_table, int32_t bt_stride,
                                       const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                                       int32_t H_I, int32_t topk, int32_t* out_idx,
                                       float* out_score, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!q_bf16 || !k_new_bf16 || !kv_new_bf16 || !slot_mapping || !kv_pool)
    return DSA_ERR_INVALID_ARG;
  // (q_bf16 stands in for the quantised-query arguments in the shared checks)
  const int st = indexer_topk_checks(q_bf16, q_bf16, w, k_pool, pool_pages, block_table, bt_stride,
                                     row_seq, row_pos, R, H_I, topk, out_idx);
  if (st != DSA_OK) return st;
  if (pool_pages > (int64_t(1) << 25)) return DSA_ERR_UNSUPPORTED;   // slots fit the kernels' int math
  if (R == 0) return DSA_OK;
  const Layout L = layout_for(std::min<int64_t>(R, kMaxRows), bt_stride);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Params P = base_params(ws + L.qcodes, ws + L.qscales, w, k_pool, pool_pages, block_table,
                         bt_stride, row_seq, row_pos, R, H_I);
  P.topk = topk;
  P.out_idx = out_idx;
  P.out_score = out_score;
  P.hdr = reinterpret_cast<uint32_t*>(ws + L.hdr);
  P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
  P.uedge = reinterpret_cast<uint32_t*>(ws + L.uedge);
  P.cand = reinterpret_cast<uint2*>(ws + L.cand);
  P.j_start = select_j_start(bt_stride, topk);
  P.q_bf16 = static_cast<const uint16_t*>(q_bf16);
  P.k_new = static_cast<const uint16_t*>(k_new_bf16);
  P.kv_new = static_cast<const uint16_t*>(kv_new_bf16);
  P.new_slot = slot_mapping;
  P.kpool_w = static_cast<uint8_t*>(k_pool);
  P.kvpool_w = static_cast<uint8_t*>(kv_pool);
  P.q_ws = ws + L.qcodes;
  P.qs_ws = ws + L.qscales;
  return run(P, false, dsa_host::as_stream(stream), true);
}

extern "C" int dsa_indexer_scores(const void* q_fp8, const void* q_e8m0, const float* w,
                                  const void* k_pool, int64_t pool_pages,
                                  const int32_t* block_table, int32_t bt_stride,
                                  const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                                  int32_t H_I, float* out_scores, int64_t ld, void* stream) {
  int st = validate(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq, row_pos,
                    R, H_I);
  if (st != DSA_OK) return st;
  if (out_scores == nullptr || ld <= 0) return DSA_ERR_INVALID_ARG;
  if (R == 0) return DSA_OK;
  hipStream_t s = dsa_host::as_stream(stream);
  const int64_t n = (int64_t)R * ld;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)), dim3(256), 0, s,
                     out_scores, n, -__builtin_huge_valf());
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  Params P = base_params(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                         row_pos, R, H_I);
  P.topk = 1;
  P.dump = out_scores;
  P.ld = ld;
  P.hdr = nullptr;   // the score dump uses no workspace
  return run(P, true, s);
}

// Rows per launch of dsa_indexer_topk_seq: at most kSeqChunkRows, a multiple
// of the tile height, and within kSeqCandBytes of candidate region.
int seq_rows_per_launch(int64_t R, int64_t n_pages) {
  const int64_t per_row = n_pages * kPage * 8;
  const int64_t fit = std::max<int64_t>(kTileRows, kSeqCandBytes / per_row / kTileRows * kTileRows);
  return (int)std::min<int64_t>(std::min<int64_t>(R, kSeqChunkRows), fit);
}

extern "C" size_t dsa_indexer_topk_seq_workspace_size(int32_t R, int32_t n_pages, int32_t H_I,
                                                      int32_t topk) {
  (void)H_I;
  (void)topk;
  if (R <= 0 || n_pages <= 0) return 256;
  return layout_for(seq_rows_per_launch(R, n_pages), n_pages).total;
}

extern "C" int dsa_indexer_topk_seq(const void* q_fp8, const void* q_e8m0, const float* w,
                                    const void* k_pool, int64_t pool_pages,
                                    const int32_t* block_table_row, int32_t n_pages,
                                    const int32_t* row_pos, int32_t R, int32_t H_I, int32_t topk,
                                    int32_t* out_idx, float* out_score, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!q_fp8 || !q_e8m0 || !w || !k_pool || !block_table_row || !row_pos || !out_idx)
    return DSA_ERR_INVALID_ARG;
  if (R < 0 || n_pages <= 0 || pool_pages <= 0) return DSA_ERR_INVALID_ARG;
  if (H_I < 1 || H_I > DSA_MAX_INDEX_HEADS) return DSA_ERR_UNSUPPORTED;
  if (n_pages > kTileMaxPages) return DSA_ERR_UNSUPPORTED;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (R == 0) return DSA_OK;
  const int per_launch = seq_rows_per_launch(R, n_pages);
  const Layout L = layout_for(per_launch, n_pages);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = dsa_host::as_stream(stream);
  const int nht = (H_I + 15) / 16;
  void* mk = pick_mq_wave_kernel(nht);
  void* sel = pick_kernel(nht, kSelect);
  const int64_t upr = units_stride(n_pages);
  for (int r0 = 0; r0 < R; r0 += per_launch) {
    const int rn = std::min(per_launch, R - r0);
    Params P = base_params(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table_row, n_pages, nullptr,
                           row_pos + r0, rn, H_I);
    P.q += (int64_t)r0 * H_I * kIdxDim;
    P.qs += (int64_t)r0 * H_I * 4;
    P.w += (int64_t)r0 * H_I;
    P.topk = topk;
    P.out_idx = out_idx + (int64_t)r0 * topk;
    P.out_score = out_score ? out_score + (int64_t)r0 * topk : nullptr;
    P.hdr = reinterpret_cast<uint32_t*>(ws + L.hdr);
    P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
    P.uedge = reinterpret_cast<uint32_t*>(ws + L.uedge);
    P.cand = reinterpret_cast<uint2*>(ws + L.cand);
    // the rows in tiles of kTileRows, one wave per (pair of rows, unit) as
    // for multi-query decode; every row reads the one block-table row
    // (chunked prefill 8192 x 131072: 8.35 -> 7.80 ms per call against the
    // row-tiled kernel that shared each page through LDS)
    P.tile_rows = kTileRows;
    const int64_t items = (rn + kTileRows - 1) / kTileRows * (kTileRows / kMqRows) * upr;
    void* args[] = {&P};
    if (hipLaunchKernel(mk, dim3((unsigned)((items + kScanWaves - 1) / kScanWaves)), dim3(kScanThreads),
                        args, 0, s) != hipSuccess)
      return DSA_ERR_HIP;
    if (hipLaunchKernel(sel, dim3((unsigned)rn), dim3(kSelThreads), args, 0, s) != hipSuccess)
      return DSA_ERR_HIP;
  }
  return DSA_OK;
}

extern "C" int dsa_indexer_topk_mq(const void* q_fp8, const void* q_e8m0, const float* w,
                                   const void* k_pool, int64_t pool_pages,
                                   const int32_t* block_table, int32_t bt_stride,
                                   const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                                   int32_t q_per_seq, int32_t H_I, int32_t topk,
                                   int32_t* out_idx, float* out_score, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  int st = validate(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq, row_pos,
                    R, H_I);
  if (st != DSA_OK) return st;
  if (out_idx == nullptr) return DSA_ERR_INVALID_ARG;
  if (q_per_seq < 1 || q_per_seq > kTileRows) return DSA_ERR_UNSUPPORTED;
  if (R % q_per_seq != 0) return DSA_ERR_INVALID_ARG;
  if (bt_stride > kTileMaxPages) return DSA_ERR_UNSUPPORTED;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (R == 0) return DSA_OK;
  const int64_t rows = std::min<int64_t>(R, kMaxRows);
  const Layout L = layout_for(rows, bt_stride);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = dsa_host::as_stream(stream);
  const int nht = (H_I + 15) / 16;
  void* mk = pick_mq_wave_kernel(nht);
  void* sel = pick_kernel(nht, kSelect);
  const int upr = units_stride(bt_stride);
  const int step = kMaxRows - kMaxRows % q_per_seq;   // whole sequences per launch
  for (int r0 = 0; r0 < R; r0 += step) {
    const int rn = std::min(step, R - r0);
    Params P = base_params(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride,
                           row_seq + r0, row_pos + r0, rn, H_I);
    P.q += (int64_t)r0 * H_I * kIdxDim;
    P.qs += (int64_t)r0 * H_I * 4;
    P.w += (int64_t)r0 * H_I;
    P.topk = topk;
    P.out_idx = out_idx + (int64_t)r0 * topk;
    P.out_score = out_score ? out_score + (int64_t)r0 * topk : nullptr;
    P.hdr = reinterpret_cast<uint32_t*>(ws + L.hdr);
    P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
    P.uedge = reinterpret_cast<uint32_t*>(ws + L.uedge);
    P.cand = reinterpret_cast<uint2*>(ws + L.cand);
    const int64_t ntiles = rn / q_per_seq;
    P.tile_rows = q_per_seq;
    void* args[] = {&P};
    // one wave per (pair of rows, unit) (decode 128K x 8, four rows per
    // sequence: 60.7-62.5 -> 56.0-57.2 us per call against the row-tiled
    // kernel's tiles; eight rows per sequence: 100.2-102.8 -> 94.6-95.4 us)
    const int64_t items = ntiles * ((q_per_seq + kMqRows - 1) / kMqRows) * upr;
    if (hipLaunchKernel(mk, dim3((unsigned)((items + kScanWaves - 1) / kScanWaves)), dim3(kScanThreads),
                        args, 0, s) != hipSuccess)
      return DSA_ERR_HIP;
    if (hipLaunchKernel(sel, dim3((unsigned)rn), dim3(kSelThreads), args, 0, s) != hipSuccess)
      return DSA_ERR_HIP;
  }
  return DSA_OK;
}
