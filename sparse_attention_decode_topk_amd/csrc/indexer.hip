// Lightning Indexer: scoring, head weighting and Top-K fused in one kernel
// over the paged MXFP8 K cache, with no score matrix written to HBM ("Deep
// Dive into Sparse Attention ...", section "1. Computation Optimization ...
// DSA Fused Kernel"; Kimi K3.1 Pro Day0 page, "Lightning Indexer
// Three-Stream Coordination": scoring, head weighting and Top-K selection
// fused, with selection pipelined with the paged K-cache reads).
//
//   I(t,s) = sum_h w[r,h] * max(0, q[r,h] . k[s]),  s <= t = row_pos[r]
//
// Work decomposition (one ordinary launch; no grid barrier, no spinning):
//  * every row's causal history is cut into units of 16 pages (1024
//    tokens); units are numbered row by row and handed out in that order by
//    one atomic counter, so rows complete in order and a row's selection
//    overlaps the scan of later rows;
//  * a unit: each wave streams pages of the unit (one page in flight ahead),
//    dequantises the MXFP8 key block exactly into bf16 (E4M3 * 2^(E-127) is
//    a bf16 value), runs v_mfma_f32_16x16x32_bf16 against the resident query
//    heads, applies ReLU and the head weights in fp32, and keeps the unit's
//    scores as order-preserving 32-bit keys in LDS;
//  * local filter: an LDS histogram of the top 14 key bits gives the bin
//    edge e_u below which the unit holds fewer than m of its largest keys (m
//    is about twice the unit's expected share of the Top-K); the unit appends
//    every key >= e_u, in position order, to its slice of the candidate
//    workspace and records e_u;
//  * the last unit of a row (ticket) selects the exact K-th key T among the
//    candidates with three LDS radix passes (12+12+8 bits) and checks that
//    no unit left out a key >= T (every e_u <= T).  A unit that fails the
//    check is rescored in full and selection is repeated, so the result is
//    always the exact Top-K; ties are broken by the lower position and the
//    positions are written in ascending order.
// No floating-point atomics are used, so results are deterministic.
#include <algorithm>

#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnitPages = 16;
constexpr int kUnitTok = kUnitPages * kPage;       // 1024 keys per unit
constexpr int kBins = 4096;                        // 12-bit histogram passes
constexpr int kCandPer = 24;                       // finisher candidates per thread
constexpr int kChunk = kCandPer * kThreads;        // candidates staged in LDS at once
constexpr int kMaxRows = 1024;                     // rows per launch
constexpr int kMaxBtStride = 16384;                // pages per row (1M tokens)
constexpr int kMaxUnitsPerRow = kMaxBtStride / kUnitPages;

enum : uint32_t { kErrBadPage = 4u, kErrFallback = 8u };

struct Params {
  const uint8_t* q;      // [R, H, 128] E4M3
  const uint8_t* qs;     // [R, H, 4]  E8M0
  const float* w;        // [R, H]
  const uint8_t* kpool;
  int64_t pool_pages;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int32_t R;
  int32_t H;
  int32_t topk;
  int32_t upr;           // units-per-row stride of ucount / uedge
  int32_t* out_idx;
  float* out_score;
  float* dump;           // score rows (test entry point only)
  int64_t ld;
  uint32_t* hdr;         // [0] next unit, [1] exited workgroups, [2] flags
  uint32_t* tick;        // [R]
  uint32_t* ucount;      // [R][upr] candidates emitted per unit
  uint32_t* uedge;       // [R][upr] every key a unit left out is below this
  uint2* cand;           // [R][bt_stride * 64] (key, position)
};

struct Smem {
  uint32_t keys[kUnitTok];            // scores of the current unit as keys
  uint2 stage[kChunk];                // finisher: a chunk of candidates
  uint32_t hist[kBins];
  uint32_t rowpre[kMaxRows + 1];      // exclusive prefix of units per row
  uint32_t cpre[kMaxUnitsPerRow + 1]; // finisher: candidate prefix per unit
  uint32_t red[2 * kWaves + 2];
  uint32_t misc[16];
};

__device__ __forceinline__ void flag_error(uint32_t* hdr, uint32_t bits) {
  if (hdr) __hip_atomic_fetch_or(&hdr[2], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

// wait until this wave's global stores have completed (vmcnt(0))
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- block primitives (256 threads) -------------------------------------

// Exclusive prefix of v over the block; *total receives the block sum.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wv] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t t = red[i];
    before += i < wv ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__device__ uint32_t block_max(uint32_t v, uint32_t* red) {
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) m = max(m, red[i]);
  __syncthreads();
  return m;
}

// Threshold search over an LDS histogram of nbins (a multiple of 256)
// counts: the largest bin b whose suffix count sum_{b'>=b} reaches `need`.
// Writes out[0] = b, out[1] = suffix(b+1), out[2] = total, out[3] = found.
__device__ void find_threshold(const uint32_t* hist, int nbins, uint32_t need, uint32_t* red,
                               uint32_t* out) {
  const int per = nbins / kThreads;
  const int b0 = threadIdx.x * per;
  auto count = [&](int b) -> uint32_t { return hist[b]; };
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += count(b0 + i);
  uint32_t total;
  const uint32_t incl = block_excl_scan(local, red, &total) + local;
  uint32_t run = total - incl;  // keys in bins above this thread's range
  if (threadIdx.x == 0) { out[2] = total; out[3] = 0; }
  __syncthreads();
  if (run < need && run + local >= need) {
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = count(b0 + i);
      if (run < need && run + c >= need) {
        out[0] = (uint32_t)(b0 + i);
        out[1] = run;
        out[3] = 1;
      }
      run += c;
    }
  }
  __syncthreads();
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

__device__ void plan_rows(const Params& P, Smem& S) {
  const int per = (P.R + kThreads - 1) / kThreads;
  const int r0 = threadIdx.x * per;
  uint32_t lu = 0;
  for (int i = 0; i < per; ++i)
    if (r0 + i < P.R) lu += (uint32_t)row_units(P.row_pos[r0 + i], P.bt_stride);
  uint32_t total;
  uint32_t run = block_excl_scan(lu, S.red, &total);
  for (int i = 0; i < per; ++i) {
    if (r0 + i < P.R) {
      S.rowpre[r0 + i] = run;
      run += (uint32_t)row_units(P.row_pos[r0 + i], P.bt_stride);
    }
  }
  if (threadIdx.x == 0) S.rowpre[P.R] = total;
  __syncthreads();
}

__device__ Unit decode_unit(const Params& P, const Smem& S, uint32_t u) {
  int lo = 0, hi = P.R - 1;     // row r with rowpre[r] <= u < rowpre[r+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.rowpre[mid] <= u) lo = mid; else hi = mid - 1;
  }
  Unit U;
  U.row = lo;
  U.uir = (int)(u - S.rowpre[lo]);
  U.units_r = (int)(S.rowpre[lo + 1] - S.rowpre[lo]);
  U.t = P.row_pos[lo];
  const int pr = row_pages(U.t, P.bt_stride);
  U.pg0 = U.uir * kUnitPages;
  U.pg1 = min(pr, U.pg0 + kUnitPages);
  return U;
}

// ---- scoring ---------------------------------------------------------------

template <int NHT>
struct QOperand {
  v8bf a[NHT][4];   // A operand per head tile and k-step
  float w[NHT][4];  // weights of heads 16i + 4g + c
};

// Query heads as the A operand of v_mfma_f32_16x16x32_bf16: lane (head
// 16i + lane%16, group g = lane/16) holds, for k-step s, dims 32g + 8s .. +7
// dequantised exactly into bf16.  The key operand uses the same k order, so
// each lane's 32 key bytes form exactly one MXFP8 group with one scale.
template <int NHT>
__device__ void load_q(const Params& P, int row, QOperand<NHT>& Q) {
  const int lane = threadIdx.x & 63, hr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < NHT; ++i) {
    const int h = 16 * i + hr;
    uint32_t dw[8];
    float sc = 1.0f;
    if (h < P.H) {
      const uint8_t* src = P.q + ((int64_t)row * P.H + h) * kIdxDim + 32 * g;
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      const uint4 b = *reinterpret_cast<const uint4*>(src + 16);
      dw[0] = a.x; dw[1] = a.y; dw[2] = a.z; dw[3] = a.w;
      dw[4] = b.x; dw[5] = b.y; dw[6] = b.z; dw[7] = b.w;
      sc = e8m0_to_f32(P.qs[((int64_t)row * P.H + h) * 4 + g]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) dw[j] = 0;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s], sc, false);
      const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s], sc, true);
      const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s + 1], sc, false);
      const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s + 1], sc, true);
      Q.a[i][s] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int hh = 16 * i + 4 * g + c;
      Q.w[i][c] = hh < P.H ? P.w[(int64_t)row * P.H + hh] : 0.f;
    }
  }
}

// Half a page (two token tiles of 16) as held by one lane: for tile
// j = 2*half + jj, d[2jj], d[2jj+1] are this lane's 32 bytes of token
// 16j + lane%16 (dims 32g..32g+31, g = lane/16) and s[jj] its E8M0 byte.
struct HalfRegs {
  uint4 d[4];
  uint32_t s[2];
};

__device__ __forceinline__ void load_half(const uint8_t* page, int half, HalfRegs& hr) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tok = 16 * (2 * half + jj) + r;
    const uint8_t* src = page + tok * kIdxDim + 32 * g;
    hr.d[2 * jj] = *reinterpret_cast<const uint4*>(src);
    hr.d[2 * jj + 1] = *reinterpret_cast<const uint4*>(src + 16);
    hr.s[jj] = page[kKScaleOff + tok * 4 + g];
  }
}

// Scores of the 32 tokens of one half page; lanes 0..15 end with token
// 16jj + lane of the half in out[jj].  Head sum: in-lane over the lane's
// heads, then across the four lane groups, in a fixed order.
template <int NHT>
__device__ __forceinline__ void score_half(const QOperand<NHT>& Q, const HalfRegs& hr,
                                           float out[2]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const float ks = e8m0_to_f32(hr.s[jj]);
    const uint32_t dw[8] = {hr.d[2 * jj].x,     hr.d[2 * jj].y,     hr.d[2 * jj].z,
                            hr.d[2 * jj].w,     hr.d[2 * jj + 1].x, hr.d[2 * jj + 1].y,
                            hr.d[2 * jj + 1].z, hr.d[2 * jj + 1].w};
    v8bf kb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s], ks, false);
      const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s], ks, true);
      const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s + 1], ks, false);
      const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * s + 1], ks, true);
      kb[s] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < NHT; ++i) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.a[i][s], kb[s], acc, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) part = __builtin_fmaf(Q.w[i][c], fmaxf(acc[c], 0.f), part);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    out[jj] = part;
  }
}

// Score one unit: keys (or dumped scores) of its (pg1-pg0)*64 positions.
// Wave w takes half pages w, w+4, w+8, ... of the unit and keeps three of
// them in flight (a ring of three register buffers, unrolled so no buffer
// is ever copied).
template <int NHT, bool DUMP>
__device__ void score_unit(const Params& P, const Unit& U, Smem& S) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int seq = P.row_seq[U.row];
  const int32_t* btrow = P.bt + (int64_t)seq * P.bt_stride;
  const int nhalf = 2 * (U.pg1 - U.pg0);
  auto fetch = [&](int h, HalfRegs& b) -> bool {
    if (U.t < 0 || h >= nhalf) return false;
    const int pg = U.pg0 + (h >> 1);
    const int32_t id = btrow[pg];
    if (id < 0 || (int64_t)id >= P.pool_pages) {
      if (lane == 0) flag_error(P.hdr, kErrBadPage);
      return false;
    }
    load_half(P.kpool + (int64_t)id * kKPageBytes, h & 1, b);
    return true;
  };
  auto consume = [&](int h, const HalfRegs& b, bool ok, const QOperand<NHT>& Q) {
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
          S.keys[tok] = valid ? score_key(sc[jj]) : 0u;
        }
      }
    }
  };
  HalfRegs b0, b1, b2;
  int h = wv;
  bool ok0 = fetch(h, b0);
  bool ok1 = fetch(h + kWaves, b1);
  QOperand<NHT> Q;
  load_q<NHT>(P, U.row, Q);
  for (; h < nhalf; h += 3 * kWaves) {
    bool ok2 = fetch(h + 2 * kWaves, b2);
    consume(h, b0, ok0, Q);
    if (h + kWaves >= nhalf) break;
    ok0 = fetch(h + 3 * kWaves, b0);
    consume(h + kWaves, b1, ok1, Q);
    if (h + 2 * kWaves >= nhalf) break;
    ok1 = fetch(h + 4 * kWaves, b1);
    consume(h + 2 * kWaves, b2, ok2, Q);
  }
}

// Keys a unit keeps: its expected share E of the Top-K (about
// topk * 1024 / (t+1)) plus four standard deviations and a margin; every key
// when the row has no more than topk positions.
__device__ __forceinline__ uint32_t unit_quota(int t, int topk) {
  const int64_t n = (int64_t)t + 1;
  if (n <= topk) return 0xFFFFFFFFu;
  const float e = (float)topk * (float)kUnitTok / (float)n;
  const float m = e + 4.0f * sqrtf(e) + 8.0f;
  return (uint32_t)fminf(ceilf(m), (float)kUnitTok);
}

// Append the unit's keys >= edge (all non-zero keys when edge is 0), in
// position order, to the unit's candidate slice.
__device__ uint32_t emit_unit_keys(const Params& P, Smem& S, const Unit& U, uint32_t edge) {
  const int ntok = (U.pg1 - U.pg0) * kPage;
  uint2* dst = P.cand + (int64_t)U.row * P.bt_stride * kPage + (int64_t)U.pg0 * kPage;
  constexpr int kPer = kUnitTok / kThreads;       // 4 consecutive keys per thread
  const int i0 = threadIdx.x * kPer;
  uint32_t k[kPer];
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    k[j] = (i0 + j < ntok) ? S.keys[i0 + j] : 0u;
    cnt += (k[j] != 0u && k[j] >= edge) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t off = block_excl_scan(cnt, S.red, &total);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (k[j] != 0u && k[j] >= edge) {
      dst[off++] = make_uint2(k[j], (uint32_t)(U.pg0 * kPage + i0 + j));
    }
  }
  return total;
}

// Local filter of a scored unit: the edge is the lower end of the 20-bit key
// bin holding the unit's quota-th largest key (two LDS histogram passes of
// 12 and 8 bits); keys at or above it are emitted, so every key left out is
// below the recorded edge.
__device__ void filter_unit(const Params& P, Smem& S, const Unit& U) {
  const int ntok = (U.pg1 - U.pg0) * kPage;
  const uint32_t quota = unit_quota(U.t, P.topk);
  uint32_t edge = 0;
  if (quota < (uint32_t)ntok) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) S.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < ntok; i += kThreads) {
      const uint32_t key = S.keys[i];
      if (key) atomicAdd(&S.hist[key >> 20], 1u);
    }
    __syncthreads();
    find_threshold(S.hist, kBins, quota, S.red, S.misc + 8);
    if (S.misc[11]) {
      const uint32_t T1 = S.misc[8], need = quota - S.misc[9];
      for (int i = threadIdx.x; i < 256; i += kThreads) S.hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < ntok; i += kThreads) {
        const uint32_t key = S.keys[i];
        if (key && (key >> 20) == T1) atomicAdd(&S.hist[(key >> 12) & 0xFFu], 1u);
      }
      __syncthreads();
      find_threshold(S.hist, 256, need, S.red, S.misc + 8);
      edge = (T1 << 20) | (S.misc[8] << 12);
    }
  }
  const uint32_t n = emit_unit_keys(P, S, U, edge);
  if (threadIdx.x == 0) {
    const int64_t slot = (int64_t)U.row * P.upr + U.uir;
    P.ucount[slot] = n;
    P.uedge[slot] = edge;   // every key left out is below this
  }
}

// ---- finisher ------------------------------------------------------------------

// prefix of the units' candidate counts (S.cpre); returns the largest edge
__device__ uint32_t load_counts(const Params& P, Smem& S, int row, int units_r) {
  const int per = (units_r + kThreads - 1) / kThreads;
  const int u0 = threadIdx.x * per;
  uint32_t local = 0, emax = 0;
  const int64_t base = (int64_t)row * P.upr;
  for (int i = 0; i < per; ++i) {
    if (u0 + i < units_r) {
      local += load_agent(&P.ucount[base + u0 + i]);
      emax = max(emax, load_agent(&P.uedge[base + u0 + i]));
    }
  }
  uint32_t total;
  uint32_t run = block_excl_scan(local, S.red, &total);
  for (int i = 0; i < per; ++i) {
    if (u0 + i < units_r) {
      S.cpre[u0 + i] = run;
      run += load_agent(&P.ucount[base + u0 + i]);
    }
  }
  if (threadIdx.x == 0) S.cpre[units_r] = total;
  __syncthreads();
  return block_max(emax, S.red);
}

// Stage candidates [ch*kChunk, ...) of the row (flat order = position
// order) into LDS.  Element f goes to thread f % 256; every element finds its
// unit by binary search over the count prefix, so all loads are independent
// and in flight together.  Returns the number staged.
__device__ uint32_t stage_chunk(const Params& P, Smem& S, int row, int units_r, uint32_t n_c,
                                uint32_t ch) {
  const uint32_t base = ch * kChunk;
  const uint32_t n = base < n_c ? min((uint32_t)kChunk, n_c - base) : 0u;
  const uint2* rowc = P.cand + (int64_t)row * P.bt_stride * kPage;
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    const uint32_t i = threadIdx.x + k * kThreads;
    if (i < n) {
      const uint32_t f = base + i;
      int u = 0, hi = units_r - 1;   // last unit with cpre[u] <= f
      while (u < hi) {
        const int mid = (u + hi + 1) >> 1;
        if (S.cpre[mid] <= f) u = mid; else hi = mid - 1;
      }
      S.stage[i] = rowc[(int64_t)u * kUnitTok + (f - S.cpre[u])];
    }
  }
  __syncthreads();
  return n;
}

// Exact key T of rank K among the candidates and the number of keys equal
// to T to keep (three histogram passes of 12, 12 and 8 bits).  Returns false
// if there are fewer than K candidates.  With more than one chunk every
// pass restages them.
__device__ bool select_threshold(const Params& P, Smem& S, int row, int units_r, uint32_t n_c,
                                 uint32_t K, uint32_t* T_out, uint32_t* ties_out) {
  const uint32_t nch = (n_c + kChunk - 1) / kChunk;
  uint32_t prefix = 0, need = K;
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = pass < 2 ? kBins : 256;
    const uint32_t shift = pass == 0 ? 20u : (pass == 1 ? 8u : 0u);
    const uint32_t mask = pass < 2 ? 0xFFFu : 0xFFu;
    const uint32_t pshift = pass == 1 ? 20u : 8u;
    for (int b = threadIdx.x; b < nb; b += kThreads) S.hist[b] = 0;
    __syncthreads();
    for (uint32_t ch = 0; ch < nch; ++ch) {
      const uint32_t n = nch > 1 ? stage_chunk(P, S, row, units_r, n_c, ch) : n_c;
      for (uint32_t f = threadIdx.x; f < n; f += kThreads) {
        const uint32_t k = S.stage[f].x;
        if (pass == 0 || (k >> pshift) == prefix) atomicAdd(&S.hist[(k >> shift) & mask], 1u);
      }
      __syncthreads();
    }
    find_threshold(S.hist, nb, need, S.red, S.misc + 8);
    if (!S.misc[11]) return false;
    need -= S.misc[9];
    prefix = (prefix << (pass < 2 ? 12 : 8)) | S.misc[8];
  }
  *T_out = prefix;
  *ties_out = need;
  return true;
}

// Ordered emission of keys > T and the first `ties` keys equal to T; each
// thread owns a contiguous segment of every staged chunk.
__device__ void emit_selection(const Params& P, Smem& S, int row, int units_r, uint32_t n_c,
                               uint32_t T, uint32_t ties) {
  const int K = P.topk;
  int32_t* oidx = P.out_idx + (int64_t)row * K;
  float* osc = P.out_score ? P.out_score + (int64_t)row * K : nullptr;
  const uint32_t nch = (n_c + kChunk - 1) / kChunk;
  uint32_t run_tie = 0, run_keep = 0;
  for (uint32_t ch = 0; ch < nch; ++ch) {
    const uint32_t n = nch > 1 ? stage_chunk(P, S, row, units_r, n_c, ch) : n_c;
    const uint32_t seg = (n + kThreads - 1) / kThreads;
    const uint32_t f0 = min(n, threadIdx.x * seg), f1 = min(n, f0 + seg);
    uint32_t eq = 0;
    for (uint32_t f = f0; f < f1; ++f) eq += S.stage[f].x == T ? 1u : 0u;
    uint32_t tot_eq;
    const uint32_t tie_base = run_tie + block_excl_scan(eq, S.red, &tot_eq);
    uint32_t keep = 0, tr = tie_base;
    for (uint32_t f = f0; f < f1; ++f) {
      const uint32_t k = S.stage[f].x;
      if (k > T) ++keep;
      else if (k == T) { if (tr < ties) ++keep; ++tr; }
    }
    uint32_t tot_keep;
    uint32_t opos = run_keep + block_excl_scan(keep, S.red, &tot_keep);
    tr = tie_base;
    for (uint32_t f = f0; f < f1; ++f) {
      const uint2 c = S.stage[f];
      bool kp = c.x > T;
      if (c.x == T) { kp = tr < ties; ++tr; }
      if (kp && opos < (uint32_t)K) {
        oidx[opos] = (int32_t)c.y;
        if (osc) osc[opos] = key_score(c.x);
        ++opos;
      }
    }
    run_tie += tot_eq;
    run_keep += tot_keep;
    __syncthreads();
  }
}

template <int NHT>
__device__ void finish_row(const Params& P, Smem& S, const Unit& U0) {
  const int row = U0.row, units_r = U0.units_r, K = P.topk;
  const uint32_t emax = load_counts(P, S, row, units_r);
  uint32_t n_c = S.cpre[units_r];
  int32_t* oidx = P.out_idx + (int64_t)row * K;
  float* osc = P.out_score ? P.out_score + (int64_t)row * K : nullptr;
  if (unit_quota(U0.t, K) == 0xFFFFFFFFu) {
    // at most topk positions: every unit kept all of its keys
    stage_chunk(P, S, row, units_r, n_c, 0);
    for (uint32_t f = threadIdx.x; f < (uint32_t)K; f += kThreads) {
      if (f < n_c) {
        oidx[f] = (int32_t)S.stage[f].y;
        if (osc) osc[f] = key_score(S.stage[f].x);
      } else {
        oidx[f] = -1;
        if (osc) osc[f] = -__builtin_huge_valf();
      }
    }
  } else {
    uint32_t T = 0, ties = 0;
    if (n_c <= (uint32_t)kChunk) stage_chunk(P, S, row, units_r, n_c, 0);
    bool ok = select_threshold(P, S, row, units_r, n_c, (uint32_t)K, &T, &ties);
    if (!ok || emax > T) {
      // Some unit may have left out a key that belongs to the Top-K: rescore
      // every such unit in full and select again (exact, rarely taken).
      if (threadIdx.x == 0) flag_error(P.hdr, kErrFallback);
      for (int u = 0; u < units_r; ++u) {
        const uint32_t e = load_agent(&P.uedge[(int64_t)row * P.upr + u]);
        const bool redo = ok ? (e > T) : (e > 0u);
        if (!redo) continue;
        __syncthreads();
        Unit V = U0;
        V.uir = u;
        V.pg0 = u * kUnitPages;
        V.pg1 = min(row_pages(V.t, P.bt_stride), V.pg0 + kUnitPages);
        score_unit<NHT, false>(P, V, S);
        __syncthreads();
        const uint32_t n = emit_unit_keys(P, S, V, 0u);
        if (threadIdx.x == 0) {
          __hip_atomic_store(&P.ucount[(int64_t)row * P.upr + u], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&P.uedge[(int64_t)row * P.upr + u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __threadfence();
      __syncthreads();
      load_counts(P, S, row, units_r);
      n_c = S.cpre[units_r];
      if (n_c <= (uint32_t)kChunk) stage_chunk(P, S, row, units_r, n_c, 0);
      select_threshold(P, S, row, units_r, n_c, (uint32_t)K, &T, &ties);
    }
    emit_selection(P, S, row, units_r, n_c, T, ties);
  }
  if (threadIdx.x == 0) P.tick[row] = 0;
}

// ---- the kernels ---------------------------------------------------------------

template <int NHT>
__global__ __launch_bounds__(kThreads, 2) void indexer_topk_kernel(Params P) {
  __shared__ Smem S;
  plan_rows(P, S);
  const uint32_t U_total = S.rowpre[P.R];
  for (;;) {
    if (threadIdx.x == 0) S.misc[0] = atomic_add_agent(&P.hdr[0], 1u);
    __syncthreads();
    const uint32_t u = S.misc[0];
    __syncthreads();
    if (u >= U_total) break;
    const Unit U = decode_unit(P, S, u);
    score_unit<NHT, false>(P, U, S);
    __syncthreads();
    filter_unit(P, S, U);
    // publish the unit's candidates, then take the row's ticket
    wait_vm();
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t old = atomic_add_agent(&P.tick[U.row], 1u);
      S.misc[1] = (old == (uint32_t)U.units_r - 1) ? 1u : 0u;
      if (S.misc[1]) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (S.misc[1]) {
      finish_row<NHT>(P, S, U);
      __syncthreads();
    }
  }
  // the last workgroup out re-arms the unit counter for the next call
  if (threadIdx.x == 0) {
    const uint32_t done = atomic_add_agent(&P.hdr[1], 1u);
    if (done == gridDim.x - 1) {
      __hip_atomic_store(&P.hdr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&P.hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Test entry: write every score of every row (units assigned statically).
template <int NHT>
__global__ __launch_bounds__(kThreads, 2) void indexer_dump_kernel(Params P) {
  __shared__ Smem S;
  plan_rows(P, S);
  const uint32_t U_total = S.rowpre[P.R];
  for (uint32_t u = blockIdx.x; u < U_total; u += gridDim.x) {
    const Unit U = decode_unit(P, S, u);
    score_unit<NHT, true>(P, U, S);
  }
}

// ---- host side ----------------------------------------------------------------

struct Layout {
  size_t hdr, tick, ucount, uedge, cand, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int units_stride(int64_t bt_stride) { return (int)((bt_stride + kUnitPages - 1) / kUnitPages); }

Layout layout_for(int64_t rows, int64_t bt_stride) {
  Layout L;
  const int64_t upr = units_stride(bt_stride);
  size_t off = 0;
  L.hdr = off; off += 256;
  L.tick = off; off += align256((size_t)rows * 4);
  L.ucount = off; off += align256((size_t)rows * upr * 4);
  L.uedge = off; off += align256((size_t)rows * upr * 4);
  L.cand = off; off += align256((size_t)rows * bt_stride * kPage * 8);
  L.total = off;
  return L;
}

void* pick_kernel(int nht, bool dump) {
  switch (nht) {
    case 1: return dump ? (void*)&indexer_dump_kernel<1> : (void*)&indexer_topk_kernel<1>;
    case 2: return dump ? (void*)&indexer_dump_kernel<2> : (void*)&indexer_topk_kernel<2>;
    case 3: return dump ? (void*)&indexer_dump_kernel<3> : (void*)&indexer_topk_kernel<3>;
    default: return dump ? (void*)&indexer_dump_kernel<4> : (void*)&indexer_topk_kernel<4>;
  }
}

// resident workgroups of a kernel on the current device (cached per device)
int resident_capacity(void* fn, int slot) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  static int cached[64][8];
  static bool have[64][8];
  if (dev < 64 && have[dev][slot]) return cached[dev][slot];
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                   kThreads, 0) != hipSuccess)
    return -1;
  const int cap = std::max(1, per_cu) * prop.multiProcessorCount;
  if (dev < 64) { cached[dev][slot] = cap; have[dev][slot] = true; }
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

int run(Params P, bool dump, hipStream_t stream) {
  const int nht = (P.H + 15) / 16;
  void* fn = pick_kernel(nht, dump);
  const int cap = resident_capacity(fn, (nht - 1) + (dump ? 4 : 0));
  if (cap <= 0) return DSA_ERR_HIP;
  const int R = P.R;
  const int upr = units_stride(P.bt_stride);
  for (int r0 = 0; r0 < R; r0 += kMaxRows) {
    Params Q = P;
    const int rn = std::min(kMaxRows, R - r0);
    Q.R = rn;
    Q.q = P.q + (int64_t)r0 * P.H * kIdxDim;
    Q.qs = P.qs + (int64_t)r0 * P.H * 4;
    Q.w = P.w + (int64_t)r0 * P.H;
    Q.row_seq = P.row_seq + r0;
    Q.row_pos = P.row_pos + r0;
    if (dump) {
      Q.dump = P.dump + (int64_t)r0 * P.ld;
    } else {
      Q.out_idx = P.out_idx + (int64_t)r0 * P.topk;
      Q.out_score = P.out_score ? P.out_score + (int64_t)r0 * P.topk : nullptr;
    }
    const int64_t G = std::min<int64_t>((int64_t)cap, (int64_t)rn * upr);
    void* args[] = {&Q};
    if (hipLaunchKernel(fn, dim3((unsigned)G), dim3(kThreads), args, 0, stream) != hipSuccess)
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
  return P;
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

extern "C" int dsa_indexer_topk(const void* q_fp8, const void* q_e8m0, const float* w,
                                const void* k_pool, int64_t pool_pages, const int32_t* block_table,
                                int32_t bt_stride, const int32_t* row_seq, const int32_t* row_pos,
                                int32_t R, int32_t H_I, int32_t topk, int32_t* out_idx,
                                float* out_score, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int st = validate(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq, row_pos,
                    R, H_I);
  if (st != DSA_OK) return st;
  if (out_idx == nullptr) return DSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (R == 0) return DSA_OK;
  const int64_t rows = std::min<int64_t>(R, kMaxRows);
  const Layout L = layout_for(rows, bt_stride);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Params P = base_params(q_fp8, q_e8m0, w, k_pool, pool_pages, block_table, bt_stride, row_seq,
                         row_pos, R, H_I);
  P.topk = topk;
  P.out_idx = out_idx;
  P.out_score = out_score;
  P.hdr = reinterpret_cast<uint32_t*>(ws + L.hdr);
  P.tick = reinterpret_cast<uint32_t*>(ws + L.tick);
  P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
  P.uedge = reinterpret_cast<uint32_t*>(ws + L.uedge);
  P.cand = reinterpret_cast<uint2*>(ws + L.cand);
  return run(P, false, dsa_host::as_stream(stream));
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
