// Lightning Indexer: scoring, head weighting and Top-K fused in one kernel
// over the paged MXFP8 K cache, with no score matrix written to HBM ("Deep
// Dive into Sparse Attention ...", section "1. Computation Optimization ...
// DSA Fused Kernel"; Kimi K3.1 Pro Day0 page, "Lightning Indexer
// Three-Stream Coordination").
//
//   I(t,s) = sum_h w[r,h] * max(0, q[r,h] . k[s]),  s <= t = row_pos[r]
//
// Work decomposition (one cooperative launch of G co-resident workgroups):
//  * every row's causal history is cut into units of `chp` pages, chp chosen
//    on the device so that there are at most G + R units; workgroup g takes
//    units g and g + G;
//  * phase 1: each wave streams pages of its unit, dequantises the MXFP8 key
//    block exactly into bf16 (E4M3 * 2^(E-127) fits bf16), runs
//    v_mfma_f32_16x16x32_bf16 against the resident query heads, applies
//    ReLU and the head weights in fp32 and keeps the unit's scores as
//    order-preserving 32-bit keys in LDS; an LDS histogram of the top 12
//    key bits is added into the row's global histogram;
//  * one grid barrier;
//  * phase 2: every unit finds the row's threshold bin from the histogram and
//    appends its keys at or above it, in position order, to its slice of the
//    candidate workspace; the last unit of a row (ticket) resolves the exact
//    K-th key with two more LDS radix passes over the candidates, breaks ties
//    by lower position, and writes the positions in ascending order.
// No floating-point atomics are used, so results are deterministic.
#include <algorithm>

#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChpMax = 64;                       // pages per unit
constexpr int kUnitsPerWg = 2;
constexpr int kKeysLds = kUnitsPerWg * kChpMax * kPage;   // 8192 keys
constexpr int kStageMax = kKeysLds / 2;           // staged candidates (uint2)
constexpr int kBins = 4096;
constexpr int kMaxRows = 1024;                    // rows per launch
constexpr int kMaxGrid = 2047;
constexpr int kMaxUnitsPerRow = kMaxGrid + 1;

enum : uint32_t { kErrBarrierTimeout = 1u, kErrPlan = 2u, kErrBadPage = 4u };

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
  int32_t* out_idx;
  float* out_score;
  float* dump;           // score rows (test entry point only)
  int64_t ld;
  uint32_t* ghist;       // [R][4096]
  uint32_t* tick;        // [R]
  uint32_t* ucount;      // [R][bt_stride]
  uint2* cand;           // [R][bt_stride * 64] (key, position)
  uint32_t* bar;         // count, generation, error flags
};

struct Smem {
  uint32_t keys[kKeysLds];            // unit scores as keys; finisher staging
  uint32_t hist[kBins];
  uint32_t rowpre[kMaxRows + 1];      // exclusive prefix of units per row
  uint32_t cpre[kMaxUnitsPerRow + 1]; // finisher: candidate prefix per unit
  uint32_t red[2 * kWaves + 2];
  uint32_t misc[16];
};

__device__ __forceinline__ void flag_error(uint32_t* bar, uint32_t bits) {
  if (bar) __hip_atomic_fetch_or(&bar[2], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

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

// Exclusive count of `flag` over the block (thread order), plus the total.
__device__ uint32_t block_excl_count(bool flag, uint32_t* red, uint32_t* total) {
  const int wv = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  if ((threadIdx.x & 63) == 0) red[wv] = (uint32_t)__popcll(b);
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
  return before + (uint32_t)__popcll(b & lanemask_lt());
}

// Threshold search over an LDS histogram of nbins (multiple of 256) counts:
// the largest bin b whose suffix count sum_{b'>=b} reaches `need`.  Writes
// out[0] = b, out[1] = suffix(b+1), out[2] = total, out[3] = found.
__device__ void find_threshold(const uint32_t* hist, int nbins, uint32_t need, uint32_t* red,
                               uint32_t* out) {
  const int per = nbins / kThreads;
  const int b0 = threadIdx.x * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[b0 + i];
  uint32_t total;
  const uint32_t incl = block_excl_scan(local, red, &total) + local;
  uint32_t run = total - incl;  // count in bins above this thread's range
  if (threadIdx.x == 0) { out[2] = total; out[3] = 0; }
  __syncthreads();
  for (int i = per - 1; i >= 0; --i) {
    const uint32_t c = hist[b0 + i];
    if (run < need && run + c >= need) {
      out[0] = (uint32_t)(b0 + i);
      out[1] = run;
      out[3] = 1;
    }
    run += c;
  }
  __syncthreads();
}

// ---- grid barrier ----------------------------------------------------------

__device__ void grid_barrier(uint32_t* bar, uint32_t G) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old =
        __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {
      __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // Co-residency is guaranteed by the cooperative launch; the time limit
      // (about 2 s of the 100 MHz constant clock) only guards against a
      // broken launch and reports it through the error word.
      const uint64_t t0 = wall_clock64();
      while (__hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(2);
        if (wall_clock64() - t0 > 200000000ull) {
          flag_error(bar, kErrBarrierTimeout);
          break;
        }
      }
    }
  }
  __syncthreads();
  __threadfence();
}

// ---- the plan ----------------------------------------------------------------

struct Unit {
  int row, uir, units_r, pg0, pg1, t, slot;
};

// Pages a row scans: positions 0..t, bounded by the block table width.
__device__ __forceinline__ int row_pages(int t, int bt_stride) {
  return t < 0 ? 1 : min(t / kPage + 1, bt_stride);
}

// ---- scoring ---------------------------------------------------------------

template <int NHT>
struct QOperand {
  v8bf a[NHT][4];   // A operand per head tile and k-step
  float w[NHT][4];  // weights of heads 16i + 4g + c
};

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

struct PageRegs {
  uint4 d[8];       // token tile j: d[2j], d[2j+1] = this lane's 32 bytes
  uint32_t s[4];    // E8M0 byte of this lane's block, per token tile
};

__device__ __forceinline__ void load_page(const uint8_t* page, PageRegs& pr) {
  const int lane = threadIdx.x & 63, hr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint8_t* src = page + (16 * j + hr) * kIdxDim + 32 * g;
    pr.d[2 * j] = *reinterpret_cast<const uint4*>(src);
    pr.d[2 * j + 1] = *reinterpret_cast<const uint4*>(src + 16);
    pr.s[j] = page[kKScaleOff + (16 * j + hr) * 4 + g];
  }
}

// Scores of the 64 tokens of one page; lanes 0..15 end with token 16j+lane
// of tile j in out[j].
template <int NHT>
__device__ __forceinline__ void score_page(const QOperand<NHT>& Q, const PageRegs& pr,
                                           float out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float ks = e8m0_to_f32(pr.s[j]);
    const uint32_t dw[8] = {pr.d[2 * j].x,     pr.d[2 * j].y,     pr.d[2 * j].z,
                            pr.d[2 * j].w,     pr.d[2 * j + 1].x, pr.d[2 * j + 1].y,
                            pr.d[2 * j + 1].z, pr.d[2 * j + 1].w};
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
    out[j] = part;
  }
}

template <int NHT, bool DUMP>
__device__ void score_unit(const Params& P, const Unit& U, Smem& S) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int seq = P.row_seq[U.row];
  const int32_t* btrow = P.bt + (int64_t)seq * P.bt_stride;
  uint32_t* keys = S.keys + U.slot * (kChpMax * kPage);
  QOperand<NHT> Q;
  load_q<NHT>(P, U.row, Q);
  PageRegs cur, nxt;
  bool cur_ok = false;
  int p = U.pg0 + wv;
  auto page_ptr = [&](int pg, bool& ok) -> const uint8_t* {
    ok = false;
    if (U.t < 0 || pg >= P.bt_stride) return nullptr;
    const int32_t id = btrow[pg];
    if (id < 0 || (int64_t)id >= P.pool_pages) {
      if (lane == 0) flag_error(P.bar, kErrBadPage);
      return nullptr;
    }
    ok = true;
    return P.kpool + (int64_t)id * kKPageBytes;
  };
  if (p < U.pg1) {
    const uint8_t* pp = page_ptr(p, cur_ok);
    if (cur_ok) load_page(pp, cur);
  }
  for (; p < U.pg1; p += kWaves) {
    bool nxt_ok = false;
    const int pn = p + kWaves;
    if (pn < U.pg1) {
      const uint8_t* pp = page_ptr(pn, nxt_ok);
      if (nxt_ok) load_page(pp, nxt);
    }
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    if (cur_ok) score_page<NHT>(Q, cur, sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = 16 * j + lane;      // valid for lanes 0..15
      const int pos = p * kPage + tok;
      const bool valid = cur_ok && pos <= U.t;
      if (lane < 16) {
        if (DUMP) {
          if (valid && pos < P.ld) P.dump[(int64_t)U.row * P.ld + pos] = sc[j] == 0.f ? 0.f : sc[j];
        } else {
          keys[(p - U.pg0) * kPage + tok] = valid ? score_key(sc[j]) : 0u;
        }
      }
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }
}

// ---- phase 2 helpers ---------------------------------------------------------

__device__ __forceinline__ uint2 cand_at(const Params& P, const Smem& S, int row, int chp,
                                         int n_units, uint32_t f) {
  int lo = 0, hi = n_units - 1;   // last unit u with cpre[u] <= f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.cpre[mid] <= f) lo = mid; else hi = mid - 1;
  }
  const int64_t base = (int64_t)row * P.bt_stride * kPage + (int64_t)lo * chp * kPage;
  return P.cand[base + (f - S.cpre[lo])];
}

__device__ void finish_row(const Params& P, Smem& S, int row, int units_r, int chp,
                           uint32_t T1, uint32_t above1, bool take_all) {
  const int K = P.topk;
  // candidate counts of the row's units -> prefix
  {
    uint32_t local = 0;
    const int per = (units_r + kThreads - 1) / kThreads;
    const int u0 = threadIdx.x * per;
    for (int i = 0; i < per; ++i)
      if (u0 + i < units_r) local += load_agent(&P.ucount[(int64_t)row * P.bt_stride + u0 + i]);
    uint32_t total;
    uint32_t run = block_excl_scan(local, S.red, &total);
    for (int i = 0; i < per; ++i) {
      if (u0 + i < units_r) {
        S.cpre[u0 + i] = run;
        run += load_agent(&P.ucount[(int64_t)row * P.bt_stride + u0 + i]);
      }
    }
    if (threadIdx.x == 0) S.cpre[units_r] = total;
    __syncthreads();
  }
  const uint32_t n_c = S.cpre[units_r];
  int32_t* oidx = P.out_idx + (int64_t)row * K;
  float* osc = P.out_score ? P.out_score + (int64_t)row * K : nullptr;
  if (take_all) {
    for (uint32_t f = threadIdx.x; f < n_c && f < (uint32_t)K; f += kThreads) {
      const uint2 c = cand_at(P, S, row, chp, units_r, f);
      oidx[f] = (int32_t)c.y;
      if (osc) osc[f] = key_score(c.x);
    }
    for (uint32_t f = n_c + threadIdx.x; f < (uint32_t)K; f += kThreads) {
      oidx[f] = -1;
      if (osc) osc[f] = -__builtin_huge_valf();
    }
  } else {
    const bool staged = n_c <= (uint32_t)kStageMax;
    uint2* stage = reinterpret_cast<uint2*>(S.keys);
    if (staged)
      for (uint32_t f = threadIdx.x; f < n_c; f += kThreads) stage[f] = cand_at(P, S, row, chp, units_r, f);
    __syncthreads();
    auto get = [&](uint32_t f) -> uint2 { return staged ? stage[f] : cand_at(P, S, row, chp, units_r, f); };
    // level 2: key bits 19..8 inside bin T1
    const uint32_t need1 = (uint32_t)K - above1;
    for (int b = threadIdx.x; b < kBins; b += kThreads) S.hist[b] = 0;
    __syncthreads();
    for (uint32_t f = threadIdx.x; f < n_c; f += kThreads) {
      const uint32_t k = get(f).x;
      if ((k >> 20) == T1) atomicAdd(&S.hist[(k >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    find_threshold(S.hist, kBins, need1, S.red, S.misc + 8);
    const uint32_t T2 = S.misc[8], need2 = need1 - S.misc[9];
    // level 3: key bits 7..0
    for (int b = threadIdx.x; b < kBins; b += kThreads) S.hist[b] = 0;
    __syncthreads();
    const uint32_t pre = (T1 << 12) | T2;
    for (uint32_t f = threadIdx.x; f < n_c; f += kThreads) {
      const uint32_t k = get(f).x;
      if ((k >> 8) == pre) atomicAdd(&S.hist[k & 0xFFu], 1u);
    }
    __syncthreads();
    find_threshold(S.hist, kBins, need2, S.red, S.misc + 8);
    const uint32_t T = (pre << 8) | S.misc[8];
    const uint32_t need3 = need2 - S.misc[9];   // ties at exactly T to keep
    // ordered emission: key > T, or key == T among the first need3 ties
    uint32_t run_keep = 0, run_tie = 0;
    for (uint32_t base = 0; base < n_c; base += kThreads) {
      const uint32_t f = base + threadIdx.x;
      uint2 c = make_uint2(0u, 0u);
      if (f < n_c) c = get(f);
      const bool eq = f < n_c && c.x == T;
      uint32_t tie_tot;
      const uint32_t tie_rank = run_tie + block_excl_count(eq, S.red, &tie_tot);
      const bool keep = f < n_c && (c.x > T || (eq && tie_rank < need3));
      uint32_t keep_tot;
      const uint32_t opos = run_keep + block_excl_count(keep, S.red, &keep_tot);
      if (keep && opos < (uint32_t)K) {
        oidx[opos] = (int32_t)c.y;
        if (osc) osc[opos] = key_score(c.x);
      }
      run_tie += tie_tot;
      run_keep += keep_tot;
    }
  }
  // leave the row's workspace zeroed for the next call
  for (int b = threadIdx.x; b < kBins; b += kThreads) P.ghist[(int64_t)row * kBins + b] = 0;
  if (threadIdx.x == 0) P.tick[row] = 0;
}

// ---- the kernel -------------------------------------------------------------

template <int NHT, bool DUMP>
__global__ __launch_bounds__(kThreads) void indexer_kernel(Params P) {
  __shared__ Smem S;
  const uint32_t G = gridDim.x;
  // plan: pages per row, units of chp pages
  {
    uint32_t local = 0;
    const int per = (P.R + kThreads - 1) / kThreads;
    const int r0 = threadIdx.x * per;
    for (int i = 0; i < per; ++i)
      if (r0 + i < P.R) local += (uint32_t)row_pages(P.row_pos[r0 + i], P.bt_stride);
    uint32_t total_pages;
    block_excl_scan(local, S.red, &total_pages);
    uint32_t chp = (total_pages + G - 1) / G;
    if (chp < 1) chp = 1;
    if (chp > (uint32_t)kChpMax) {
      if (threadIdx.x == 0) flag_error(P.bar, kErrPlan);
      chp = kChpMax;
    }
    uint32_t lu = 0;
    for (int i = 0; i < per; ++i)
      if (r0 + i < P.R) lu += ((uint32_t)row_pages(P.row_pos[r0 + i], P.bt_stride) + chp - 1) / chp;
    uint32_t total_units;
    uint32_t run = block_excl_scan(lu, S.red, &total_units);
    for (int i = 0; i < per; ++i) {
      if (r0 + i < P.R) {
        S.rowpre[r0 + i] = run;
        run += ((uint32_t)row_pages(P.row_pos[r0 + i], P.bt_stride) + chp - 1) / chp;
      }
    }
    if (threadIdx.x == 0) {
      S.rowpre[P.R] = total_units;
      S.misc[0] = chp;
      if (total_units > kUnitsPerWg * G) flag_error(P.bar, kErrPlan);
    }
    __syncthreads();
  }
  const int chp = (int)S.misc[0];
  const uint32_t U_total = S.rowpre[P.R];
  Unit units[kUnitsPerWg];
  int n_my = 0;
#pragma unroll
  for (int k = 0; k < kUnitsPerWg; ++k) {
    const uint32_t u = blockIdx.x + k * G;
    Unit& U = units[k];
    U.slot = k;
    if (u >= U_total) { U.row = -1; continue; }
    n_my = k + 1;
    int lo = 0, hi = P.R - 1;     // row r with rowpre[r] <= u < rowpre[r+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (S.rowpre[mid] <= u) lo = mid; else hi = mid - 1;
    }
    U.row = lo;
    U.uir = (int)(u - S.rowpre[lo]);
    U.units_r = (int)(S.rowpre[lo + 1] - S.rowpre[lo]);
    U.t = P.row_pos[lo];
    const int pr = row_pages(U.t, P.bt_stride);
    U.pg0 = U.uir * chp;
    U.pg1 = min(pr, U.pg0 + chp);
  }
  // phase 1: scores
#pragma unroll
  for (int k = 0; k < kUnitsPerWg; ++k)
    if (k < n_my) score_unit<NHT, DUMP>(P, units[k], S);
  if (DUMP) return;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kUnitsPerWg; ++k) {
    if (k >= n_my) break;
    const Unit& U = units[k];
    const uint32_t* keys = S.keys + U.slot * (kChpMax * kPage);
    const int ntok = (U.pg1 - U.pg0) * kPage;
    for (int b = threadIdx.x; b < kBins; b += kThreads) S.hist[b] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < ntok; i += kThreads) {
      const uint32_t key = keys[i];
      if (key) atomicAdd(&S.hist[key >> 20], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kBins; b += kThreads) {
      const uint32_t c = S.hist[b];
      if (c) atomic_add_agent(&P.ghist[(int64_t)U.row * kBins + b], c);
    }
    __syncthreads();
  }
  grid_barrier(P.bar, G);
  // phase 2: per-unit threshold and ordered candidate emission
  uint32_t T1s[kUnitsPerWg], above1s[kUnitsPerWg];
  bool take_alls[kUnitsPerWg];
#pragma unroll
  for (int k = 0; k < kUnitsPerWg; ++k) {
    if (k >= n_my) break;
    const Unit& U = units[k];
    for (int b = threadIdx.x; b < kBins; b += kThreads)
      S.hist[b] = load_agent(&P.ghist[(int64_t)U.row * kBins + b]);
    __syncthreads();
    find_threshold(S.hist, kBins, (uint32_t)P.topk, S.red, S.misc + 8);
    const bool take_all = S.misc[11] == 0;     // fewer valid keys than topk
    const uint32_t T1 = take_all ? 0u : S.misc[8];
    T1s[k] = T1;
    above1s[k] = take_all ? 0u : S.misc[9];
    take_alls[k] = take_all;
    const uint32_t* keys = S.keys + U.slot * (kChpMax * kPage);
    const int ntok = (U.pg1 - U.pg0) * kPage;
    uint2* dst = P.cand + (int64_t)U.row * P.bt_stride * kPage + (int64_t)U.pg0 * kPage;
    uint32_t run = 0;
    for (int base = 0; base < ntok; base += kThreads) {
      const int i = base + threadIdx.x;
      const uint32_t key = i < ntok ? keys[i] : 0u;
      const bool f = key != 0u && (key >> 20) >= T1;
      uint32_t tot;
      const uint32_t off = run + block_excl_count(f, S.red, &tot);
      if (f) dst[off] = make_uint2(key, (uint32_t)(U.pg0 * kPage + i));
      run += tot;
    }
    if (threadIdx.x == 0) P.ucount[(int64_t)U.row * P.bt_stride + U.uir] = run;
    __syncthreads();
  }
  // tickets: the last unit of a row finishes it
#pragma unroll
  for (int k = 0; k < kUnitsPerWg; ++k) {
    if (k >= n_my) break;
    const Unit& U = units[k];
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = atomic_add_agent(&P.tick[U.row], 1u);
      S.misc[1] = (old == (uint32_t)U.units_r - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (S.misc[1]) {
      __threadfence();
      if (U.units_r <= kMaxUnitsPerRow)
        finish_row(P, S, U.row, U.units_r, chp, T1s[k], above1s[k], take_alls[k]);
      else if (threadIdx.x == 0)
        flag_error(P.bar, kErrPlan);
      __syncthreads();
    }
  }
}

// ---- host side ----------------------------------------------------------------

struct Layout {
  size_t bar, ghist, tick, ucount, cand, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout layout_for(int64_t rows, int64_t bt_stride) {
  Layout L;
  size_t off = 0;
  L.bar = off; off += 256;
  L.ghist = off; off += align256((size_t)rows * kBins * 4);
  L.tick = off; off += align256((size_t)rows * 4);
  L.ucount = off; off += align256((size_t)rows * bt_stride * 4);
  L.cand = off; off += align256((size_t)rows * bt_stride * kPage * 8);
  L.total = off;
  return L;
}

template <int NHT, bool DUMP>
void* kernel_ptr() { return reinterpret_cast<void*>(&indexer_kernel<NHT, DUMP>); }

void* pick_kernel(int nht, bool dump) {
  switch (nht) {
    case 1: return dump ? kernel_ptr<1, true>() : kernel_ptr<1, false>();
    case 2: return dump ? kernel_ptr<2, true>() : kernel_ptr<2, false>();
    case 3: return dump ? kernel_ptr<3, true>() : kernel_ptr<3, false>();
    default: return dump ? kernel_ptr<4, true>() : kernel_ptr<4, false>();
  }
}

// co-resident workgroups of the fused kernel on the current device
int coresident_capacity(void* fn) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  static int cached[64][4];
  static bool have[64][4];
  int nht_slot = 0;
  for (int i = 1; i <= 4; ++i)
    if (fn == pick_kernel(i, false)) nht_slot = i - 1;
  if (dev < 64 && have[dev][nht_slot]) return cached[dev][nht_slot];
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                   kThreads, 0) != hipSuccess)
    return -1;
  int cap = per_cu * prop.multiProcessorCount;
  if (cap > kMaxGrid) cap = kMaxGrid;
  if (dev < 64) { cached[dev][nht_slot] = cap; have[dev][nht_slot] = true; }
  return cap;
}

int validate(const void* q, const void* qs, const float* w, const void* kpool, int64_t pool_pages,
             const int32_t* bt, int32_t bt_stride, const int32_t* row_seq, const int32_t* row_pos,
             int32_t R, int32_t H) {
  if (!q || !qs || !w || !kpool || !bt || !row_seq || !row_pos) return DSA_ERR_INVALID_ARG;
  if (R < 0 || bt_stride <= 0 || pool_pages <= 0) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > DSA_MAX_INDEX_HEADS) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

int run(Params P, bool dump, hipStream_t stream) {
  const int nht = (P.H + 15) / 16;
  void* fn = pick_kernel(nht, dump);
  const int cap = coresident_capacity(pick_kernel(nht, false));
  if (cap <= 0) return DSA_ERR_HIP;
  const int64_t rows_by_pages = (int64_t)cap * kChpMax / P.bt_stride;
  int64_t rpl = std::min<int64_t>({(int64_t)kMaxRows, (int64_t)cap, rows_by_pages});
  if (rpl < 1) return DSA_ERR_UNSUPPORTED;   // one row's history exceeds one launch
  const int R = P.R;
  for (int r0 = 0; r0 < R; r0 += (int)rpl) {
    Params Q = P;
    const int rn = (int)std::min<int64_t>(rpl, R - r0);
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
    const int64_t G = std::min<int64_t>((int64_t)cap, std::max<int64_t>((int64_t)rn, (int64_t)rn * P.bt_stride));
    void* args[] = {&Q};
    hipError_t e;
    if (dump)
      e = hipLaunchKernel(fn, dim3((unsigned)G), dim3(kThreads), args, 0, stream);
    else
      e = hipLaunchCooperativeKernel(fn, dim3((unsigned)G), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
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
  P.topk = topk;
  P.out_idx = out_idx;
  P.out_score = out_score;
  P.bar = reinterpret_cast<uint32_t*>(ws + L.bar);
  P.ghist = reinterpret_cast<uint32_t*>(ws + L.ghist);
  P.tick = reinterpret_cast<uint32_t*>(ws + L.tick);
  P.ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
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
  P.topk = 1;
  P.dump = out_scores;
  P.ld = ld;
  P.bar = nullptr;   // the score dump uses no workspace
  return run(P, true, s);
}
