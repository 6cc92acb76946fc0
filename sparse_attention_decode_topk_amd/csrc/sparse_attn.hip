// Sparse Flash Attention over the Top-K positions of an FP8 MLA latent
// cache ("Deep Dive into Sparse Attention ...", section 1; "Adapting and
// Optimizing Kimi K3.1 Pro for Long-Sequence Inference", section 2: gather
// the cache entries of the selected indices, then attention; Kimi K3.1 Pro
// Day0 page, "FP8 KVCache ..." and "Preserving a Mixed-Precision Path").
//
// One workgroup = (query row, group of 32 heads, split of the index list);
// the groups of one (row, split) are placed on one XCD so the records they
// all read are served by that XCD's L2.  The waves form G groups of four:
// group g takes tile g (32 tokens) of every step of 32G tokens and keeps its
// own softmax state, and the groups are merged in LDS at the end.  A split
// list takes G = 2 (one work-group per CU, two waves per SIMD); a list taken
// whole takes G = 1 with a smaller ring, so that two independent
// work-groups share every CU (again two waves per SIMD, but not tied by each
// other's barriers, and one's start and end overlap the other's steps).  In
// a group, wave (ht, dh)
// owns head tile ht (16 heads) and latent half dh (256 of the 512 dims,
// plus half of the rope dims).
//  * up front, every entry of the split is translated position -> page ->
//    record slot (two dependent loads, all entries in flight together);
//  * the selected 656-byte records are copied 32 per tile straight from
//    global memory into LDS (global_load_lds_dwordx4, no registers), into a
//    ring of six tiles (three steps, two ahead of the compute) for G = 2, of
//    two (two steps, one ahead) for G = 1; a group's four waves copy its tile;
//  * logits S^T = K Q^T on v_mfma_f32_16x16x32_bf16, each wave over its
//    half of the 576 dims: E4M3 latent -> bf16 is exact, each 128-wide
//    latent tile accumulates separately and is scaled by its fp32 tile
//    scale in fp32, the bf16 rope part adds on top; the two halves are
//    summed through LDS in a fixed order (partner waves end with identical
//    logits), times softmax_scale*log2(e);
//  * online softmax per head inside the wave (a head's 32 logits of a tile
//    live in its four lanes);
//  * O^T += V^T P'^T on v_mfma_f32_16x16x32_f16: V is the exact E4M3 code in
//    f16 read transposed from LDS by ds_read_b64_tr_b8, and the tile scale
//    of every token is folded into P (P' = p * scale * 2^(8-E), E a running
//    power-of-two reference so P' stays well inside fp16).  P' never leaves
//    the registers: the logits' output layout is the B-operand layout of
//    the P.V product once the tile's 32 tokens are ordered to match.
// With one split the workgroup writes out and lse; otherwise it writes (O, m, l) partials and a
// second launch combines the splits of every (row, head) in split order
// (deterministic).
#include <algorithm>

#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kCombineThreads = 256;
constexpr int kHeadsWG = 32;                  // heads per workgroup (two MFMA tiles)
constexpr int kTileTok = 32;                  // tokens per tile
constexpr int kPieces = kRec / 16;            // 41 16-byte pieces per record
constexpr int kDmaPerTile = 21;               // ceil(32 * 41 / 64) DMA instructions per tile
constexpr int kDmaPerWave = 6;                // per wave per step (the last ones are padding)
constexpr int kSlotBytes = kDmaPerTile * 1024;  // 21504: 32 records + padding
constexpr int kRingBytes = 6 * kSlotBytes;    // 129024: six tiles of records
constexpr int kMaxEntries = DSA_MAX_TOPK;     // entries of one split
constexpr int kMaxSplits = 16;                // a row of 2048 entries: two 64-entry steps per split
constexpr int kWideSplits = 8;                // splits the eight-dim combine holds in registers
constexpr int kTargetWgs = 256;
constexpr int kZeroBytes = 1024;              // zero record in the workspace
constexpr int kMargin = 6;                    // logits may exceed the softmax reference by 2^6
constexpr int kPBias = 8;                     // P' = p * scale * 2^(kPBias - E) < 2^(kMargin+1+kPBias)
constexpr int kMergeWords = 66;               // per lane: 64 output accumulators, m, l
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(kDmaPerWave * 4 >= kDmaPerTile, "a group's DMA assignment covers its tile");
static_assert(32 * kPieces <= kDmaPerTile * 64, "a tile fits its DMA instructions");
static_assert(kMargin + 1 + kPBias < 16, "P' stays below the fp16 maximum");
static_assert(4 * kMergeWords * 64 * 4 <= kRingBytes, "the merge fits the ring");

// An attention work-group is G wave groups of four waves, each group taking
// one tile of 32 records per step.  G = 2: eight waves (two per SIMD), a
// ring of three steps, two copied ahead, one work-group per CU.  G = 1: four
// waves, a ring of two steps, one copied ahead, in about 60 KB of LDS: two
// work-groups per CU.
template <int G>
struct Cfg {
  static constexpr int kThreads = 256 * G;
  static constexpr int kStepTok = G * kTileTok;                 // tokens per step
  static constexpr int kRing = G == 1 ? 2 * kSlotBytes : kRingBytes;   // ring bytes
  static constexpr int kRingSteps = kRing / (G * kSlotBytes);   // 2 or 3
  static constexpr int kAhead = kRingSteps - 1;                 // steps copied ahead
  static constexpr int kSlotCap = (kMaxEntries + kStepTok - 1) / kStepTok * kStepTok;   // whole steps
};
static_assert(Cfg<1>::kRingSteps == 2 && Cfg<2>::kRingSteps == 3, "ring depths");

struct Params {
  const uint16_t* q;      // [R, H, 576] bf16
  const uint8_t* pool;
  int64_t pool_pages;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* row_seq;
  const int32_t* idx;     // [R, topk]
  int32_t R, H, topk;
  float scale_log2;       // softmax_scale * log2(e)
  float* out;             // [R, H, 512]
  float* lse;             // [R, H] or null
  int32_t S, per_split;   // splits and entries per split (multiple of 64)
  int32_t HGn;            // head groups of 32
  float* part_o;          // [R][H][S][512]
  float* part_ml;         // [R][H][S][2]
  const uint8_t* zero;    // kZeroBytes of zeros
  uint32_t* err;
};

template <int G>
struct Smem {
  uint8_t ring[Cfg<G>::kRing];         // record tiles; the group merge at the end
  uint8_t junk[1024];                  // target of padding DMA instructions
  int32_t slot[Cfg<G>::kSlotCap];      // record slot per entry of the split, -1 = none
  float zx[G][2][2][8 * 64];           // partial logits [group][ht][dh], swapped between partners
  uint32_t vmask[Cfg<G>::kSlotCap / 32];   // entry validity, one bit per entry of the split
};

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bits) {
  if (err) __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 8 and 16 bytes at LDS byte address a (the loop addresses the ring by
// 32-bit LDS offsets, so that the constant part of every read folds into its
// offset field).
typedef unsigned int lds_v2u __attribute__((ext_vector_type(2)));
typedef unsigned int lds_v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_u2(uint32_t a) {
  const lds_v2u v = *(const __attribute__((address_space(3))) lds_v2u*)(size_t)a;
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 lds_u4(uint32_t a) {
  const lds_v4u v = *(const __attribute__((address_space(3))) lds_v4u*)(size_t)a;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16 bytes per lane from global memory into LDS at lds_base + 16*lane.  Issued
// as inline assembly so that the compiler does not pair it with automatic
// waits; completion is tracked by the explicit vmcnt waits of the main loop.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// Maximum / sum of a value over the four 16-lane rows of a wave (every lane
// receives it), by v_permlane16_swap / v_permlane32_swap instead of LDS
// round trips.  The sum is (row0 + row1) + (row2 + row3) in every lane, as
// the pairwise exchange by lane xor 16 then 32 gives up to the order of
// each (commutative) addition.
__device__ __forceinline__ float rows_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ uint32_t rows_umax(uint32_t u) {
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t m = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return max((uint32_t)b[0], (uint32_t)b[1]);
}
__device__ __forceinline__ float rows_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The tokens of a tile in the order of the P.V contraction: k = 8g + i is
// token 4g + i for i < 4 and 16 + 4g + (i - 4) otherwise, which is where the
// logits of those tokens land in the output of the two 16-token MFMAs.
__device__ __forceinline__ int ktok(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

template <int G>
__global__ __launch_bounds__(256 * G, G == 1 ? 2 : 1) void sfa_kernel(Params P) {
  constexpr int kGroups = G, kThreads = Cfg<G>::kThreads, kStepTok = Cfg<G>::kStepTok;
  constexpr int kRingSteps = Cfg<G>::kRingSteps, kSlotCap = Cfg<G>::kSlotCap;
  __shared__ __attribute__((aligned(16))) Smem<G> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hr = lane & 15, g = lane >> 4;
  const int grp = wv >> 2, ht = wv & 1, dh = (wv >> 1) & 1;
  // blockIdx -> (row, head group, split).  Work-groups are dealt to the 8
  // XCDs round-robin (block b to XCD b % 8).  When the rows divide evenly
  // among the XCDs, every work-group of a row goes to one XCD (row r to XCD
  // r % 8): the row's records and its split partials then stay in that
  // XCD's L2, where the combine launch (whose blocks of row r also run on
  // XCD r % 8) reads them.  Otherwise the head groups of one (row, split)
  // are R*S blocks apart, a multiple of 8 when R*S is, so at least the
  // records they share come from one L2.
  int row, hg, sp;
  {
    const int per_row = P.HGn * P.S;
    const int b = blockIdx.x;
    if ((P.R & 7) == 0) {
      const int x = b & 7, j = b >> 3;
      row = x + 8 * (j / per_row);
      const int rem = j % per_row;
      hg = rem / P.S;
      sp = rem % P.S;
    } else {
      const int pairs = P.R * P.S;
      const int pair = b % pairs;
      hg = b / pairs;
      row = pair / P.S;
      sp = pair % P.S;
    }
  }
  const int seq = P.row_seq[row];
  const int j0 = sp * P.per_split;
  const int jend = min(P.topk, j0 + P.per_split);
  const int nent = max(0, jend - j0);
  const int nsteps = (nent + kStepTok - 1) / kStepTok;

  // ---- query operand: B operand of S^T = K Q^T for head tile ht over the
  //      wave's half of the dims.  Lane (head hr, group g) holds, for k-step
  //      j < 8, latent dims 256dh+32j+8g..+7 and for j = 8 rope dims
  //      32dh+8g..+7.  Issued first so the slot resolution's waits cover them.
  const int head = kHeadsWG * hg + 16 * ht + hr;
  const bool head_ok = head < P.H;
  v8bf qv[9];
  {
    const uint16_t* qrow = P.q + ((int64_t)row * P.H + (head_ok ? head : 0)) * kQK;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int d = j < 8 ? 256 * dh + 32 * j + 8 * g : kLatent + 32 * dh + 8 * g;
      uint4 v = *reinterpret_cast<const uint4*>(qrow + d);
      if (!head_ok) v = make_uint4(0, 0, 0, 0);
      qv[j] = __builtin_bit_cast(v8bf, v);
    }
  }

  // ---- record slots of the split's entries ----
  {
    const int32_t* idxrow = P.idx + (int64_t)row * P.topk + j0;
    const int32_t* btrow = P.bt + (int64_t)seq * P.bt_stride;
    constexpr int kPer = (kSlotCap + kThreads - 1) / kThreads;   // 4 or 3
    int32_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * kThreads;
      v[i] = e < nent ? idxrow[e] : -1;
    }
    int32_t pid[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool in = v[i] >= 0 && (v[i] >> 6) < P.bt_stride;
      pid[i] = in ? btrow[v[i] >> 6] : -1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * kThreads;
      int32_t s = -1;
      if (v[i] >= 0) {
        if (pid[i] >= 0 && (int64_t)pid[i] < P.pool_pages && (v[i] >> 6) < P.bt_stride)
          s = pid[i] * kPage + (v[i] & 63);
        else
          flag(P.err, 1u);
      }
      if (e < nsteps * kStepTok) S.slot[e] = s;
      // validity of the wave's 64 consecutive entries, one bit per entry
      const uint64_t vb = __builtin_amdgcn_ballot_w64(s >= 0);
      const int e0 = (tid & ~63) + i * kThreads;
      if (lane == 0 && e0 < nsteps * kStepTok) {
        S.vmask[e0 >> 5] = (uint32_t)vb;
        S.vmask[(e0 >> 5) + 1] = (uint32_t)(vb >> 32);
      }
    }
  }
  __syncthreads();

  // ---- DMA of one step into ring slot k % kRingSteps: the four waves of
  //      group grp copy tile grp of the step, each issuing exactly kDmaPerWave instructions per step,
  //      padding ones included, so the waits below can count them.
  //      Instruction m of a wave covers pieces 64j + lane (j = wv%4 + 4m) of
  //      the tile: record rec_m, 16-byte piece part_m.
  const uint32_t ring0 = lds_addr(S.ring), junk = lds_addr(S.junk);
  const int wq = wv & 3;
  auto issue_step = [&](int k) {
    const uint32_t ln = (uint32_t)lane;
    uint32_t ro_m[kDmaPerWave];
#pragma unroll
    for (int m = 0; m < kDmaPerWave; ++m) {
      const uint32_t piece = 64u * (uint32_t)(wq + 4 * m) + ln;
      const uint32_t rec = piece / (uint32_t)kPieces;
      ro_m[m] = rec | ((piece - (uint32_t)kPieces * rec) * 16u) << 16;
    }
    int32_t sl[kDmaPerWave];
#pragma unroll
    for (int m = 0; m < kDmaPerWave; ++m) {
      const int rec = (int)(ro_m[m] & 0xFFFFu);
      const bool live = wq + 4 * m < kDmaPerTile && k < nsteps && rec < kTileTok;
      sl[m] = live ? S.slot[(kGroups * k + grp) * kTileTok + rec] : -1;
    }
    const uint32_t base = ring0 + (uint32_t)(((k % kRingSteps) * kGroups + grp) * kSlotBytes);
#pragma unroll
    for (int m = 0; m < kDmaPerWave; ++m) {
      const bool inst = wq + 4 * m < kDmaPerTile && k < nsteps;   // wave-uniform
      const int32_t sv = sl[m];
      const uint8_t* rb = sv >= 0 ? P.pool + (int64_t)sv * kRec : P.zero;   // the record, or zeros
      const uint8_t* src = rb + (ro_m[m] >> 16);
      dma16(src, inst ? base + (uint32_t)((wq + 4 * m) * 1024) : junk);
    }
  };

  // m_ref / l_run: softmax reference and running sum of head hr over the
  // group's tiles (identical in the four lanes of a head and in both
  // partners; l_run and O are relative to m_ref); eref: power-of-two
  // references of the wave's two latent tiles (wave-uniform).  The
  // references move only when a logit exceeds m_ref by more than kMargin or
  // a tile scale exceeds its reference, so O is rescaled rarely.
  // o[d][c] = dim 256dh + 16d + 4g + c of head hr.
  float m_ref = -__builtin_huge_valf(), l_run = 0.f;
  int eref[2] = {-1000, -1000};
  v4f o[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) o[d] = v4f{0.f, 0.f, 0.f, 0.f};
  float* zx = S.zx[grp][ht][dh];
  const float* zpart = S.zx[grp][ht][dh ^ 1];

#pragma unroll
  for (int a = 0; a < Cfg<G>::kAhead; ++a) issue_step(a);
  // Group g runs g barriers behind group 0: every s_barrier of the loop is
  // then one group's step-top barrier and another's mid-step barrier, so the
  // waves sharing a SIMD are not all in the same phase.  A group's ring
  // slots, partial logits and DMA are its own, so only its own waves'
  // ordering matters; the counts match through the extra barriers after the
  // loop.
  for (int b = 0; b < grp; ++b) __builtin_amdgcn_s_barrier();
  for (int k = 0; k < nsteps; ++k) {
    // this step's copies are complete once only the later steps' remain
    // (kDmaPerWave per step copied ahead of this one); the barrier also
    // releases the slots of step k-1, which take step k + kAhead
    static_assert(Cfg<G>::kAhead == 1 || Cfg<G>::kAhead == 2, "the wait below");
    if constexpr (Cfg<G>::kAhead == 2)
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    issue_step(k + Cfg<G>::kAhead);
    const uint32_t tq = ring0 + (uint32_t)(((k % kRingSteps) * kGroups + grp) * kSlotBytes);   // the group's tile
    const int eq0 = (kGroups * k + grp) * kTileTok;   // its first entry
    // this step's base addresses of the lane's reads, built from an opaque
    // lane id so that the compiler rebuilds them per step instead of holding
    // one hoisted address per read: the constant parts of every read fold
    // into its offset field and neighbouring reads pair up
    uint32_t ln = (uint32_t)lane;
    asm volatile("" : "+v"(ln));
    const uint32_t hr_ = ln & 15u, g_ = ln >> 4;
    const uint32_t rec0 = tq + hr_ * kRec + 256u * dh + 8u * g_;
    const uint32_t rope0 = tq + hr_ * kRec + kRecRopeOff + 64u * dh + 16u * g_;
    const uint32_t scl0 = tq + 4u * g_ * kRec + kRecScaleOff + 8u * dh;
    const uint32_t vrow0 = tq + (uint32_t)ktok((int)g_, (int)(hr_ >> 1)) * kRec + 8u * (hr_ & 1u) + 256u * dh;

    // ---- partial logits over the wave's half of the dims: accumulators
    //      acc[u][t] of token rows 16u + (0..15), latent tile 2dh + t (t < 2)
    //      or the rope half (t = 2); consecutive MFMAs feed different ones
    v4f acc[2][3];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 3; ++t) acc[u][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = 4 * t + jj;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint2 raw = lds_u2(rec0 + (uint32_t)(u * 16 * kRec + 32 * j));
          const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
          const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
          const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
          const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
          const v8bf a = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[j], acc[u][t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 r4 = lds_u4(rope0 + (uint32_t)(16 * u * kRec));
      acc[u][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r4), qv[8],
                                                          acc[u][2], 0, 0, 0);
    }
    // scales of the wave's two latent tiles for the lane's 8 tokens (k order)
    float sc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint2 s2 = lds_u2(scl0 + (uint32_t)(ktok(0, i) * kRec));
      sc[i][0] = __uint_as_float(s2.x);
      sc[i][1] = __uint_as_float(s2.y);
    }
    // this half's part of the logits of the lane's 8 tokens, shared with the
    // partner (same heads, other half)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i >> 2, c = i & 3;
      float v = acc[u][2][c];
      v = __builtin_fmaf(sc[i][0], acc[u][0][c], v);
      v = __builtin_fmaf(sc[i][1], acc[u][1][c], v);
      zx[i * 64 + lane] = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float z[8];
    // validity of the tile's 32 entries, shifted so that bit i (i < 4) and
    // bit 12 + i (i >= 4) are token ktok(g, i)'s
    const uint32_t tmask = S.vmask[eq0 >> 5] >> (4 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float own = zx[i * 64 + lane], other = zpart[i * 64 + lane];
      const float v = dh ? other + own : own + other;   // half 0 first in both partners
      z[i] = (tmask >> ktok(0, i)) & 1u ? v * P.scale_log2 : -__builtin_huge_valf();
    }
    uint32_t smax[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      smax[0] = max(smax[0], __float_as_uint(sc[i][0]));
      smax[1] = max(smax[1], __float_as_uint(sc[i][1]));
    }

    // ---- online softmax of head hr over the tile (lazy references) ----
    float zm = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) zm = fmaxf(zm, z[i]);
    zm = rows_max(zm);
    int et[2];
    bool egrow = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t b = smax[t];
      b = rows_umax(b);
      et[t] = (b & 0x7FFFFFFFu) ? (int)((b >> 23) & 0xFF) - 127 : -1000;
      egrow |= et[t] > eref[t];
    }
    const bool grow = zm > m_ref + (float)kMargin;   // false while zm is -inf
    if (__builtin_amdgcn_ballot_w64(grow) || egrow) {
      const float m_new = grow ? zm : m_ref;
      const float fh = m_ref == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      float ft[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int en = max(eref[t], et[t]);
        ft[t] = eref[t] > -1000 ? pow2f(max(-126, eref[t] - en)) : 0.f;
        eref[t] = en;
      }
      if (__builtin_amdgcn_ballot_w64(l_run != 0.f)) {
#pragma unroll
        for (int d = 0; d < 16; ++d) {
          const float f = fh * ft[d >> 3];
#pragma unroll
          for (int c = 0; c < 4; ++c) o[d][c] *= f;
        }
      }
      l_run *= fh;
      m_ref = m_new;
    }
    float pr[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = z[i] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(z[i] - m_ref);   // <= 2^kMargin
      ps += pr[i];
    }
    ps = rows_sum(ps);
    l_run += ps;

    // ---- O^T += V^T P'^T over the tile (one k-step of 32 tokens) ----
    typedef __attribute__((address_space(3))) v2i lds_v2i;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float mul = eref[t] > -1000 ? pow2f(max(-126, min(127, kPBias - eref[t]))) : 0.f;
      _Float16 h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (_Float16)(pr[i] * sc[i][t] * mul);
      const v8h b = v8h{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
      const uint32_t vrow = vrow0 + (uint32_t)(128 * t);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(size_t)(vrow + 16 * dd));
        const v2h v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, false);
        const v2h v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, true);
        const v2h v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, false);
        const v2h v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, true);
        const v8h a = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        o[8 * t + dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, o[8 * t + dd], 0, 0, 0);
      }
    }
  }
  // no copy may still be landing in LDS when the ring is reused or the
  // workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int b = grp; b < kGroups - 1; ++b) __builtin_amdgcn_s_barrier();

  // ---- true O relative to m_ref: o * 2^(eref - kPBias) ----
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float f = eref[t] > -1000 ? pow2f(max(-126, min(127, eref[t] - kPBias))) : 0.f;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd)
#pragma unroll
      for (int c = 0; c < 4; ++c) o[8 * t + dd][c] *= f;
  }
  // ---- merge groups 1 .. kGroups-1 into group 0 (same lane, same wave
  //      role), one group at a time through the ring ----
  float* mg = reinterpret_cast<float*>(S.ring) + (wv & 3) * kMergeWords * 64 + lane;
  for (int src = 1; src < kGroups; ++src) {
    __syncthreads();   // the ring (and the previous group's copy) is free
    if (grp == src) {
#pragma unroll
      for (int d = 0; d < 16; ++d)
#pragma unroll
        for (int c = 0; c < 4; ++c) mg[(4 * d + c) * 64] = o[d][c];
      mg[64 * 64] = m_ref;
      mg[65 * 64] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = mg[64 * 64], l1 = mg[65 * 64];
      const float M = fmaxf(m_ref, m1);
      const float f0 = m_ref == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
      const float f1 = m1 == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
      for (int d = 0; d < 16; ++d)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[d][c] = o[d][c] * f0 + mg[(4 * d + c) * 64] * f1;
      l_run = l_run * f0 + l1 * f1;
      m_ref = M;
    }
  }
  if (grp != 0) return;
  if (!head_ok) return;
  if (P.S == 1) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float4* dst = reinterpret_cast<float4*>(P.out + ((int64_t)row * P.H + head) * kLatent) + 64 * dh;
#pragma unroll
    for (int d = 0; d < 16; ++d)
      dst[4 * d + g] = make_float4(o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv);
    if (P.lse && g == 0 && dh == 0)
      P.lse[(int64_t)row * P.H + head] =
          l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : -__builtin_huge_valf();
    return;
  }
  const int64_t ph = ((int64_t)row * P.H + head) * P.S + sp;
  float4* po = reinterpret_cast<float4*>(P.part_o + ph * kLatent) + 64 * dh;
#pragma unroll
  for (int d = 0; d < 16; ++d)
    __builtin_nontemporal_store(v4f{o[d][0], o[d][1], o[d][2], o[d][3]}, reinterpret_cast<v4f*>(po + 4 * d + g));
  if (g == 0 && dh == 0) {
    P.part_ml[2 * ph] = m_ref;
    P.part_ml[2 * ph + 1] = l_run;
  }
}

// Combines the S partials of every (row, head) in split order.  A thread takes
// V consecutive dims of one head (512/V threads per head), so a block of 256
// threads covers 2 heads for V = 4 and 4 heads for V = 8.  V = 4 is used when
// the V = 8 grid would have fewer blocks than the chip has CUs (one row of
// 128 heads: 32 blocks): twice the blocks put more loads in flight (0.4 us
// less per call for one row of 128 heads in eight splits); with a block per
// CU the two measure the same.  The arithmetic per element is the same for
// both.
// SMAX is the most splits the block holds in registers (8, or 16 for a batch
// of a few rows whose lists are cut into two steps per split).
template <int V, int SMAX>
__global__ __launch_bounds__(kCombineThreads) void sfa_combine_kernel(Params P) {
  constexpr int kF4 = V / 4;                          // float4 per thread
  constexpr int kTPH = kLatent / V;                   // threads per head
  const int row = blockIdx.x, h = (kCombineThreads / kTPH) * blockIdx.y + threadIdx.x / kTPH;
  const int c = threadIdx.x % kTPH;
  if (h >= P.H) return;
  const int64_t ph0 = ((int64_t)row * P.H + h) * P.S;
  // every split's loads first (S <= SMAX), then the fixed-order sums
  float2 ml[SMAX];
  float4 x[SMAX][kF4];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    if (s < P.S) {
      ml[s] = reinterpret_cast<const float2*>(P.part_ml)[ph0 + s];
      const float4* src = reinterpret_cast<const float4*>(P.part_o + (ph0 + s) * kLatent) + kF4 * c;
#pragma unroll
      for (int f = 0; f < kF4; ++f) x[s][f] = src[f];
    }
  }
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < SMAX; ++s)
    if (s < P.S) M = fmaxf(M, ml[s].x);
  float L = 0.f;
  float4 a[kF4];
#pragma unroll
  for (int f = 0; f < kF4; ++f) a[f] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    if (s >= P.S) continue;
    const float m = ml[s].x;
    const float w = (M == -__builtin_huge_valf() || m == -__builtin_huge_valf()) ? 0.f : exp2f(m - M);
    L += w * ml[s].y;
#pragma unroll
    for (int f = 0; f < kF4; ++f) {
      a[f].x += w * x[s][f].x; a[f].y += w * x[s][f].y;
      a[f].z += w * x[s][f].z; a[f].w += w * x[s][f].w;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float4* dst = reinterpret_cast<float4*>(P.out + ((int64_t)row * P.H + h) * kLatent) + kF4 * c;
#pragma unroll
  for (int f = 0; f < kF4; ++f)
    dst[f] = make_float4(a[f].x * inv, a[f].y * inv, a[f].z * inv, a[f].w * inv);
  if (P.lse && c == 0)
    P.lse[(int64_t)row * P.H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -__builtin_huge_valf();
}

struct Plan {
  int S, per_split, hg;
};

Plan plan_for(int R, int H, int topk) {
  Plan p;
  p.hg = (H + kHeadsWG - 1) / kHeadsWG;
  // splits are whole steps of the two-group form (64 records)
  constexpr int kSplitTok = Cfg<2>::kStepTok;
  const int steps = (topk + kSplitTok - 1) / kSplitTok;
  const int64_t groups = (int64_t)R * p.hg;
  int S = (int)std::min<int64_t>((kTargetWgs + groups - 1) / groups, (int64_t)steps);
  S = std::max(1, std::min(S, kMaxSplits));
  const int steps_per = (steps + S - 1) / S;
  p.per_split = steps_per * kSplitTok;
  p.S = (topk + p.per_split - 1) / p.per_split;
  return p;
}

struct Layout {
  size_t err, zero, part_ml, part_o, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout layout_for(int R, int H, int topk) {
  const Plan p = plan_for(R, H, topk);
  Layout L;
  size_t off = 0;
  L.err = off; off += 256;
  L.zero = off; off += kZeroBytes;
  const bool split = p.S > 1;
  const size_t heads = (size_t)R * H;
  L.part_ml = off; off += split ? align256(heads * p.S * 2 * 4) : 0;
  L.part_o = off; off += split ? align256(heads * p.S * kLatent * 4) : 0;
  L.total = off;
  return L;
}

}  // namespace

extern "C" size_t dsa_sparse_attn_workspace_size(int32_t R, int32_t H, int32_t topk) {
  if (R <= 0 || H <= 0 || topk <= 0) return 256 + kZeroBytes;
  return layout_for(R, H, topk).total;
}

extern "C" int dsa_sparse_attn(const void* q_bf16, const void* kv_pool, int64_t pool_pages,
                               const int32_t* block_table, int32_t bt_stride,
                               const int32_t* row_seq, const int32_t* idx, int32_t R, int32_t H,
                               int32_t topk, float softmax_scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_bf16 || !kv_pool || !block_table || !row_seq || !idx || !out) return DSA_ERR_INVALID_ARG;
  if (R < 0 || bt_stride <= 0 || pool_pages <= 0) return DSA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > DSA_MAX_ATTN_HEADS) return DSA_ERR_UNSUPPORTED;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (pool_pages > (int64_t(1) << 25)) return DSA_ERR_UNSUPPORTED;   // slots fit int32
  if (R == 0) return DSA_OK;
  const Layout L = layout_for(R, H, topk);
  if (workspace == nullptr || workspace_bytes < L.total) return DSA_ERR_WORKSPACE;
  const Plan pl = plan_for(R, H, topk);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Params P{};
  P.q = static_cast<const uint16_t*>(q_bf16);
  P.pool = static_cast<const uint8_t*>(kv_pool);
  P.pool_pages = pool_pages;
  P.bt = block_table;
  P.bt_stride = bt_stride;
  P.row_seq = row_seq;
  P.idx = idx;
  P.R = R;
  P.H = H;
  P.topk = topk;
  P.scale_log2 = softmax_scale * kLog2e;
  P.out = out;
  P.lse = lse;
  P.S = pl.S;
  P.per_split = pl.per_split;
  P.HGn = pl.hg;
  P.err = reinterpret_cast<uint32_t*>(ws + L.err);
  P.zero = ws + L.zero;
  P.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
  P.part_o = reinterpret_cast<float*>(ws + L.part_o);
  const int64_t grid = (int64_t)R * pl.hg * pl.S;
  if (grid > 0x7FFFFFFF) return DSA_ERR_UNSUPPORTED;
  hipStream_t s = dsa_host::as_stream(stream);
  // one group (two work-groups per CU) for lists taken whole, two for
  // splits (one group there would need twice the splits, and partials, for
  // chains as short: decode 128K x 8 26.0 -> 31.1 us per call)
  if (pl.S == 1)
    hipLaunchKernelGGL(sfa_kernel<1>, dim3((unsigned)grid), dim3(Cfg<1>::kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(sfa_kernel<2>, dim3((unsigned)grid), dim3(Cfg<2>::kThreads), 0, s, P);
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  if (pl.S > 1) {
    // V = 8 needs a block per CU and at most 8 splits; more than 8 splits
    // only arise with fewer than 32 (row, head group) pairs, where V = 4
    // is the faster form anyway
    const bool wide = (int64_t)R * ((H + 3) / 4) >= 256 && pl.S <= kWideSplits;
    const dim3 g4((unsigned)R, (unsigned)((H + 1) / 2));
    if (wide)
      hipLaunchKernelGGL((sfa_combine_kernel<8, kWideSplits>), dim3((unsigned)R, (unsigned)((H + 3) / 4)), dim3(kCombineThreads), 0, s, P);
    else if (pl.S <= kWideSplits)
      hipLaunchKernelGGL((sfa_combine_kernel<4, kWideSplits>), g4, dim3(kCombineThreads), 0, s, P);
    else
      hipLaunchKernelGGL((sfa_combine_kernel<4, kMaxSplits>), g4, dim3(kCombineThreads), 0, s, P);
    if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}
