// Sparse Flash Attention over the Top-K positions of an FP8 MLA latent
// cache ("Deep Dive into Sparse Attention ...", section 1; "Adapting and
// Optimizing Kimi K3.1 Pro for Long-Sequence Inference", section 2: gather
// the cache entries of the selected indices, then attention; Kimi K3.1 Pro
// Day0 page, "FP8 KVCache ..." and "Preserving a Mixed-Precision Path").
//
// One workgroup = (query row, group of 16 heads, split of the index list).
//  * up front, every entry of the split is translated position -> page ->
//    record slot in one parallel pass (slots kept in LDS);
//  * per 64-token tile: the 64 selected 656-byte records are fetched one
//    tile ahead into registers and staged in LDS (latent rows padded to 528
//    bytes);
//  * logits: wave w owns tokens 16w..16w+15.  S^T = K Q^T on
//    v_mfma_f32_16x16x32_bf16: E4M3 latent -> bf16 is exact, each 128-wide
//    tile accumulates separately and is multiplied by its fp32 tile scale in
//    fp32, the bf16 rope part adds on top; times softmax_scale*log2(e);
//  * online softmax shared by the four waves through LDS (fp32);
//  * P.V: wave w owns latent tile w (dims 128w..128w+127).  The tile scale
//    of every token is folded into P (P' = p * scale * 2^(8-E), E a running
//    power-of-two reference so P' stays well inside fp16), V is the exact
//    E4M3 code in f16, fetched transposed by ds_read_tr8_b64;
//    v_mfma_f32_16x16x32_f16 accumulates in fp32.
// Splits write (O, m, l) partials; the last split of a (row, head group)
// combines them in split order (deterministic).
#include <algorithm>

#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTile = 64;
constexpr int kHG = 16;                 // heads per workgroup
constexpr int kLatStride = 528;         // LDS bytes per staged latent row
constexpr int kPPStride = 72;           // fp16 per P' row (64 + 8 pad)
constexpr int kQStride = 584;           // bf16 per staged query row (576 + 8 pad)
constexpr int kChunks = kRec / 16;      // 41 16-byte pieces per record
constexpr int kLoads = (kTile * kChunks + kThreads - 1) / kThreads;   // 11
constexpr int kMaxTiles = DSA_MAX_TOPK / kTile;                       // 32
constexpr int kSlotsPerThread = kMaxTiles * kTile / kThreads;         // 8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 64;
constexpr int kTargetWgs = 512;

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
  int32_t S, per_split;   // splits and tokens per split (multiple of 64)
  float* part_o;          // [R*HG][S][16][512]
  float* part_ml;         // [R*HG][S][16][2]
  uint32_t* tick;         // [R*HG]
  uint32_t* err;
};

struct Smem {
  uint8_t lat[kTile * kLatStride];          // 33792 (combine: normalised split weights)
  uint16_t rope[kTile * kRope];             // 8192
  float scl[kTile * 4];                     // 1024
  _Float16 pp[4][kHG][kPPStride];           // P' per latent tile, 9216
  int32_t slot[kMaxTiles * kTile];          // record slot per entry of the split, -1 = none
  uint16_t qs[kHG * kQStride];              // the workgroup's 16 query rows (bf16), 18688
  float wmax[kWaves][kHG];
  float wsum[kWaves][kHG];
  float alpha[kHG];
  int32_t emax[4];
  uint32_t last;
};

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bits) {
  if (err) __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__global__ __launch_bounds__(kThreads, 2) void sfa_kernel(Params P) {
  __shared__ Smem S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hr = lane & 15, g = lane >> 4;
  const int HGn = (P.H + kHG - 1) / kHG;
  const int sp = blockIdx.x % P.S;
  const int hg = (blockIdx.x / P.S) % HGn;
  const int row = blockIdx.x / (P.S * HGn);
  const int seq = P.row_seq[row];
  const int32_t* idxrow = P.idx + (int64_t)row * P.topk;
  const int32_t* btrow = P.bt + (int64_t)seq * P.bt_stride;
  const int j0 = sp * P.per_split;
  const int jend = min(P.topk, j0 + P.per_split);
  const int ntiles = jend > j0 ? (jend - j0 + kTile - 1) / kTile : 0;

  // ---- record slots of every entry of the split (two dependent loads, all
  //      entries in flight together) ----
  {
    int32_t v[kSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int e = tid + i * kThreads;
      v[i] = (e < ntiles * kTile && j0 + e < jend) ? idxrow[j0 + e] : -1;
    }
    int32_t pid[kSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      pid[i] = -1;
      if (v[i] >= 0) {
        if ((v[i] >> 6) < P.bt_stride) pid[i] = btrow[v[i] >> 6];
        else flag(P.err, 1u);
      }
    }
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int e = tid + i * kThreads;
      int32_t s = -1;
      if (v[i] >= 0 && pid[i] >= 0 && (int64_t)pid[i] < P.pool_pages) s = pid[i] * kPage + (v[i] & 63);
      else if (v[i] >= 0 && (v[i] >> 6) < P.bt_stride) flag(P.err, 1u);
      if (e < kMaxTiles * kTile) S.slot[e] = s;
    }
  }

  // the 16 query rows of this head group, staged in LDS; as the B operand,
  // k-step (t, j) of head hr holds dims 128t + 32g + 8j .. +7 and rope step r
  // holds dims 512 + 32r + 8g .. +7
  const int head = kHG * hg + hr;
  const bool head_ok = head < P.H;
  for (int c = tid; c < kHG * (kQK / 8); c += kThreads) {
    const int h = c / (kQK / 8), part = c % (kQK / 8);
    const int hh = kHG * hg + h;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hh < P.H) v = *reinterpret_cast<const uint4*>(P.q + ((int64_t)row * P.H + hh) * kQK + 8 * part);
    *reinterpret_cast<uint4*>(S.qs + h * kQStride + 8 * part) = v;
  }
  auto qop = [&](int off) -> v8bf {
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(S.qs + hr * kQStride + off));
  };
  __syncthreads();

  // running softmax state of head hr (identical in every wave), running
  // power-of-two references of the four latent tiles (identical in every
  // wave), and this wave's output block: dims 128*wv + 16d + hr, heads 4g+c
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  int eref[4] = {-1000, -1000, -1000, -1000};
  v4f o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 buf[kLoads];
  auto issue_loads = [&](int it) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      buf[i] = make_uint4(0, 0, 0, 0);
      if (c < kTile * kChunks) {
        const int32_t s = S.slot[it * kTile + c / kChunks];
        if (s >= 0) buf[i] = *reinterpret_cast<const uint4*>(P.pool + (int64_t)s * kRec + (c % kChunks) * 16);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kTile * kChunks) {
        const int tok = c / kChunks, part = c % kChunks;
        if (part < 32)
          *reinterpret_cast<uint4*>(S.lat + tok * kLatStride + part * 16) = buf[i];
        else if (part == 32)
          *reinterpret_cast<uint4*>(S.scl + tok * 4) = buf[i];
        else
          *reinterpret_cast<uint4*>(S.rope + tok * kRope + (part - 33) * 8) = buf[i];
      }
    }
  };

  if (ntiles > 0) issue_loads(0);

  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();                      // previous tile fully consumed
    stage();
    __syncthreads();
    if (it + 1 < ntiles) issue_loads(it + 1);
    if (wv == 0) {
      // largest scale exponent of each latent tile over the tile's tokens:
      // positive fp32 bit patterns order like integers, so a wave-wide
      // integer max of the bits gives the largest scale
      const bool ok = S.slot[it * kTile + lane] >= 0;
      const uint4 sb = *reinterpret_cast<const uint4*>(S.scl + lane * 4);
      uint32_t m[4] = {ok ? sb.x : 0u, ok ? sb.y : 0u, ok ? sb.z : 0u, ok ? sb.w : 0u};
#pragma unroll
      for (int d = 1; d < 64; d <<= 1)
#pragma unroll
        for (int t = 0; t < 4; ++t) m[t] = max(m[t], (uint32_t)__shfl_xor((int)m[t], d));
      if (lane < 4) {
        const uint32_t b = lane == 0 ? m[0] : lane == 1 ? m[1] : lane == 2 ? m[2] : m[3];
        S.emax[lane] = (b & 0x7FFFFFFFu) ? (int)((b >> 23) & 0xFF) - 127 : -1000;
      }
    }

    // ---- logits of tokens 16wv .. 16wv+15 (lane: head hr, tokens 4g+c) ----
    const int tok_a = 16 * wv + hr;       // A-operand row of this lane
    v4f acc[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* src = S.lat + tok_a * kLatStride + 128 * t + 32 * g;
      const uint4 a0 = *reinterpret_cast<const uint4*>(src);
      const uint4 a1 = *reinterpret_cast<const uint4*>(src + 16);
      const uint32_t dw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * j], 1.0f, false);
        const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * j], 1.0f, true);
        const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * j + 1], 1.0f, false);
        const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw[2 * j + 1], 1.0f, true);
        const v8bf a = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop(128 * t + 32 * g + 8 * j), acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint4 v = *reinterpret_cast<const uint4*>(S.rope + tok_a * kRope + 32 * r + 8 * g);
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, v), qop(kLatent + 32 * r + 8 * g), acc[4], 0, 0, 0);
    }
    float z[4];
    float zmax = -__builtin_huge_valf();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int tok = 16 * wv + 4 * g + c;
      const float* sc = S.scl + tok * 4;
      float v = acc[4][c];
#pragma unroll
      for (int t = 0; t < 4; ++t) v = __builtin_fmaf(sc[t], acc[t][c], v);
      z[c] = S.slot[it * kTile + tok] >= 0 ? v * P.scale_log2 : -__builtin_huge_valf();
      zmax = fmaxf(zmax, z[c]);
    }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
    if (lane < 16) S.wmax[wv][hr] = zmax;
    __syncthreads();
    float m_new = m_run;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m_new = fmaxf(m_new, S.wmax[w][hr]);
    const bool any = m_new != -__builtin_huge_valf();
    const float alpha = any ? exp2f(m_run - m_new) : 1.0f;   // exp2(-inf) = 0
    float p[4], psum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      p[c] = any ? exp2f(z[c] - m_new) : 0.f;
      psum += p[c];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    if (lane < 16) S.wsum[wv][hr] = psum;
    if (wv == 0 && lane < 16) S.alpha[hr] = alpha;
    // running references: largest scale exponent seen so far per latent tile
    int eold_w = eref[0];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t == wv) eold_w = eref[t];
      eref[t] = max(eref[t], S.emax[t]);
    }
    // P' for every latent tile t: p * scale[t] * 2^(8 - Eref_t)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = eref[t];
      const float mul = e > -1000 ? pow2f(max(-126, min(127, 8 - e))) : 0.f;
      _Float16 h[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tok = 16 * wv + 4 * g + c;
        h[c] = (_Float16)(p[c] * S.scl[tok * 4 + t] * mul);
      }
      *reinterpret_cast<uint2*>(&S.pp[t][hr][16 * wv + 4 * g]) = __builtin_bit_cast(uint2, h);
    }
    __syncthreads();
    float tile_sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tile_sum += S.wsum[w][hr];
    l_run = alpha * l_run + tile_sum;
    m_run = m_new;

    // ---- P'.V for latent tile wv ----
    int enew_w = eref[0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t == wv) enew_w = eref[t];
    const float resc = (eold_w > -1000 && enew_w > eold_w) ? pow2f(max(-126, eold_w - enew_w)) : 1.0f;
    float al[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) al[c] = S.alpha[4 * g + c] * resc;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int c = 0; c < 4; ++c) o[d][c] *= al[c];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pa = *reinterpret_cast<const uint4*>(&S.pp[wv][hr][32 * ks + 8 * g]);
      const v8h a = __builtin_bit_cast(v8h, pa);
      typedef __attribute__((address_space(3))) v2i lds_v2i;
      const int vtok = 32 * ks + 8 * g + (hr >> 1);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint8_t* src = S.lat + vtok * kLatStride + 128 * wv + 16 * d + 8 * (hr & 1);
        const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_v2i*)((__attribute__((address_space(3))) uint8_t*)(src)));
        const v2h v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, false);
        const v2h v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, true);
        const v2h v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, false);
        const v2h v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, true);
        const v8h b = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, o[d], 0, 0, 0);
      }
    }
  }

  // ---- epilogue ----
  // o holds sum_j p_j * v_j / 2^(eref_w - 8) for heads 4g+c, dims 128wv+16d+hr
  int ew = eref[0];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t == wv) ew = eref[t];
  const float oscale = ew > -1000 ? pow2f(max(-126, min(127, ew - 8))) : 0.f;
  const int64_t pair = (int64_t)row * HGn + hg;
  if (P.S == 1) {
    // l and m of head 4g+c live in lanes whose hr == 4g+c: share via LDS
    __syncthreads();
    if (wv == 0 && lane < 16) { S.wsum[0][hr] = l_run; S.wmax[0][hr] = m_run; }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int hh = kHG * hg + 4 * g + c;
      if (hh >= P.H) continue;
      const float l = S.wsum[0][4 * g + c];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float* dst = P.out + ((int64_t)row * P.H + hh) * kLatent + 128 * wv + hr;
#pragma unroll
      for (int d = 0; d < 8; ++d) dst[16 * d] = o[d][c] * oscale * inv;
    }
    if (P.lse && wv == 0 && lane < 16 && head_ok) {
      P.lse[(int64_t)row * P.H + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -__builtin_huge_valf();
    }
    return;
  }
  // split: write partial (O, m, l), the last split of the pair combines
  float* po = P.part_o + (pair * P.S + sp) * (kHG * kLatent);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int d = 0; d < 8; ++d) po[(4 * g + c) * kLatent + 128 * wv + 16 * d + hr] = o[d][c] * oscale;
  if (wv == 0 && lane < 16) {
    float* pm = P.part_ml + (pair * P.S + sp) * (kHG * 2);
    pm[2 * hr] = m_run;
    pm[2 * hr + 1] = l_run;
  }
  wait_vm();
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    S.last = atomic_add_agent(&P.tick[pair], 1u) == (uint32_t)P.S - 1 ? 1u : 0u;
    if (S.last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!S.last) return;
  // normalised weights of every (split, head) in LDS; lse per head
  float* cw = reinterpret_cast<float*>(S.lat);        // [S][16]
  if (tid < kHG) {
    const int h = tid;
    const float* pm = P.part_ml + pair * P.S * (kHG * 2);
    float M = -__builtin_huge_valf();
    for (int s = 0; s < P.S; ++s) M = fmaxf(M, pm[(s * kHG + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < P.S; ++s) {
      const float m = pm[(s * kHG + h) * 2];
      const float wgt = (M == -__builtin_huge_valf() || m == -__builtin_huge_valf()) ? 0.f : exp2f(m - M);
      cw[s * kHG + h] = wgt;
      L += wgt * pm[(s * kHG + h) * 2 + 1];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    for (int s = 0; s < P.S; ++s) cw[s * kHG + h] *= inv;
    const int hh = kHG * hg + h;
    if (P.lse && hh < P.H)
      P.lse[(int64_t)row * P.H + hh] = L > 0.f ? (M + log2f(L)) * kLn2 : -__builtin_huge_valf();
  }
  __syncthreads();
  // 16 heads x 128 float4 per split; thread owns 8 float4 (q = tid + 256 j)
  const float4* src4 = reinterpret_cast<const float4*>(P.part_o + pair * P.S * (kHG * kLatent));
  float4 acc4[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < P.S; s0 += 4) {
    float4 v[4][8];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[ds][j] = (s0 + ds < P.S) ? src4[(s0 + ds) * (kHG * kLatent / 4) + tid + 256 * j]
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      if (s0 + ds >= P.S) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float wgt = cw[(s0 + ds) * kHG + (tid + 256 * j) / 128];
        acc4[j].x += wgt * v[ds][j].x;
        acc4[j].y += wgt * v[ds][j].y;
        acc4[j].z += wgt * v[ds][j].z;
        acc4[j].w += wgt * v[ds][j].w;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = tid + 256 * j;
    const int h = q / 128, col = q % 128;
    const int hh = kHG * hg + h;
    if (hh < P.H) reinterpret_cast<float4*>(P.out + ((int64_t)row * P.H + hh) * kLatent)[col] = acc4[j];
  }
  if (tid == 0) P.tick[pair] = 0;
}

struct Plan {
  int S, per_split, hg;
};

Plan plan_for(int R, int H, int topk) {
  Plan p;
  p.hg = (H + kHG - 1) / kHG;
  const int tiles = (topk + kTile - 1) / kTile;
  const int64_t pairs = (int64_t)R * p.hg;
  int S = (int)std::min<int64_t>((kTargetWgs + pairs - 1) / pairs, (int64_t)tiles);
  S = std::max(1, std::min(S, kMaxSplits));
  const int tiles_per = (tiles + S - 1) / S;
  p.per_split = tiles_per * kTile;
  p.S = (topk + p.per_split - 1) / p.per_split;
  return p;
}

struct Layout {
  size_t err, tick, part_ml, part_o, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout layout_for(int R, int H, int topk) {
  const Plan p = plan_for(R, H, topk);
  const int64_t pairs = (int64_t)R * p.hg;
  Layout L;
  size_t off = 0;
  L.err = off; off += 256;
  L.tick = off; off += align256((size_t)pairs * 4);
  const bool split = p.S > 1;
  L.part_ml = off; off += split ? align256((size_t)pairs * p.S * kHG * 2 * 4) : 0;
  L.part_o = off; off += split ? align256((size_t)pairs * p.S * kHG * kLatent * 4) : 0;
  L.total = off;
  return L;
}

}  // namespace

extern "C" size_t dsa_sparse_attn_workspace_size(int32_t R, int32_t H, int32_t topk) {
  if (R <= 0 || H <= 0 || topk <= 0) return 256;
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
  P.err = reinterpret_cast<uint32_t*>(ws + L.err);
  P.tick = reinterpret_cast<uint32_t*>(ws + L.tick);
  P.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
  P.part_o = reinterpret_cast<float*>(ws + L.part_o);
  const int64_t grid = (int64_t)R * pl.hg * pl.S;
  if (grid > 0x7FFFFFFF) return DSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(sfa_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     dsa_host::as_stream(stream), P);
  return dsa_host::launch_status(hipGetLastError());
}
