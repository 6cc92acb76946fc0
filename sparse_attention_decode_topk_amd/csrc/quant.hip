// MXFP8 quantisation (indexer q / paged indexer k) and FP8 per-tile KV
// quantisation into the paged SFA cache.
//
// MXFP8: one E8M0 scale per 32 elements ("Full MXFP8 Quantization with
// Per-Group Dynamic Scaling for LI", Kimi K3.1 Pro Day0 page).  KV: one fp32
// scale amax/448 per 128-element tile of each token's latent, rope kept in
// bf16 ("FP8 KVCache with Per-Token-Head-Tile Quantization for SFA" and
// "Preserving a Mixed-Precision Path", same page).
#include "quant_dev.hpp"

namespace {

using namespace dsa;

__global__ __launch_bounds__(256) void mxfp8_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int cols, uint8_t* __restrict__ out,
    uint8_t* __restrict__ out_scale, uint8_t* __restrict__ kpool,
    const int64_t* __restrict__ slots, int64_t pool_slots) {
  mxfp8_quant_range((int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x,
                    x, rows, cols, out, out_scale, kpool, slots, pool_slots);
}

__global__ __launch_bounds__(256) void kv_quant_kernel(
    const uint16_t* __restrict__ kv, int64_t n, const int64_t* __restrict__ slots,
    uint8_t* __restrict__ pool, int64_t pool_slots) {
  kv_quant_range((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6),
                 (int64_t)gridDim.x * (blockDim.x >> 6), kv, n, slots, pool, pool_slots);
}

// The decode step's three quantisations in one launch: blocks [0, nb_q)
// quantise the indexer queries, the next nb_k blocks write the new indexer
// keys into the K cache, the remaining blocks write the new KV records.
struct PrologParams {
  const uint16_t* q;      // [q_rows, q_cols] bf16
  int64_t q_rows;
  int q_cols;
  uint8_t* q_fp8;
  uint8_t* q_e8m0;
  const uint16_t* k;      // [n, 128] bf16
  const uint16_t* kv;     // [n, 576] bf16
  int64_t n;
  const int64_t* slots;   // [n]
  uint8_t* k_pool;
  uint8_t* kv_pool;
  int64_t pool_slots;
  int nb_q, nb_k;
};

__global__ __launch_bounds__(256) void prolog_kernel(PrologParams P) {
  const int b = blockIdx.x;
  if (b < P.nb_q) {
    mxfp8_quant_range((int64_t)b * 256 + threadIdx.x, (int64_t)P.nb_q * 256, P.q, P.q_rows, P.q_cols,
                      P.q_fp8, P.q_e8m0, nullptr, nullptr, 0);
  } else if (b < P.nb_q + P.nb_k) {
    const int bk = b - P.nb_q;
    mxfp8_quant_range((int64_t)bk * 256 + threadIdx.x, (int64_t)P.nb_k * 256, P.k, P.n, kIdxDim,
                      nullptr, nullptr, P.k_pool, P.slots, P.pool_slots);
  } else {
    const int bv = b - P.nb_q - P.nb_k;
    const int nb_v = (int)gridDim.x - P.nb_q - P.nb_k;
    kv_quant_range((int64_t)bv * 4 + (threadIdx.x >> 6), (int64_t)nb_v * 4, P.kv, P.n, P.slots,
                   P.kv_pool, P.pool_slots);
  }
}

int grid_for(int64_t threads, int block) {
  int64_t g = (threads + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

}  // namespace

extern "C" int mxfp8_quant(const void* x_bf16, int64_t rows, int32_t cols, void* out_fp8,
                           void* out_e8m0, void* k_pool, const int64_t* slot_mapping,
                           int64_t pool_pages, void* stream) {
  if (x_bf16 == nullptr || rows < 0 || cols <= 0) return DSA_ERR_INVALID_ARG;
  if (cols % 32 != 0 || cols > 65536) return DSA_ERR_UNSUPPORTED;
  const bool paged = k_pool != nullptr || slot_mapping != nullptr;
  if (paged) {
    if (k_pool == nullptr || slot_mapping == nullptr || out_fp8 != nullptr || out_e8m0 != nullptr)
      return DSA_ERR_INVALID_ARG;
    if (cols != DSA_INDEX_DIM) return DSA_ERR_UNSUPPORTED;
    if (pool_pages <= 0) return DSA_ERR_INVALID_ARG;
  } else if (out_fp8 == nullptr || out_e8m0 == nullptr) {
    return DSA_ERR_INVALID_ARG;
  }
  if (rows == 0) return DSA_OK;
  const int64_t threads = rows * (cols / 8);
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3(grid_for(threads, 256)), dim3(256), 0,
                     dsa_host::as_stream(stream), static_cast<const uint16_t*>(x_bf16), rows,
                     (int)cols, static_cast<uint8_t*>(out_fp8), static_cast<uint8_t*>(out_e8m0),
                     static_cast<uint8_t*>(k_pool), slot_mapping,
                     paged ? pool_pages * DSA_PAGE_TOKENS : (int64_t)0);
  return dsa_host::launch_status(hipGetLastError());
}

extern "C" int kv_fp8_quant_paged_write(const void* kv_bf16, int64_t n_tokens,
                                        const int64_t* slot_mapping, void* kv_pool,
                                        int64_t pool_pages, void* stream) {
  if (kv_bf16 == nullptr || slot_mapping == nullptr || kv_pool == nullptr || n_tokens < 0 ||
      pool_pages <= 0)
    return DSA_ERR_INVALID_ARG;
  if (n_tokens == 0) return DSA_OK;
  hipLaunchKernelGGL(kv_quant_kernel, dim3(grid_for(n_tokens * 64, 256)), dim3(256), 0,
                     dsa_host::as_stream(stream), static_cast<const uint16_t*>(kv_bf16), n_tokens,
                     slot_mapping, static_cast<uint8_t*>(kv_pool), pool_pages * DSA_PAGE_TOKENS);
  return dsa_host::launch_status(hipGetLastError());
}

extern "C" int dsa_decode_prolog(const void* q_bf16, int64_t q_rows, int32_t q_cols,
                                 void* q_fp8, void* q_e8m0, const void* k_bf16,
                                 const void* kv_bf16, int64_t n_tokens,
                                 const int64_t* slot_mapping, void* k_pool, void* kv_pool,
                                 int64_t pool_pages, void* stream) {
  if (q_bf16 == nullptr || q_fp8 == nullptr || q_e8m0 == nullptr || q_rows < 0 || q_cols <= 0)
    return DSA_ERR_INVALID_ARG;
  if (q_cols % 32 != 0 || q_cols > 65536) return DSA_ERR_UNSUPPORTED;
  if (n_tokens < 0) return DSA_ERR_INVALID_ARG;
  if (n_tokens > 0 && (k_bf16 == nullptr || kv_bf16 == nullptr || slot_mapping == nullptr ||
                       k_pool == nullptr || kv_pool == nullptr || pool_pages <= 0))
    return DSA_ERR_INVALID_ARG;
  PrologParams P;
  P.q = static_cast<const uint16_t*>(q_bf16);
  P.q_rows = q_rows;
  P.q_cols = (int)q_cols;
  P.q_fp8 = static_cast<uint8_t*>(q_fp8);
  P.q_e8m0 = static_cast<uint8_t*>(q_e8m0);
  P.k = static_cast<const uint16_t*>(k_bf16);
  P.kv = static_cast<const uint16_t*>(kv_bf16);
  P.n = n_tokens;
  P.slots = slot_mapping;
  P.k_pool = static_cast<uint8_t*>(k_pool);
  P.kv_pool = static_cast<uint8_t*>(kv_pool);
  P.pool_slots = pool_pages * DSA_PAGE_TOKENS;
  P.nb_q = q_rows > 0 ? grid_for(q_rows * (q_cols / 8), 256) : 0;
  P.nb_k = n_tokens > 0 ? grid_for(n_tokens * (DSA_INDEX_DIM / 8), 256) : 0;
  const int nb_v = n_tokens > 0 ? grid_for(n_tokens * 64, 256) : 0;
  const int64_t grid = (int64_t)P.nb_q + P.nb_k + nb_v;
  if (grid == 0) return DSA_OK;
  hipLaunchKernelGGL(prolog_kernel, dim3((unsigned)grid), dim3(256), 0, dsa_host::as_stream(stream), P);
  return dsa_host::launch_status(hipGetLastError());
}
