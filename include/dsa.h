/*
 * dsa.h - C ABI of the MI355X (gfx950) DSA hot path library
 *         (libdsa_mi355x.so, built from sparse_attention_decode_topk_amd/csrc).
 *
 * DeepSeek-style sparse attention in two stages: a Lightning Indexer scores
 * every causal history position of each query and keeps the Top-K; Sparse
 * Flash Attention then attends only to those positions of an MLA latent
 * cache ("Deep Dive into Sparse Attention and Engineering Optimizations for
 * Efficient Inference in Kimi K3.1 Pro", section 1 "Hybrid Architecture";
 * "Kimi K3.1 Pro Inference Acceleration: Day0 Optimization on Heterogeneous
 * AI Hardware", sections "Lightning Indexer Three-Stream Coordination",
 * "Full MXFP8 Quantization ...", "FP8 KVCache ..." and "Preserving a
 * Mixed-Precision Path").
 *
 * Conventions shared by every entry point
 *  - Memory: every array argument is a DEVICE pointer owned by the caller.
 *    The library allocates nothing and keeps no pointer after returning.
 *  - Execution: work is enqueued asynchronously on `stream` (a hipStream_t
 *    passed as void*; NULL = the null stream).  No call synchronises.
 *  - Return value: DSA_OK, or an error code returned BEFORE any device work
 *    is enqueued (argument checks are pure host code), or DSA_ERR_HIP when a
 *    launch fails.  Faults inside kernels surface at the caller's next
 *    synchronisation, as usual for HIP.
 *  - Inputs must be finite.  bf16/fp32 arrays are little-endian, row-major.
 *  - Threads: entry points are re-entrant; two calls that share a workspace
 *    must not run concurrently.
 *
 * Cache layouts (one block table of physical page ids serves both caches;
 * token s of sequence b lives in page block_table[b*bt_stride + s/64] at
 * offset s%64):
 *  - indexer K page, DSA_K_PAGE_BYTES = 8448 bytes, in tiles of 16 tokens:
 *      bytes [0, 8192): codes, tile j (tokens 16j..16j+15) at 2048j; code d
 *        of the tile's token n at 1024*(d/64) + 256*((d%64)/16) + 16*n + d%16
 *        (16-byte pieces of the 16 tokens side by side, dims 0-15, 16-31,
 *        32-47, 48-63, then the same for dims 64-127);
 *      bytes [8192, 8448): E8M0 scales, tile j at 8192 + 64j; byte b (dims
 *        32b..32b+31) of the tile's token n at 16*b + n.
 *    (A 16-token MFMA operand then reads one contiguous kilobyte per load.)
 *  - SFA KV record, DSA_KV_RECORD_BYTES = 656 bytes per token (slot p*64+o
 *    at byte offset (p*64+o)*656 of the pool):
 *      [512 E4M3 latent codes][4 x fp32 tile scales][64 x bf16 rope]
 *  E4M3 is the OCP "FN" variant (max 448, no infinities); E8M0 is 2^(E-127).
 */
#ifndef DSA_MI355X_H
#define DSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_OK              0
#define DSA_ERR_INVALID_ARG 1  /* null pointer, non-positive size, bad stride */
#define DSA_ERR_UNSUPPORTED 2  /* a dimension the kernels are not built for   */
#define DSA_ERR_WORKSPACE   3  /* workspace missing or smaller than required  */
#define DSA_ERR_HIP         4  /* a HIP launch/runtime call failed            */

#define DSA_PAGE_TOKENS      64
#define DSA_INDEX_DIM        128
#define DSA_MX_GROUP         32
#define DSA_K_PAGE_BYTES     8448
#define DSA_LATENT_DIM       512
#define DSA_ROPE_DIM         64
#define DSA_KV_TILE          128
#define DSA_KV_RECORD_BYTES  656
#define DSA_KV_PAGE_BYTES    41984
#define DSA_MAX_TOPK         2048
#define DSA_MAX_INDEX_HEADS  64
#define DSA_MAX_ATTN_HEADS   128

/* Human-readable name of a status code (static string, never NULL). */
const char* dsa_status_str(int status);

/* Library version, major*10000 + minor*100 + patch. */
int dsa_version(void);

/*
 * MXFP8 quantisation of bf16 rows: every 32 consecutive elements share one
 * E8M0 scale X = 2^e, e the smallest integer with amax <= 448*2^e (clamped
 * to [-127,127]; e = 0 when amax is 0), and each element becomes the E4M3
 * code of x/X rounded to nearest-even, saturating.  Defined for the indexer
 * by "Full MXFP8 Quantization with Per-Group Dynamic Scaling for LI" (Kimi
 * K3.1 Pro Day0 page; group size 32) and "2. Memory Optimization" of the
 * "Deep Dive into Sparse Attention" page.
 *
 *   x_bf16   [rows, cols] bf16, cols % 32 == 0 (cols <= 65536)
 *   Contiguous mode (indexer q): out_fp8 [rows, cols] E4M3 and
 *     out_e8m0 [rows, cols/32] non-NULL; k_pool and slot_mapping NULL.
 *   Paged mode (indexer k written into the K cache): cols == 128, k_pool and
 *     slot_mapping [rows] (int64) non-NULL, out_* NULL; row i goes to slot
 *     slot_mapping[i]; slots < 0 or >= pool_pages*64 are skipped.
 */
int mxfp8_quant(const void* x_bf16, int64_t rows, int32_t cols,
                void* out_fp8, void* out_e8m0,
                void* k_pool, const int64_t* slot_mapping, int64_t pool_pages,
                void* stream);

/*
 * FP8 quantisation of KV rows into the paged SFA cache: each token's
 * 512-wide latent is cut into four tiles of 128; a tile's scale is the IEEE
 * float32 quotient amax/448 (1.0 when amax is 0) and each element becomes
 * the E4M3 code of the float32 quotient x/scale, nearest-even, saturating.
 * The 64-wide rope part is copied as bf16.  Defined by "FP8 KVCache with
 * Per-Token-Head-Tile Quantization for SFA" (Kimi K3.1 Pro Day0 page, tile
 * 128) and the multi-stream note that KV writes happen during decode
 * ("System-Level Coordination", same page).
 *
 *   kv_bf16       [n_tokens, 576] bf16 = latent 512 | rope 64
 *   slot_mapping  [n_tokens] int64; slots < 0 or >= pool_pages*64 skipped
 *   kv_pool       pool of pool_pages pages of 41984 bytes
 */
int kv_fp8_quant_paged_write(const void* kv_bf16, int64_t n_tokens,
                             const int64_t* slot_mapping, void* kv_pool,
                             int64_t pool_pages, void* stream);

/*
 * The quantisations of one decode step in a single launch (the fused-prolog
 * direction of "Lightning Indexer Three-Stream Coordination" and "System-
 * Level Coordination", Kimi K3.1 Pro Day0 page: the quantisation prolog was
 * a serial wait before the indexer).  Results are bit-identical to
 *   mxfp8_quant(q_bf16, q_rows, q_cols, q_fp8, q_e8m0, NULL, NULL, 0)
 *   mxfp8_quant(k_bf16, n_tokens, 128, NULL, NULL, k_pool, slot_mapping, pool_pages)
 *   kv_fp8_quant_paged_write(kv_bf16, n_tokens, slot_mapping, kv_pool, pool_pages)
 * with the same rules for skipped slots.  The K and KV caches share page ids
 * (one slot_mapping, one pool_pages for both).  n_tokens may be 0 (then the
 * k/kv/slot/pool arguments may be NULL).
 */
int dsa_decode_prolog(const void* q_bf16, int64_t q_rows, int32_t q_cols,
                      void* q_fp8, void* q_e8m0,
                      const void* k_bf16, const void* kv_bf16, int64_t n_tokens,
                      const int64_t* slot_mapping, void* k_pool, void* kv_pool,
                      int64_t pool_pages, void* stream);

/*
 * Bytes of workspace dsa_indexer_topk needs for R query rows whose block
 * tables have bt_stride entries.
 */
size_t dsa_indexer_topk_workspace_size(int32_t R, int32_t bt_stride,
                                       int32_t H_I, int32_t topk);

/*
 * Lightning Indexer with fused head weighting and Top-K, no score matrix in
 * HBM ("Deep Dive into Sparse Attention", section "1. Computation
 * Optimization: ... DSA Fused Kernel"; Kimi K3.1 Pro Day0 page, "Lightning
 * Indexer Three-Stream Coordination").  Two launches per 1024 rows on the
 * caller's stream: a scan that scores the K pages and keeps each 1024-position
 * unit's candidates (keys at or above a per-unit edge), then a select that
 * takes the exact Top-K of every row from them.  The second launch starts
 * when the first has drained (at 8 rows of 128K positions: about 33 us of
 * scan, then about 7 us of select); no work-group waits on another inside a
 * launch.
 *
 *   I(t,s) = sum_h w[r,h] * max(0, q[r,h] . k[s]),  0 <= s <= t = row_pos[r]
 *
 * over the dequantised MXFP8 q and k; keeps the topk largest scores, ties
 * broken by the lower position; writes the kept positions in ascending
 * order, padded with -1 when fewer than topk positions exist.
 *
 *   q_fp8      [R, H_I, 128] E4M3      q_e8m0 [R, H_I, 4] E8M0
 *   w          [R, H_I] fp32 head weights
 *   k_pool     indexer K cache, pool_pages pages of 8448 bytes
 *   block_table[B, bt_stride] int32 page ids; row_seq[R] int32 selects the
 *              sequence (row of block_table); row_pos[R] int32 is t
 *   H_I        1..64;  topk 1..2048
 *   out_idx    [R, topk] int32 ascending positions, then -1
 *   out_score  [R, topk] fp32 scores aligned with out_idx (-inf padding);
 *              may be NULL
 *   workspace  >= dsa_indexer_topk_workspace_size(...) bytes.  Its
 *              contents need no initialisation: every call writes what it
 *              reads.  Bytes [8,12) hold a sticky status word that the
 *              kernels only OR bits into (the caller clears it to start
 *              afresh and reads it after the call): bit 2 = a page id
 *              outside [0, pool_pages) was skipped, bit 3 = a row needed
 *              the exact rescoring path (informational).
 * Results are exact and deterministic (no floating-point atomics).  A page id
 * outside [0, pool_pages) or a row with row_pos < 0 contributes no positions.
 * block_table widths up to 16384 pages (1M tokens) are supported.
 */
int dsa_indexer_topk(const void* q_fp8, const void* q_e8m0, const float* w,
                     const void* k_pool, int64_t pool_pages,
                     const int32_t* block_table, int32_t bt_stride,
                     const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                     int32_t H_I, int32_t topk,
                     int32_t* out_idx, float* out_score,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes exactly what dsa_indexer_topk
 * computes (the same kernels) and allocates nothing: its workspace is a
 * 64 MiB array inside the library, one per GPU, held until the process ends.
 *   - Limit: the workspace dsa_indexer_topk_workspace_size(R, bt_stride, ...)
 *     reports must be at most 64 MiB (e.g. 32 rows of 1024 pages, or 8 rows
 *     of 2048 pages, need 16.8 MB / 8.4 MB); larger launches return
 *     DSA_ERR_WORKSPACE before any device work.
 *   - Every call on a GPU shares that GPU's array: calls that overlap on one
 *     GPU (two streams, two host threads) race and must be serialised by the
 *     caller.  Nothing in the array has to start at zero; the status bits of
 *     dsa_indexer_topk's workspace word are kept there and not reported.
 *   - The first call on each device looks up the array's device address
 *     (no allocation) and returns DSA_ERR_HIP if that fails.
 */
int dsa_indexer_topk_noalloc(const void* q_fp8, const void* q_e8m0, const float* w,
                             const void* k_pool, int64_t pool_pages,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                             int32_t H_I, int32_t topk, int32_t* out_idx, float* out_score,
                             void* stream);

/*
 * One decode step's indexer with the quantisation prolog folded into the
 * same launch ("Lightning Indexer Three-Stream Coordination" and "System-
 * Level Coordination", Kimi K3.1 Pro Day0 page: Q quantisation feeds the
 * scoring directly, and the KV-cache writes of the new token happen during
 * the step instead of as a serial prolog).  Row r brings its new token: the
 * bf16 indexer key k_new[r], the bf16 KV row kv_new[r] and its cache slot
 * slot_mapping[r] (int64).  The call computes exactly what
 *   dsa_decode_prolog(q_bf16, R*H_I, 128, q_fp8, q_e8m0, k_new, kv_new, R,
 *                     slot_mapping, k_pool, kv_pool, pool_pages)
 *   dsa_indexer_topk(q_fp8, q_e8m0, w, k_pool, ...)
 * computes (same cache bytes written, same indices and scores bit for bit),
 * in the launches of dsa_indexer_topk alone:
 *   - the queries are quantised to MXFP8 inside the scan (no q_fp8 array);
 *   - the new keys and KV records are written into the caches by the scan
 *     (read by later launches), and each row's new key is scored from the
 *     launch's own copy.
 * Preconditions: slot_mapping[r] is the slot of position row_pos[r] of
 * sequence row_seq[r] (the decode token at the row's causal limit), and the
 * rows name distinct sequences (multi-query groups and prefill chunks use
 * dsa_decode_prolog and dsa_indexer_topk_mq / _seq).  A slot < 0 or >=
 * pool_pages*64 means the row writes nothing and position row_pos[r] is
 * scored from the cache as it is.
 *
 *   q_bf16       [R, H_I, 128] bf16 indexer queries
 *   k_new_bf16   [R, 128] bf16;  kv_new_bf16 [R, 576] bf16 (latent | rope)
 *   k_pool, kv_pool  the two caches (pool_pages pages each), written
 *   other arguments, outputs and status bits as for dsa_indexer_topk; the
 *   workspace is sized by dsa_indexer_topk_workspace_size.
 */
int dsa_decode_indexer_topk(const void* q_bf16, const float* w, const void* k_new_bf16,
                            const void* kv_new_bf16, const int64_t* slot_mapping,
                            void* k_pool, void* kv_pool, int64_t pool_pages,
                            const int32_t* block_table, int32_t bt_stride,
                            const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                            int32_t H_I, int32_t topk, int32_t* out_idx, float* out_score,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace dsa_indexer_topk_seq needs for R query rows of a
 * sequence of n_pages pages.  The rows are taken in launches of at most 4096
 * rows, and of few enough that a launch's candidate region (8 bytes per
 * history slot of every row) stays within 512 MiB: about 537 MB at 2048
 * pages (512 rows per launch), whatever R is.
 */
size_t dsa_indexer_topk_seq_workspace_size(int32_t R, int32_t n_pages,
                                           int32_t H_I, int32_t topk);

/*
 * dsa_indexer_topk for R query rows that all belong to ONE sequence: a chunk
 * of a causal prefill (each query scores its own history, "Lightning Indexer
 * ... scores every causal history position" with the triangular workload of
 * the chunked-prefill case) or the several query tokens of one sequence.  The
 * rows are taken in tiles of 8 consecutive rows; one wave scores one 16-page
 * unit for a pair of rows of a tile, and the four pairs of a unit run side
 * by side in one work-group, so the unit's pages are streamed together.
 * Every work item is one unit of one pair, so the triangle's long rows do
 * not leave a tail of long work items (the load-balancing concern of the
 * pages' context-parallel zigzag split, "Adapting and Optimizing Kimi K3.1
 * Pro for Long-Sequence Inference", met on one GPU by that granularity).
 *
 *   block_table_row [n_pages] int32 page ids of the sequence (n_pages <= 4096)
 *   row_pos         [R] int32, t of each row (any order; < 0 = no positions)
 *   other arguments, outputs, status bits and workspace rules as for
 *   dsa_indexer_topk, with the workspace from
 *   dsa_indexer_topk_seq_workspace_size.
 * Scores are computed with the same operations in the same order as
 * dsa_indexer_topk, so both entry points return identical bits.
 */
int dsa_indexer_topk_seq(const void* q_fp8, const void* q_e8m0, const float* w,
                         const void* k_pool, int64_t pool_pages,
                         const int32_t* block_table_row, int32_t n_pages,
                         const int32_t* row_pos, int32_t R, int32_t H_I,
                         int32_t topk, int32_t* out_idx, float* out_score,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk for multi-query decode: each of B sequences brings
 * q_per_seq consecutive query rows, as when the target model verifies
 * several drafted tokens in one pass (speculative decoding: "Deep Dive into
 * Sparse Attention", section "3. Decoding Phase Optimization"; Day0 page,
 * "System-Level Coordination").  Rows
 * r = b*q_per_seq .. b*q_per_seq + q_per_seq - 1 form one tile whose K pages
 * are read once per pair of rows (one wave scores a 16-page unit for two
 * rows of the tile; the pairs of one unit run side by side in one
 * work-group); each row keeps its own causal limit row_pos[r] and its own
 * Top-K.
 *
 *   R          B * q_per_seq (a multiple of q_per_seq, else
 *              DSA_ERR_INVALID_ARG);  q_per_seq 1..8
 *   row_seq    [R] int32; the rows of one tile must name the same sequence
 *              (the tile reads the pages of its first row's sequence; a tile
 *              whose rows differ sets status bit 4 and is scored against
 *              those pages)
 *   bt_stride  <= 4096 pages (256K tokens)
 *   other arguments, outputs, status bits and workspace (sized by
 *   dsa_indexer_topk_workspace_size) as for dsa_indexer_topk.
 * Scores are computed with the same operations in the same order as
 * dsa_indexer_topk, so both entry points return identical bits.
 */
int dsa_indexer_topk_mq(const void* q_fp8, const void* q_e8m0, const float* w,
                        const void* k_pool, int64_t pool_pages,
                        const int32_t* block_table, int32_t bt_stride,
                        const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                        int32_t q_per_seq, int32_t H_I, int32_t topk,
                        int32_t* out_idx, float* out_score,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * TEST ONLY: the full score rows of dsa_indexer_topk, computed by the same
 * device code: out_scores[r*ld + s] = I(t,s) for s <= t, -inf for
 * t < s < ld.  Requires ld >= max(row_pos)+1 (positions beyond ld are not
 * written).  Arguments as for dsa_indexer_topk.
 */
int dsa_indexer_scores(const void* q_fp8, const void* q_e8m0, const float* w,
                       const void* k_pool, int64_t pool_pages,
                       const int32_t* block_table, int32_t bt_stride,
                       const int32_t* row_seq, const int32_t* row_pos, int32_t R,
                       int32_t H_I, float* out_scores, int64_t ld, void* stream);

/* Bytes of workspace dsa_sparse_attn needs (zeroed once before first use). */
size_t dsa_sparse_attn_workspace_size(int32_t R, int32_t H, int32_t topk);

/*
 * Sparse Flash Attention over the selected positions ("Deep Dive into
 * Sparse Attention", section 1; "Adapting and Optimizing Kimi K3.1 Pro for
 * Long-Sequence Inference", section 2: gather by the indices of the
 * previous step, then attention):
 *
 *   z_j = scale * (q[r,h,:512] . latent_j + q[r,h,512:] . rope_j)
 *   out[r,h,:] = sum_j softmax(z)_j * latent_j ,  lse[r,h] = ln sum_j e^{z_j}
 *
 * latent_j = E4M3 codes times their tile scale, rope_j bf16, for every entry
 * j of idx[r,:] that is >= 0 (duplicates count as listed); no other mask.
 *
 *   q_bf16     [R, H, 576] bf16 (latent 512 | rope 64)
 *   kv_pool    SFA cache, pool_pages pages of 41984 bytes
 *   idx        [R, topk] int32 positions of sequence row_seq[r]; -1 = skip
 *   H          1..128;  topk 1..2048
 *   softmax_scale  the logit scale (1/sqrt(576) for this model)
 *   out        [R, H, 512] fp32;  lse [R, H] fp32 (may be NULL)
 *   A row with no valid entry gets out = 0 and lse = -inf.  Entries whose
 *   position maps to no page, or to a page id outside [0, pool_pages), are
 *   skipped and set bit 0 of the status word at workspace bytes [0,4).
 *   workspace  >= dsa_sparse_attn_workspace_size(...) bytes, zero-filled once
 *              by the caller before first use: bytes [256, 1280) must stay
 *              zero (no call writes them); the rest holds per-call partial
 *              results.
 * Results are deterministic (splits are combined in a fixed order).
 */
int dsa_sparse_attn(const void* q_bf16, const void* kv_pool, int64_t pool_pages,
                    const int32_t* block_table, int32_t bt_stride,
                    const int32_t* row_seq, const int32_t* idx, int32_t R,
                    int32_t H, int32_t topk, float softmax_scale,
                    float* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement utility (not part of the hot path): reads `bytes` (a multiple
 * of 16) from the device buffer `src` once with streaming 16-byte loads on
 * `grid` work-groups of 256 threads and writes one folded word per
 * work-group to out[grid] (device, caller-owned).  Its duration gives the
 * plain streaming-read bandwidth of the GPU, the practical ceiling next to
 * the HBM datasheet figure for the indexer's K-cache scan ("Adapting and
 * Optimizing Kimi K3.1 Pro for Long-Sequence Inference", section 3: memory
 * bandwidth is one of the primary bottlenecks of long sequences).
 */
int dsa_probe_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_MI355X_H */
