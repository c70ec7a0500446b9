/*
 * fp4idx: FP4 lightning-indexer hot path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp4idx.so. Every pointer argument marked "device" is a device address on the
 * current HIP device; the library never allocates, frees or synchronises. All calls are
 * asynchronous on `stream` (a hipStream_t; NULL is the legacy default stream) and results are
 * valid once the stream has reached the call. Arguments are validated on the host before any
 * HIP call; a failing call returns a negative status, enqueues nothing and records a message
 * for idx_last_error(). Nothing is thrown or aborted across this boundary.
 *
 * Sources, cited by page title and section:
 *  [P1] "DeepSeek-V4.1 model structure (3): sequence dimension, Hierarchical Sparse Indexer and
 *       FP4 KV cache" (blog.javazero.top)
 *  [P3] "DeepSeek-V4 model structure (2): Lightning Indexer and sparse selection" (xhh.club)
 *
 * Data layout shared by every entry point ("indexer rows"):
 *  - an indexer row is one 128-dim vector (a query head or a key) in MXFP4: 64 code bytes, two
 *    E2M1 codes per byte with element 2i in the low nibble of byte i, plus 4 UE8M0 scale bytes,
 *    one per group of 32 elements (byte value = exponent + 127, 0 .. 254; 255, the E8M0 NaN, is
 *    outside the contract) ([P1] "the scale format decides precision": groups of 32 with an E8M0
 *    scale, 4.25 bits per element, 68 bytes per key);
 *  - codes live in one array [rows][64] and scales in another [rows][4];
 *  - a query is 32 consecutive rows (heads 0..31), weights are fp32 [nq][32].
 */
#ifndef FP4IDX_H
#define FP4IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t idx_status;

#define IDX_OK 0
#define IDX_EINVAL (-1)        /* null pointer, negative size, inconsistent strides */
#define IDX_EALIGN (-2)        /* a device pointer is not aligned as documented */
#define IDX_EUNSUPPORTED (-3)  /* a parameter outside what the kernels implement */
#define IDX_EHIP (-4)          /* a HIP launch failed; the message names the HIP error */
#define IDX_EWORKSPACE (-5)    /* workspace missing or smaller than idx_workspace_size() */

#define IDX_ABI_VERSION 1

#define IDX_HEADS 32
#define IDX_DIM 128
#define IDX_MAX_K 2048

/* operation codes for idx_workspace_size */
#define IDX_OP_BUILD_POOL 1
#define IDX_OP_TOPK 2

/* Version of this ABI (IDX_ABI_VERSION). */
int32_t idx_abi_version(void);

/* Message of the last failing call on this host thread ("" if none). The string is owned by
 * the library and stays valid until the next call on the same thread. */
const char* idx_last_error(void);

/* Bytes of workspace that `op` needs for nq rows of at most max_n values and selection size k
 * (k = topk_blocks for IDX_OP_BUILD_POOL). Returns 0 for an unknown op or invalid sizes. */
size_t idx_workspace_size(int32_t op, int32_t nq, int64_t max_n, int32_t k);

/*
 * idx_quantize_q: random-Hadamard rotation followed by MXFP4 quantisation of 128-dim rows.
 *
 * Implements the quantise rule q_c = round_E2M1(x_c / s) with s a power of two ([P1] "E2M1 has
 * only 15 values" and "the scale format decides precision": the ideal max/6 is rounded up to a
 * power of two) after the rotation that reduces quantisation error ([P3], Q&A on the indexer's
 * quantisation). Used for the indexer queries and, with the same math, for the key cache rows.
 *
 *   y   = fl32( fl32(S) * fl32(2^-3.5) ),  S_i = sum_c H[i][c] * signs[c] * x[c]  (exact sum),
 *         H[i][c] = (-1)^popcount(i & c) (Sylvester order);
 *   e_g = smallest integer with 6 * 2^e_g >= max_{c in group g} |y_c|, clamped to [-127, 127],
 *         -127 for an all-zero group; scales[g] = e_g + 127;
 *   code_c = E2M1 of y_c / 2^e_g, round to nearest, ties to the even mantissa bit; zero is +0.
 *
 *   x_bf16 : device, bf16 bit patterns [rows][128], 16-byte aligned.
 *   rows   : number of rows, >= 0 (0 enqueues nothing).
 *   signs  : device int8 [128], each +1 or -1 (other values give unspecified codes).
 *   codes  : device uint8 [rows][64], 16-byte aligned (written).
 *   scales : device uint8 [rows][4], 4-byte aligned (written).
 * Inputs must be finite and the 128 values of a row must span at most 38 binades (the sum S is
 * then exact in fp64); otherwise the result is unspecified.
 */
idx_status idx_quantize_q(const uint16_t* x_bf16, int64_t rows, const int8_t* signs, uint8_t* codes,
                          uint8_t* scales, void* stream);

/*
 * idx_score_full: Full-layer scan. For every query t and visible key position s < n_t:
 *
 *   I_{t,s} = sum_{j=0..31} w_{t,j} * ReLU(q_{t,j} . k_s)
 *
 * ([P1] "Reindex layers score a million entries per token": the score equation with 32 heads of
 * 128 dims; [P3] Q&A: ReLU instead of softmax, query-generated weights), with q and k in MXFP4,
 * per-head dots computed by scaled-FP4 matrix instructions and the head sum in fp32;
 * fused with the block maxima of the candidate pool, B_b = max_{8b <= s < 8b+8, s < n_t} I_{t,s}
 * with positions past n_t counting as -inf ([P1] "use shallow-layer scores to limit
 * deep-layer scoring" and the walk-through of the official pool code). The newest-block pin is
 * applied by idx_build_pool, not here.
 *
 *   k_codes, k_scales : device key cache, [N][64] and [N][4] (16- and 4-byte aligned).
 *   k_base  : device int64 [nq]; query t reads key rows k_base[t] .. k_base[t] + n_t - 1.
 *   n_vis   : device int32 [nq]; n_t = min(max(n_vis[t], 0), max_n).
 *   nq      : number of queries, >= 0.
 *   group   : >= 1 and divides nq; each run of `group` consecutive queries shares one key range
 *             (k_base equal within a run): 1 for batched decode, the chunk size for prefill.
 *   max_n   : host upper bound on n_vis, 0 .. 2^24 (sizes the launch grid; one query's key range
 *             is addressed with 32-bit offsets).
 *   q_codes, q_scales : device, [nq][32][64] and [nq][32][4] (16- and 4-byte aligned).
 *   w       : device fp32 [nq][32], 4-byte aligned.
 *   scores  : device fp32 [nq][score_stride] or NULL; written for s < n_t only.
 *   score_stride : >= max_n when scores or head_dots is given.
 *   block_max : device fp32 [nq][bm_stride] or NULL; written for b < ceil(n_t / 8) only.
 *   bm_stride : >= ceil(max_n / 8) when block_max is given.
 *   head_dots : device fp32 [nq][32][score_stride] or NULL: the per-head dots q_{t,j}.k_s
 *               (a debugging output; slow).
 * At least one of scores, block_max, head_dots must be non-NULL.
 *
 * Exactness precondition. For query head j and key s let the spread be the largest exponent sum
 * (e_q[j][g] + e_k[s][g]) over the four groups g minus the smallest such sum among the groups whose
 * 32 code products do not sum to zero. The matrix instruction aligns the four group sums to the
 * largest group's exponent (also when that group sums to zero), so:
 *  - spread <= 14: the dot is exact (hence the same fp32 value as the exact sum whenever that is
 *    representable) and I is the fp32 head sum of exact terms, within 1e-5 * sum_j |w_j| ReLU(d_j)
 *    of the exact score (measured on MI355X over random codes at every spread up to 40);
 *  - spread > 14: low-order group sums may be dropped (entirely when the largest group cancels), so
 *    dots, scores and block maxima are unspecified.
 * Rows written by idx_quantize_q from activations have group exponents within a few units of each
 * other (the rotation spreads a row's energy over all four groups); the seeded workloads of this
 * library never exceed a spread of 9.
 * Summation order. Scores, and block maxima computed alongside scores, are bit-identical across
 * group values and with idx_score_pool_gather. Block maxima requested without scores at group > 1
 * sum the same exact per-head terms in another fp32 order (within the same tolerance).
 */
idx_status idx_score_full(const uint8_t* k_codes, const uint8_t* k_scales, const int64_t* k_base,
                          const int32_t* n_vis, int32_t nq, int32_t group, int64_t max_n, const uint8_t* q_codes,
                          const uint8_t* q_scales, const float* w, float* scores, int64_t score_stride,
                          float* block_max, int64_t bm_stride, float* head_dots, void* stream);

/*
 * idx_build_pool: candidate pool of the Hierarchical Sparse Indexer from the Full layer's block
 * maxima ([P1] "use shallow-layer scores to limit deep-layer scoring" and "three details of the
 * pool in the code"): the block holding position n_t - 1 gets +inf, blocks are ranked by
 * (value desc, block id asc), the first min(topk_blocks, ceil(n_t / block)) are kept (those
 * whose value is above -inf). With at most topk_blocks blocks every block is kept.
 *
 *   block_max  : device fp32 [nq][bm_stride], raw maxima as written by idx_score_full.
 *   n_vis      : device int32 [nq]; n_t = min(max(n_vis[t], 0), max_n).
 *   max_n      : host upper bound on n_vis.
 *   topk_blocks: 1 .. 2048 (2048 in the method).
 *   block      : must be 8 (the method's block size).
 *   pool_blocks: device int32 [nq][pool_stride], ascending block ids, -1 after pool_count[t].
 *   pool_stride: >= topk_blocks.
 *   pool_count : device int32 [nq] (written).
 *   ws, ws_bytes : device workspace of at least idx_workspace_size(IDX_OP_BUILD_POOL, nq, max_n,
 *                  topk_blocks) bytes, 16-byte aligned. It must be zero-filled before its first
 *                  use (e.g. when allocated); every call restores the counters and histograms it
 *                  holds to zero before it completes, so the workspace can be reused without
 *                  clearing (also inside a captured graph). Calls that may run concurrently need
 *                  separate workspaces.
 */
idx_status idx_build_pool(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq,
                          int64_t max_n, int32_t topk_blocks, int32_t block, int32_t* pool_blocks,
                          int64_t pool_stride, int32_t* pool_count, void* ws, size_t ws_bytes, void* stream);

/*
 * idx_build_pool_noalloc: idx_build_pool for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * semantics and results as idx_build_pool, without the workspace: the selection's scratch is a
 * fixed 80 MiB array inside the library, one copy per GPU, held until the process ends. The call
 * allocates and frees nothing. The scratch is enough for nq rows of ceil(max_n / 8) block maxima
 * up to idx_workspace_size(IDX_OP_BUILD_POOL, nq, max_n, topk_blocks) <= 80 MiB (e.g. 76 rows at
 * max_n = 2^20); larger requests return IDX_EUNSUPPORTED before any HIP call.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents: calls
 * that may overlap on one GPU (different streams without ordering) race and give unspecified
 * results. The first call on a device (and any call with more rows than every call before it on
 * that device) also enqueues a small kernel that clears the per-row counters it is about to use.
 */
idx_status idx_build_pool_noalloc(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq,
                                  int64_t max_n, int32_t topk_blocks, int32_t block, int32_t* pool_blocks,
                                  int64_t pool_stride, int32_t* pool_count, void* stream);

/*
 * idx_top_blocks: the k blocks of 8 positions with the largest block maxima, ranked by (value desc,
 * block id asc) without any pin, for a layer's own top-k reached through its block maxima (a key
 * among the top k outranks every other key of at most k - 1 blocks, so its block is among the top
 * k blocks: [P1] "use shallow-layer scores to limit deep-layer scoring", the nesting argument of the
 * pool). Used by chunked prefill: the top-512 blocks of each query, then idx_score_pool_gather over
 * them and idx_topk with the block map. Row t holds ceil(n_t / 8) maxima; blocks whose maximum is
 * -inf are never selected.
 *
 *   block_max, bm_stride, n_vis, max_n, block : as for idx_build_pool (n_vis counts positions).
 *   k           : 1 .. 2048.
 *   blocks      : device int32 [nq][blocks_stride], blocks_stride >= k: ascending block ids, -1 after
 *                 count[t] (count[t] = min(k, blocks above -inf)).
 *   count       : device int32 [nq] (written).
 *   ws, ws_bytes: at least idx_workspace_size(IDX_OP_BUILD_POOL, nq, max_n, k) bytes, as for
 *                 idx_build_pool.
 */
idx_status idx_top_blocks(const float* block_max, int64_t bm_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                          int32_t k, int32_t block, int32_t* blocks, int64_t blocks_stride, int32_t* count, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * idx_score_pool_gather: Reindex-layer scoring restricted to the candidate pool. Only the key
 * rows of the listed blocks are read and scored with the layer's own q and w ([P1] "use
 * shallow-layer scores to limit deep-layer scoring": Reindex layers score only pool positions,
 * 16384 x 4096 MACs per query independent of context length; and the remark that the saving
 * needs a kernel that reads only pooled keys, after the mask-form reference code).
 *
 *   k_codes, k_scales, k_base, n_vis, q_codes, q_scales, w : as for idx_score_full (group 1);
 *                 n_vis values above 2^24 are clamped to 2^24. The per-key arithmetic is the
 *                 scan's, bit for bit, under the same exactness precondition (spread <= 14).
 *   blocks      : device int32 [nq][blocks_stride]; block ids (any order) of query t are
 *                 blocks[t][0 .. block_count[t] - 1].
 *   block_count : device int32 [nq]; values are clamped to [0, max_blocks].
 *   max_blocks  : host bound, 0 .. 1 << 20.
 *   block       : must be 8.
 *   scores      : device fp32 [nq][score_stride], score_stride >= 8 * max_blocks; slot 8 * i + r
 *                 holds the score of position 8 * blocks[t][i] + r, or -inf when i >=
 *                 block_count[t] or the position is >= n_t (all 8 * max_blocks slots written).
 *   head_dots   : device fp32 [nq][32][score_stride] or NULL (debugging output).
 */
idx_status idx_score_pool_gather(const uint8_t* k_codes, const uint8_t* k_scales, const int64_t* k_base,
                                 const int32_t* n_vis, int32_t nq, const int32_t* blocks, int64_t blocks_stride,
                                 const int32_t* block_count, int32_t max_blocks, int32_t block,
                                 const uint8_t* q_codes, const uint8_t* q_scales, const float* w, float* scores,
                                 int64_t score_stride, float* head_dots, void* stream);

/*
 * idx_topk: the k largest values of each row ([P1] "use shallow-layer scores...": each layer keeps
 * its own top-512), ranked by (value desc, index asc) so that ties at the k-th value go to the
 * lower index; -inf (and NaN) values never enter the selection. Output per row: the
 * min(k, number of eligible values) selected indices in ascending index order (the order in
 * which a consumer gathers the selected keys), then -1. With a block map the order is ascending
 * slot order, which is ascending position when the map is ascending (as idx_build_pool and
 * idx_topk produce it); rows longer than 16384 values are always reported by ascending position.
 *
 *   scores       : device fp32 [nq][score_stride]; row t uses values 0 .. n_t - 1.
 *   n_valid      : device int32 [nq] or NULL (NULL means max_n for every row);
 *                  n_t = min(max(n_valid[t], 0), max_n).
 *   max_n        : host upper bound, 0 .. 1 << 30.
 *   k            : 1 .. 2048.
 *   blocks       : NULL, or a device int32 [nq][blocks_stride] block map as produced by
 *                  idx_build_pool: value slot s of row t stands for position
 *                  blocks[t][s / block] * block + s % block, and that position is both the
 *                  reported index and the tie-break key. The ids of a row must be distinct (as
 *                  idx_build_pool writes them); a repeated id gives an unspecified selection.
 *   block        : 8 when blocks is given (ignored otherwise).
 *   out_idx      : device int32 [nq][out_stride], out_stride >= k.
 *   out_val      : device fp32 [nq][out_stride] or NULL: the selected values in the same order
 *                  (-0 and +0 are equal values and a selected zero is reported as +0), -inf
 *                  after them.
 *   ws, ws_bytes : at least idx_workspace_size(IDX_OP_TOPK, nq, max_n, k) bytes, 16-byte aligned,
 *                  zero-filled before first use; every call restores its counters (as for
 *                  idx_build_pool); separate workspaces for calls that may run concurrently.
 */
idx_status idx_topk(const float* scores, int64_t score_stride, const int32_t* n_valid, int32_t nq, int64_t max_n,
                    int32_t k, const int32_t* blocks, int64_t blocks_stride, int32_t block, int32_t* out_idx,
                    int64_t out_stride, float* out_val, void* ws, size_t ws_bytes, void* stream);

/*
 * idx_mask_pool: the candidate pool in its training form ([P1] "three details of the pool in the
 * code": the official code turns the pool into a boolean table and a Reindex layer sets every
 * score outside it to -inf before its top-512; "the pool also acts in training": post-training
 * applies the same restriction). In place: with p = t / group, scores[t][s] = -inf for every
 * visible position s < n_t whose block s / block is not among pool_blocks[p][0 .. pool_count[p] - 1];
 * pooled positions and positions >= n_t are left as they are. With idx_score_full (scores)
 * before it and idx_topk after it, this is the mask-form Reindex layer; its top-512 equals the
 * gather form (idx_score_pool_gather + idx_topk with the block map). `group` lets the rows of
 * several layers of one query (consecutive rows) share that query's pool.
 *
 *   scores      : device fp32 [nq][score_stride], read and written; score_stride >= max_n.
 *   n_vis, max_n: as for idx_score_full (max_n up to 2^30).
 *   pool_blocks : device int32 [nq / group][pool_stride] block ids in any order (ids outside the
 *                 row are ignored); pool_count : device int32 [nq / group], clamped to
 *                 [0, pool_stride].
 *   group       : >= 1 and divides nq.
 *   block       : must be 8.
 * Errors: IDX_EINVAL (null pointer, score_stride < max_n, negative pool_stride, group not
 * dividing nq), IDX_EALIGN (pointers not 4-byte aligned), IDX_EUNSUPPORTED (nq > 65535,
 * max_n > 2^30, block != 8); nothing is launched on error. nq == 0 or max_n == 0 is a no-op.
 */
idx_status idx_mask_pool(float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                         const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count, int32_t group,
                         int32_t block, void* stream);

/*
 * idx_topk_pool: the top-k of full score rows restricted to the candidate pool ([P1] "three details
 * of the pool in the code": a layer's scores outside the pooled blocks count as -inf before its
 * top-512). The result equals idx_mask_pool followed by idx_topk on the same rows, but the rows
 * are read only at the pooled positions and left unchanged. With p = t / group, row t's
 * candidates are the positions 8 * pool_blocks[p][i] + r (i < min(pool_count[p], max_blocks),
 * r < 8) below n_t; ids outside [0, ceil(n_t / 8)) contribute nothing. Ranking, ties and the -1 /
 * -inf padding are those of idx_topk; indices are absolute positions, in ascending order when
 * the block ids are ascending (as idx_build_pool writes them). The block ids of a pool must be
 * distinct: the ranking assumes that every position appears once, so a repeated id gives an
 * unspecified selection.
 *
 *   scores       : device fp32 [nq][score_stride], score_stride >= max_n (read only).
 *   n_vis, max_n : device int32 [nq]; n_t = min(max(n_vis[t], 0), max_n); max_n 0 .. 2^28.
 *   pool_blocks  : device int32 [nq / group][pool_stride]; pool_count: device int32 [nq / group].
 *   max_blocks   : 0 .. 2048, <= pool_stride: the pool width read (one block of threads per row).
 *   group        : >= 1 and divides nq (rows of several layers of one query share its pool).
 *   block        : must be 8.
 *   k            : 1 .. 2048.
 *   out_idx      : device int32 [nq][out_stride], out_stride >= k; out_val: fp32, same shape, or NULL.
 * No workspace: every row is handled by one block of threads in LDS.
 * Errors: IDX_EINVAL (null pointer, a stride too small, group not dividing nq), IDX_EALIGN
 * (pointers not 4-byte aligned), IDX_EUNSUPPORTED (k, nq, max_n, max_blocks out of range,
 * block != 8); nothing is launched on error. nq == 0 is a no-op.
 */
idx_status idx_topk_pool(const float* scores, int64_t score_stride, const int32_t* n_vis, int32_t nq, int64_t max_n,
                         const int32_t* pool_blocks, int64_t pool_stride, const int32_t* pool_count,
                         int32_t max_blocks, int32_t group, int32_t block, int32_t k, int32_t* out_idx,
                         int64_t out_stride, float* out_val, void* stream);

/*
 * Main-KV FP4 storage ([P1] "the scale format decides precision" and "removing the global scale
 * still leaves enough range"): a main-KV entry is 512 values stored as E2M1 codes (element 2i in
 * the low nibble of byte i) with one E4M3 scale per group of 16 values and no global scale,
 * 256 code bytes + 32 scale bytes = 288 bytes. Codes live in [rows][256], scales in [rows][32].
 * E4M3 is the OCP FP8 "fn" variant (bias 7, subnormals, no infinities); scale bytes 0x7f and 0xff
 * (NaN) are outside the contract.
 */

/*
 * idx_quantize_kv: write main-KV rows in the storage format.
 *
 *   s_g    = the smallest E4M3 value s >= 0 with 6 * s >= max_{c in group g} |x_c| (448 at most);
 *            the page rounds the ideal max/6 up, as for the indexer's power-of-two scales;
 *   code_c = E2M1 of x_c / s_g, round to nearest, ties to the even mantissa bit, zero is +0;
 *            an all-zero group gets s_g = 0 and zero codes.
 *
 *   x_bf16 : device, bf16 bit patterns [rows][512], 16-byte aligned, finite values.
 *   rows   : 0 .. 2^31 (0 enqueues nothing).
 *   codes  : device uint8 [rows][256], 4-byte aligned (written).
 *   scales : device uint8 [rows][32] (written).
 */
idx_status idx_quantize_kv(const uint16_t* x_bf16, int64_t rows, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * idx_gather_kv: the selected main-KV entries of each query, dequantised to bf16 for core
 * attention (the cache stores FP4; attention reads dequantised values, [P1] "the scale format
 * decides precision": the main-KV format is read back before attention, the multiplication does
 * not happen in 4 bits). Every value is an E2M1 value times an E4M3 scale, exact in bf16.
 *
 *   codes, scales : device main-KV cache, [N][256] (4-byte aligned) and [N][32].
 *   kv_base : device int64 [nq]; position p of query t is cache row kv_base[t] + p.
 *   n_vis   : device int32 [nq]; positions outside [0, n_vis[t]) (e.g. the -1 padding of
 *             idx_topk) give rows of zeros.
 *   nq, k   : queries (at most 65535) and entries per query, nq * k <= 2^31.
 *   idx     : device int32 [nq][idx_stride] positions (e.g. idx_topk's out_idx), idx_stride >= k.
 *   out     : device bf16 bit patterns [nq][k][512], 16-byte aligned (written).
 */
idx_status idx_gather_kv(const uint8_t* codes, const uint8_t* scales, const int64_t* kv_base, const int32_t* n_vis,
                         int32_t nq, const int32_t* idx, int64_t idx_stride, int32_t k, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4IDX_H */
