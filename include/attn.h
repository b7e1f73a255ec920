/*
 * attn.h -- C ABI of libattn.so, a flash-attention forward library for
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The operation (all entry points): for each (batch b, head h),
 *     O = softmax(Q K^T * scale, masked) V
 * computed tile by tile with an online softmax so the N x N score matrix is
 * never stored: "Flash MSA Attention Kernel Implementation Tutorial",
 * sections "Why We Needed a New Attention Kernel" and "Understanding Flash
 * MSA Core Mechanics". Scores are accumulated in fp32; the running row max
 * m and row sum l are fp32.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc'd or equivalent) unless noted.
 *     The caller owns every buffer; the library allocates nothing, frees
 *     nothing and keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is only enqueued; the library never synchronises.
 *   - Every argument is checked on the host before anything is enqueued: a
 *     return value other than ATTN_OK means no device work was issued and
 *     no memory was touched (so these paths work without a GPU).
 *     ATTN_ERR_LAUNCH is the exception: it reports a failed launch.
 *     Device faults surface at the caller's next synchronisation.
 *   - Base pointers must be 16-byte aligned. Outputs must not alias inputs.
 *   - Tensors are dense, row-major, innermost dimension last.
 *   - Sizes: d (head dim) in {64, 128}; N >= 1; B*H*N < 2^31.
 *   - No C++ exception crosses this interface. Every call is thread-safe and
 *     the library holds no state, with one exception: attn_decode_paged_noalloc
 *     keeps a fixed device array per GPU (and its address), whose calls race
 *     when they overlap on one GPU (see there).
 */
#ifndef TILED_ATTENTION_AMD_ATTN_H
#define TILED_ATTENTION_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 2

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,  /* null pointer, size <= 0, misalignment, bad enum, window out of range */
  ATTN_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d = 96, 32-token pages) */
  ATTN_ERR_WORKSPACE = 3,    /* workspace smaller than the size query returns */
  ATTN_ERR_LAUNCH = 4        /* the HIP runtime reported a launch failure */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_FP8_E4M3 = 2 } attn_dtype;

/* Visibility of key j to query i (square masks, positions 0..N-1):
 *   NONE      every key;
 *   CAUSAL    j <= i;
 *   SLIDING   i - window < j <= i  (one-sided causal window of `window` keys,
 *             the query included; window >= 1);
 *   BAND      |i - j| <= window  (two-sided window of `window` neighbours on
 *             each side; window >= 0);
 *   PREFIX_LM j <= i or j < window  (the first `window` positions are a
 *             prefix every query sees; window >= 0, 0 is CAUSAL);
 *   DOCUMENT  i and j lie in the same document of doc_offsets (see below);
 *   DOCUMENT_CAUSAL  same document and j <= i (packed variable-length
 *             causal sequences).
 * The window masks are "Optimizing Triton kernels for custom attention
 * patterns on H100", Pattern B (which also names prefix-LM masks); the
 * document masks are Pattern A of that page.
 *
 * Documents: doc_offsets is a device array of num_docs + 1 int32 with
 * doc_offsets[0] = 0, doc_offsets[num_docs] = N, non-decreasing; document d
 * holds positions [doc_offsets[d], doc_offsets[d+1]) (it may be empty), and
 * every (batch, head) uses the same documents. A packed batch of sequences of
 * different lengths is B = 1 with one document per sequence. The contents
 * are the caller's contract and are not checked: other contents give
 * unspecified results, but no access outside the arguments' buffers. For
 * the other masks doc_offsets is ignored (may be NULL). */
typedef enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING = 2,
  ATTN_MASK_BAND = 3,
  ATTN_MASK_PREFIX_LM = 4,
  ATTN_MASK_DOCUMENT = 5,
  ATTN_MASK_DOCUMENT_CAUSAL = 6
} attn_mask;

/*
 * attn_fwd -- prefill under any attn_mask (dense, causal, windows, prefix-LM,
 * documents).
 *   q, k, v : [B, H, N, d], dtype in_dtype (ATTN_F32 or ATTN_BF16, all three alike).
 *   o       : [B, H, N, d], dtype out_dtype (ATTN_F32 or ATTN_BF16); every
 *             element is written (a row with no visible key, impossible for
 *             these masks, would be written as 0).
 *   scale   : multiplies Q K^T; the pages use 1/sqrt(d) (kernel listing in
 *             "Flash MSA ...", "Implementation Step-by-Step with Triton").
 *             Must be positive and finite, else ATTN_ERR_INVALID_ARG (the
 *             same holds for every entry point below that takes a scale);
 *             scaled scores must stay finite (inputs whose scores overflow
 *             fp32 give unspecified results).
 *   mask, window : see attn_mask; window is read by SLIDING, BAND and
 *             PREFIX_LM only.
 *   doc_offsets, num_docs : the documents of DOCUMENT / DOCUMENT_CAUSAL
 *             (device int32 [num_docs + 1], num_docs >= 1); ignored otherwise.
 *   lse     : NULL, or [B, H, N] fp32 receiving log(sum_j exp(S_ij)) per row
 *             (natural log, scaled scores), -inf for a row with no visible key.
 * bf16 inputs run on bf16 MFMA with fp32 accumulation; fp32 inputs run in
 * fp32 throughout. The K/V loop skips tiles with no visible pair and applies
 * the mask only on tiles that straddle its edge ("Optimizing Triton kernels
 * ...", Patterns A and B); document bounds are found on the device by a
 * search of doc_offsets, once per query tile.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int N, int d,
                     attn_dtype in_dtype, attn_dtype out_dtype,
                     float scale, attn_mask mask, int window,
                     const int32_t* doc_offsets, int num_docs,
                     float* lse, void* stream);

/*
 * attn_fwd_split_workspace_size -- bytes of workspace attn_fwd_split needs
 * for this shape and mask: 0 when the launch is not split, else B*H * (split
 * tiles) * 2 * 128 * (d + 1) * 4 bytes. It splits only bf16 CAUSAL and
 * PREFIX_LM launches with at most half a query tile (128 rows) per workgroup
 * slot of the GPU (512 slots) whose costliest tile holds at least 32 key tiles
 * of 64 (16 at d = 128), or at most 1.5 tiles per slot with at least 128 (64);
 * elsewhere the merge does not pay. The query tiles that cost more than half
 * the costliest are split. Host-only; 0 for arguments attn_fwd would reject.
 */
size_t attn_fwd_split_workspace_size(int B, int H, int N, int d, attn_dtype in_dtype,
                                     attn_mask mask, int window);

/*
 * attn_fwd_split -- attn_fwd, with the key range of the costliest query tiles
 * split in two for grids with few query tiles per workgroup slot (there the
 * costliest tile alone sets the launch time). Each part runs the same online
 * softmax over its keys and writes its normalised output and LSE to the
 * workspace; a second kernel merges the two parts of each split tile as
 * O = sum_i exp(L_i - L) O_i with L = log sum_i exp(L_i) (the split-KV merge
 * of "Flash MSA ...", "Understanding Flash MSA Core Mechanics", applied to the
 * key dimension of prefill), and writes O and the LSE.
 *   Arguments as attn_fwd, plus:
 *   workspace, workspace_bytes : device memory of at least
 *             attn_fwd_split_workspace_size(...) bytes, 16-byte aligned, owned
 *             by the caller; contents need not be initialised. When that size
 *             is 0 the call is attn_fwd and the workspace is not touched (it
 *             may be NULL). Too small or NULL otherwise -> ATTN_ERR_WORKSPACE.
 * Two kernels are enqueued on the stream; calls that share a workspace must
 * not overlap.
 */
attn_status attn_fwd_split(const void* q, const void* k, const void* v, void* o,
                           int B, int H, int N, int d,
                           attn_dtype in_dtype, attn_dtype out_dtype,
                           float scale, attn_mask mask, int window,
                           const int32_t* doc_offsets, int num_docs,
                           float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * attn_fwd_fp8 -- prefill with block-quantised fp8 Q and K and bf16 V
 * ("FlashAttention-3: Warp Specialization ...", "FP8 Block Quantization").
 *   q8, k8   : [B, H, N, d] OCP E4M3FN bytes.
 *   q_scale, k_scale : [B, H, ceil(N/qk_block)] fp32; the value of element
 *              x is e4m3(code) * scale of its qk_block-row block. Block
 *              scales must be positive and finite (device contents are not
 *              checked; others give unspecified results).
 *   v        : [B, H, N, d] bf16.   o : [B, H, N, d] bf16.
 *   S_ij = (sum_k q8_ik k8_jk) * q_scale[i/qk_block] * k_scale[j/qk_block] * scale,
 *   with the fp8 product accumulated in fp32; the rescale is folded into the
 *   exponent of the online softmax. P is rounded to bf16 for P V.
 *   qk_block must be 128. mask, window, doc_offsets, num_docs as in
 *   attn_fwd. lse: NULL or [B,H,N].
 */
attn_status attn_fwd_fp8(const uint8_t* q8, const float* q_scale,
                         const uint8_t* k8, const float* k_scale,
                         const void* v, void* o,
                         int B, int H, int N, int d, int qk_block,
                         float scale, attn_mask mask, int window,
                         const int32_t* doc_offsets, int num_docs,
                         float* lse, void* stream);

/*
 * attn_fwd_fp8_full -- prefill with Q, K and V all fp8: S as in attn_fwd_fp8,
 * and P V on the fp8 matrix cores with P rounded to E4M3 (P <= 448 is kept by
 * the softmax reference). This extends the block quantisation of
 * "FlashAttention-3 ...", "FP8 Block Quantization", which the page applies
 * to Q and K, to the second product.
 *   v8      : [B, H, N, d] E4M3FN codes.
 *   v_scale : [B, H, ceil(N/qk_block)] fp32, each a power of two in
 *             [2^-127, 2^127] (attn_quant_fp8_block_pow2 writes such scales);
 *             the matrix core applies it as an exponent, so a scale that is
 *             not a power of two acts as the power of two at or below it.
 *   other arguments and the output as attn_fwd_fp8 (o bf16).
 */
attn_status attn_fwd_fp8_full(const uint8_t* q8, const float* q_scale,
                              const uint8_t* k8, const float* k_scale,
                              const uint8_t* v8, const float* v_scale, void* o,
                              int B, int H, int N, int d, int qk_block,
                              float scale, attn_mask mask, int window,
                              const int32_t* doc_offsets, int num_docs,
                              float* lse, void* stream);

/*
 * attn_quant_fp8_block -- per-block E4M3FN quantisation of x [B, H, N, d] fp32
 * ("FlashAttention-3 ...", "FP8 Block Quantization"): for every 128-row
 * block (the last may be ragged) s = fp32(absmax) / 448 (IEEE fp32 division;
 * s = 1 for an all-zero block), code = e4m3(x / s) rounded to nearest, ties
 * to even, saturating at +-448.
 *   codes  : [B, H, N, d] uint8 out.   scales : [B, H, ceil(N/block)] fp32 out.
 *   block must be 128.
 */
attn_status attn_quant_fp8_block(const float* x, uint8_t* codes, float* scales,
                                 int B, int H, int N, int d, int block, void* stream);

/*
 * attn_quant_fp8_block_pow2 -- as attn_quant_fp8_block, with each block's
 * scale rounded up to a power of two: s = 2^k, the smallest with
 * absmax / s <= 448 (k >= -127; s = 1 for an all-zero block), decided on the
 * exact binary mantissa of absmax. code = e4m3(x / s) (an exact division).
 * For V of attn_fwd_fp8_full.
 */
attn_status attn_quant_fp8_block_pow2(const float* x, uint8_t* codes, float* scales,
                                      int B, int H, int N, int d, int block, void* stream);

/*
 * Paged KV cache ("Optimizing Triton kernels ...", Pattern C).
 *   k_pool, v_pool : [num_pages, H, page_size, d] bf16; page p, head h holds
 *                    rows t % page_size of the tokens mapped to it.
 *   block_table    : [S, max_pages] int32 (device); token t of sequence s is
 *                    in page block_table[s, t / page_size], row t % page_size.
 *                    Entries at or past ceil(seq_lens[s] / page_size) are
 *                    never read. Page ids must lie in [0, num_pages).
 *   seq_lens       : [S] int32 (device), 1 <= seq_lens[s] <= max_pages*page_size.
 *   page_size      : 16 or 64 tokens (other sizes -> ATTN_ERR_UNSUPPORTED).
 * The device contents are the caller's contract and are not checked: the
 * kernels clamp page ids into [0, num_pages) (and the decode clamps lengths
 * into [0, max_pages * page_size]), so other contents give unspecified
 * results but no access outside the buffers.
 */

/* Bytes of workspace attn_decode_paged uses to split long sequences. */
size_t attn_decode_paged_workspace_size(int S, int H, int d, int max_pages, int page_size);

/*
 * attn_decode_paged -- one new query token per sequence at position
 * seq_lens[s] - 1, attending to all seq_lens[s] cached keys.
 *   q, o : [S, H, d] bf16.
 *   workspace : NULL (each (sequence, head) is one pass over its pages) or at
 *               least attn_decode_paged_workspace_size(...) bytes (sequences
 *               are split into page ranges processed in parallel and merged
 *               with the online-softmax rescale). Smaller -> ATTN_ERR_WORKSPACE.
 *   lse : NULL or [S, H] fp32.
 */
attn_status attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* o, int S, int H, int d, int page_size,
                              int max_pages, int num_pages, float scale,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged with the split path, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). The split ranges'
 * partial states live in a fixed 16 MiB array of device memory inside the
 * library (one per GPU, held until the process ends) instead of a caller
 * workspace; the call itself allocates nothing.
 *   Arguments and results as attn_decode_paged (without the workspace).
 *   If attn_decode_paged_workspace_size(S, H, d, max_pages, page_size)
 *   exceeds 16 MiB (2^24 bytes) the call returns ATTN_ERR_WORKSPACE and
 *   nothing runs.
 *   Every call on one GPU uses that GPU's one array: calls whose work can
 *   overlap on a GPU (different streams, or host threads, without ordering
 *   between them) race and give unspecified results. Calls ordered on one
 *   stream are safe; nothing from an earlier call's contents is read.
 */
attn_status attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      void* o, int S, int H, int d, int page_size,
                                      int max_pages, int num_pages, float scale,
                                      float* lse, void* stream);

/*
 * attn_prefill_paged -- causal prefill over a paged KV cache ("Optimizing
 * Triton kernels ...", Pattern C, its prefix-caching use), with the page
 * gather fused into the attention's tile loads instead of a separate
 * gather-then-attend pass. It reads the decode's 16-token pool as well as a
 * 64-token one.
 *   The last q_len positions of every sequence are the query rows: row i of
 *   sequence s sits at position seq_lens[s] - q_len + i and sees the keys at
 *   positions 0 .. that position (the new rows' own K/V already in the pool).
 *   q, o : [S, H, q_len, d]; q bf16, o of out_dtype (ATTN_BF16 or ATTN_F32).
 *   k_pool, v_pool : [num_pages, H, page_size, d] bf16; page_size 64 (one
 *            page of one head is one 64-key tile) or 16 (the decode's pages,
 *            four per tile); any other size -> ATTN_ERR_UNSUPPORTED.
 *   block_table : [S, max_pages] int32 (device), as for attn_decode_paged.
 *   seq_lens : [S] int32 (device), q_len <= seq_lens[s] <= max_pages * page_size.
 *   max_pages <= 4096 (a list is staged on chip). lse : NULL or [S, H, q_len] fp32.
 * The device contents (page ids, lengths) are the caller's contract and are
 * not checked: lengths are clamped to [0, max_pages * page_size] and page ids into
 * [0, num_pages), so other contents give unspecified results but no access
 * outside the buffers.
 */
attn_status attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens, void* o,
                               int S, int H, int q_len, int d, int page_size, int max_pages,
                               int num_pages, attn_dtype out_dtype, float scale, float* lse,
                               void* stream);

/*
 * attn_cross_paged -- block-sparse paged cross-attention ("Optimizing Triton
 * kernels ...", Pattern C: each query block reads its own set of pages, as in
 * retrieval). Query block b of sequence s, rows 128b .. 128b + 127 of q[s],
 * attends with no mask to the first kv_lens[s, b] tokens of the
 * concatenation of pages page_table[s, b, 0], page_table[s, b, 1], ...
 *   q, o, pools, page_size (16 or 64), max_pages (<= 4096) as for attn_prefill_paged.
 *   page_table : [S, ceil(q_len / 128), max_pages] int32 (device).
 *   kv_lens : [S, ceil(q_len / 128)] int32 (device), 0 <= kv_lens <= max_pages * page_size;
 *            a block with no key gets O = 0 and LSE = -inf.
 * Device contents are handled as for attn_prefill_paged. The keys of a block
 * form a set, so the kernel visits the whole pages among its first 256 list
 * entries in ascending id order (blocks of one head that share pages then
 * read them from the L2 together); the result equals the list order's up to
 * fp32 rounding, and does not depend on how those pages are ordered.
 */
attn_status attn_cross_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* page_table, const int32_t* kv_lens, void* o,
                             int S, int H, int q_len, int d, int page_size, int max_pages,
                             int num_pages, attn_dtype out_dtype, float scale, float* lse,
                             void* stream);

/*
 * attn_gather_paged -- stage one of the two-stage paged route: a bit copy
 *   k_out[s, h, t, :] = k_pool[block_table[s, t / page_size], h, t % page_size, :]
 * (same for v) for t < seq_lens[s]. k_out, v_out: [S, H, max_pages*page_size, d]
 * of `dtype` (ATTN_BF16 or ATTN_F32, element size only); rows t >= seq_lens[s]
 * are left untouched. page_size 16 (the decode's pages) or 64.
 */
attn_status attn_gather_paged(const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* k_out, void* v_out, int S, int H, int d,
                              int page_size, int max_pages, int num_pages,
                              attn_dtype dtype, void* stream);

/*
 * Host-side tile planning (no device access). For every mask the keys
 * visible to row i form one interval holding i whose ends never decrease
 * with i, so a tile's class follows from the intervals of its first and last
 * rows. Tiles of query rows [m0, m1) against keys [n0, n1) are EMPTY (0: no
 * visible pair, never loaded), PARTIAL (1: the mask is applied element by
 * element) or FULL (2: every pair visible, no mask work). Keys >= N do not
 * exist, so a tile reaching past N is at most PARTIAL; rows >= N are ignored.
 * doc_offsets here is a HOST array (num_docs + 1 entries, checked: 0 first,
 * N last, non-decreasing) for the document masks and ignored otherwise.
 * attn_tile_class returns -1 on invalid arguments.
 */
int attn_tile_class(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs,
                    int N, int m0, int m1, int n0, int n1);

/* K-tile index range [*t_lo, *t_hi) (tiles of bn keys) that can hold a key
 * visible to some row of [m0, m1); tiles outside it are EMPTY and none inside
 * it is. An empty row range gives *t_lo == *t_hi == 0. */
attn_status attn_k_tile_range(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs,
                              int N, int m0, int m1, int bn, int* t_lo, int* t_hi);

/* Global K-tile index range [*f_lo, *f_hi) of the tiles of bn keys that are
 * FULL for the rows [m0, m1) (every pair visible: the kernels skip the mask
 * there). They are contiguous; an empty range is returned as *f_lo == *f_hi. */
attn_status attn_full_tile_range(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs,
                                 int N, int m0, int m1, int bn, int* f_lo, int* f_hi);

/* Host copy of the heaviest-first dispatch ranking that the document-masked
 * and paged prefill kernels compute on the device (the same code): groups of
 * work (query tiles, sequences) are ranked by cost, descending, ties by
 * index, and workgroup id r takes the group of rank r, so the hardware's
 * in-order dispatch runs the costliest first (the longest-first rule for
 * load balance; the pages' Pattern A, "Optimizing Triton kernels ...",
 * notes that a document mask makes tile costs uneven).
 *   costs : host int32 [groups], each in [0, 2^23).   groups : 1 .. 256.
 *   ranks : host int32 [groups] out; ranks[g] = number of groups ranked
 *           before group g.
 * Returns ATTN_ERR_INVALID_ARG for other arguments. */
attn_status attn_dispatch_ranks(const int32_t* costs, int groups, int32_t* ranks);

const char* attn_status_str(attn_status s);
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_AMD_ATTN_H */
