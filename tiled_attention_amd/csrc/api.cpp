// C ABI of libattn.so: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is enqueued, so a non-OK
// status means no device work was issued.
#include "attn.h"

#include <stdint.h>

#include <cmath>

#include "attn_common.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Mask kind and window; the document masks also need their offsets array
// (device or host pointer, 4-byte aligned) and num_docs >= 1.
bool valid_mask(int mask, int window, const int32_t* doc_offsets, int num_docs) {
  switch (mask) {
    case ATTN_MASK_NONE:
    case ATTN_MASK_CAUSAL: return true;
    case ATTN_MASK_SLIDING: return window >= 1;
    case ATTN_MASK_BAND:
    case ATTN_MASK_PREFIX_LM: return window >= 0;
    case ATTN_MASK_DOCUMENT:
    case ATTN_MASK_DOCUMENT_CAUSAL:
      return doc_offsets != nullptr && ((uintptr_t)doc_offsets & 3u) == 0 && num_docs >= 1 &&
             num_docs < (1 << 30);
  }
  return false;
}

// Host document offsets: 0 first, N last, never decreasing.
bool valid_host_docs(const int32_t* offs, int num_docs, int N) {
  if (offs[0] != 0 || offs[num_docs] != N) return false;
  for (int d = 0; d < num_docs; ++d)
    if (offs[d + 1] < offs[d]) return false;
  return true;
}

// Fills the mask fields of a launch.
void set_mask(attn::FwdArgs& a, int mask, int window, const int32_t* doc_offsets, int num_docs, int N) {
  a.mask = mask;
  a.window = attn::clamp_window(mask, window, N);
  a.doc = attn::is_document(mask) ? doc_offsets : nullptr;
  a.num_docs = attn::is_document(mask) ? num_docs : 0;
}

// Shared size checks: B, H, N >= 1; d > 0; B*H*N fits in 31 bits.
attn_status check_dims(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * H * N >= (1LL << 31)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// The kernels give invisible keys a score of -inf before the scale multiplies
// the scores, and take the running maximum over unscaled scores: both need a
// positive scale (a zero or negative one would turn -inf into NaN or +inf).
bool valid_scale(float scale) { return scale > 0.f && std::isfinite(scale); }

attn_status launched(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

// Shared by attn_fwd and attn_fwd_split: validation, then the launch (with
// the split-key plan when a workspace is given and the plan splits).
static attn_status fwd_dense(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                             attn_dtype in_dtype, attn_dtype out_dtype, float scale, attn_mask mask, int window,
                             const int32_t* doc_offsets, int num_docs, float* lse, void* workspace,
                             size_t workspace_bytes, bool split, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID_ARG;
  if (in_dtype != ATTN_F32 && in_dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!valid_mask(mask, window, doc_offsets, num_docs)) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_dims(B, H, N, d);
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.N = N;
  a.d = d;
  set_mask(a, mask, window, doc_offsets, num_docs, N);
  a.scale = scale;
  a.in_f32 = in_dtype == ATTN_F32;
  a.out_f32 = out_dtype == ATTN_F32;
  a.fp8 = false;
  if (split) {
    const size_t need = attn::fwd_split_workspace_bytes(a);
    if (need > 0) {
      if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
      if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
      a.workspace = workspace;
    }
  }
  return launched(attn::launch_fwd(a, (hipStream_t)stream));
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                     attn_dtype in_dtype, attn_dtype out_dtype, float scale, attn_mask mask, int window,
                     const int32_t* doc_offsets, int num_docs, float* lse, void* stream) {
  return fwd_dense(q, k, v, o, B, H, N, d, in_dtype, out_dtype, scale, mask, window, doc_offsets, num_docs, lse,
                   nullptr, 0, false, stream);
}

size_t attn_fwd_split_workspace_size(int B, int H, int N, int d, attn_dtype in_dtype, attn_mask mask, int window) {
  if (check_dims(B, H, N, d) != ATTN_OK) return 0;
  if (in_dtype != ATTN_F32 && in_dtype != ATTN_BF16) return 0;
  if (mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_PREFIX_LM) return 0;
  if (!valid_mask(mask, window, nullptr, 0)) return 0;
  attn::FwdArgs a{};
  a.BH = B * H;
  a.N = N;
  a.d = d;
  set_mask(a, mask, window, nullptr, 0, N);
  a.in_f32 = in_dtype == ATTN_F32;
  return attn::fwd_split_workspace_bytes(a);
}

attn_status attn_fwd_split(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                           attn_dtype in_dtype, attn_dtype out_dtype, float scale, attn_mask mask, int window,
                           const int32_t* doc_offsets, int num_docs, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return fwd_dense(q, k, v, o, B, H, N, d, in_dtype, out_dtype, scale, mask, window, doc_offsets, num_docs, lse,
                   workspace, workspace_bytes, true, stream);
}

static attn_status fwd_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                           const void* v, const float* v_scale, bool v8, void* o, int B, int H, int N, int d,
                           int qk_block, float scale, attn_mask mask, int window, const int32_t* doc_offsets,
                           int num_docs, float* lse, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v || !o || (v8 && !v_scale)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID_ARG;
  if (!valid_mask(mask, window, doc_offsets, num_docs)) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (qk_block < 1) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_dims(B, H, N, d);
  if (st != ATTN_OK) return st;
  if (qk_block != 128) return ATTN_ERR_UNSUPPORTED;
  attn::FwdArgs a{};
  a.q = q8;
  a.k = k8;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v8 ? v_scale : nullptr;
  a.BH = B * H;
  a.N = N;
  a.d = d;
  set_mask(a, mask, window, doc_offsets, num_docs, N);
  a.scale = scale;
  a.in_f32 = false;
  a.out_f32 = false;
  a.fp8 = true;
  a.v8 = v8;
  return launched(attn::launch_fwd(a, (hipStream_t)stream));
}

attn_status attn_fwd_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                         const void* v, void* o, int B, int H, int N, int d, int qk_block, float scale,
                         attn_mask mask, int window, const int32_t* doc_offsets, int num_docs, float* lse,
                         void* stream) {
  return fwd_fp8(q8, q_scale, k8, k_scale, v, nullptr, false, o, B, H, N, d, qk_block, scale, mask, window,
                 doc_offsets, num_docs, lse, stream);
}

attn_status attn_fwd_fp8_full(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                              const uint8_t* v8, const float* v_scale, void* o, int B, int H, int N, int d,
                              int qk_block, float scale, attn_mask mask, int window, const int32_t* doc_offsets,
                              int num_docs, float* lse, void* stream) {
  return fwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, true, o, B, H, N, d, qk_block, scale, mask, window,
                 doc_offsets, num_docs, lse, stream);
}

static attn_status quant(const float* x, uint8_t* codes, float* scales, int B, int H, int N, int d, int block,
                         bool pow2, void* stream) {
  if (!x || !codes || !scales) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 3u)) return ATTN_ERR_INVALID_ARG;
  if (block < 1) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_dims(B, H, N, d);
  if (st != ATTN_OK) return st;
  if (block != 128) return ATTN_ERR_UNSUPPORTED;
  return launched(attn::launch_quant_fp8(x, codes, scales, B * H, N, d, pow2, (hipStream_t)stream));
}

attn_status attn_quant_fp8_block(const float* x, uint8_t* codes, float* scales, int B, int H, int N, int d,
                                 int block, void* stream) {
  return quant(x, codes, scales, B, H, N, d, block, false, stream);
}

attn_status attn_quant_fp8_block_pow2(const float* x, uint8_t* codes, float* scales, int B, int H, int N, int d,
                                      int block, void* stream) {
  return quant(x, codes, scales, B, H, N, d, block, true, stream);
}

size_t attn_decode_paged_workspace_size(int S, int H, int d, int max_pages, int page_size) {
  if (S < 1 || H < 1 || max_pages < 1 || (d != 64 && d != 128) || (page_size != 16 && page_size != 64)) return 0;
  return attn::decode_workspace_bytes(S, H, d, max_pages, page_size);
}

static attn_status check_paged(const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, int S, int H, int d, int page_size, int max_pages,
                               int num_pages) {
  if (!k_pool || !v_pool || !block_table || !seq_lens) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)block_table & 3u) || ((uintptr_t)seq_lens & 3u)) return ATTN_ERR_INVALID_ARG;
  if (S < 1 || H < 1 || d < 1 || page_size < 1 || max_pages < 1 || num_pages < 1) return ATTN_ERR_INVALID_ARG;
  if ((long long)S * max_pages >= (1LL << 31) || (long long)num_pages * H * page_size >= (1LL << 31))
    return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (page_size != 16 && page_size != 64) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status attn_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, int S, int H, int d, int page_size, int max_pages,
                              int num_pages, float scale, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!q || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o)) return ATTN_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_paged(k_pool, v_pool, block_table, seq_lens, S, H, d, page_size, max_pages, num_pages);
  if (st != ATTN_OK) return st;
  if (workspace) {
    if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
    if (workspace_bytes < attn::decode_workspace_bytes(S, H, d, max_pages, page_size)) return ATTN_ERR_WORKSPACE;
  }
  attn::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.workspace = workspace;
  a.S = S;
  a.H = H;
  a.d = d;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.scale = scale;
  return launched(attn::launch_decode(a, (hipStream_t)stream));
}

attn_status attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* seq_lens, void* o, int S, int H,
                                      int d, int page_size, int max_pages, int num_pages, float scale, float* lse,
                                      void* stream) {
  if (!q || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o)) return ATTN_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_paged(k_pool, v_pool, block_table, seq_lens, S, H, d, page_size, max_pages, num_pages);
  if (st != ATTN_OK) return st;
  // the partial states must fit the library's fixed device array
  if (attn::decode_workspace_bytes(S, H, d, max_pages, page_size) > attn::kNoAllocScratchBytes)
    return ATTN_ERR_WORKSPACE;
  attn::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.workspace = nullptr;
  a.S = S;
  a.H = H;
  a.d = d;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.scale = scale;
  return launched(attn::launch_decode_noalloc(a, (hipStream_t)stream));
}

// Shared checks of the two paged prefill entry points (16- or 64-token pages).
static attn_status paged_fwd(const void* q, const void* k_pool, const void* v_pool, const int32_t* table,
                             const int32_t* lens, void* o, int S, int H, int q_len, int d, int page_size,
                             int max_pages, int num_pages, attn_dtype out_dtype, float scale, float* lse,
                             void* stream, bool causal) {
  if (!q || !o || !k_pool || !v_pool || !table || !lens) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_pool) || !aligned16(v_pool)) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)table & 3u) || ((uintptr_t)lens & 3u)) return ATTN_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID_ARG;
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (page_size < 1 || max_pages < 1 || num_pages < 1) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_dims(S, H, q_len, d);
  if (st != ATTN_OK) return st;
  const int qb = (q_len + 127) / 128;
  if ((long long)S * qb * max_pages >= (1LL << 31)) return ATTN_ERR_INVALID_ARG;
  if (page_size != attn::kPrefillPageSize && page_size != attn::kPrefillSmallPage) return ATTN_ERR_UNSUPPORTED;
  if (max_pages > attn::kPrefillMaxPages) return ATTN_ERR_UNSUPPORTED;
  if ((long long)num_pages * H * page_size * d >= (1LL << 40)) return ATTN_ERR_INVALID_ARG;
  attn::PagedFwdArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.o = o;
  a.lse = lse;
  a.table = table;
  a.lens = lens;
  a.S = S;
  a.H = H;
  a.q_len = q_len;
  a.d = d;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.table_stride_s = causal ? max_pages : qb * max_pages;
  a.table_stride_b = causal ? 0 : max_pages;
  a.lens_stride_s = causal ? 1 : qb;
  a.lens_stride_b = causal ? 0 : 1;
  a.causal = causal;
  a.out_f32 = out_dtype == ATTN_F32;
  a.scale = scale;
  return launched(attn::launch_fwd_paged(a, (hipStream_t)stream));
}

attn_status attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, int S, int H, int q_len, int d, int page_size,
                               int max_pages, int num_pages, attn_dtype out_dtype, float scale, float* lse,
                               void* stream) {
  return paged_fwd(q, k_pool, v_pool, block_table, seq_lens, o, S, H, q_len, d, page_size, max_pages, num_pages,
                   out_dtype, scale, lse, stream, true);
}

attn_status attn_cross_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                             const int32_t* kv_lens, void* o, int S, int H, int q_len, int d, int page_size,
                             int max_pages, int num_pages, attn_dtype out_dtype, float scale, float* lse,
                             void* stream) {
  return paged_fwd(q, k_pool, v_pool, page_table, kv_lens, o, S, H, q_len, d, page_size, max_pages, num_pages,
                   out_dtype, scale, lse, stream, false);
}

attn_status attn_gather_paged(const void* k_pool, const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, void* k_out, void* v_out, int S, int H, int d,
                              int page_size, int max_pages, int num_pages, attn_dtype dtype, void* stream) {
  if (!k_out || !v_out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_out) || !aligned16(v_out)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_paged(k_pool, v_pool, block_table, seq_lens, S, H, d, page_size, max_pages, num_pages);
  if (st != ATTN_OK) return st;
  if ((long long)S * H * max_pages * page_size >= (1LL << 31)) return ATTN_ERR_INVALID_ARG;
  attn::GatherArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.k_out = k_out;
  a.v_out = v_out;
  a.S = S;
  a.H = H;
  a.d = d;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.elem_bytes = dtype == ATTN_F32 ? 4 : 2;
  a.page_size = page_size;
  return launched(attn::launch_gather(a, (hipStream_t)stream));
}

// Spans of the first and last rows of [m0, m1) clipped to N (m0 < min(m1, N)).
static void plan_spans(int mask, int window, const int32_t* offs, int num_docs, int N, int m0, int m1,
                       attn::KeySpan* first, attn::KeySpan* last) {
  if (m1 > N) m1 = N;
  *first = attn::host_span(mask, window, offs, num_docs, N, m0);
  *last = attn::host_span(mask, window, offs, num_docs, N, m1 - 1);
}

static bool valid_plan(int mask, int window, const int32_t* offs, int num_docs, int N) {
  if (N < 1 || !valid_mask(mask, window, offs, num_docs)) return false;
  return !attn::is_document(mask) || valid_host_docs(offs, num_docs, N);
}

int attn_tile_class(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs, int N, int m0, int m1,
                    int n0, int n1) {
  if (!valid_plan(mask, window, doc_offsets, num_docs, N) || m0 < 0 || n0 < 0 || m1 < m0 || n1 < n0) return -1;
  if (m0 >= (m1 < N ? m1 : N)) return attn::TILE_EMPTY;
  attn::KeySpan first, last;
  plan_spans(mask, window, doc_offsets, num_docs, N, m0, m1, &first, &last);
  return attn::span_tile_class(first, last, N, n0, n1);
}

attn_status attn_k_tile_range(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs, int N, int m0,
                              int m1, int bn, int* t_lo, int* t_hi) {
  if (!t_lo || !t_hi || !valid_plan(mask, window, doc_offsets, num_docs, N) || bn < 1 || m0 < 0 || m1 < m0)
    return ATTN_ERR_INVALID_ARG;
  *t_lo = *t_hi = 0;
  if (m0 >= (m1 < N ? m1 : N)) return ATTN_OK;
  attn::KeySpan first, last;
  plan_spans(mask, window, doc_offsets, num_docs, N, m0, m1, &first, &last);
  attn::touched_tiles(first, last, bn, t_lo, t_hi);
  return ATTN_OK;
}

attn_status attn_full_tile_range(attn_mask mask, int window, const int32_t* doc_offsets, int num_docs, int N,
                                 int m0, int m1, int bn, int* f_lo, int* f_hi) {
  if (!f_lo || !f_hi || !valid_plan(mask, window, doc_offsets, num_docs, N) || bn < 1 || m0 < 0 || m1 < m0)
    return ATTN_ERR_INVALID_ARG;
  *f_lo = *f_hi = 0;
  if (m0 >= (m1 < N ? m1 : N)) return ATTN_OK;
  attn::KeySpan first, last;
  plan_spans(mask, window, doc_offsets, num_docs, N, m0, m1, &first, &last);
  attn::full_tiles(first, last, bn, f_lo, f_hi);
  return ATTN_OK;
}

attn_status attn_dispatch_ranks(const int32_t* costs, int groups, int32_t* ranks) {
  if (!costs || !ranks || groups < 1 || groups > attn::kRankMaxGroups) return ATTN_ERR_INVALID_ARG;
  for (int g = 0; g < groups; ++g)
    if (costs[g] < 0 || costs[g] >= (1 << 23)) return ATTN_ERR_INVALID_ARG;
  // the workgroup's key array, as its threads fill it
  alignas(16) int keys[attn::kRankMaxGroups];
  const int padded = attn::rank_padded(groups);
  for (int t = 0; t < padded; ++t) keys[t] = t < groups ? (int)attn::rank_key(costs[t], t) : 0;
  for (int g = 0; g < groups; ++g) ranks[g] = 0;
  // every counting thread in turn (their sums do not depend on the order)
  const int parts = attn::rank_parts(groups, attn::kRankMaxGroups);
  for (int t = 0; t < parts * groups; ++t) {
    const int part = attn::rank_part(t, groups);
    const int g = t - part * groups;
    ranks[g] += attn::rank_count((const attn::i32x4*)keys, groups, part, parts, (unsigned)keys[g]);
  }
  return ATTN_OK;
}

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: valid but not implemented";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace too small";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: kernel launch failed";
  }
  return "unknown attn_status";
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
