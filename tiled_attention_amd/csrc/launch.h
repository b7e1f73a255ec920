// Internal launcher interface between the host API (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;        // [BH, N, d] bf16 / f32 / fp8 bytes
  const void* k;
  const void* v;        // bf16 (f32 for the f32 path)
  void* o;
  float* lse;           // nullable
  const float* q_scale; // fp8 only: [BH, ceil(N/128)]
  const float* k_scale;
  const float* v_scale; // all-fp8 path: V codes' power-of-two block scales (else null)
  const int32_t* doc;   // document masks: [num_docs + 1] start offsets
  int num_docs;
  int BH, N, d, mask, window;  // window clamped (clamp_window)
  float scale;
  bool in_f32, out_f32, fp8, v8;
  void* workspace;      // nullable: split key ranges (attn_fwd_split) when the plan asks for it
};

// Prefill / cross-attention over a paged pool of 64-token pages.
struct PagedFwdArgs {
  const void* q;        // [S, H, q_len, d] bf16
  const void* k_pool;   // [num_pages, H, page_size, d] bf16
  const void* v_pool;
  void* o;
  float* lse;           // nullable
  const int32_t* table; // page lists (device)
  const int32_t* lens;  // list lengths (device)
  int S, H, q_len, d, max_pages, num_pages, page_size;   // page_size 16 or 64
  int table_stride_s, table_stride_b, lens_stride_s, lens_stride_b;
  bool causal, out_f32;
  float scale;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  void* workspace;      // nullable
  int S, H, d, max_pages, num_pages, page_size;   // page_size 16 or 64
  float scale;
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* k_out;
  void* v_out;
  int S, H, d, max_pages, num_pages, elem_bytes, page_size;
};

// 16-token units per split of the split-KV decode, and the resulting
// workspace size for block-table rows of max_pages pages of page_size tokens.
constexpr int kDecodeSplitPages = 64;
size_t decode_workspace_bytes(int S, int H, int d, int max_pages, int page_size);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Workspace of the split-key prefill for this launch (0: the plan does not split).
size_t fwd_split_workspace_bytes(const FwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The split-KV decode with its partial states in the library's static device
// array (kNoAllocScratchBytes per GPU); a.workspace is ignored.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fwd_paged(const PagedFwdArgs& a, hipStream_t stream);
constexpr int kPrefillPageSize = 64;     // one page of one head is one 64-key tile
constexpr int kPrefillSmallPage = 16;    // the decode's pages: four per tile
constexpr int kPrefillMaxPages = 4096;  // page ids of one list staged in LDS
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_quant_fp8(const float* x, uint8_t* codes, float* scales, int BH, int N, int d, bool pow2,
                            hipStream_t stream);

}  // namespace attn
