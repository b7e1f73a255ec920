// Shared definitions for the gfx950 attention kernels and the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// MFMA operand / accumulator vector types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

enum MaskKind {
  MASK_NONE = 0,
  MASK_CAUSAL = 1,
  MASK_SLIDING = 2,
  MASK_BAND = 3,
  MASK_PREFIX_LM = 4,
  MASK_DOCUMENT = 5,
  MASK_DOCUMENT_CAUSAL = 6
};
enum TileClass { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__host__ __device__ inline bool is_document(int mask) {
  return mask == MASK_DOCUMENT || mask == MASK_DOCUMENT_CAUSAL;
}

// The keys visible to a query row i form one interval [lo, hi] for every mask
// here: the band masks by definition, the document masks because a document
// is a run of consecutive positions. The interval holds i itself, and lo and
// hi never decrease as i grows. Hence the keys visible to some row of
// [m0, m1) are exactly [lo(m0), hi(m1 - 1)], and the keys visible to every
// row of it are [lo(m1 - 1), hi(m0)]: tile classification and loop bounds
// need the spans of the first and last rows only ("Optimizing Triton kernels
// for custom attention patterns on H100", Patterns A and B).
struct KeySpan {
  int lo, hi;
};

// Window argument clamped to what changes the mask, so that i + window and
// i - window stay within [-N, 2N] (SLIDING: more than N keys is causal; BAND
// and PREFIX_LM: N covers every key).
__host__ __device__ inline int clamp_window(int mask, int window, int N) {
  if (mask == MASK_SLIDING) return window <= N ? window : N + 1;
  if (mask == MASK_BAND || mask == MASK_PREFIX_LM) return window <= N ? window : N;
  return 0;
}

// Span of row i for the closed-form masks (window already clamped).
//   NONE: every key. CAUSAL: j <= i. SLIDING: i - w < j <= i.
//   BAND: |i - j| <= w. PREFIX_LM: j <= i or j < w.
__host__ __device__ inline KeySpan band_span(int mask, int w, int N, int i) {
  switch (mask) {
    case MASK_NONE: return {0, N - 1};
    case MASK_SLIDING: return {i - w + 1 > 0 ? i - w + 1 : 0, i};
    case MASK_BAND: return {i - w > 0 ? i - w : 0, i + w < N - 1 ? i + w : N - 1};
    case MASK_PREFIX_LM: return {0, w - 1 > i ? w - 1 : i};
    default: return {0, i};  // CAUSAL
  }
}

// Span of row i inside the document [start, end). Out-of-range offsets are
// clamped so that the span always holds i and stays inside [0, N): any
// offsets array then gives in-bounds loop ranges.
__host__ __device__ inline KeySpan doc_span(bool causal, int start, int end, int N, int i) {
  KeySpan s;
  s.lo = start < 0 ? 0 : (start > i ? i : start);
  if (causal) {
    s.hi = i;
  } else {
    const int e = end > N ? N : end;
    s.hi = (e > i + 1 ? e : i + 1) - 1;
  }
  return s;
}

// Host: span of row i of any mask; offs / nd describe the documents (host
// memory): row i lies in the last document d with offs[d] <= i.
inline KeySpan host_span(int mask, int window, const int32_t* offs, int nd, int N, int i) {
  if (!is_document(mask)) return band_span(mask, clamp_window(mask, window, N), N, i);
  int lo = 0, hi = nd - 1;  // the document is the last d in [0, nd) with offs[d] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (offs[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return doc_span(mask == MASK_DOCUMENT_CAUSAL, offs[lo], offs[lo + 1], N, i);
}

// Tiles of bn keys [lo, hi) that hold a key visible to some row whose spans
// of the first and last rows are `first` and `last`.
__host__ __device__ inline void touched_tiles(KeySpan first, KeySpan last, int bn, int* lo, int* hi) {
  *lo = first.lo / bn;
  *hi = last.hi / bn + 1;
}

// Tiles [lo, hi) of bn keys in which every pair is visible to every row of
// the rows with those first/last spans (a contiguous run; empty as lo == hi).
__host__ __device__ inline void full_tiles(KeySpan first, KeySpan last, int bn, int* lo, int* hi) {
  const int l = (last.lo + bn - 1) / bn;
  const int h = (first.hi + 1) / bn;
  *lo = l < h ? l : h;
  *hi = h;
}

// Class of the tile (rows [m0, m1), clipped to N, with those first / last
// spans) x (keys [n0, n1)). Keys >= N do not exist, so a tile reaching past N
// is at most PARTIAL.
__host__ __device__ inline int span_tile_class(KeySpan first, KeySpan last, int N, int n0, int n1) {
  if (n0 >= N || n0 >= n1) return TILE_EMPTY;
  const bool ragged = n1 > N;
  const int n_last = (ragged ? N : n1) - 1;
  if (n0 > last.hi || n_last < first.lo) return TILE_EMPTY;
  if (!ragged && last.lo <= n0 && n_last <= first.hi) return TILE_FULL;
  return TILE_PARTIAL;
}

// Number of entries <= x among offs[0..n), n >= 1, offs ascending, x the same
// in every lane of the wave. A 64-ary search: each level probes 64 evenly
// spaced entries (one load per lane) and a ballot counts those <= x, so the
// answer is found in ceil(log64(n)) + 1 rounds of independent loads. Reads
// stay inside offs[0..n) whatever its contents.
__device__ inline int doc_count_le(const int32_t* offs, int n, int x) {
  const int lane = __lane_id();
  int base = 0, span = n;
  while (span > 64) {
    const int stride = (span + 63) >> 6;
    const int pos = base + (lane + 1) * stride - 1;
    const bool le = pos < base + span && offs[pos] <= x;
    const int k = __popcll(__ballot(le));
    base += k * stride;
    span = min(stride - 1, span - k * stride);
  }
  const bool le = lane < span && offs[base + lane] <= x;
  return base + __popcll(__ballot(le));
}

// Document of row x given count = doc_count_le(offs, nd + 1, x), clamped to a
// valid document index.
__device__ inline int doc_index(int count, int nd) {
  const int d = count - 1;
  return d < 0 ? 0 : (d > nd - 1 ? nd - 1 : d);
}

// Spans a workgroup and its waves need, for rows of one wave:
//   tile_first / tile_last: first and last row of the workgroup's Q tile,
//   wave_first / wave_last: first and last row of this wave,
//   lane: this lane's row.
// Every row argument is < N; all but `row` are uniform across the wave.
struct RowSpans {
  KeySpan lane, lane2, wave_first, wave_last, tile_first, tile_last;
};

// Spans of a workgroup's first and last rows, of a wave's first and last
// rows, and of the lane's rows `row` and `row2` (both inside the wave's rows).
__device__ inline RowSpans row_spans(int mask, int window, const int32_t* offs, int nd, int N, int tile_r0,
                                     int tile_r1, int wave_r0, int wave_r1, int row, int row2) {
  RowSpans r;
  if (!is_document(mask)) {
    r.lane = band_span(mask, window, N, row);
    r.lane2 = band_span(mask, window, N, row2);
    r.wave_first = band_span(mask, window, N, wave_r0);
    r.wave_last = band_span(mask, window, N, wave_r1);
    r.tile_first = band_span(mask, window, N, tile_r0);
    r.tile_last = band_span(mask, window, N, tile_r1);
    return r;
  }
  const bool causal = mask == MASK_DOCUMENT_CAUSAL;
  const int ct0 = doc_count_le(offs, nd + 1, tile_r0);
  const int ct1 = doc_count_le(offs, nd + 1, tile_r1);
  const int cw0 = doc_count_le(offs, nd + 1, wave_r0);
  const int cw1 = doc_count_le(offs, nd + 1, wave_r1);
  int d = doc_index(ct0, nd);
  r.tile_first = doc_span(causal, offs[d], offs[d + 1], N, tile_r0);
  d = doc_index(ct1, nd);
  r.tile_last = doc_span(causal, offs[d], offs[d + 1], N, tile_r1);
  d = doc_index(cw0, nd);
  r.wave_first = doc_span(causal, offs[d], offs[d + 1], N, wave_r0);
  d = doc_index(cw1, nd);
  r.wave_last = doc_span(causal, offs[d], offs[d + 1], N, wave_r1);
  // the lane's rows: the document starts between the wave's first and last
  // rows (usually none or one) decide them
  int c = cw0, c2 = cw0;
  for (int t = cw0; t < cw1; ++t) {
    c += offs[t] <= row ? 1 : 0;
    c2 += offs[t] <= row2 ? 1 : 0;
  }
  d = doc_index(c, nd);
  r.lane = doc_span(causal, offs[d], offs[d + 1], N, row);
  d = doc_index(c2, nd);
  r.lane2 = doc_span(causal, offs[d], offs[d + 1], N, row2);
  return r;
}

__device__ inline RowSpans row_spans(int mask, int window, const int32_t* offs, int nd, int N, int tile_r0,
                                     int tile_r1, int wave_r0, int wave_r1, int row) {
  return row_spans(mask, window, offs, nd, N, tile_r0, tile_r1, wave_r0, wave_r1, row, row);
}

// Workgroup id -> work unit, so that consecutive units land on one XCD.
// Workgroups are dealt to the 8 XCDs round-robin by id; unit u is given to
// workgroup (u % per_xcd) * 8 + u / per_xcd, i.e. XCD u / per_xcd, so a run
// of per_xcd consecutive units (the tiles of a few heads) shares one L2.
__device__ inline int xcd_unit(int wg, int grid) {
  const int per_xcd = grid >> 3;  // grid is a multiple of 8
  return (wg & 7) * per_xcd + (wg >> 3);
}

__host__ inline int round_up8(int x) { return (x + 7) & ~7; }

// Heaviest-first ranking of G <= 256 groups of work by cost (descending,
// ties by group index), shared by the kernels that order their dispatch and
// by a host copy that tests it. Group g's key is (cost + 1) * 256 + (255 - g):
// distinct per group, larger for a larger cost and, at equal cost, for a
// lower index; costs must lie in [0, 2^23). The keys are stored padded with
// zeros (below every key) to a multiple of sixteen, and a group's rank is the
// number of keys above its own, counted sixteen at a time by `parts`
// threads, each taking every parts-th round of sixteen.
constexpr int kRankMaxGroups = 256;   // one thread per group in a 256-thread workgroup
__host__ __device__ inline unsigned rank_key(int cost, int g) {
  return (unsigned)(cost + 1) * 256u + (unsigned)(255 - g);
}
__host__ __device__ inline int rank_padded(int G) { return (G + 15) & ~15; }
__host__ __device__ inline int rank_parts(int G, int threads) {
  return G <= threads / 4 ? 4 : G <= threads / 2 ? 2 : 1;
}
// part of thread t (t < parts * G) and the group it counts for: t = part * G + g
__host__ __device__ inline int rank_part(int t, int G) { return (t >= G) + (t >= 2 * G) + (t >= 3 * G); }
// keys above `key` in rounds part, part + parts, ... of the padded keys
// (keys4: the padded keys as 16-byte vectors, rank_padded(G) / 4 of them)
__host__ __device__ inline int rank_count(const i32x4* keys4, int G, int part, int parts, unsigned key) {
  int r = 0;
  const int n16 = rank_padded(G) >> 4;
  for (int round = part; round < n16; round += parts) {
    const i32x4 v0 = keys4[4 * round], v1 = keys4[4 * round + 1], v2 = keys4[4 * round + 2],
                v3 = keys4[4 * round + 3];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r += ((unsigned)v0[e] > key) + ((unsigned)v1[e] > key) + ((unsigned)v2[e] > key) + ((unsigned)v3[e] > key);
  }
  return r;
}

}  // namespace attn
