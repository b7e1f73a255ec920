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

enum MaskKind { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_SLIDING = 2 };
enum TileClass { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Window length in keys: SLIDING's window clamped to N + 1 (a longer window
// sees the same keys), CAUSAL's is N + 1. All mask arithmetic then stays in
// [-N, 2N] and fits in 32 bits.
__host__ __device__ inline int effective_window(int mask, int window, int N) {
  return (mask == MASK_SLIDING && window <= N) ? window : N + 1;
}

// Key j visible to query i (both < N)? NONE: always; CAUSAL: j <= i;
// SLIDING: i - window < j <= i. w is effective_window().
__host__ __device__ inline bool key_visible(int mask, int w, int i, int j) {
  if (mask == MASK_NONE) return true;
  return j <= i && j > i - w;
}

// Class of the tile (query rows [m0, m1)) x (keys [n0, n1)).
// Rows >= N are ignored; keys >= N do not exist (a tile reaching past N is
// at most PARTIAL). The visible region of a causal/sliding mask is a band
// monotone in i, so the tile misses it iff it lies wholly above the diagonal
// (n0 > last row) or wholly below the window (last key < first row - w + 1),
// and lies inside it iff the last key is <= the first row and the first key
// is > last row - w.
__host__ __device__ inline int tile_class(int mask, int window, int N, int m0, int m1, int n0,
                                          int n1) {
  if (m1 > N) m1 = N;
  if (m0 >= m1 || n0 >= N || n0 >= n1) return TILE_EMPTY;
  const bool ragged = n1 > N;
  const int n_last = (ragged ? N : n1) - 1;
  if (mask == MASK_NONE) return ragged ? TILE_PARTIAL : TILE_FULL;
  const int w = effective_window(mask, window, N);
  if (n0 > m1 - 1) return TILE_EMPTY;
  if (n_last < m0 - w + 1) return TILE_EMPTY;
  if (!ragged && n_last <= m0 && n0 > (m1 - 1) - w) return TILE_FULL;
  return TILE_PARTIAL;
}

// K-tile index range [lo, hi) of tiles of bn keys that may hold a key visible
// to a row of [m0, m1). Causal: keys <= m1-1. Sliding: keys >= m0 - w + 1.
__host__ __device__ inline void k_tile_range(int mask, int window, int N, int m0, int m1, int bn,
                                             int* lo, int* hi) {
  const int nt = (N + bn - 1) / bn;
  if (m1 > N) m1 = N;
  if (m0 >= m1) {
    *lo = 0;
    *hi = 0;
    return;
  }
  if (mask == MASK_NONE) {
    *lo = 0;
    *hi = nt;
    return;
  }
  int h = (m1 - 1) / bn + 1;
  if (h > nt) h = nt;
  int first = mask == MASK_SLIDING ? m0 - effective_window(mask, window, N) + 1 : 0;
  if (first < 0) first = 0;
  *lo = first / bn;
  *hi = h;
}

// Global K-tile index range [lo, hi) of tiles of bn keys that are FULL (every
// pair visible) for the rows [m0, m1): wholly inside [0, N), every key at or
// before the first row (causal/sliding), and every key inside the last row's
// window (sliding). A band mask's FULL tiles are contiguous.
__host__ __device__ inline void full_tile_range(int mask, int window, int N, int m0, int m1, int bn, int* lo,
                                                int* hi) {
  if (m1 > N) m1 = N;
  if (m0 >= m1) {
    *lo = 0;
    *hi = 0;
    return;
  }
  int h = N / bn;
  int l = 0;
  if (mask != MASK_NONE) {
    const int c = (m0 + 1) / bn;  // n1 - 1 <= m0
    if (c < h) h = c;
    const int first = m1 - effective_window(mask, window, N);  // n0 >= m1 - w
    if (first > 0) l = (first + bn - 1) / bn;
  }
  if (l > h) l = h;
  *lo = l;
  *hi = h;
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

}  // namespace attn
