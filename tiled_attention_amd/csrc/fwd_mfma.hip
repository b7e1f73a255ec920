// Flash-attention forward on gfx950 MFMA: bf16 Q/K/V, or fp8 (E4M3FN) Q/K with
// per-128-row-block scales and bf16 or fp8 V; K/V dense or in a paged pool.
//
// Method: "Flash MSA Attention Kernel Implementation Tutorial", "Understanding
// Flash MSA Core Mechanics" -- a Q tile stays on chip while K/V tiles stream
// past it; each tile updates a running reference m and row sum l, rescales the
// accumulator by exp(m - m_new) when m moves, adds P V, and O = acc / l is
// written once. fp8 scores: "FlashAttention-3 ...", "FP8 Block Quantization"
// -- the product of the two blocks' scales multiplies the fp8 dot products; it
// is folded into the exponent's scale factor.
//
// Mapping onto CDNA4 (a workgroup is 4 waves = 128 query rows, 32 per wave;
// bf16 d = 64 dense: 64 rows and one 32-key half of every tile per wave, below):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x64_f8f6f4 for
//    fp8): K is the A operand, read from LDS; Q is the B operand, held in
//    VGPRs for the whole K loop. In the 32x32 result lane l owns query row
//    l%32 and 16 of the 32 keys; the other 16 keys of that row are in lane
//    l^32, so a row reduction needs one v_permlane32_swap.
//  * O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: P (rounded to bf16) is
//    already laid out as the B operand -- the MFMA's k index is matched to
//    the keys each lane holds -- and V^T comes from the row-major V tile
//    through ds_read_b64_tr_b16 (16 lanes read a 4x16 block, each receives a
//    column). O^T has the same lane -> row ownership as S^T, so a rescale is
//    lane-local.
//  * K and V tiles (64 keys) stream through LDS rings of NS slots filled by
//    LDS DMA (buffer_load_dwordx4 ... lds) NS-1 tiles ahead of use. The main
//    loop is unrolled so that every slot is a compile-time LDS offset, and the
//    buffer descriptors advance by one tile per step with scalar adds; a
//    descriptor clipped at the Q tile's last key tile (or the end of the
//    sequence) reads the rows past it as zeros, with no memory traffic.
//    Rows are stored unpadded with the 16-byte chunks XOR-swizzled by row, so
//    the 16-byte K reads and the transposed V reads hit distinct banks.
//  * Software pipeline: while the VALU computes the exponentials of tile i,
//    the matrix cores run S = K Q^T of tile i+1 and O += P V of tile i-1 (P V
//    is one tile behind, so neither depends on the softmax in flight), in one
//    interleaved block.
//  * bf16 d = 64, dense K/V, from 4096 keys (key split): wave w takes rows
//    64 (w & 1) .. +63 as two 32-row blocks and keys 32 (w >> 1) .. +31 of
//    every tile, so each K / V operand read from LDS feeds two MFMAs (one per
//    row block): half the LDS reads per MFMA, at the same MFMA and softmax
//    work per step. The scores fit in one buffer per row block (the step runs
//    in three phases, each block's scores overwritten after their use). The
//    two waves that share rows keep separate references and sums over their
//    key halves; the epilogue merges them through LDS, each wave finishing
//    one row block. That merge is a per-Q-tile cost: below 4096 keys the
//    32-row layout is as fast or faster.
//  * Reference without a per-tile max: P = 2^(S*c - m) against a reference m
//    that is the exact row max when it is set. A tile whose sum of P stays
//    below 2^24 per lane keeps it (no overflow is possible in fp32 / bf16 and
//    no precision is lost: only the ratio P / l enters O). When a tile's sum
//    exceeds that (or the row has no reference yet) a rare slow path takes the
//    exact row max of the tile, moves m, recomputes the tile's P and rescales
//    l and acc by 2^(m_old - m_new). O = acc / l does not depend on the
//    reference used. l sums P in fp32 with plain adds; P V applies P rounded
//    to bf16, so the weights O uses sum to 1 within the bf16 rounding of P.
//  * Masks: the keys a row sees form one interval whose ends never decrease
//    with the row (every mask kind, documents included), so the tiles the
//    workgroup must visit and the tiles fully visible to a wave's 32 rows are
//    two contiguous ranges set once per Q tile; only tiles outside the
//    latter evaluate the mask, as a compare of each key against the lane's
//    interval ("Optimizing Triton kernels for custom attention patterns on
//    H100", Patterns A and B: loop bounds, edge-only masking, document bounds
//    found by a search of the document offsets). The mask kind is a run-time
//    value: it only changes this set-up.
//  * Causal and prefix-LM: one Q tile per workgroup, dispatched costliest
//    first (tile-major from the last tile down, heads innermost, so that a
//    head's tiles share an XCD and its L2).
//  * Paged K/V ("Optimizing Triton kernels ...", Pattern C, fused instead of
//    gather-then-attend): with 64-token pages of a [pages, H, 64, d] pool one
//    page of one head is exactly one K (or V) tile, contiguous, so the same
//    LDS DMA fetches it from its page's address. With 16-token pages a tile
//    spans four pages; the rows of one DMA instruction lie in one of them, so
//    each instruction takes its own page's descriptor. A Q tile's page list
//    is staged in LDS once; each issue reads its page ids from there and
//    clips the descriptors at the list's last valid token (later rows load as
//    zeros).
#include <type_traits>
#include <utility>

#include "attn_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per K/V tile
constexpr int NW = 4;         // waves per workgroup
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 (gfx9 raw buffer)
// A lane's partial sum of one tile's P above this moves the reference. P <=
// 2^24 leaves acc and l far from the fp32 range for any sequence length.
constexpr float kSumLimit = 16777216.f;
// With P in fp8 (E4M3, largest value 448) the same bound is 448: it caps every P.
constexpr float kSumLimitFp8 = 448.f;
// With P in fp8, P is formed scaled by 2^3 (and the matrix core scales the
// product back by 2^-3): E4M3 is normal only from 2^-6, and over long rows most
// weights are small. 2^3 is the largest factor that keeps 32 weights of at
// most 1 (a lane's share of a tile right after the reference moved) under the
// 448 bound, so it adds no reference moves.
constexpr int kPShiftFp8 = 3;

// V8: V is fp8 too (codes with power-of-two block scales) and P V runs on the
// fp8 matrix cores.
template <int D, bool FP8, bool V8 = false>
struct Cfg {
  static constexpr int KROW = FP8 ? D : 2 * D;  // bytes per K row
  static constexpr int VROW = V8 ? D : 2 * D;   // bytes per V row
  static constexpr int K_SLOT = BN * KROW;
  static constexpr int V_SLOT = BN * VROW;
  static constexpr int KLD = K_SLOT / (16 * NT);  // DMA loads per thread per K tile
  static constexpr int VLD = V_SLOT / (16 * NT);
  // LDS ring slots (K and V alike): four for bf16 d = 64 (half of a CU's
  // 160 KB per workgroup, two workgroups per CU), two otherwise. Measured
  // with the mask-free loop: a 3-slot fp8 ring (a 6-step unroll) spilled
  // VGPRs and ran 3% slower than two slots on the all-fp8 kernel; at d = 64
  // four slots are 1% faster than two.
  static constexpr int NS = (!FP8 && 4 * (K_SLOT + V_SLOT) <= 80 * 1024) ? 4 : 2;
  // main-loop unroll: a multiple of NS (compile-time slots) and of 2 (the S / P double buffers)
  static constexpr int U = NS;
  static constexpr int LDS = NS * (K_SLOT + V_SLOT);
  static constexpr int QK_STEPS = FP8 ? D / 64 : D / 16;
  static constexpr int DE = D / 32;             // 32-row blocks of O^T
};

// 16-byte-chunk swizzles (chunk ^ swz(row)). The 64 banks span 256 bytes:
// four 64-byte rows, two 128-byte rows or one 256-byte row.
//  K (16-byte reads of one chunk by 16 consecutive rows): rows that share
//    bank positions get distinct chunks.
//  V (transposed reads: 4 consecutive rows x 32 bytes, two such groups side
//    by side): the 32-byte windows of the rows land on distinct banks.
template <int ROWB>
__device__ __forceinline__ int swz_k(int row) {
  static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "row size");
  return ROWB == 64 ? (row >> 2) & 3 : ROWB == 128 ? (row >> 1) & 7 : row & 15;
}
template <int ROWB>
__device__ __forceinline__ int swz_v(int row) {
  static_assert(ROWB == 128 || ROWB == 256, "row size");
  return ROWB == 128 ? ((row >> 1) & 1) << 2 : (row & 3) << 2;
}
//  K with fp8 V (rows read in the order 0-3, 32-35, 4-7, 36-39, ... by 16
//    lanes): row bit 5 joins the swizzle so rows 32 apart differ too; rows 16
//    apart (the second key block) keep the same swizzle.
template <int ROWB>
__device__ __forceinline__ int swz_k8(int row) {
  static_assert(ROWB == 64 || ROWB == 128, "row size");
  return ROWB == 64 ? ((row >> 2) & 1) | (((row >> 5) & 1) << 1) : ((row >> 1) & 3) | (((row >> 5) & 1) << 2);
}
//  fp8 V (8-bit transposed reads: 8 consecutive rows x 16 bytes per 16 lanes):
//    the even rows (and the odd rows) of an 8-row run land on distinct chunks.
//    Only row bits 1-2 (64-byte rows: bit 2) are used, so rows 8 apart share
//    the swizzle.
template <int ROWB>
__device__ __forceinline__ int swz_v8(int row) {
  static_assert(ROWB == 64 || ROWB == 128, "row size");
  return ROWB == 64 ? (row >> 2) & 1 : (row >> 1) & 3;
}

constexpr int kMaxSplitUnits = 256;   // units per head of a split launch (entries of unit_tab)

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* doc;
  int N, mask, window, nd, n_qtiles, units_per_bh, units, nsb;
  // paged K/V: k, v are [pool pages, H, pg_page, d] pools (pg_page 16 or
  // 64 tokens); (sequence s, query block b) reads the page list
  // pg_table + s * pg_stride_s + b * pg_stride_b and its length
  // pg_lens[s * len_stride_s + b * len_stride_b] (the sequence length when
  // pg_causal, else the number of keys)
  const int32_t* pg_table;
  const int32_t* pg_lens;
  int H, pg_stride_s, pg_stride_b, len_stride_s, len_stride_b, pg_max, pg_pool, pg_causal, pg_page;
  int pg_cap;          // pg_max * pg_page: the longest list in tokens
  // heaviest-first dispatch (order != ORDER_NONE): units come in `groups`
  // groups of `per_group` equal-cost units
  int order, groups, per_group;
  float scale_log2;
  // split key ranges (ORDER_SPLIT): group r of units is entry r of unit_tab
  // (Q tile | split << 12 | part << 13); the two parts of a split tile
  // t >= split_t0 write their normalised outputs (fp32 [BM, d]) and LSEs to
  // part_o / part_lse, at rows ((bh n_split + t - split_t0) 2 + part) BM
  float* part_o;
  float* part_lse;
  int split_t0, n_split, split_units;
  uint16_t unit_tab[kMaxSplitUnits];
};

enum UnitOrder {
  ORDER_NONE = 0,    // unit u -> (bh, w) = (u / units_per_bh, u % units_per_bh), XCD-grouped
  ORDER_DOC = 1,     // groups = Q tiles, costed by the keys their documents span; per group: the heads
  ORDER_SEQ = 2,     // groups = sequences of a paged prefill, costed by length; per group: heads x units
  ORDER_TILES = 3,   // one Q tile per unit, tile-major from the last tile down (costs never fall with
                     // the tile index for these masks), heads innermost so a head stays on one XCD
  ORDER_SPLIT = 4,   // as ORDER_TILES, with the costliest tiles split into two key ranges (unit_tab)
  ORDER_HEADS = 5    // paged cross-attention: head-major (per_group = sequences x query blocks), each XCD
                     // taking a contiguous run, so the blocks that read one head's pages share an L2
};
constexpr int kKeySplitMinN = 4096;   // bf16 d = 64: the key-split layout from this length
constexpr int kOrderMaxDocs = 8192;  // document offsets staged in LDS for the costing (and the LDS
                                     // must hold them behind the 2 NT ints of costs and ranks)

__device__ __forceinline__ float half_swap_max(float x) {
  // max over lane l and lane l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one v_max3_f32. Scores are finite or -inf (never NaN), so
// the IEEE-mode canonicalisation the compiler adds around fmaxf is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from buffer offset voff to LDS at m0 + lane * 16. The
// compiler does not see this load: its completion is waited for explicitly
// (sync_tiles). The s_nop covers the SALU-writes-M0 -> LDS DMA hazard; M0 is
// declared clobbered. No memory clobber: the slot written is one no wave
// reads until a later sync_tiles (whose clobber orders the LDS reads), and
// volatile asm keeps its place after the sync_tiles that freed the slot.
__device__ __forceinline__ void dma16(uint32_t m0v, int voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "m0");
}

// Wait until at most N of this wave's loads are outstanding, then barrier.
// One asm statement with a memory clobber, so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void sync_tiles() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// A stream of K (or V) tiles of one head through its LDS ring: a raw buffer
// descriptor whose base walks one tile per issue and whose size is clipped at
// the Q tile's last key tile or the sequence (rows past it load as zeros).
template <int ROWB>
struct TileStream {
  uint64_t base;    // global address of the next tile to issue
  int rows;         // rows from base to the end of the head (may go <= 0)
  // The descriptor's size field is 32 bits and a head can hold 2^31 bytes or
  // more: the row count is clamped first, which loses nothing, since one
  // issue reads one tile (BN rows) past base. Scalar 32-bit operations only.
  __device__ __forceinline__ i32x4 rsrc() const {
    constexpr int kMaxRows = 0x7fffffff / ROWB;
    // scalar instructions, so the descriptor stays in SGPRs (the compiler
    // would fold min and max into a vector med3). s_max / s_min write SCC,
    // which the compiler may hold live across this statement (the carry of a
    // 64-bit address add split around it): it is declared clobbered.
    int n;
    asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2\n\ts_mul_i32 %0, %0, %3"
        : "=&s"(n)
        : "s"(rows), "i"(kMaxRows), "i"(ROWB)
        : "scc");
    return (i32x4){(int)(uint32_t)base, (int)(uint32_t)(base >> 32), n, kBufferFlags};
  }
};

// Sorts the first min(n, NT) page ids of an LDS list into ascending order
// (equal ids keep their order; the rest of the list is left as it is), by
// rank: each thread counts the entries that precede its own. Called by the
// whole workgroup; ends with a barrier.
constexpr int kSortedPages = NT;
__device__ void sort_ids(int* ids, int n) {
  n = min(n, kSortedPages);
  const int i = threadIdx.x;
  const int key = i < n ? ids[i] : 0;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int x = ids[j];
    rank += (x < key) | ((x == key) & (j < i));
  }
  __syncthreads();
  if (i < n) ids[rank] = key;
  __syncthreads();
}

template <int D, bool FP8, bool OUT_F32, int PG, bool V8, bool KSPLIT>
struct QTile {
  static_assert(!(PG && FP8), "paged K/V is bf16");
  static_assert(!V8 || FP8, "fp8 V comes with fp8 Q and K");
  using C = Cfg<D, FP8, V8>;
  static constexpr int KROW = C::KROW, VROW = C::VROW, QK_STEPS = C::QK_STEPS, DE = C::DE;
  static constexpr int KLD = C::KLD, VLD = C::VLD, L = KLD + VLD, NS = C::NS, U = C::U;
  static constexpr float kLimit = V8 ? kSumLimitFp8 : kSumLimit;
  // key split (bf16 d = 64, dense K/V): two 32-row blocks per wave, 32 keys of each tile
  static constexpr bool KS = KSPLIT;
  static_assert(!KS || (D == 64 && !FP8 && !PG), "the key split is the bf16 d = 64 dense layout");
  static constexpr int NJ = KS ? 2 : 1;     // 32-row blocks per wave
  // LDS bytes of one row block's partial state handed over in the key-split epilogue
  static constexpr int kXchgBytes = DE * 16 * 64 * 4 + 64 * 8;
  // the schedule's run of softmax VALU instructions after each MFMA of a step
  // (d = 64: four measured 0.9-1.4% faster than six on the causal workload;
  // d = 128: no difference)
  static constexpr int kValuPerMfma = D == 64 ? 4 : 6;
  // per step: LDS operand reads and MFMAs
  static constexpr int kStepReads = KS ? QK_STEPS + 4 * DE : 2 * QK_STEPS * (FP8 ? 2 : 1) + (V8 ? 4 : 8) * DE;
  static constexpr int kStepMfma = 2 * QK_STEPS + (V8 ? 1 : 4) * DE;
  static constexpr int kFirstReads = KS ? QK_STEPS : 2 * QK_STEPS * (FP8 ? 2 : 1);
  // S^T rows of key block 1 sit this many K rows after block 0's
  static constexpr int kBlock1Rows = V8 ? 16 : 32;
  static __device__ __forceinline__ int kswz(int row) {
    if constexpr (V8)
      return swz_k8<KROW>(row);
    else
      return swz_k<KROW>(row);
  }
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QFrag;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

  const Params& p;
  unsigned char* smem;
  int lane, wave, l32, hl, N, bh, m0, wrow0, t_lo, NK;
  int kh;                   // key split: the 32-key half of every tile this wave takes
  int part;                 // -1, or the key range (0, 1) of a split Q tile this workgroup takes
  int qrow[NJ], qsrc[NJ];   // the lane's row in each row block
  int klo_m1[NJ], khi[NJ];  // keys visible to the lane's rows: klo_m1 < key <= khi
  int f_lo, f_hi;           // local tiles [f_lo, f_hi) are FULL for this wave
  size_t head;
  QFrag qf[NJ * QK_STEPS];  // [row block][k-step]
  // Q as loaded: 16-byte pieces, two per k-step for fp8
  static constexpr int QRAW = NJ * (FP8 ? 2 * QK_STEPS : QK_STEPS);
  i32x4 qraw[QRAW];
  float qscale;
  int kdma[KLD], vdma[VLD];
  int kread[QK_STEPS * (FP8 ? 2 : 1)];
  int vread[DE];
  uint32_t lds_k, lds_v;    // this wave's DMA destinations in slot 0 (K, V)
  TileStream<KROW> ks;
  TileStream<VROW> vs;
  // paged mode: pools, page ids in LDS, valid keys of the list, next tile of each stream
  uint64_t pool_k, pool_v;
  const int* pg_ids;
  int pg_h, pg_len, k_next, v_next;

  // per row block of the lane:
  float m_ref[NJ];          // reference (log2 units) of the exponentials; -inf: none yet
  float m_use[NJ];          // m_ref, or 0 while it is -inf
  float limit[NJ];          // largest tile sum of P that keeps m_ref (-1 while it is -inf)
  float l_run[NJ];          // this lane's share of the row sum
  float c_next;             // fp8: score scale of the next tile, loaded a step ahead
  int vq0, vq1;             // fp8 V: scale exponents (E8M0) of tiles i and i+1 at step i+1
  f32x16 oacc[NJ * DE];     // [row block][32-dim block]
  f32x16 S[2][2];           // S^T of two tiles: [buffer][key block] (key split: [buffer][row block])
  bf16x8 P[2][4];           // P of two tiles: [buffer][k-step] (key split: [buffer][2 row block + k-step])
  i32x8 P8[2];              // fp8 V: P of two tiles as fp8 bytes, byte k = key 32 hl + k

  // offs: the document offsets (p.doc, or a copy of them in LDS that the
  // ring does not overwrite before the workgroup's next barrier).
  // early (bf16 Q/K and dense K/V only; the ring must be free): Q is loaded
  // and the tile stream started from inside the set-up, as soon as their
  // addresses are known, instead of after it. The set-up runs once per Q
  // tile and takes microseconds of issue time; its memory latency then
  // overlaps it.
  __device__ __forceinline__ QTile(const Params& p_, unsigned char* smem_, int bh_, int qt, const int32_t* offs,
                                   bool early = false, int part_ = -1, int seq = 0)
      : p(p_), smem(smem_) {
    part = part_;
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave logic scalar
    l32 = lane & 31;
    hl = lane >> 5;
    N = p.N;
    bh = bh_;
    m0 = qt * BM;
    const int m1 = min(m0 + BM, N);
    kh = KS ? wave >> 1 : 0;
    wrow0 = m0 + (KS ? (wave & 1) * 64 : wave * 32);
    // a row past N (ragged last Q tile) computes row N - 1's result, which is
    // never stored: it stays finite and takes no extra slow-path steps
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      qrow[j] = wrow0 + 32 * j + l32;
      qsrc[j] = min(qrow[j], N - 1);
    }
    head = (size_t)bh * N;
    if constexpr (!FP8 && !PG) {
      if (early) load_q();
    }

    const int wr0 = min(wrow0, N - 1), wr1 = min(wrow0 + 32 * NJ - 1, N - 1);
    RowSpans sp;
    if constexpr (PG) {
      // keys [0, hi(row)]: causal prefill rows sit at positions len - N + row
      // seq = bh / H, from the caller (computed once, in the kernel's entry)
      const int s = seq;
      pg_h = bh - s * p.H;
      const int32_t* list = p.pg_table + (size_t)s * p.pg_stride_s + (size_t)qt * p.pg_stride_b;
      pg_len = min(max(p.pg_lens[s * p.len_stride_s + qt * p.len_stride_b], 0), p.pg_cap);
      const int pos0 = pg_len - N;
      auto span = [&](int r) -> KeySpan { return {0, p.pg_causal ? min(pg_len - 1, pos0 + r) : pg_len - 1}; };
      sp.lane = span(qsrc[0]);
      sp.lane2 = sp.lane;
      sp.wave_first = span(wr0);
      sp.wave_last = span(wr1);
      sp.tile_first = span(m0);
      sp.tile_last = span(m1 - 1);
      t_lo = 0;
      NK = sp.tile_last.hi >= 0 ? sp.tile_last.hi / BN + 1 : 0;
      // stage the page ids of the tiles this Q tile visits (clamped into the
      // pool): one per tile, or four with 16-token pages, at most the list's
      // pg_max <= kPrefillMaxPages entries
      int* ids = (int*)(smem + C::LDS);
      const int n_ids = min(NK * (BN / PG), p.pg_max);   // PG: the page size
      for (int i = tid; i < n_ids; i += NT) ids[i] = min(max(list[i], 0), p.pg_pool - 1);
      __syncthreads();
      // a cross-attention list is a set of keys, so its whole pages may be
      // visited in any order: ascending ids let the blocks of one head that
      // list the same page (running side by side on one XCD) read it close
      // together in time, from the L2. The partial last page stays last
      if (!p.pg_causal) sort_ids(ids, min(pg_len / PG, n_ids));
      pg_ids = ids;
      pool_k = (uint64_t)(uintptr_t)p.k;
      pool_v = (uint64_t)(uintptr_t)p.v;
      k_next = 0;
      v_next = 0;
    } else {
      sp = row_spans(p.mask, p.window, offs, p.nd, N, m0, m1 - 1, wr0, wr1, qsrc[0], qsrc[NJ - 1]);
      // the tile's and the wave's spans are uniform; offsets read through a
      // pointer that may be in LDS come back in VGPRs, so say so
      auto uniform = [](KeySpan k) {
        return KeySpan{__builtin_amdgcn_readfirstlane(k.lo), __builtin_amdgcn_readfirstlane(k.hi)};
      };
      sp.tile_first = uniform(sp.tile_first);
      sp.tile_last = uniform(sp.tile_last);
      sp.wave_first = uniform(sp.wave_first);
      sp.wave_last = uniform(sp.wave_last);
      touched_tiles(sp.tile_first, sp.tile_last, BN, &t_lo, &NK);
      NK -= t_lo;
      if (part >= 0) {
        // one of the two key ranges of a split Q tile: part 0 takes the first
        // half (rounded up) of its tiles, part 1 the rest
        const int h = (NK + 1) >> 1;
        t_lo += part ? h : 0;
        NK = part ? NK - h : h;
      }
    }
    // opaque to the optimizer: bounds it can reason about (NK >= 1, t_lo = 0
    // for causal masks) let it restructure the tile loop of the fp8 kernels
    // in a way that overflows the VGPRs
    asm volatile("" : "+s"(t_lo), "+s"(NK));

    // ---- the tile stream: DMA offsets, LDS slots, K/V descriptors
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int off = (u * NW + wave) * 1024 + lane * 16;
      const int row = off / KROW, ch = (off % KROW) / 16;
      kdma[u] = row * KROW + 16 * (ch ^ kswz(row));
    }
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      const int off = (u * NW + wave) * 1024 + lane * 16;
      const int row = off / VROW, ch = (off % VROW) / 16;
      if constexpr (V8)
        vdma[u] = row * VROW + 16 * (ch ^ swz_v8<VROW>(row));
      else
        vdma[u] = row * VROW + 16 * (ch ^ swz_v<VROW>(row));
    }
    const uint32_t lds0 = lds_addr(smem);
    lds_k = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
    lds_v = __builtin_amdgcn_readfirstlane(lds0 + NS * C::K_SLOT + wave * 1024);
    const uint64_t kb = PG ? 0 : (uint64_t)(uintptr_t)p.k + (head + (size_t)t_lo * BN) * KROW;
    const uint64_t vb = PG ? 0 : (uint64_t)(uintptr_t)p.v + (head + (size_t)t_lo * BN) * VROW;
    // the streams end with the Q tile's last tile (or the head): the ring's
    // refills past it (NS - 1 K tiles, NS - 2 V tiles) then read nothing
    const int rem = __builtin_amdgcn_readfirstlane(min(N - t_lo * BN, NK * BN));
    ks.base = ((uint64_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(kb >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)kb);
    vs.base = ((uint64_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(vb >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)vb);
    ks.rows = rem;
    vs.rows = rem;

    if constexpr (!FP8 && !PG) {
      if (early) start_stream();
    }

    // ---- per-lane state of the loop
    klo_m1[0] = sp.lane.lo - 1;
    khi[0] = sp.lane.hi;
    if constexpr (KS) {
      klo_m1[NJ - 1] = sp.lane2.lo - 1;
      khi[NJ - 1] = sp.lane2.hi;
    }
    // FULL range of this wave's 32 rows (a contiguous run of tiles), local indices
    full_tiles(sp.wave_first, sp.wave_last, BN, &f_lo, &f_hi);
    f_lo = min(max(f_lo - t_lo, 0), NK);
    f_hi = min(max(f_hi - t_lo, f_lo), NK);
    qscale = 1.f;
    if constexpr (V8) P8[0] = P8[1] = (i32x8){};   // defined words for the conversions to start from
    if constexpr (FP8) qscale = p.q_scale[bh * p.nsb + m0 / 128];

    // K read of k-step t: lane l32 supplies S^T row l32 of block 0 (block 1:
    // kBlock1Rows further, same swizzle), chunk of half hl. With fp8 V the
    // rows are permuted so that lane (row l32, half hl) ends up holding keys
    // 32 hl .. 32 hl + 31 of the tile: row 8j + 4h + t reads key 32h + 4j + t.
    const int krow = V8 ? 32 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3) : 32 * kh + l32;
    constexpr int KCH_STEP = FP8 ? 4 : 2;  // 16-byte chunks per k-step
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) {
      if constexpr (FP8) {
        const int c0 = KCH_STEP * t + 2 * hl;
        kread[2 * t] = krow * KROW + 16 * (c0 ^ kswz(krow));
        kread[2 * t + 1] = krow * KROW + 16 * ((c0 + 1) ^ kswz(krow));
      } else {
        kread[t] = krow * KROW + 16 * ((KCH_STEP * t + hl) ^ kswz(krow));
      }
    }
    if constexpr (V8) {
      // 8-bit transposed V reads: in each 16-lane group, output lane j takes
      // byte j % 8 of the 8 bytes that lanes 2m + j / 8 (m = 0..7) point at.
      // Lane l points at key 32 hl + 8 i + (l % 16) / 2 (read i = 0..3) and at
      // dims 32 e + 16 ((l >> 4) & 1) + 8 (l & 1) .. + 7, so lane l receives
      // dim 32 e + l % 32 of keys 32 hl + 8 i .. + 7: the A operand of the fp8
      // MFMA (row = dim, k = key - 32 hl). Row bases for even and odd e: the
      // swizzle flips chunk bit 1 (dim block parity) and bit 0 (half).
      const int row0 = 32 * hl + ((lane & 15) >> 1);
      const int g1 = (lane >> 4) & 1;
      const int sw = swz_v8<VROW>(row0);
      const int base = row0 * VROW + 16 * (g1 ^ (sw & 1)) + 8 * (lane & 1);
      const int s1 = VROW == 128 ? (sw >> 1) & 1 : 0;
      vread[0] = base + 32 * s1;
      vread[1] = base - 32 * s1;
    } else {
      // transposed V read: 16-lane group g, row rr of 4, 8-byte column piece cc
      const int g = lane >> 4, rr = (lane >> 2) & 3, cc = lane & 3;
      const int sv = swz_v<VROW>(4 * hl + rr);   // same for rows +16q and +8
      // (key split: the wave's half starts 32 rows in; rows 32 apart share the swizzle)
#pragma unroll
      for (int e = 0; e < DE; ++e)
        vread[e] = (32 * kh + 4 * hl + rr) * VROW + 16 * ((4 * e + 2 * (g & 1) + (cc >> 1)) ^ sv) + 8 * (cc & 1);
    }

#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      m_ref[j] = -INFINITY;
      m_use[j] = 0.f;
      limit[j] = -1.f;
      l_run[j] = 0.f;
    }
    c_next = tile_scale(0);
    vq0 = 127;                // the tile before the first (no P V there)
    vq1 = v_exponent(0);
  }

  // Q fragments: lane (row l32, half hl) holds the k-slots of half hl. The
  // loads are issued before the tile stream's first DMAs and are not tracked
  // by the compiler, so the loop's first wait can let the later prologue DMAs
  // stay in flight (a compiler-inserted wait for Q would drain them all).
  static __device__ __forceinline__ i32x4 gload16(const void* ptr) {
    i32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(ptr) : "memory");
    return r;
  }
  __device__ __forceinline__ void load_q() {
    if constexpr (FP8) {
      const unsigned char* qp = (const unsigned char*)p.q + (head + qsrc[0]) * D + 32 * hl;
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t) {
        qraw[2 * t] = gload16(qp + 64 * t);
        qraw[2 * t + 1] = gload16(qp + 64 * t + 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const __bf16* qp = (const __bf16*)p.q + (head + qsrc[j]) * D + 8 * hl;
#pragma unroll
        for (int t = 0; t < QK_STEPS; ++t) qraw[j * QK_STEPS + t] = gload16(qp + 16 * t);
      }
    }
  }
  // waits until at most N vector-memory operations of this wave are
  // outstanding, then for every wave; the Q registers are operands, so no
  // read of them is scheduled before the wait
  template <int N>
  __device__ __forceinline__ void q_landed() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    static_assert(QRAW == 2 || QRAW == 4 || QRAW == 8, "Q pieces");
    if constexpr (QRAW == 2)
      asm volatile("s_waitcnt vmcnt(%2)\n\ts_barrier" : "+v"(qraw[0]), "+v"(qraw[1]) : "n"(N) : "memory");
    else if constexpr (QRAW == 4)
      asm volatile("s_waitcnt vmcnt(%4)\n\ts_barrier"
                   : "+v"(qraw[0]), "+v"(qraw[1]), "+v"(qraw[2]), "+v"(qraw[3])
                   : "n"(N)
                   : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%8)\n\ts_barrier"
                   : "+v"(qraw[0]), "+v"(qraw[1]), "+v"(qraw[2]), "+v"(qraw[3]), "+v"(qraw[4]), "+v"(qraw[5]),
                     "+v"(qraw[6]), "+v"(qraw[7])
                   : "n"(N)
                   : "memory");
#pragma unroll
    for (int t = 0; t < NJ * QK_STEPS; ++t) {
      if constexpr (FP8) {
        const i32x4 a = qraw[2 * t], b = qraw[2 * t + 1];
        qf[t] = (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      } else {
        qf[t] = __builtin_bit_cast(bf16x8, qraw[t]);
      }
    }
  }

  // DMA of the next K tile into ring slot SLOT; the stream moves one tile on.
  // descriptor of paged tile j (page pg_ids[j] of this head), clipped at the list's length
  __device__ __forceinline__ i32x4 page_rsrc(uint64_t pool, int j, int slot_bytes, int row_bytes) const {
    const int jc = max(min(j, NK - 1), 0);
    const int pid = __builtin_amdgcn_readfirstlane(pg_ids[jc]);
    const uint64_t base = pool + ((uint64_t)pid * p.H + pg_h) * (uint64_t)slot_bytes;
    const int rows = min(max(pg_len - j * BN, 0), BN);
    // every word is wave-uniform; readfirstlane keeps the descriptor in SGPRs
    return (i32x4){__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                   __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)),
                   __builtin_amdgcn_readfirstlane(rows * row_bytes), kBufferFlags};
  }

  // 16-token pages: a tile spans four pages, and each DMA instruction's rows
  // (1024 bytes, at most 16 rows) lie in one of them, so every instruction
  // takes the descriptor of its own page (rows clipped at the list's length)
  // and an offset within that page
  template <int ROWB, int NLD>
  __device__ __forceinline__ void issue_paged16(uint64_t pool, int j, uint32_t lds, const int (&off)[NLD]) const {
    static_assert(1024 / ROWB <= 16, "a DMA instruction spans one 16-row page");
    // ids 4j .. 4j + 3 (16-byte aligned); entries past the staged ones only
    // reach pages with no rows to load
    const int jc = max(min(j, NK - 1), 0);
    const i32x4 q4 = *(const i32x4*)(pg_ids + 4 * jc);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int pi = (((u * NW + wave) * 1024) / ROWB) >> 4;   // page of the tile, scalar
      const int pid = __builtin_amdgcn_readfirstlane(pi == 0 ? q4[0] : pi == 1 ? q4[1] : pi == 2 ? q4[2] : q4[3]);
      const uint64_t base = pool + ((uint64_t)pid * p.H + pg_h) * (uint64_t)(16 * ROWB);
      const int rows = min(max(pg_len - (j * BN + 16 * pi), 0), 16);
      const i32x4 rs = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                        __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)),
                        __builtin_amdgcn_readfirstlane(rows * ROWB), kBufferFlags};
      dma16(lds + u * NW * 1024, off[u] & (16 * ROWB - 1), rs);
    }
  }

  template <int SLOT>
  __device__ __forceinline__ void issue_k() {
    if constexpr (PG == kPrefillSmallPage) {
      issue_paged16<KROW, KLD>(pool_k, k_next++, lds_k + SLOT * C::K_SLOT, kdma);
      return;
    } else if constexpr (PG) {
      const i32x4 rs = page_rsrc(pool_k, k_next++, C::K_SLOT, KROW);
#pragma unroll
      for (int u = 0; u < KLD; ++u) dma16(lds_k + SLOT * C::K_SLOT + u * NW * 1024, kdma[u], rs);
      return;
    }
    const i32x4 rs = ks.rsrc();
#pragma unroll
    for (int u = 0; u < KLD; ++u) dma16(lds_k + SLOT * C::K_SLOT + u * NW * 1024, kdma[u], rs);
    ks.base += BN * KROW;
    ks.rows -= BN;
  }
  template <int SLOT>
  __device__ __forceinline__ void issue_v() {
    if constexpr (PG == kPrefillSmallPage) {
      issue_paged16<VROW, VLD>(pool_v, v_next++, lds_v + SLOT * C::V_SLOT, vdma);
      return;
    } else if constexpr (PG) {
      const i32x4 rs = page_rsrc(pool_v, v_next++, C::V_SLOT, VROW);
#pragma unroll
      for (int u = 0; u < VLD; ++u) dma16(lds_v + SLOT * C::V_SLOT + u * NW * 1024, vdma[u], rs);
      return;
    }
    const i32x4 rs = vs.rsrc();
#pragma unroll
    for (int u = 0; u < VLD; ++u) dma16(lds_v + SLOT * C::V_SLOT + u * NW * 1024, vdma[u], rs);
    vs.base += BN * VROW;
    vs.rows -= BN;
  }
  // zero-size loads into V slot SLOT (the V of the tile before the first)
  template <int SLOT>
  __device__ __forceinline__ void issue_v_zero() {
    const i32x4 rs = {(int)(uint32_t)vs.base, (int)(uint32_t)(vs.base >> 32), 0, kBufferFlags};
#pragma unroll
    for (int u = 0; u < VLD; ++u) dma16(lds_v + SLOT * C::V_SLOT + u * NW * 1024, vdma[u], rs);
  }

  // S^T of the K tile in slot SLOT into S[B]: keys n0..n0+31 in S[B][0], n0+32..n0+63 in S[B][1]
  template <int SLOT, int B>
  __device__ __forceinline__ void qk() {
    const unsigned char* ksl = smem + SLOT * C::K_SLOT;
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) {
      if constexpr (FP8) {
        const i32x4 a0l = *(const i32x4*)(ksl + kread[2 * t]);
        const i32x4 a0h = *(const i32x4*)(ksl + kread[2 * t + 1]);
        const i32x4 a1l = *(const i32x4*)(ksl + kread[2 * t] + kBlock1Rows * KROW);
        const i32x4 a1h = *(const i32x4*)(ksl + kread[2 * t + 1] + kBlock1Rows * KROW);
        const i32x8 a0 = {a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]};
        const i32x8 a1 = {a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]};
        s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[t], s0, 0, 0, 0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[t], s1, 0, 0, 0, 0, 0, 0);
      } else if constexpr (KS) {
        // one read of the wave's 32 keys serves both row blocks
        const bf16x8 a = *(const bf16x8*)(ksl + kread[t]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[QK_STEPS + t], s1, 0, 0, 0);
      } else {
        const bf16x8 a0 = *(const bf16x8*)(ksl + kread[t]);
        const bf16x8 a1 = *(const bf16x8*)(ksl + kread[t] + kBlock1Rows * KROW);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[t], s1, 0, 0, 0);
      }
    }
    S[B][0] = s0;
    S[B][1] = s1;
  }

  // O^T += V^T P^T for the V tile in slot SLOT and the P in P[B] (fp8 V: the
  // tile's scale exponent vexp is applied by the matrix core)
  template <int SLOT, int B>
  __device__ __forceinline__ void pv(int vexp) {
    const unsigned char* vsl = smem + NS * C::K_SLOT + SLOT * C::V_SLOT;
    if constexpr (V8) {
      typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
#pragma unroll
      for (int e = 0; e < DE; ++e) {
        const unsigned char* vp = vsl + vread[e & 1] + 32 * e;
        i32x2 r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vp + 8 * i * VROW));
        const i32x8 a = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        oacc[e] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, P8[B], oacc[e], 0, 0, 0, vexp, 0,
                                                                 127 - kPShiftFp8);
      }
      return;
    }
    // key split: the wave's 32 keys are k-steps 0 and 1 (rows 16 q from its
    // half's start); each V^T operand serves both row blocks
#pragma unroll
    for (int q = 0; q < (KS ? 2 : 4); ++q) {
#pragma unroll
      for (int e = 0; e < DE; ++e) {
        const unsigned char* vp = vsl + vread[e] + 16 * q * VROW;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * VROW));
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, vv);
        oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[B][q], oacc[e], 0, 0, 0);
        if constexpr (KS) oacc[DE + e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[B][2 + q], oacc[DE + e], 0, 0, 0);
      }
    }
  }

  // reference the exponentials subtract: fp8 P is formed 2^kPShiftFp8 times larger
  __device__ __forceinline__ float m_exp(int j) const { return V8 ? m_use[j] - (float)kPShiftFp8 : m_use[j]; }

  // fp8 V: E8M0 exponent (biased by 127) of local tile i's power-of-two V scale
  __device__ __forceinline__ int v_exponent(int i) const {
    if constexpr (!V8) return 127;
    const float s = p.v_scale[bh * p.nsb + ((t_lo + max(min(i, NK - 1), 0)) * BN) / 128];
    return (int)((__float_as_uint(s) >> 23) & 0xFFu);
  }

  // log2-domain score scale of local tile i (fp8: times the two blocks' scales)
  __device__ __forceinline__ float tile_scale(int i) const {
    float c = p.scale_log2;
    if constexpr (FP8) c *= qscale * p.k_scale[bh * p.nsb + ((t_lo + max(min(i, NK - 1), 0)) * BN) / 128];
    return c;
  }

  // S[B] of local tile i: -inf where the key is not visible to the lane's row
  template <int B>
  __device__ __forceinline__ void mask(int i) {
    // key of S[B][b][r] is n0 + 32b + 8(r/4) + r%4 (fp8 V: n0 + 16b + r; key
    // split: n0 + 8(r/4) + r%4 in both row blocks b, n0 past the wave's half)
    // visible offsets kc: lo < kc <= hi (the interval ends before N)
    const int n0 = (t_lo + i) * BN + (V8 ? 32 : 4) * hl + 32 * kh;
    int lo[NJ], hi[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      hi[j] = khi[j] - n0;
      lo[j] = klo_m1[j] - n0;
    }
    // a bound no lane's keys of this tile cross is not tested (the causal
    // diagonal needs only the upper one, a window's far edge only the lower)
    constexpr int kMaxKc = KS ? 27 : V8 ? 31 : 59;
    const bool need_lo = __any(max(lo[0], lo[NJ - 1]) >= 0), need_hi = __any(min(hi[0], hi[NJ - 1]) < kMaxKc);
    if (need_lo && need_hi)
      mask_with<B, true, true>(lo, hi);
    else if (need_hi)
      mask_with<B, false, true>(lo, hi);
    else if (need_lo)
      mask_with<B, true, false>(lo, hi);
  }
  template <int B, bool LO, bool HI>
  __device__ __forceinline__ void mask_with(const int (&lo)[NJ], const int (&hi)[NJ]) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        constexpr int j0 = 0;
        const int j = KS ? b : j0;
        const int kc = KS ? 8 * (r >> 2) + (r & 3) : V8 ? 16 * b + r : 32 * b + 8 * (r >> 2) + (r & 3);
        const bool vis = (!HI || kc <= hi[j]) && (!LO || kc > lo[j]);
        S[B][b][r] = vis ? S[B][b][r] : -INFINITY;
      }
  }

  // P[B] = 2^(S[B] c - m_use) rounded to bf16 as the B operand (k-step q covers
  // keys 16q..16q+15 of the tile); psum gets the lane's fp32 sum of the
  // values. The sum is a tree of plain adds: v_dot2 on the packed bf16 values
  // would not issue while an MFMA is executing, these do. (The key-split
  // layout forms its exponentials per row block: ks_exps.)
  template <int B>
  __device__ __forceinline__ void exponentials(float c, float (&psum)[NJ]) {
    static_assert(!KS, "the key-split step uses ks_exps");
    float e[32];
    const float m0v = m_exp(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[8 * q + j] = fast_exp2(__builtin_fmaf(S[B][q >> 1][8 * (q & 1) + j], c, -m0v));
        if constexpr (!V8) P[B][q][j] = (__bf16)e[8 * q + j];
      }
    if constexpr (V8) {
      // byte k of the B operand is e[k] (key 32 hl + k), rounded to E4M3; the
      // two conversions write the low and the high half of the word, so its
      // starting value does not matter (and takes no instruction to set)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w], e[4 * w + 1], P8[B][w], false);
        P8[B][w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w + 2], e[4 * w + 3], d, true);
      }
    }
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
      for (int j = 0; j < w; ++j) e[j] += e[j + w];
    psum[0] = e[0];
  }

  // the row max of S[B] over the lane pair (l, l^32) for row block j (unscaled)
  template <int B>
  __device__ __forceinline__ float tile_row_max(int j) const {
    float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if constexpr (KS) {
#pragma unroll
      for (int r = 0; r < 8; ++r) mq[r & 3] = max3(mq[r & 3], S[B][j][r], S[B][j][r + 8]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) mq[r & 3] = max3(mq[r & 3], S[B][0][r], S[B][1][r]);
    }
    return half_swap_max(max3(mq[0], mq[1], fmaxf(mq[2], mq[3])));
  }

  // First tile of the Q tile: the reference is the exact row max of its
  // scores (none yet: a row that sees no key here keeps -inf, so its next
  // tile takes the slow path). Nothing is rescaled: l and acc are still 0.
  template <int B>
  __device__ __forceinline__ void set_reference(float c) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      m_ref[j] = tile_row_max<B>(j) * c;
      m_use[j] = m_ref[j] == -INFINITY ? 0.f : m_ref[j];
      limit[j] = m_ref[j] == -INFINITY ? -1.f : kLimit;
    }
  }

  // Slow path for tile i in S[B]/P[B]: the reference becomes the exact row max
  // (if it rises), P is recomputed against it, and l and acc (which holds P V
  // of the tiles before i) are rescaled.
  template <int B>
  __device__ __forceinline__ void rebase(float c, float (&psum)[NJ]) {
    float alpha[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float mt = tile_row_max<B>(j) * c;
      const float m_new = fmaxf(m_ref[j], mt);
      // 0 on a first move from -inf; 1 when nothing moves
      alpha[j] = m_new == m_ref[j] ? 1.f : fast_exp2(m_ref[j] - m_new);
      m_ref[j] = m_new;
      m_use[j] = m_ref[j] == -INFINITY ? 0.f : m_ref[j];
      limit[j] = m_ref[j] == -INFINITY ? -1.f : kLimit;
    }
    exponentials<B>(c, psum);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      l_run[j] *= alpha[j];
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j * DE + e][r] *= alpha[j];
    }
  }

  // One pipeline step at local tile i (PH = i mod U): S of tile i+1 and P V of
  // tile i-1 on the matrix cores, the exponentials of tile i on the VALU.
  // FIRST (i = 0): there is no P V yet, and the row max of the tile sets the
  // reference before the exponentials, which are then formed once.
  // MASK: the step tests whether tile i is outside this wave's FULL range and
  // masks it then; the loop's bulk runs without (see loop()).
  // ---- key split: one S buffer per row block, the step in three phases
  // K operands of the wave's 32 keys of the tile in slot SLOT (both row blocks use them)
  template <int SLOT>
  __device__ __forceinline__ void ks_kread(bf16x8 (&kop)[QK_STEPS]) const {
    const unsigned char* ksl = smem + SLOT * C::K_SLOT;
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) kop[t] = *(const bf16x8*)(ksl + kread[t]);
  }
  template <int J>
  __device__ __forceinline__ void ks_qk(const bf16x8 (&kop)[QK_STEPS]) {
    f32x16 s0 = {};
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t)
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[t], qf[J * QK_STEPS + t], s0, 0, 0, 0);
    S[0][J] = s0;
  }
  // P[B][2J + q] = 2^(S[0][J] c - m_use[J]) as bf16; returns the lane's sum
  template <int B, int J>
  __device__ __forceinline__ float ks_exps(float c) {
    float e[16];
    const float mj = m_use[J];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        e[8 * q + jj] = fast_exp2(__builtin_fmaf(S[0][J][8 * q + jj], c, -mj));
        P[B][2 * J + q][jj] = (__bf16)e[8 * q + jj];
      }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int jj = 0; jj < w; ++jj) e[jj] += e[jj + w];
    return e[0];
  }
  template <int J>
  __device__ __forceinline__ void ks_set_reference(float c) {
    m_ref[J] = tile_row_max<0>(J) * c;
    m_use[J] = m_ref[J] == -INFINITY ? 0.f : m_ref[J];
    limit[J] = m_ref[J] == -INFINITY ? -1.f : kLimit;
  }
  template <int B, int J>
  __device__ __forceinline__ void ks_rebase(float c, float& psum) {
    const float mt = tile_row_max<0>(J) * c;
    const float m_new = fmaxf(m_ref[J], mt);
    const float alpha = m_new == m_ref[J] ? 1.f : fast_exp2(m_ref[J] - m_new);
    m_ref[J] = m_new;
    m_use[J] = m_ref[J] == -INFINITY ? 0.f : m_ref[J];
    limit[J] = m_ref[J] == -INFINITY ? -1.f : kLimit;
    psum = ks_exps<B, J>(c);
    l_run[J] *= alpha;
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[J * DE + e][r] *= alpha;
  }
  // Step at local tile i, S_i in S[0]: (1) P V of tile i-1 beside the
  // exponentials of row block 0, (2) S of tile i+1 for block 0 beside the
  // exponentials of block 1, (3) S of tile i+1 for block 1. A block's scores
  // are overwritten only after its reference test (and rare rebase) used them.
  template <int PH, bool FIRST, bool MASK>
  __device__ __forceinline__ void ks_step(int i) {
    constexpr int B = PH & 1;          // P[B] receives P_i
    constexpr int BO = B ^ 1;          // P[BO] holds P_{i-1}
    sync_tiles<(NS - 2) * L>();
    const float c = p.scale_log2;
    if constexpr (kEarlyRefill) refill<PH>();
    if constexpr (MASK) {
      if ((unsigned)(i - f_lo) >= (unsigned)(f_hi - f_lo)) mask<0>(i);
    }
    bf16x8 kop[QK_STEPS];
    ks_kread<(PH + 1) % NS>(kop);
    if constexpr (!FIRST) pv<(PH + NS - 1) % NS, BO>(127);
    if constexpr (FIRST) ks_set_reference<0>(c);
    float ps0 = ks_exps<B, 0>(c);
    __builtin_amdgcn_sched_group_barrier(0x100, FIRST ? QK_STEPS : kStepReads, 0);
    if constexpr (!FIRST) {
#pragma unroll
      for (int k = 0; k < 4 * DE; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
      }
      if (__builtin_expect(__any(!(ps0 <= limit[0])), 0)) ks_rebase<B, 0>(c, ps0);
    }
    l_run[0] += ps0;
    ks_qk<0>(kop);
    if constexpr (FIRST) ks_set_reference<1>(c);
    float ps1 = ks_exps<B, 1>(c);
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
    if constexpr (!FIRST) {
      if (__builtin_expect(__any(!(ps1 <= limit[1])), 0)) ks_rebase<B, 1>(c, ps1);
    }
    l_run[1] += ps1;
    ks_qk<1>(kop);
    if constexpr (!kEarlyRefill) refill<PH>();
  }

  template <int PH, bool FIRST = false, bool MASK = true>
  __device__ __forceinline__ void step(int i) {
    if constexpr (KS)
      ks_step<PH, FIRST, MASK>(i);
    else
      step32<PH, FIRST, MASK>(i);
  }
  // the 32-row layout's step
  template <int PH, bool FIRST, bool MASK>
  __device__ __forceinline__ void step32(int i) {
    constexpr int B = PH & 1;          // S[B] holds S_i, P[B] receives P_i
    constexpr int BO = B ^ 1;          // S[BO] receives S_{i+1}, P[BO] holds P_{i-1}
    // {K_{i+1}, V_{i-1}} landed; every wave is done with K_i and V_{i-2}
    sync_tiles<(NS - 2) * L>();
    float c = p.scale_log2;
    int vpv = 127;
    if constexpr (FP8) {
      // the scales loaded a step ago: waited for here, before this step's LDS reads
      c = c_next;
      asm volatile("" : "+v"(c));
      c_next = tile_scale(i + 1);
      if constexpr (V8) {
        asm volatile("" : "+v"(vq1));
        vpv = vq0;            // tile i - 1, whose P V runs now
        vq0 = vq1;            // tile i
        vq1 = v_exponent(i + 1);
      }
    }
    // refill the slots freed at this step's sync_tiles. A ring of 2 slots
    // is refilled at once, so the tiles have a whole step to land
    // before the next step waits for them; a 4-slot ring has slack to spare
    // and refills after the MFMA block, where a stall on the texture-address
    // queue overlaps the MFMAs in flight.
    if constexpr (kEarlyRefill) refill<PH>();
    if constexpr (MASK) {
      if ((unsigned)(i - f_lo) >= (unsigned)(f_hi - f_lo)) mask<B>(i);
    }
    // unconditional, so the block has no branch: for i + 1 == NK the slot
    // holds zeros (the stream ends at tile NK - 1) whose scores are never used
    qk<(PH + 1) % NS, BO>();
    if constexpr (!FIRST) pv<(PH + NS - 1) % NS, BO>(vpv);
    if constexpr (FIRST) set_reference<B>(c);
    float psum[NJ];
    exponentials<B>(c, psum);
    // issue order: every LDS operand read of the step first, then each MFMA
    // followed by a run of the softmax VALU work
    constexpr int kReads = FIRST ? kFirstReads : kStepReads;
    constexpr int kMfma = FIRST ? 2 * QK_STEPS : kStepMfma;
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
    for (int k = 0; k < kMfma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    // P is converted before the test below, not sunk past its branch: the
    // conversions then issue while the sum's add tree completes (1-3% at
    // d = 64; the bf16 d = 128 kernels would spill the extra live values)
    if constexpr (V8) {
      asm volatile("" ::"v"(P8[B]));
    } else if constexpr (D == 64) {
#pragma unroll
      for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(P[B][q]));
    }
    // a lane without a reference yet, or a tile sum past the limit, moves it
    // (before P V of the tile, which the next step issues)
    if constexpr (!FIRST) {
      bool over = !(psum[0] <= limit[0]);
      if constexpr (KS) over = over || !(psum[1] <= limit[1]);
      if (__builtin_expect(__any(over), 0)) rebase<B>(c, psum);
    }
    // the sum of P itself (fp8 P: the sum of the scaled values times 2^-3)
#pragma unroll
    for (int j = 0; j < NJ; ++j) l_run[j] += V8 ? psum[j] * (1.f / (1 << kPShiftFp8)) : psum[j];
    if constexpr (!kEarlyRefill) refill<PH>();
  }

  static constexpr bool kEarlyRefill = NS == 2;
  template <int PH>
  __device__ __forceinline__ void refill() {
    issue_k<PH % NS>();                // K_{i+NS} into K_i's slot
    issue_v<(PH + NS - 2) % NS>();     // V_{i+NS-2} into V_{i-2}'s slot
  }

  template <int PH>
  __device__ __forceinline__ void step_if(int i) {
    if (i < NK) step<PH>(i);
  }
  // steps 1 .. U-1 (the first group after step 0)
  template <int... PHS>
  __device__ __forceinline__ void run_head(std::integer_sequence<int, PHS...>) {
    (step_if<PHS + 1>(PHS + 1), ...);
  }

  // P V of the last tile (local NK - 1, phase PH)
  template <int PH>
  __device__ __forceinline__ void drain() {
    sync_tiles<(NS - 2) * L>();
    pv<PH % NS, PH & 1>(vq0);
  }

  template <int... PHS>
  __device__ __forceinline__ void run_steps(int i, std::integer_sequence<int, PHS...>) {
    (step<PHS>(i + PHS), ...);
  }
  template <int... PHS>
  __device__ __forceinline__ void run_steps_full(int i, std::integer_sequence<int, PHS...>) {
    (step<PHS, false, false>(i + PHS), ...);
  }
  template <int... PHS>
  __device__ __forceinline__ void run_tail(int i, std::integer_sequence<int, PHS...>) {
    (step_if<PHS>(i + PHS), ...);
  }
  template <int... PHS>
  __device__ __forceinline__ void run_drain(int ph, std::integer_sequence<int, PHS...>) {
    ((ph == PHS ? drain<PHS>() : (void)0), ...);
  }
  // batch {K_{x+NS}, V_{x+NS-2}} of step x = XS + 1 - NS. V_{-1} is never
  // read (step 0 has no P V); its zero-size loads keep every batch at the
  // same count of loads, which the waits rely on
  template <int XS>
  __device__ __forceinline__ void prologue_batch() {
    issue_k<XS + 1>();
    if constexpr (XS == 0) {
      issue_v_zero<NS - 1>();
    } else {
      issue_v<XS - 1>();
    }
  }
  template <int... XS>
  __device__ __forceinline__ void prologue(std::integer_sequence<int, XS...>) {
    (prologue_batch<XS>(), ...);
  }

  // DMA of the first tiles: K_0, then K_1..K_{NS-1} with V_{-1}..V_{NS-3}.
  // The ring must be free (every wave past its last read of a previous Q tile).
  __device__ __forceinline__ void start_stream() {
    issue_k<0>();
    prologue(std::make_integer_sequence<int, NS - 1>{});
  }

  // The K loop: S_0, the pipeline steps, then P V of the last tile; ends with
  // every DMA landed and every wave past its last LDS read.
  __device__ __forceinline__ void loop() {
#pragma unroll
    for (int e = 0; e < NJ * DE; ++e) oacc[e] = (f32x16){};
    // Q (issued first) and K_0 have landed once no more than the NS - 1
    // later prologue batches are outstanding (the counter drains in order);
    // those batches keep streaming under the first steps
    q_landed<(NS - 1) * L>();
    if (NK > 0) {
      qk<0, 0>();
      step<0, true>(0);
    }
    run_head(std::make_integer_sequence<int, U - 1>{});

    // The bulk: tiles every row of this wave sees in full, in a loop with no
    // mask code. A conditional mask inside the step made the compiler move
    // the 32 scores between registers at the join on every step (measured
    // 3-4% of the causal d = 64 launch); the tiles around the bulk go through
    // steps that test for the mask. Waves may split their steps differently:
    // each still runs one barrier per step.
    int i = U;
    const int bulk_end = f_lo <= U ? f_hi : U;
    for (; i + U <= bulk_end; i += U) run_steps_full(i, std::make_integer_sequence<int, U>{});
    for (; i + U <= NK; i += U) run_steps(i, std::make_integer_sequence<int, U>{});
    run_tail(i, std::make_integer_sequence<int, U - 1>{});
    {
      // the count re-read through an opaque copy: a test of it formed before
      // the loop would otherwise be held (and spilled) across it
      int nk = NK;
      asm volatile("" : "+s"(nk));
      if (nk > 0) run_drain((nk - 1) % U, std::make_integer_sequence<int, U>{});
    }
    // drain the DMA tail before the LDS is reused
    sync_tiles<0>();
  }

  // O = acc / l, written once (and the LSE)
  __device__ __forceinline__ void epilogue() {
    if constexpr (KS) {
      // the two waves of a row pair each finish one row block: a wave hands
      // over the other block's (acc, m, l) through LDS (the ring is free: the
      // loop ended with every wave past its last read) and merges its own
      // block with its partner's
      const float l0 = half_swap_sum(l_run[0]), l1 = half_swap_sum(l_run[1]);
      if (kh)
        handover<0>(l0);
      else
        handover<1>(l1);
      __syncthreads();
      if (kh)
        finish<1>(l1);
      else
        finish<0>(l0);
      return;
    }
    const float l_tot = half_swap_sum(l_run[0]);
    if (qrow[0] < N) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float x0 = oacc[e][4 * g4 + 0] * inv, x1 = oacc[e][4 * g4 + 1] * inv;
          const float x2 = oacc[e][4 * g4 + 2] * inv, x3 = oacc[e][4 * g4 + 3] * inv;
          store_o(qrow[0], 32 * e + 8 * g4 + 4 * hl, x0, x1, x2, x3);
        }
      if (hl == 0) store_lse(qrow[0], l_tot > 0.f ? (m_ref[0] + __log2f(l_tot)) * kLn2 : -INFINITY);
    }
  }

  // first row of this part's slice of the split outputs
  __device__ __forceinline__ size_t part_row0() const {
    return ((size_t)(bh * p.n_split + (m0 / BM - p.split_t0)) * 2 + part) * BM;
  }
  // O (or, for a part of a split Q tile, its normalised fp32 output) of one row, dims d0 .. d0 + 3
  __device__ __forceinline__ void store_o(int row, int d0, float x0, float x1, float x2, float x3) const {
    if (part >= 0) {
      *(float4*)(p.part_o + (part_row0() + (row - m0)) * D + d0) = make_float4(x0, x1, x2, x3);
    } else if constexpr (OUT_F32) {
      *(float4*)((float*)p.o + (head + row) * D + d0) = make_float4(x0, x1, x2, x3);
    } else {
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
      const bf16x4 ov = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
      *(bf16x4*)((__bf16*)p.o + (head + row) * D + d0) = ov;
    }
  }
  // the row's LSE (natural log): to lse if asked for; a split part's always goes to part_lse
  __device__ __forceinline__ void store_lse(int row, float v) const {
    if (part >= 0)
      p.part_lse[part_row0() + (row - m0)] = v;
    else if (p.lse != nullptr)
      p.lse[head + row] = v;
  }

  // key split: LDS region of row pair (wave & 1), row block J: the state of
  // block J from the wave that does not finish it. Accumulators lane-major in
  // 16-byte pieces (piece k of every lane, then piece k + 1), then (m, l) per lane.
  __device__ __forceinline__ unsigned char* xchg(int J) const { return smem + ((wave & 1) * 2 + J) * kXchgBytes; }
  template <int J>
  __device__ __forceinline__ void handover(float l_tot) {
    unsigned char* x = xchg(J);
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = oacc[J * DE + e];
        *(f32x4*)(x + ((e * 4 + g) * 64 + lane) * 16) = (f32x4){a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
      }
    *(float2*)(x + DE * 16 * 64 * 4 + lane * 8) = make_float2(m_ref[J], l_tot);
  }
  template <int J>
  __device__ __forceinline__ void finish(float l_own) {
    const unsigned char* x = xchg(J);
    const float2 ml = *(const float2*)(x + DE * 16 * 64 * 4 + lane * 8);
    // the merge of two partial states over disjoint keys (the combine of
    // split-key attention): both to the larger reference
    const float m1 = m_ref[J], m2 = ml.x;
    const float m = fmaxf(m1, m2);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
    const float a2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - m);
    const float l_tot = l_own * a1 + ml.y * a2;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float w1 = a1 * inv, w2 = a2 * inv;
    const int row = qrow[J];
    if (row < N) {
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 o2 = *(const f32x4*)(x + ((e * 4 + g4) * 64 + lane) * 16);
          const f32x16& a = oacc[J * DE + e];
          store_o(row, 32 * e + 8 * g4 + 4 * hl, a[4 * g4] * w1 + o2[0] * w2, a[4 * g4 + 1] * w1 + o2[1] * w2,
                  a[4 * g4 + 2] * w1 + o2[2] * w2, a[4 * g4 + 3] * w1 + o2[3] * w2);
        }
      if (hl == 0) store_lse(row, l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY);
    }
  }
};

// Last document d in [0, nd) whose start offs[d] is <= x (offs in LDS).
__device__ __forceinline__ int lds_doc_of(const int* offs, int nd, int x) {
  int lo = 0, hi = nd - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Heaviest-first dispatch. Workgroups are handed out in id order as slots
// free up, so giving the lowest ids to the costliest units makes that
// greedy dispatch longest-first. Every workgroup costs all groups (one per
// thread, groups <= NT), ranks them in LDS (cost descending, then index) and
// takes the group of rank u / per_group. Uses the LDS before any tile lands.
__device__ void ordered_unit(const Params& p, unsigned char* smem, int u, int* bh, int* w) {
  int* cost = (int*)smem;
  int* order = cost + NT;
  int* offs = order + NT;
  const int tid = threadIdx.x;
  const int G = p.groups;
  if (p.order == ORDER_DOC) {
    for (int i = tid; i <= p.nd; i += NT) offs[i] = p.doc[i];
    __syncthreads();
  }
  if (tid < G) {
    int c;
    if (p.order == ORDER_DOC) {
      // keys touched by Q tile tid: from the first row's document start to the
      // last row's document end (or the last row itself when causal)
      const int m0 = tid * BM, m1 = min(m0 + BM, p.N);
      const bool causal = p.mask == MASK_DOCUMENT_CAUSAL;
      int d = lds_doc_of(offs, p.nd, m0);
      const KeySpan f = doc_span(causal, offs[d], offs[d + 1], p.N, m0);
      d = lds_doc_of(offs, p.nd, m1 - 1);
      const KeySpan l = doc_span(causal, offs[d], offs[d + 1], p.N, m1 - 1);
      c = l.hi / BN - f.lo / BN + 1;
    } else {
      c = min(max(p.pg_lens[tid], 0), p.pg_cap);
    }
    // the ranking's key (attn_common.h): by cost, then by index
    cost[tid] = (int)rank_key(c, tid);
    order[tid] = 0;                        // rank counter of group tid
  } else if (tid < rank_padded(G)) {
    cost[tid] = 0;                         // padding to whole rounds of sixteen; below every key
  }
  __syncthreads();
  // rank = number of larger keys. The keys are read sixteen at a time (four
  // broadcast 16-byte LDS reads in flight per round), and with G <= 128
  // groups two or four threads share a group's rounds and add their counts:
  // one read per group in turn took about 8000 cycles at 128 groups, and
  // every workgroup ranks all groups.
  const int parts = rank_parts(G, NT);
  if (tid < parts * G) {
    const int part = rank_part(tid, G);
    const int g = tid - part * G;
    const int r = rank_count((const i32x4*)cost, G, part, parts, (unsigned)cost[g]);
    atomicAdd(&order[g], r);
  }
  __syncthreads();
  // the ranks are a permutation of [0, G); the clamps keep a mistake in them
  // from turning into an access outside the table or a tile index outside
  // the tensors. The keys are dead: their array takes the group of each rank.
  if (tid < G) cost[min(max(order[tid], 0), G - 1)] = tid;
  __syncthreads();
  const int grp = min(max(cost[u / p.per_group], 0), G - 1);
  const int sub = u - (u / p.per_group) * p.per_group;
  // no barrier here: nothing writes these arrays before the caller's next
  // barrier (the page-id staging, or the one after the document spans), and
  // the ring's DMA starts only after it
  if (p.order == ORDER_DOC) {             // group = Q tile, sub = head
    *bh = sub;
    *w = p.n_qtiles - 1 - grp;
  } else {                                // ORDER_SEQ: group = sequence, sub = (unit, head)
    // heads innermost: the waves reading one page's head slices, adjacent in
    // the pool, run side by side (3-4% faster than units innermost)
    *bh = grp * p.H + sub % p.H;
    *w = sub / p.H;
  }
}

template <int D, bool FP8, bool OUT_F32, int PG, bool V8, bool KSPLIT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_mfma_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg<D, FP8, V8>::LDS + (PG ? 4 * kPrefillMaxPages : 0)];
  int bh, w, part = -1;
  // the set-up's kernel arguments in one batch of loads before the first
  // branch: the compiler otherwise loads each field where it is first used,
  // each behind a wait of its own (a chain of scalar round trips)
  asm volatile("" ::"s"(p.order), "s"(p.units), "s"(p.per_group), "s"(p.n_qtiles), "s"(p.N), "s"(p.mask),
               "s"(p.window), "s"(p.nd), "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.H), "s"(p.o), "s"(p.lse));
  if (p.order == ORDER_TILES || p.order == ORDER_SPLIT) {
    const int u = blockIdx.x;
    if (u >= p.units) return;
    const int r = u / p.per_group;       // per_group = B*H
    bh = u - r * p.per_group;
    w = r;                               // tile n_qtiles - 1 - r
    if (p.order == ORDER_SPLIT) {
      const int e = p.unit_tab[r];
      w = p.n_qtiles - 1 - min(e & 0xfff, p.n_qtiles - 1);
      part = (e >> 12) & 1 ? (e >> 13) & 1 : -1;
    }
  } else if (p.order == ORDER_HEADS) {
    const int u = xcd_unit(blockIdx.x, gridDim.x);
    if (u >= p.units) return;
    const int h = u / p.per_group;
    const int r = u - h * p.per_group;
    const int s = r / p.n_qtiles;
    bh = s * p.H + h;
    w = r - s * p.n_qtiles;
  } else if (p.order != ORDER_NONE) {
    // ranks follow workgroup ids (the dispatch order); each XCD takes every 8th
    const int u = blockIdx.x;
    if (u >= p.units) return;
    ordered_unit(p, smem, u, &bh, &w);
  } else {
    const int u = xcd_unit(blockIdx.x, gridDim.x);
    if (u >= p.units) return;
    bh = u / p.units_per_bh;
    w = u - bh * p.units_per_bh;
  }
  bh = __builtin_amdgcn_readfirstlane(bh);
  w = __builtin_amdgcn_readfirstlane(w);
  // unit w is Q tile n_qtiles - 1 - w: the costlier tiles come first in
  // the orders that rank them
  const int tile = p.n_qtiles - 1 - w;
  const int seq = PG ? __builtin_amdgcn_readfirstlane(bh / p.H) : 0;   // paged: the sequence
  {
    // with the ordering's LDS copy of the document offsets, the spans are
    // searched there (a search in global memory costs several dependent
    // round trips per workgroup); a barrier then frees the LDS for the ring
    const bool lds_offs = p.order == ORDER_DOC;
    const bool early = !FP8 && !PG && !lds_offs;
    QTile<D, FP8, OUT_F32, PG, V8, KSPLIT> a(p, smem, bh, tile, lds_offs ? (const int32_t*)(smem + 2 * NT * sizeof(int)) : p.doc,
                                     early, part, seq);
    if (!early) {
      a.load_q();
      if (lds_offs) __syncthreads();
      a.start_stream();
    }
    a.loop();
    a.epilogue();
  }
}

Params base_params(const void* q, const void* k, const void* v, void* o, float* lse, int N, float scale) {
  Params p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.N = N;
  p.n_qtiles = (N + BM - 1) / BM;
  p.nsb = (N + 127) / 128;
  p.scale_log2 = scale * kLog2e;
  return p;
}

// Merge of the two key ranges of each split Q tile (one workgroup per tile):
// from the parts' normalised outputs O_i and LSEs L_i, O = sum_i w_i O_i with
// w_i = exp(L_i - L) and L = log sum_i exp(L_i) -- the combine of split-key
// attention, as in the decode's combine. A row no part sees keys of gets
// O = 0 and L = -inf.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(NT) void split_combine_kernel(Params p) {
  const int bh = blockIdx.x / p.n_split;
  const int m0 = (p.split_t0 + blockIdx.x % p.n_split) * BM;
  const size_t r0 = (size_t)blockIdx.x * 2 * BM;     // part 0's rows; part 1's follow
  const size_t head = (size_t)bh * p.N;
  constexpr int C4 = D / 4;
  for (int i = threadIdx.x; i < BM * C4; i += NT) {
    const int r = i / C4, c = i - r * C4;
    const int row = m0 + r;
    if (row >= p.N) break;
    const float l0 = p.part_lse[r0 + r], l1 = p.part_lse[r0 + BM + r];
    const float L = fmaxf(l0, l1);
    float w0 = 0.f, w1 = 0.f, lse = -INFINITY;
    if (L != -INFINITY) {
      w0 = fast_exp2((l0 - L) * kLog2e);
      w1 = fast_exp2((l1 - L) * kLog2e);
      const float sum = w0 + w1;
      lse = L + __log2f(sum) * kLn2;
      w0 /= sum;
      w1 /= sum;
    }
    const float4 a = *(const float4*)(p.part_o + (r0 + r) * D + 4 * c);
    const float4 b = *(const float4*)(p.part_o + (r0 + BM + r) * D + 4 * c);
    const float x0 = w0 * a.x + w1 * b.x, x1 = w0 * a.y + w1 * b.y;
    const float x2 = w0 * a.z + w1 * b.z, x3 = w0 * a.w + w1 * b.w;
    if constexpr (OUT_F32) {
      *(float4*)((float*)p.o + (head + row) * D + 4 * c) = make_float4(x0, x1, x2, x3);
    } else {
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
      const bf16x4 ov = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
      *(bf16x4*)((__bf16*)p.o + (head + row) * D + 4 * c) = ov;
    }
    if (c == 0 && p.lse != nullptr) p.lse[head + row] = lse;
  }
}

template <int D, bool FP8, bool OUT_F32, int PG, bool V8 = false, bool KSPLIT = false>
hipError_t launch_p(Params& p, int BH, hipStream_t stream) {
  if (p.order == ORDER_SPLIT) {
    p.units_per_bh = p.split_units;
    p.units = BH * p.units_per_bh;
    hipLaunchKernelGGL((fwd_mfma_kernel<D, FP8, OUT_F32, PG, V8, KSPLIT>), dim3(round_up8(p.units)), dim3(NT), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((split_combine_kernel<D, OUT_F32>), dim3(BH * p.n_split), dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  p.units_per_bh = p.n_qtiles;
  p.units = BH * p.units_per_bh;
  const int grid = round_up8(p.units);
  hipLaunchKernelGGL((fwd_mfma_kernel<D, FP8, OUT_F32, PG, V8, KSPLIT>), dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

// Split key ranges for grids of few Q tiles per workgroup slot (causal and
// prefix-LM, bf16): with at most about one tile per slot the costliest tile
// sets the launch time. Tiles costing more than half the costliest are cut
// into two key ranges, and all units are dispatched costliest first. The
// merge costs a second launch and a pass over the parts, so the plan splits
// only where that measured faster: up to half a tile per slot when the
// costliest tile holds at least 32 steps' worth of work (64-key tiles at
// d = 64; half as many at d = 128), and up to 1.5 tiles per slot from 128.
// A workgroup left alone on a CU runs faster than a paired one, which evens
// out much of the imbalance below that. The plan depends only on the shape
// and mask, so the size query and the launch agree.
struct SplitPlan {
  int units, t0, n_split;
  uint16_t tab[kMaxSplitUnits];
};
constexpr int kSplitSlots = 512;            // workgroup slots: 256 CUs x 2 workgroups
bool plan_split(const FwdArgs& a, SplitPlan* sp) {
  if (a.in_f32 || a.fp8 || a.v8) return false;
  if (a.mask != MASK_CAUSAL && a.mask != MASK_PREFIX_LM) return false;
  const int T = (a.N + BM - 1) / BM;
  if ((long long)a.BH * T * 2 > 3LL * kSplitSlots || 2 * T > kMaxSplitUnits || T > 0xfff) return false;
  int cost[kMaxSplitUnits / 2];
  int cmax = 0;
  for (int t = 0; t < T; ++t) {
    const int m1 = (t * BM + BM < a.N ? t * BM + BM : a.N) - 1;
    int lo, hi;
    touched_tiles(band_span(a.mask, a.window, a.N, t * BM), band_span(a.mask, a.window, a.N, m1), BN, &lo, &hi);
    cost[t] = hi - lo;
    cmax = cost[t] > cmax ? cost[t] : cmax;
  }
  const long long tiles = (long long)a.BH * T;
  const int work = cmax * (a.d / 64);       // the costliest tile, in d = 64 steps
  if (!((2 * tiles <= kSplitSlots && work >= 32) || (2 * tiles <= 3LL * kSplitSlots && work >= 128))) return false;
  const int lim = (cmax + 1) / 2;
  // the split tiles must be the last ones (costs never fall with t for these masks)
  int t0 = T;
  while (t0 > 0 && cost[t0 - 1] > lim) --t0;
  for (int t = 0; t < t0; ++t)
    if (cost[t] > lim) return false;
  if (t0 == T) return false;
  // units (cost, entry), costliest first; ties: later tile, then part 0
  struct U { int c, e; };
  U u[kMaxSplitUnits];
  int n = 0;
  for (int t = 0; t < T; ++t) {
    if (t < t0) {
      u[n++] = {cost[t], t};
    } else {
      const int h = (cost[t] + 1) / 2;
      u[n++] = {h, t | 1 << 12};
      u[n++] = {cost[t] - h, t | 1 << 12 | 1 << 13};
    }
  }
  for (int i = 1; i < n; ++i) {            // insertion sort, n <= 256
    const U x = u[i];
    int j = i;
    auto before = [](const U& p, const U& q) {
      return p.c != q.c ? p.c > q.c : (p.e & 0xfff) != (q.e & 0xfff) ? (p.e & 0xfff) > (q.e & 0xfff) : p.e < q.e;
    };
    while (j > 0 && before(x, u[j - 1])) {
      u[j] = u[j - 1];
      --j;
    }
    u[j] = x;
  }
  sp->units = n;
  sp->t0 = t0;
  sp->n_split = T - t0;
  for (int i = 0; i < n; ++i) sp->tab[i] = (uint16_t)u[i].e;
  return true;
}

template <int D, bool FP8, bool OUT_F32, bool V8 = false>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  Params p = base_params(a.q, a.k, a.v, a.o, a.lse, a.N, a.scale);
  p.q_scale = a.q_scale;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.doc = a.doc;
  p.mask = a.mask;
  p.window = a.window;
  p.nd = a.num_docs;
  if (is_document(a.mask)) {
    if (p.n_qtiles <= NT && a.num_docs + 1 <= kOrderMaxDocs &&
        (2 * NT + a.num_docs + 1) * (int)sizeof(int) <= Cfg<D, FP8, V8>::LDS) {
      p.order = ORDER_DOC;
      p.groups = p.n_qtiles;
      p.per_group = a.BH;
    }
  } else if (a.mask == MASK_CAUSAL || a.mask == MASK_PREFIX_LM) {
    // Q tiles of rising cost: single tiles, costliest first, so a slot that
    // frees early takes a cheap tile (a pair of tiles t and T-1-t per
    // workgroup left one of the two workgroups of a CU running alone at the
    // end: they share the CU unevenly)
    p.order = ORDER_TILES;
    p.per_group = a.BH;
    SplitPlan sp;
    if (a.workspace != nullptr && plan_split(a, &sp)) {
      p.order = ORDER_SPLIT;
      p.split_units = sp.units;
      p.split_t0 = sp.t0;
      p.n_split = sp.n_split;
      for (int i = 0; i < sp.units; ++i) p.unit_tab[i] = sp.tab[i];
      p.part_o = (float*)a.workspace;
      p.part_lse = p.part_o + (size_t)a.BH * sp.n_split * 2 * BM * D;
    }
  }
  // the key-split layout for bf16 d = 64 from kKeySplitMinN keys: fewer LDS
  // reads per step, at a per-Q-tile cost (the epilogue's merge) that short
  // loops do not recover
  if constexpr (D == 64 && !FP8) {
    if (a.N >= kKeySplitMinN) return launch_p<D, FP8, OUT_F32, false, false, true>(p, a.BH, stream);
  }
  return launch_p<D, FP8, OUT_F32, false, V8>(p, a.BH, stream);
}

template <int D, bool OUT_F32>
hipError_t launch_pg(const PagedFwdArgs& a, hipStream_t stream) {
  Params p = base_params(a.q, a.k_pool, a.v_pool, a.o, a.lse, a.q_len, a.scale);
  p.pg_table = a.table;
  p.pg_lens = a.lens;
  p.H = a.H;
  p.pg_stride_s = a.table_stride_s;
  p.pg_stride_b = a.table_stride_b;
  p.len_stride_s = a.lens_stride_s;
  p.len_stride_b = a.lens_stride_b;
  p.pg_max = a.max_pages;
  p.pg_pool = a.num_pages;
  p.pg_causal = a.causal ? 1 : 0;
  p.pg_page = a.page_size;
  p.pg_cap = a.max_pages * a.page_size;
  // causal prefill: single Q tiles, sequences ranked by length and each
  // sequence's tiles costliest first (pairs of tiles t and T-1-t per
  // workgroup measured 9-11% slower: the two workgroups of a CU share it
  // unevenly). Cross-attention: head-major, so that the blocks which read
  // one head's pages run side by side on one XCD (ranking the lists by
  // length measured slower with lists of about equal length)
  if (a.causal && a.S <= NT) {
    p.order = ORDER_SEQ;
    p.groups = a.S;
    p.per_group = a.H * p.n_qtiles;
  } else if (!a.causal) {
    p.order = ORDER_HEADS;
    p.per_group = a.S * p.n_qtiles;
  }
  if (a.page_size == kPrefillSmallPage) return launch_p<D, false, OUT_F32, kPrefillSmallPage>(p, a.S * a.H, stream);
  return launch_p<D, false, OUT_F32, kPrefillPageSize>(p, a.S * a.H, stream);
}

}  // namespace

size_t fwd_split_workspace_bytes(const FwdArgs& a) {
  SplitPlan sp;
  if (!plan_split(a, &sp)) return 0;
  return (size_t)a.BH * sp.n_split * 2 * BM * (a.d + 1) * sizeof(float);
}

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t stream) {
  if (a.v8) {
    return a.d == 64 ? launch_t<64, true, false, true>(a, stream) : launch_t<128, true, false, true>(a, stream);
  }
  if (a.fp8) {
    return a.d == 64 ? launch_t<64, true, false>(a, stream) : launch_t<128, true, false>(a, stream);
  }
  if (a.out_f32) {
    return a.d == 64 ? launch_t<64, false, true>(a, stream) : launch_t<128, false, true>(a, stream);
  }
  return a.d == 64 ? launch_t<64, false, false>(a, stream) : launch_t<128, false, false>(a, stream);
}

hipError_t launch_fwd_paged(const PagedFwdArgs& a, hipStream_t stream) {
  if (a.out_f32) return a.d == 64 ? launch_pg<64, true>(a, stream) : launch_pg<128, true>(a, stream);
  return a.d == 64 ? launch_pg<64, false>(a, stream) : launch_pg<128, false>(a, stream);
}

}  // namespace attn
