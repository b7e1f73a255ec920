// Flash-attention forward on gfx950 MFMA: bf16 Q/K/V, or fp8 (E4M3FN) Q/K with
// per-128-row-block scales and bf16 V.
//
// Method: "Flash MSA Attention Kernel Implementation Tutorial", "Understanding
// Flash MSA Core Mechanics" -- a Q tile stays on chip while K/V tiles stream
// past it; each tile updates a running row max m and row sum l, rescales the
// accumulator by exp(m - m_new), adds P V, and O = acc / l is written once.
// fp8 scores: "FlashAttention-3 ...", "FP8 Block Quantization" -- the product
// of the two blocks' scales multiplies the fp8 dot products; it is folded
// into the exponent's scale factor.
//
// Mapping onto CDNA4 (a workgroup is 4 waves = 128 query rows, 32 per wave):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x64_f8f6f4 for
//    fp8): K is the A operand, read from LDS; Q is the B operand, held in
//    VGPRs for the whole K loop. In the 32x32 result lane l owns query row
//    l%32 and 16 of the 32 keys; the other 16 keys of that row are in lane
//    l^32, so a row reduction needs one v_permlane32_swap.
//  * O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: P (rounded to bf16) is
//    already laid out as the B operand -- the MFMA's k index is matched to
//    the keys each lane holds -- and V^T comes from the row-major V tile
//    through ds_read_b64_tr_b16 (16 lanes read a 4x16 block, each receives a
//    column). O^T has the same lane -> row ownership as S^T, so the rescale
//    is lane-local.
//  * K and V tiles (64 keys) stream through LDS rings (3 slots, or 2 for
//    d = 128 bf16) filled by LDS DMA (buffer_load_dwordx4 ... lds) ahead of
//    use; a buffer
//    descriptor per tile makes rows past the end read as zeros. Rows are
//    stored unpadded with the 16-byte chunks XOR-swizzled by row, so the
//    16-byte K reads and the transposed V reads hit distinct banks.
//  * Software pipeline: while the VALU computes the softmax of tile i, the
//    matrix cores run S = K Q^T of tile i+1 and O += P V of tile i-1 (P V is
//    one tile behind, so neither depends on the softmax in flight); on full
//    tiles the 16 MFMAs are interleaved with the VALU work in one block.
//  * Lazy rescale: P = 2^(S*c - m_ref) against a reference max that moves
//    only when a row max exceeds it by more than 2^8, so the exponentials
//    stay <= 2^8 and the rescale of acc by 2^(m_old - m_new) is skipped on
//    almost every tile; O = acc / l does not depend on the reference used.
//    l sums the bf16-rounded P (v_dot2_f32_bf16), the weights P V applies.
//  * Per wave, each K tile is classified EMPTY / PARTIAL / FULL against the
//    wave's 32 rows: EMPTY tiles skip the MFMA and softmax work, only PARTIAL
//    tiles evaluate the mask, and the tile loop never visits tiles outside
//    the mask's band ("Optimizing Triton kernels for custom attention
//    patterns on H100", Pattern B: loop bounds and edge-only masking).
//  * Causal: a workgroup takes Q tiles t and T-1-t so all carry equal work;
//    workgroup ids are mapped so that a head's tiles share an XCD (its L2).
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per K/V tile
constexpr int NW = 4;         // waves per workgroup
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr float kLazy = 8.f;              // log2 headroom before the reference max moves
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 (gfx9 raw buffer)

template <int D, bool FP8>
struct Cfg {
  static constexpr int KROW = FP8 ? D : 2 * D;  // bytes per K row
  static constexpr int VROW = 2 * D;            // bytes per V row
  static constexpr int K_SLOT = BN * KROW;
  static constexpr int V_SLOT = BN * VROW;
  static constexpr int KLD = K_SLOT / (16 * NT);  // DMA loads per thread per K tile
  static constexpr int VLD = V_SLOT / (16 * NT);
  // LDS ring slots for K and for V: loads run NS-1 tiles ahead. Three slots
  // when two workgroups still fit in a CU's 160 KB, else two.
  static constexpr int NS = 3 * (K_SLOT + V_SLOT) <= 80 * 1024 ? 3 : 2;
  static constexpr int LDS = NS * (K_SLOT + V_SLOT);
  static constexpr int QK_STEPS = FP8 ? D / 64 : D / 16;
  static constexpr int DE = D / 32;             // 32-row blocks of O^T
  // Occupancy the register allocation aims at (waves per SIMD). d = 64: two,
  // although the LDS ring would admit three workgroups per CU, so that the
  // scheduler may keep a step's LDS operand reads in flight together.
  static constexpr int WAVES_MIN = D == 64 ? 2 : 1;
  static constexpr int WAVES_MAX = D == 64 ? 2 : 2;
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

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_scale;
  const float* k_scale;
  int N, window, n_qtiles, units_per_bh, units, pair, nsb;
  float scale_log2;
};

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

// Raw buffer descriptor over [base, base + bytes).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r = {(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, kBufferFlags};
  r[0] = __builtin_amdgcn_readfirstlane(r[0]);
  r[1] = __builtin_amdgcn_readfirstlane(r[1]);
  r[2] = __builtin_amdgcn_readfirstlane(r[2]);
  return r;
}

// 16 bytes per lane from buffer offset voff to LDS at m0 + lane * 16. The
// compiler does not see this load: its completion is waited for explicitly
// (sync_tiles). The s_nop covers the SALU-writes-M0 -> LDS DMA hazard.
__device__ __forceinline__ void dma16(uint32_t m0v, int voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "memory");
}

// Wait until at most N of this wave's loads are outstanding, then barrier.
// One asm statement with a memory clobber, so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void sync_tiles() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int D, int MASK, bool FP8, bool OUT_F32>
__device__ __forceinline__ void process_qtile(const Params& p, unsigned char* smem, int bh, int qt) {
  using C = Cfg<D, FP8>;
  constexpr int KROW = C::KROW, VROW = C::VROW, QK_STEPS = C::QK_STEPS, DE = C::DE;
  constexpr int KLD = C::KLD, VLD = C::VLD, L = KLD + VLD, NS = C::NS;
  // per step: LDS reads (K: 2 x QK_STEPS x (fp8: 2); V: 2 x 4 x DE) and MFMAs
  constexpr int kStepReads = 2 * QK_STEPS * (FP8 ? 2 : 1) + 8 * DE;
  constexpr int kStepMfma = 2 * QK_STEPS + 4 * DE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave logic scalar
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int N = p.N;
  const int m0 = qt * BM;
  const int m1 = min(m0 + BM, N);
  const int wrow0 = m0 + wave * 32;
  const int qrow = wrow0 + l32;
  const size_t head = (size_t)bh * N;
  const unsigned char* kbase = (const unsigned char*)p.k + head * KROW;
  const unsigned char* vbase = (const unsigned char*)p.v + head * VROW;

  // ---- Q fragments: lane (row l32, half hl) holds the k-slots of half hl.
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QFrag;
  QFrag qf[QK_STEPS];
  if (qrow < N) {
    if constexpr (FP8) {
      const unsigned char* qp = (const unsigned char*)p.q + (head + qrow) * D + 32 * hl;
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t) {
        const i32x4 a = *(const i32x4*)(qp + 64 * t);
        const i32x4 b = *(const i32x4*)(qp + 64 * t + 16);
        qf[t] = (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      }
    } else {
      const __bf16* qp = (const __bf16*)p.q + (head + qrow) * D + 8 * hl;
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t) qf[t] = *(const bf16x8*)(qp + 16 * t);
    }
  } else {
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) qf[t] = (QFrag){};
  }
  // The Q loads complete here: an outstanding one inside the loop would make
  // the in-order wait counter stall on the K/V prefetch as well.
#pragma unroll
  for (int t = 0; t < QK_STEPS; ++t) asm volatile("" ::"v"(qf[t]));

  int t_lo, t_hi;
  k_tile_range(MASK, p.window, N, m0, m1, BN, &t_lo, &t_hi);
  const int NK = t_hi - t_lo;
  const int wlen = effective_window(MASK, p.window, N);
  float qscale = 1.f;
  if constexpr (FP8) qscale = p.q_scale[bh * p.nsb + m0 / 128];

  // ---- per-lane offsets (loop invariant)
  int kdma[KLD], vdma[VLD];
#pragma unroll
  for (int u = 0; u < KLD; ++u) {
    const int off = (u * NW + wave) * 1024 + lane * 16;
    const int row = off / KROW, ch = (off % KROW) / 16;
    kdma[u] = row * KROW + 16 * (ch ^ swz_k<KROW>(row));
  }
#pragma unroll
  for (int u = 0; u < VLD; ++u) {
    const int off = (u * NW + wave) * 1024 + lane * 16;
    const int row = off / VROW, ch = (off % VROW) / 16;
    vdma[u] = row * VROW + 16 * (ch ^ swz_v<VROW>(row));
  }
  // K read of k-step t: row l32 (block b adds 32 rows, same swizzle), chunk of half hl
  constexpr int KCH_STEP = FP8 ? 4 : 2;  // 16-byte chunks per k-step
  int kread[QK_STEPS * (FP8 ? 2 : 1)];
#pragma unroll
  for (int t = 0; t < QK_STEPS; ++t) {
    if constexpr (FP8) {
      const int c0 = KCH_STEP * t + 2 * hl;
      kread[2 * t] = l32 * KROW + 16 * (c0 ^ swz_k<KROW>(l32));
      kread[2 * t + 1] = l32 * KROW + 16 * ((c0 + 1) ^ swz_k<KROW>(l32));
    } else {
      kread[t] = l32 * KROW + 16 * ((KCH_STEP * t + hl) ^ swz_k<KROW>(l32));
    }
  }
  // transposed V read: 16-lane group g, row rr of 4, 8-byte column piece cc
  const int g = lane >> 4, rr = (lane >> 2) & 3, cc = lane & 3;
  const int sv = swz_v<VROW>(4 * hl + rr);   // same for rows +16q and +8
  int vread[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e)
    vread[e] = (4 * hl + rr) * VROW + 16 * ((4 * e + 2 * (g & 1) + (cc >> 1)) ^ sv) + 8 * (cc & 1);

  const uint32_t lds0 = lds_addr(smem);
  auto kslot = [&](int i) { return smem + ((i + NS) % NS) * C::K_SLOT; };
  auto vslot = [&](int i) { return smem + NS * C::K_SLOT + ((i + NS) % NS) * C::V_SLOT; };

  // DMA of K tile i (local index) and V tile j into their ring slots; tiles
  // outside [0, NK) get an empty descriptor and write zeros to a free slot.
  auto issue_k = [&](int i) {
    const int n0 = (t_lo + i) * BN;
    const bool live = i >= 0 && i < NK;
    const i32x4 rs = make_rsrc(kbase + (size_t)(live ? n0 : 0) * KROW, live ? (uint32_t)(N - n0) * KROW : 0u);
    const uint32_t base = lds0 + (uint32_t)(((i + NS) % NS) * C::K_SLOT);
#pragma unroll
    for (int u = 0; u < KLD; ++u)
      dma16(__builtin_amdgcn_readfirstlane(base + (u * NW + wave) * 1024), kdma[u], rs);
  };
  auto issue_v = [&](int i) {
    const int n0 = (t_lo + i) * BN;
    const bool live = i >= 0 && i < NK;
    const i32x4 rs = make_rsrc(vbase + (size_t)(live ? n0 : 0) * VROW, live ? (uint32_t)(N - n0) * VROW : 0u);
    const uint32_t base = lds0 + (uint32_t)(NS * C::K_SLOT + ((i + NS) % NS) * C::V_SLOT);
#pragma unroll
    for (int u = 0; u < VLD; ++u)
      dma16(__builtin_amdgcn_readfirstlane(base + (u * NW + wave) * 1024), vdma[u], rs);
  };

  auto wave_class = [&](int i) {
    const int n0 = (t_lo + i) * BN;
    return tile_class(MASK, p.window, N, wrow0, wrow0 + 32, n0, n0 + BN);
  };

  // S^T for keys n0..n0+31 (s[0]) and n0+32..n0+63 (s[1]) of the tile in K slot of i
  auto qk = [&](int i, f32x16 (&s)[2]) {
    const unsigned char* ks = kslot(i);
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) {
      if constexpr (FP8) {
        const i32x4 a0l = *(const i32x4*)(ks + kread[2 * t]);
        const i32x4 a0h = *(const i32x4*)(ks + kread[2 * t + 1]);
        const i32x4 a1l = *(const i32x4*)(ks + kread[2 * t] + 32 * KROW);
        const i32x4 a1h = *(const i32x4*)(ks + kread[2 * t + 1] + 32 * KROW);
        const i32x8 a0 = {a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]};
        const i32x8 a1 = {a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]};
        s[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[t], s[0], 0, 0, 0, 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[t], s[1], 0, 0, 0, 0, 0, 0);
      } else {
        const bf16x8 a0 = *(const bf16x8*)(ks + kread[t]);
        const bf16x8 a1 = *(const bf16x8*)(ks + kread[t] + 32 * KROW);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[t], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[t], s[1], 0, 0, 0);
      }
    }
  };

  float m_ref = -INFINITY;  // reference max (log2 units) of the exponentials
  float l_run = 0.f;
  f32x16 oacc[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) oacc[e] = (f32x16){};
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  // P = 2^(s*c - m_use) rounded to bf16 as the B operand (k-step q covers keys
  // 16q..16q+15 of the tile); returns the sum of the rounded values (four
  // independent partial sums keep the dependency chains short).
  auto exponentials = [&](const f32x16 (&s)[2], float c, float m_use, bf16x8 (&pf)[4]) {
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[q][j] = (__bf16)fast_exp2(__builtin_fmaf(s[q >> 1][8 * (q & 1) + j], c, -m_use));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 pr = {pf[q][2 * j], pf[q][2 * j + 1]};
        ps[j] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[j], false);
      }
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // log2-domain score scale of local tile i (i == NK, the zero tile past the
  // end, takes the last tile's: its scores are all masked anyway)
  auto tile_scale = [&](int i) {
    float c = p.scale_log2;
    if constexpr (FP8) c *= qscale * p.k_scale[bh * p.nsb + ((t_lo + min(i, NK - 1)) * BN) / 128];
    return c;
  };

  // O^T += V^T P^T for the tile whose V sits in the slot of local index j
  auto pv = [&](int j, const bf16x8 (&pf)[4]) {
    const unsigned char* vs = vslot(j);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < DE; ++e) {
        const unsigned char* vp = vs + vread[e] + 16 * q * VROW;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * VROW));
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[q], oacc[e], 0, 0, 0);
      }
    }
  };

  // The reference for tile i (m_use) and its factor alpha = 2^(m_prev - m_new)
  // are decided as soon as S_i exists, at the end of step i-1; l takes alpha
  // in step i, acc at the start of step i+1 (just before P_i V joins it, while
  // P_{i-1} V, taken against the previous reference, is already in).
  float m_use = 0.f, alpha_cur = 1.f, alpha_acc = 1.f;

  // mask (edge tiles), row max and reference update for the scores s of tile j
  auto prepare = [&](int j, f32x16 (&s)[2], int cls_j) {
    if (cls_j != TILE_FULL) {
      // key of s[b][r] is n0 + 32b + 8(r/4) + 4hl + r%4 (an EMPTY tile masks everything)
      const int n0 = (t_lo + j) * BN;
      const bool partial = cls_j == TILE_PARTIAL;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * b + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool vis = partial & (key < N) & key_visible(MASK, wlen, qrow, key);
          s[b][r] = vis ? s[b][r] : -INFINITY;
        }
    }
    // row max over the lane's 32 scores: three-input maxes in four chains
    // (fmaxf would first canonicalise every MFMA result)
    float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int r = 0; r < 16; ++r) mq[r & 3] = max3(mq[r & 3], s[0][r], s[1][r]);
    const float mt = half_swap_max(max3(mq[0], mq[1], fmaxf(mq[2], mq[3]))) * tile_scale(j);
    const bool move = mt > m_ref + kLazy;
    alpha_cur = move ? fast_exp2(m_ref - mt) : 1.f;   // 0 on a first move from -inf
    m_ref = move ? mt : m_ref;
    m_use = m_ref == -INFINITY ? 0.f : m_ref;
  };

  // One pipeline step at local tile i: S of tile i+1 and P V of tile i-1 on
  // the matrix cores, the exponentials of tile i on the VALU, in one
  // branch-free block; then the next tile's mask/max. sc holds S_i (masked,
  // reference decided), sn receives S_{i+1}; pp holds P_{i-1}, pc receives P_i.
  auto step = [&](int i, f32x16 (&sc)[2], f32x16 (&sn)[2], const bf16x8 (&pp)[4], bf16x8 (&pc)[4], int& cls) {
    // {K_{i+1}, V_{i-1}} landed; every wave is done with K_i and V_{i-2}
    sync_tiles<(NS - 2) * L>();
    issue_k(i + NS);
    issue_v(i + NS - 2);
    if (__any(alpha_acc != 1.f)) {
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha_acc;
    }
    const int cls_n = i + 1 < NK ? wave_class(i + 1) : TILE_EMPTY;
    const float c = tile_scale(i);
    // unconditional, so the block has no branch: for i + 1 == NK the slot holds
    // the zeros loaded for the tile past the end (masked as EMPTY below)
    qk(i + 1, sn);
    pv(i - 1, pp);
    const float psum = exponentials(sc, c, m_use, pc);
    // issue order: every LDS operand read of the step first, then each MFMA
    // followed by a run of exponentials
    __builtin_amdgcn_sched_group_barrier(0x100, kStepReads, 0);
#pragma unroll
    for (int k = 0; k < kStepMfma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    l_run = l_run * alpha_cur + psum;
    alpha_acc = alpha_cur;
    // keep this step's results here: otherwise the exponentials sink to their
    // use in the next step and no longer overlap this step's MFMAs
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(pc[q]));
    asm volatile("" ::"v"(l_run));
    prepare(i + 1, sn, cls_n);
    cls = cls_n;
  };

  // ---- prologue: K_0, then batches {K_{x+NS}, V_{x+NS-2}} for x = 1-NS .. -1
  issue_k(0);
#pragma unroll
  for (int x = 1 - NS; x < 0; ++x) {
    issue_k(x + NS);
    issue_v(x + NS - 2);
  }
  sync_tiles<(NS - 1) * L>();
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pb[q] = (bf16x8){};
  int cls = NK > 0 ? wave_class(0) : TILE_EMPTY;
  if (NK > 0) {
    qk(0, sa);
    prepare(0, sa, cls);
  }

  int i = 0;
  for (; i + 1 < NK; i += 2) {
    step(i, sa, sb, pb, pa, cls);
    step(i + 1, sb, sa, pa, pb, cls);
  }
  if (i < NK) step(i, sa, sb, pb, pa, cls);
  if (NK > 0) {
    // P V of the last tile (its V is in the oldest outstanding batch)
    sync_tiles<(NS - 2) * L>();
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha_acc;
    pv(NK - 1, (NK & 1) ? pa : pb);
  }
  // drain the DMA tail before the LDS is reused
  sync_tiles<0>();

  // ---- epilogue: O = acc / l, written once
  const float l_tot = half_swap_sum(l_run);
  if (qrow < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * e + 8 * g4 + 4 * hl;
        const float x0 = oacc[e][4 * g4 + 0] * inv, x1 = oacc[e][4 * g4 + 1] * inv;
        const float x2 = oacc[e][4 * g4 + 2] * inv, x3 = oacc[e][4 * g4 + 3] * inv;
        if constexpr (OUT_F32) {
          *(float4*)((float*)p.o + (head + qrow) * D + d0) = make_float4(x0, x1, x2, x3);
        } else {
          typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
          const bf16x4 ov = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
          *(bf16x4*)((__bf16*)p.o + (head + qrow) * D + d0) = ov;
        }
      }
    if (p.lse != nullptr && hl == 0)
      p.lse[head + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int MASK, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(Cfg<D, FP8>::WAVES_MIN, Cfg<D, FP8>::WAVES_MAX))) void fwd_mfma_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg<D, FP8>::LDS];
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  if (u >= p.units) return;
  const int bh = u / p.units_per_bh;
  const int w = u - bh * p.units_per_bh;
  if (p.pair) {
    const int ta = w, tb = p.n_qtiles - 1 - w;
    process_qtile<D, MASK, FP8, OUT_F32>(p, smem, bh, tb);
    if (ta != tb) process_qtile<D, MASK, FP8, OUT_F32>(p, smem, bh, ta);
  } else {
    process_qtile<D, MASK, FP8, OUT_F32>(p, smem, bh, p.n_qtiles - 1 - w);
  }
}

template <int D, int MASK, bool FP8, bool OUT_F32>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.q_scale = a.q_scale;
  p.k_scale = a.k_scale;
  p.N = a.N;
  p.window = a.window;
  p.n_qtiles = (a.N + BM - 1) / BM;
  p.pair = (MASK == MASK_CAUSAL) ? 1 : 0;
  p.units_per_bh = p.pair ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  p.units = a.BH * p.units_per_bh;
  p.nsb = (a.N + 127) / 128;
  p.scale_log2 = a.scale * kLog2e;
  const int grid = round_up8(p.units);
  hipLaunchKernelGGL((fwd_mfma_kernel<D, MASK, FP8, OUT_F32>), dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8, bool OUT_F32>
hipError_t launch_mask(const FwdArgs& a, hipStream_t stream) {
  switch (a.mask) {
    case MASK_NONE: return launch_t<D, MASK_NONE, FP8, OUT_F32>(a, stream);
    case MASK_CAUSAL: return launch_t<D, MASK_CAUSAL, FP8, OUT_F32>(a, stream);
    default: return launch_t<D, MASK_SLIDING, FP8, OUT_F32>(a, stream);
  }
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t stream) {
  if (a.fp8) {
    return a.d == 64 ? launch_mask<64, true, false>(a, stream) : launch_mask<128, true, false>(a, stream);
  }
  if (a.out_f32) {
    return a.d == 64 ? launch_mask<64, false, true>(a, stream) : launch_mask<128, false, true>(a, stream);
  }
  return a.d == 64 ? launch_mask<64, false, false>(a, stream) : launch_mask<128, false, false>(a, stream);
}

}  // namespace attn
