// Flash-attention forward on gfx950 MFMA: bf16 Q/K/V, or fp8 (E4M3FN) Q/K with
// per-128-row-block scales and bf16 V.
//
// Method: "Flash MSA Attention Kernel Implementation Tutorial", "Understanding
// Flash MSA Core Mechanics" -- a Q tile stays on chip while K/V tiles stream
// past it; each tile updates a running row max m and row sum l, rescales the
// accumulator by exp(m - m_new), adds P V, and O = acc / l is written once.
// fp8 scores: "FlashAttention-3 ...", "FP8 Block Quantization" -- the product
// of the two blocks' scales multiplies the fp8 dot products, folded here into
// the exponent's scale factor.
//
// Mapping onto CDNA4 (one workgroup = 4 waves = 128 query rows, 32 per wave):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (or v_mfma_f32_32x32x64_f8f6f4):
//    K is the A operand, read from LDS; Q is the B operand, held in VGPRs for
//    the whole K loop. In the 32x32 result, lane l owns query row l%32 and 16
//    of the 32 keys; the other 16 keys of that row sit in lane l^32. The row
//    max and row sum therefore need one cross-half exchange
//    (v_permlane32_swap) per tile, the rest is in-lane.
//  * O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: the exponentials P (rounded to
//    bf16) are already laid out as the B operand -- the k index of the MFMA
//    is matched to the keys each lane holds -- and V^T is read from a
//    row-major V tile with ds_read_b64_tr_b16 (16 lanes read a 4x16 block and
//    each receives one column). The accumulator O^T has the same lane ->
//    query-row ownership as S^T, so the exp(m - m_new) rescale is lane-local.
//  * K/V tiles of 64 keys are double-buffered in LDS: tile j+1 is fetched
//    from HBM into registers while tile j is consumed, then stored to the
//    other LDS slot; one barrier per tile.
//  * Per wave, each K tile is classified EMPTY / PARTIAL / FULL against the
//    wave's 32 rows: EMPTY tiles are skipped, only PARTIAL tiles evaluate the
//    mask, and the tile loop never visits tiles outside the mask's band
//    ("Optimizing Triton kernels for custom attention patterns on H100",
//    Pattern B, loop bounds and edge-only masking).
//  * Causal: each workgroup takes Q tiles t and T-1-t so all workgroups carry
//    equal work; workgroup ids are mapped so that a head's tiles share an XCD
//    (and its L2).
#include "attn_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BM = 128;      // query rows per workgroup
constexpr int BN = 64;       // keys per K/V tile
constexpr int NT = 256;      // threads per workgroup
constexpr float kLazy = 8.f; // log2 headroom before the reference max moves
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for gfx9 raw buffers

template <int D, bool FP8>
struct Lds {
  // K tile: bf16 rows padded by 16 B, or fp8 rows padded by 16 B; V tile:
  // bf16 rows padded by 32 B. The paddings keep the 16-byte K reads of 16
  // consecutive rows and the transposed V reads on distinct banks.
  static constexpr int K_PITCH = FP8 ? D + 16 : (D + 8) * 2;  // bytes
  static constexpr int V_PITCH = D + 16;                     // bf16 elements
  static constexpr int K_BYTES = BN * K_PITCH;
  static constexpr int V_BYTES = BN * V_PITCH * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

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

template <int D, int MASK, bool FP8, bool OUT_F32>
__device__ __forceinline__ void process_qtile(const Params& p, unsigned char* smem, int bh, int qt) {
  using L = Lds<D, FP8>;
  constexpr int QK_STEPS = FP8 ? D / 64 : D / 16;  // MFMA k-steps for S
  constexpr int KCH = FP8 ? D / 16 : D / 8;         // 16-byte chunks per K row
  constexpr int VCH = D / 8;                        // 16-byte chunks per V row
  constexpr int KLOADS = BN * KCH / NT;
  constexpr int VLOADS = BN * VCH / NT;
  constexpr int KROW = FP8 ? D : 2 * D;             // bytes per K row in HBM
  constexpr int DE = D / 32;                        // 32-wide d blocks of O

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int N = p.N;
  const int m0 = qt * BM;
  const int m1 = min(m0 + BM, N);
  const int wrow0 = m0 + wave * 32;
  const int qrow = wrow0 + l32;

  const size_t head = (size_t)bh * N;
  const unsigned char* kbase = (const unsigned char*)p.k + head * KROW;
  const unsigned char* vbase = (const unsigned char*)p.v + head * (2 * D);

  // ---- Q fragments: lane (row l32, half hl) holds the k-slots of half hl.
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QFrag;
  QFrag qf[QK_STEPS];
  if (qrow < N) {
    if constexpr (FP8) {
      const unsigned char* qp = (const unsigned char*)p.q + (head + qrow) * D + 32 * hl;
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t) {
        i32x4 a = *(const i32x4*)(qp + 64 * t);
        i32x4 b = *(const i32x4*)(qp + 64 * t + 16);
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

  // Complete the Q loads here: the wait counter is in-order, so a Q load still
  // pending inside the loop would make every tile wait for its own prefetch.
#pragma unroll
  for (int t = 0; t < QK_STEPS; ++t) asm volatile("" ::"v"(qf[t]));

  int t_lo, t_hi;
  k_tile_range(MASK, p.window, N, m0, m1, BN, &t_lo, &t_hi);
  const long long wlen = effective_window(MASK, p.window, N);
  float qscale = 1.f;
  if constexpr (FP8) qscale = p.q_scale[bh * p.nsb + m0 / 128];

  float m_ref = -INFINITY;   // reference max (log2 units) the exponentials are taken against
  float l_run = 0.f;
  f32x16 oacc[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) oacc[e] = (f32x16){};

  // Buffer resources over this head's K and V rows: loads past row N return 0.
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, N * KROW, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vres =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, N * (2 * D), kBufferFlags);
  i32x4 kreg[KLOADS], vreg[VLOADS];
  auto gload = [&](int kt) {
    const int n0 = kt * BN;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int c = tid + i * NT, row = c / KCH, col = c % KCH;
      kreg[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, (n0 + row) * KROW + col * 16, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int c = tid + i * NT, row = c / VCH, col = c % VCH;
      vreg[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, (n0 + row) * (2 * D) + col * 16, 0, 0));
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* ks = smem + buf * L::STAGE;
    unsigned char* vs = ks + L::K_BYTES;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int c = tid + i * NT, row = c / KCH, col = c % KCH;
      *(i32x4*)(ks + row * L::K_PITCH + col * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int c = tid + i * NT, row = c / VCH, col = c % VCH;
      *(i32x4*)(vs + row * (2 * L::V_PITCH) + col * 16) = vreg[i];
    }
  };

  // lane roles in the transposed V read: 16-lane group g, row rr, 4-column chunk cc
  const int g = lane >> 4;
  const int rr = (lane >> 2) & 3;
  const int cc = lane & 3;
  const int v_lane_off = (4 * hl + rr) * L::V_PITCH + 16 * (g & 1) + 4 * cc;  // elements

  if (t_lo < t_hi) {
    gload(t_lo);
    lstore(0);
  }
  __syncthreads();

  for (int kt = t_lo; kt < t_hi; ++kt) {
    const int buf = (kt - t_lo) & 1;
    const bool more = kt + 1 < t_hi;
    if (more) gload(kt + 1);
    const int n0 = kt * BN;
    const int cls = tile_class(MASK, p.window, N, wrow0, wrow0 + 32, n0, n0 + BN);
    if (cls != TILE_EMPTY) {
      const unsigned char* ks = smem + buf * L::STAGE;
      const __bf16* vs = (const __bf16*)(ks + L::K_BYTES);

      // ---- S^T for keys n0..n0+31 (s[0]) and n0+32..n0+63 (s[1])
      f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t) {
        if constexpr (FP8) {
          const unsigned char* a0p = ks + l32 * L::K_PITCH + 64 * t + 32 * hl;
          const unsigned char* a1p = a0p + 32 * L::K_PITCH;
          i32x4 a0l = *(const i32x4*)a0p, a0h = *(const i32x4*)(a0p + 16);
          i32x4 a1l = *(const i32x4*)a1p, a1h = *(const i32x4*)(a1p + 16);
          i32x8 a0 = {a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], a0h[2], a0h[3]};
          i32x8 a1 = {a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], a1h[2], a1h[3]};
          s[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[t], s[0], 0, 0, 0, 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[t], s[1], 0, 0, 0, 0, 0, 0);
        } else {
          const unsigned char* a0p = ks + l32 * L::K_PITCH + (16 * t + 8 * hl) * 2;
          bf16x8 a0 = *(const bf16x8*)a0p;
          bf16x8 a1 = *(const bf16x8*)(a0p + 32 * L::K_PITCH);
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[t], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[t], s[1], 0, 0, 0);
        }
      }

      float c = p.scale_log2;
      if constexpr (FP8) c *= qscale * p.k_scale[bh * p.nsb + n0 / 128];

      // ---- mask (edge tiles only): key of s[b][r] is n0 + 32b + 8(r/4) + 4hl + r%4
      if (cls == TILE_PARTIAL) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + 32 * b + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (!(key < N && key_visible(MASK, wlen, qrow, key))) s[b][r] = -INFINITY;
          }
      }

      // ---- online softmax (log2 domain). The reference max m_ref only moves
      // when a row's max exceeds it by more than 2^kLazy: the exponentials
      // then stay <= 2^kLazy and the final O = acc / l is unchanged, while
      // the rescale of acc by 2^(m_old - m_new) is skipped on most tiles.
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      const float mt = half_swap_max(mx) * c;
      const bool move = mt > m_ref + kLazy;
      if (__any(move)) {
        const float m_new = move ? mt : m_ref;
        // 1 for rows that keep their reference (also while it is still -inf), 0 for a first move
        const float alpha = move ? fast_exp2(m_ref - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < DE; ++e)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha;
        m_ref = m_new;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

      // ---- P = 2^(s*c - m) rounded to bf16, laid out as the B operand: k-step q
      // covers keys 16q..16q+15 of the tile. l sums the rounded values, so O is
      // an exact convex combination of the V rows P multiplies.
      bf16x8 pf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pf[q][j] = (__bf16)fast_exp2(__builtin_fmaf(s[q >> 1][8 * (q & 1) + j], c, -m_use));
      {
        typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
        const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
        float psum = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 pr = {pf[q][2 * j], pf[q][2 * j + 1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum, false);
          }
        l_run += psum;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < DE; ++e) {
          const __bf16* vp = vs + v_lane_off + 16 * q * L::V_PITCH + 32 * e;
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vp));
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vp + 8 * L::V_PITCH));
          s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[q],
                                                            oacc[e], 0, 0, 0);
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

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
          bf16x4 ov = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
          *(bf16x4*)((__bf16*)p.o + (head + qrow) * D + d0) = ov;
        }
      }
    if (p.lse != nullptr && hl == 0)
      p.lse[head + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int MASK, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(NT) void fwd_mfma_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lds<D, FP8>::TOTAL];
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  if (u >= p.units) return;
  const int bh = u / p.units_per_bh;
  const int w = u - bh * p.units_per_bh;
  if (p.pair) {
    const int ta = w, tb = p.n_qtiles - 1 - w;
    process_qtile<D, MASK, FP8, OUT_F32>(p, smem, bh, tb);
    if (ta != tb) {
      __syncthreads();
      process_qtile<D, MASK, FP8, OUT_F32>(p, smem, bh, ta);
    }
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
