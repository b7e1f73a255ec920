// Flash-attention forward with fp32 Q/K/V, computed in fp32 on the vector ALUs.
//
// Same tiled online-softmax method as the MFMA kernel ("Flash MSA Attention
// Kernel Implementation Tutorial", "Understanding Flash MSA Core Mechanics"),
// kept in full fp32 because gfx950 has no reduced-precision path that would
// preserve fp32 inputs. A workgroup of 256 threads owns 128 query rows; two
// lanes share a row (each holds half of q and of the accumulator), so the
// running m and l of a row are computed redundantly in both lanes and never
// leave registers. K/V tiles of 32 keys are staged in LDS and read as
// broadcasts (all lanes of a half read the same address). Grids too small to
// fill the chip run a split-key layout instead (below).
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace attn {

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t stream);

namespace {

constexpr int BMF = 128;
constexpr int BNF = 32;
constexpr int NTF = 256;
// below this many 128-row workgroups (one per CU) the split-key layout runs instead
constexpr int kSmallGridWorkgroups = 256;

struct ParamsF {
  const float* q;
  const float* k;
  const float* v;
  void* o;
  float* lse;
  const int32_t* doc;
  int N, mask, window, nd, n_qtiles, bh_count, desc;
  float scale_log2;
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(NTF) void fwd_f32_kernel(ParamsF p) {
  constexpr int HALF = D / 2;
  constexpr int PITCH = D + 4;  // floats; keeps 16-byte row starts off one bank
  __shared__ __attribute__((aligned(16))) float ks[BNF * PITCH];
  __shared__ __attribute__((aligned(16))) float vs[BNF * PITCH];

  // costliest first for the masks whose Q tiles cost more the later they
  // are (tile-major from the last tile down, heads innermost); else in order
  const int u = blockIdx.x;
  const int r = u / p.bh_count;
  const int bh = u - r * p.bh_count;
  const int qt = p.desc ? p.n_qtiles - 1 - r : r;
  const int tid = threadIdx.x;
  const int row_in = tid >> 1;
  const int half = tid & 1;
  const int N = p.N;
  const int m0 = qt * BMF;
  const int m1 = min(m0 + BMF, N);
  const int qrow = m0 + row_in;
  const size_t head = (size_t)bh * N;
  // keys visible to this thread's row: [span.lo, span.hi]; a wave holds 32 rows
  const int wrow0 = m0 + 32 * __builtin_amdgcn_readfirstlane(tid >> 6);
  const RowSpans sp = row_spans(p.mask, p.window, p.doc, p.nd, N, m0, m1 - 1, min(wrow0, N - 1),
                                min(wrow0 + 31, N - 1), min(qrow, N - 1));

  float q[HALF];
  float acc[HALF];
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    q[i] = qrow < N ? p.q[(head + qrow) * D + half * HALF + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  int t_lo, t_hi;
  touched_tiles(sp.tile_first, sp.tile_last, BNF, &t_lo, &t_hi);
  constexpr int CH = D / 4;  // float4 per row
  for (int kt = t_lo; kt < t_hi; ++kt) {
    const int n0 = kt * BNF;
    for (int c = tid; c < BNF * CH; c += NTF) {
      const int r = c / CH, col = c % CH;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (n0 + r < N) {
        kv = *(const float4*)(p.k + (head + n0 + r) * D + 4 * col);
        vv = *(const float4*)(p.v + (head + n0 + r) * D + 4 * col);
      }
      *(float4*)(ks + r * PITCH + 4 * col) = kv;
      *(float4*)(vs + r * PITCH + 4 * col) = vv;
    }
    __syncthreads();
    float s[BNF];
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < HALF; i += 4) {
        const float4 kk = *(const float4*)(ks + j * PITCH + half * HALF + i);
        dot = __builtin_fmaf(q[i], kk.x, dot);
        dot = __builtin_fmaf(q[i + 1], kk.y, dot);
        dot = __builtin_fmaf(q[i + 2], kk.z, dot);
        dot = __builtin_fmaf(q[i + 3], kk.w, dot);
      }
      dot += __shfl_xor(dot, 1);
      const int key = n0 + j;
      s[j] = (key >= sp.lane.lo && key <= sp.lane.hi) ? dot : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < BNF; ++j) mx = fmaxf(mx, s[j]);
    const float c = p.scale_log2;
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      s[j] = exp2f(__builtin_fmaf(s[j], c, -m_use));
      psum += s[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < HALF; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
#pragma unroll
      for (int i = 0; i < HALF; i += 4) {
        const float4 vv = *(const float4*)(vs + j * PITCH + half * HALF + i);
        acc[i] = __builtin_fmaf(s[j], vv.x, acc[i]);
        acc[i + 1] = __builtin_fmaf(s[j], vv.y, acc[i + 1]);
        acc[i + 2] = __builtin_fmaf(s[j], vv.z, acc[i + 2]);
        acc[i + 3] = __builtin_fmaf(s[j], vv.w, acc[i + 3]);
      }
    }
    __syncthreads();
  }
  if (qrow < N) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const float x = acc[i] * inv;
      if constexpr (OUT_F32)
        ((float*)p.o)[(head + qrow) * D + half * HALF + i] = x;
      else
        ((__bf16*)p.o)[(head + qrow) * D + half * HALF + i] = (__bf16)x;
    }
    if (p.lse != nullptr && half == 0)
      p.lse[head + qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// Small grids (fewer workgroups of 128 rows than CUs): a workgroup owns 4
// query rows, sixteen lanes per row (a sixteenth of d each), and its NW waves
// split the key tiles among themselves (tile t_lo + j goes to wave j % NW),
// each wave staging its tiles in its own LDS region, so the waves need no
// workgroup barrier in the loop. The NW partial states (m, l, acc) per row
// are merged at the end with the same rescale algebra as the split-KV
// decode. Such a grid is latency-bound: a lane's serial work per key tile
// (d / 16 multiply-adds for the score and as many for P V, plus a 4-step
// shuffle sum) is what sets its time, and the grid has 32x the workgroups of
// the 128-row layout. (16 rows with four lanes each ran the single-head
// 256 x 64 case in 16.9 us; this layout takes 10.8 us.)
constexpr int BMS = 4;   // query rows per workgroup
constexpr int LPR = 16;  // lanes per query row
static_assert(BMS * LPR == 64, "one wave covers the workgroup's rows");
template <int D>
constexpr int split_waves() { return D == 64 ? 8 : 4; }

// orders the LDS writes of a wave's lanes before their reads by other lanes
// of the same wave (and the reads before the next writes)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * split_waves<D>()) void fwd_f32_split_kernel(ParamsF p) {
  constexpr int NWS = split_waves<D>();
  constexpr int DQ = D / LPR;   // dims per lane
  constexpr int PITCH = D + 4;  // floats; keeps 16-byte row starts off one bank
  constexpr int TILE = BNF * PITCH;
  static_assert(64 * (DQ + 2) <= TILE, "a wave's merge record fits its tile region");
  static_assert(2 * NWS * TILE * sizeof(float) <= 160 * 1024, "K and V regions fit the LDS");
  __shared__ __attribute__((aligned(16))) float ks[NWS * TILE];
  __shared__ __attribute__((aligned(16))) float vs[NWS * TILE];

  const int bh = blockIdx.y;
  const int m0 = blockIdx.x * BMS;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int part = lane % LPR;
  const int N = p.N;
  const int m1 = min(m0 + BMS, N);
  const int qrow = m0 + lane / LPR;
  const size_t head = (size_t)bh * N;
  const RowSpans sp = row_spans(p.mask, p.window, p.doc, p.nd, N, m0, m1 - 1, m0, m1 - 1, min(qrow, N - 1));

  float q[DQ];
  float acc[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    q[i] = qrow < N ? p.q[(head + qrow) * D + part * DQ + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  int t_lo, t_hi;
  touched_tiles(sp.tile_first, sp.tile_last, BNF, &t_lo, &t_hi);
  float* kw = ks + wave * TILE;
  float* vw = vs + wave * TILE;
  constexpr int CH = D / 4;  // float4 per row
  const float c = p.scale_log2;
  for (int kt = t_lo + wave; kt < t_hi; kt += NWS) {
    const int n0 = kt * BNF;
#pragma unroll
    for (int u = 0; u < BNF * CH / 64; ++u) {
      const int cc = lane + 64 * u;
      const int r = cc / CH, col = cc % CH;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (n0 + r < N) {
        kv = *(const float4*)(p.k + (head + n0 + r) * D + 4 * col);
        vv = *(const float4*)(p.v + (head + n0 + r) * D + 4 * col);
      }
      *(float4*)(kw + r * PITCH + 4 * col) = kv;
      *(float4*)(vw + r * PITCH + 4 * col) = vv;
    }
    wave_lds_sync();
    float s[BNF];
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 kk = *(const float4*)(kw + j * PITCH + part * DQ + i);
        dot = __builtin_fmaf(q[i], kk.x, dot);
        dot = __builtin_fmaf(q[i + 1], kk.y, dot);
        dot = __builtin_fmaf(q[i + 2], kk.z, dot);
        dot = __builtin_fmaf(q[i + 3], kk.w, dot);
      }
#pragma unroll
      for (int x = 1; x < LPR; x <<= 1) dot += __shfl_xor(dot, x);
      const int key = n0 + j;
      s[j] = (key >= sp.lane.lo && key <= sp.lane.hi) ? dot : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < BNF; ++j) mx = fmaxf(mx, s[j]);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      s[j] = exp2f(__builtin_fmaf(s[j], c, -m_use));
      psum += s[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DQ; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 vv = *(const float4*)(vw + j * PITCH + part * DQ + i);
        acc[i] = __builtin_fmaf(s[j], vv.x, acc[i]);
        acc[i + 1] = __builtin_fmaf(s[j], vv.y, acc[i + 1]);
        acc[i + 2] = __builtin_fmaf(s[j], vv.z, acc[i + 2]);
        acc[i + 3] = __builtin_fmaf(s[j], vv.w, acc[i + 3]);
      }
    }
    wave_lds_sync();
  }
  // merge: each wave leaves (m, l, acc) per lane in its K region; wave 0
  // combines m* = max m_w, l* = sum 2^(m_w - m*) l_w, acc* likewise
  __syncthreads();
  float* rec = kw + lane * (DQ + 2);
  rec[0] = m_run;
  rec[1] = l_run;
#pragma unroll
  for (int i = 0; i < DQ; ++i) rec[2 + i] = acc[i];
  __syncthreads();
  if (wave != 0 || qrow >= N) return;
  float m_star = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWS; ++w) m_star = fmaxf(m_star, ks[w * TILE + lane * (DQ + 2)]);
  const float m_use = m_star == -INFINITY ? 0.f : m_star;
  float l_tot = 0.f;
  float o[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) o[i] = 0.f;
#pragma unroll
  for (int w = 0; w < NWS; ++w) {
    const float* r = ks + w * TILE + lane * (DQ + 2);
    const float wt = exp2f(r[0] - m_use);
    l_tot += wt * r[1];
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] += wt * r[2 + i];
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    const float x = o[i] * inv;
    if constexpr (OUT_F32)
      ((float*)p.o)[(head + qrow) * D + part * DQ + i] = x;
    else
      ((__bf16*)p.o)[(head + qrow) * D + part * DQ + i] = (__bf16)x;
  }
  if (p.lse != nullptr && part == 0)
    p.lse[head + qrow] = l_tot > 0.f ? (m_star + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool OUT_F32>
hipError_t launch_f32_d(const FwdArgs& a, hipStream_t stream) {
  ParamsF p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.doc = a.doc;
  p.N = a.N;
  p.mask = a.mask;
  p.window = a.window;
  p.nd = a.num_docs;
  p.n_qtiles = (a.N + BMF - 1) / BMF;
  p.scale_log2 = a.scale * kLog2e;
  if ((long long)p.n_qtiles * a.BH < kSmallGridWorkgroups) {
    dim3 grid((a.N + BMS - 1) / BMS, a.BH);
    hipLaunchKernelGGL((fwd_f32_split_kernel<D, OUT_F32>), grid, dim3(64 * split_waves<D>()), 0, stream, p);
    return hipGetLastError();
  }
  p.bh_count = a.BH;
  p.desc = (a.mask == MASK_CAUSAL || a.mask == MASK_PREFIX_LM) ? 1 : 0;
  hipLaunchKernelGGL((fwd_f32_kernel<D, OUT_F32>), dim3(p.n_qtiles * a.BH), dim3(NTF), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (!a.in_f32) return launch_fwd_mfma(a, stream);
  if (a.out_f32) return a.d == 64 ? launch_f32_d<64, true>(a, stream) : launch_f32_d<128, true>(a, stream);
  return a.d == 64 ? launch_f32_d<64, false>(a, stream) : launch_f32_d<128, false>(a, stream);
}

}  // namespace attn
