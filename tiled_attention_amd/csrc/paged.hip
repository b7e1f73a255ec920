// Paged-KV decode and page gather on gfx950.
//
// Pool layout [num_pages, H, 16, d] bf16 with a per-sequence block table
// ("Optimizing Triton kernels for custom attention patterns on H100",
// Pattern C, gather_pages). Decode is bound by HBM bandwidth: every cached
// K/V byte is read once, so the kernels are built around keeping enough bytes
// in flight, not around the matrix cores.
//
// decode_split: one wave per (sequence, head, range of 32 pages). The page id
//   is read once per page as a scalar (it is uniform across the wave) and the
//   page gather is fused into the K/V loads ("the naive gather-then-attend
//   route wastes bandwidth", Pattern C). Lane l owns key l/4 of a 16-token
//   page and a quarter of the head dimension, so each (page, head) slice --
//   4 KB contiguous for d = 128 -- is read with 16-byte loads that together
//   cover it exactly once. q.k uses v_dot2_f32_bf16 on packed bf16; the online
//   softmax ("Flash MSA ...", "Understanding Flash MSA Core Mechanics") runs
//   over two pages per step. Each range writes its un-normalised state
//   (m, l, acc) to the workspace.
// decode_combine: merges the ranges of a (sequence, head) with the same
//   rescale algebra: m* = max m_i, l* = sum 2^(m_i - m*) l_i,
//   O = sum 2^(m_i - m*) acc_i / l*.
// With no workspace the whole sequence is one range and decode_split writes
// O directly.
#include "attn_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int PAGE = 16;

struct DecParams {
  const __bf16* q;
  const __bf16* kp;
  const __bf16* vp;
  const int32_t* bt;
  const int32_t* lens;
  __bf16* o;
  float* lse;
  float* ws_acc;   // [S, H, max_splits, d]
  float* ws_ml;    // [S, H, max_splits, 2]
  int H, max_pages, split_pages, max_splits, direct;
  float scale_log2;
};

__device__ __forceinline__ float dpp_quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Reduce over the 16 lanes that share lane % 4 (xor 4, 8, 16, 32).
__device__ __forceinline__ float key_lanes_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 8));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float key_lanes_sum(float x) {
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecParams p) {
  constexpr int E = D / 4;        // head-dim elements per lane
  constexpr int W = E / 2;        // packed bf16 pairs per lane
  constexpr int LD = E / 8;       // 16-byte loads per lane per page
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int key = lane >> 2;
  const int ch = lane & 3;
  const int H = p.H;
  const int len = p.lens[s];
  const int npages = (len + PAGE - 1) / PAGE;
  const int pg0 = split * p.split_pages;
  if (pg0 >= npages) return;
  const int pg1 = min(pg0 + p.split_pages, npages);

  uint32_t qw[W];
  {
    const uint4* qp = (const uint4*)(p.q + ((size_t)s * H + h) * D + ch * E);
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const uint4 t = qp[i];
      qw[4 * i] = t.x;
      qw[4 * i + 1] = t.y;
      qw[4 * i + 2] = t.z;
      qw[4 * i + 3] = t.w;
    }
  }
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;
  const int32_t* bt = p.bt + (size_t)s * p.max_pages;
  const size_t lane_off = (size_t)key * D + ch * E;   // elements within a (page, head) slice

  for (int pg = pg0; pg < pg1; pg += 2) {
    const bool two = pg + 1 < pg1;
    const int pid0 = __builtin_amdgcn_readfirstlane(bt[pg]);
    const int pid1 = two ? __builtin_amdgcn_readfirstlane(bt[pg + 1]) : pid0;
    const uint4* k0 = (const uint4*)(p.kp + ((size_t)pid0 * H + h) * (PAGE * D) + lane_off);
    const uint4* v0 = (const uint4*)(p.vp + ((size_t)pid0 * H + h) * (PAGE * D) + lane_off);
    const uint4* k1 = (const uint4*)(p.kp + ((size_t)pid1 * H + h) * (PAGE * D) + lane_off);
    const uint4* v1 = (const uint4*)(p.vp + ((size_t)pid1 * H + h) * (PAGE * D) + lane_off);
    uint4 kr0[LD], kr1[LD], vr0[LD], vr1[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      kr0[i] = k0[i];
      kr1[i] = k1[i];
    }
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      vr0[i] = v0[i];
      vr1[i] = v1[i];
    }
    // q . k over this lane's quarter of d, then over the 4 lanes of the key
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const uint32_t a0[4] = {kr0[i].x, kr0[i].y, kr0[i].z, kr0[i].w};
      const uint32_t a1[4] = {kr1[i].x, kr1[i].y, kr1[i].z, kr1[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
        d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[4 * i + j]),
                                             __builtin_bit_cast(bf16x2, a0[j]), d0, false);
        d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[4 * i + j]),
                                             __builtin_bit_cast(bf16x2, a1[j]), d1, false);
      }
    }
    d0 += dpp_quad_xor1(d0);
    d1 += dpp_quad_xor1(d1);
    d0 += dpp_quad_xor2(d0);
    d1 += dpp_quad_xor2(d1);
    const int t0 = pg * PAGE + key;
    const bool ok0 = t0 < len;
    const bool ok1 = two && (t0 + PAGE) < len;
    const float s0 = ok0 ? d0 * c : -INFINITY;
    const float s1 = ok1 ? d1 * c : -INFINITY;
    const float mx = key_lanes_max(fmaxf(s0, s1));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    const float p0 = ok0 ? __builtin_amdgcn_exp2f(s0 - m_use) : 0.f;
    const float p1 = ok1 ? __builtin_amdgcn_exp2f(s1 - m_use) : 0.f;
    l_run = l_run * alpha + p0 + p1;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= alpha;
    if (ok0) {
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        const uint32_t w[4] = {vr0[i].x, vr0[i].y, vr0[i].z, vr0[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[8 * i + 2 * j] = __builtin_fmaf(p0, bf16_lo(w[j]), acc[8 * i + 2 * j]);
          acc[8 * i + 2 * j + 1] = __builtin_fmaf(p0, bf16_hi(w[j]), acc[8 * i + 2 * j + 1]);
        }
      }
    }
    if (ok1) {
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        const uint32_t w[4] = {vr1[i].x, vr1[i].y, vr1[i].z, vr1[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[8 * i + 2 * j] = __builtin_fmaf(p1, bf16_lo(w[j]), acc[8 * i + 2 * j]);
          acc[8 * i + 2 * j + 1] = __builtin_fmaf(p1, bf16_hi(w[j]), acc[8 * i + 2 * j + 1]);
        }
      }
    }
  }
  // sum l and acc over the 16 keys
  const float l_tot = key_lanes_sum(l_run);
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = key_lanes_sum(acc[i]);
  if (key != 0) return;   // lanes 0..3 hold the full row, a quarter of d each
  const size_t sh = (size_t)s * H + h;
  if (p.direct) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* op = p.o + sh * D + ch * E;
#pragma unroll
    for (int i = 0; i < E; ++i) op[i] = (__bf16)(acc[i] * inv);
    if (p.lse != nullptr && ch == 0)
      p.lse[sh] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const size_t slot = sh * p.max_splits + split;
    float* ap = p.ws_acc + slot * D + ch * E;
#pragma unroll
    for (int i = 0; i < E; i += 4) *(float4*)(ap + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    if (ch == 0) *(float2*)(p.ws_ml + 2 * slot) = make_float2(m_run, l_tot);
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecParams p) {
  const int sh = blockIdx.x;
  const int s = sh / p.H;
  const int len = p.lens[s];
  const int npages = (len + PAGE - 1) / PAGE;
  const int nsplit = (npages + p.split_pages - 1) / p.split_pages;
  const size_t base = (size_t)sh * p.max_splits;
  float m_star = -INFINITY;
  for (int i = 0; i < nsplit; ++i) m_star = fmaxf(m_star, p.ws_ml[2 * (base + i)]);
  const float m_use = m_star == -INFINITY ? 0.f : m_star;
  float l = 0.f, acc = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const float w = __builtin_amdgcn_exp2f(p.ws_ml[2 * (base + i)] - m_use);
    l += w * p.ws_ml[2 * (base + i) + 1];
    acc += w * p.ws_acc[(base + i) * D + threadIdx.x];
  }
  p.o[(size_t)sh * D + threadIdx.x] = (__bf16)(l > 0.f ? acc / l : 0.f);
  if (p.lse != nullptr && threadIdx.x == 0) p.lse[sh] = l > 0.f ? (m_star + __log2f(l)) * kLn2 : -INFINITY;
}

// One workgroup per (page slot, sequence) copies that page's rows t < L for
// every head: a bit copy with 16-byte loads and stores.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int slot = blockIdx.x;
  const int s = blockIdx.y;
  const int len = a.seq_lens[s];
  if (slot * PAGE >= len) return;
  const int rows = min(PAGE, len - slot * PAGE);
  const int pid = a.block_table[(size_t)s * a.max_pages + slot];
  const int row_chunks = a.d * a.elem_bytes / 16;
  const int per_head = rows * row_chunks;
  const int total = a.H * per_head;
  const size_t row_bytes = (size_t)a.d * a.elem_bytes;
  for (int c = threadIdx.x; c < total; c += 256) {
    const int h = c / per_head;
    const int rem = c - h * per_head;
    const int r = rem / row_chunks;
    const int col = rem - r * row_chunks;
    const size_t src = (((size_t)pid * a.H + h) * PAGE + r) * row_bytes + (size_t)col * 16;
    const size_t dst = (((size_t)s * a.H + h) * ((size_t)a.max_pages * PAGE) + (size_t)slot * PAGE + r) * row_bytes +
                       (size_t)col * 16;
    *(uint4*)((char*)a.k_out + dst) = *(const uint4*)((const char*)a.k_pool + src);
    *(uint4*)((char*)a.v_out + dst) = *(const uint4*)((const char*)a.v_pool + src);
  }
}

int split_count(int max_pages) { return (max_pages + kDecodeSplitPages - 1) / kDecodeSplitPages; }

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = (const __bf16*)a.q;
  p.kp = (const __bf16*)a.k_pool;
  p.vp = (const __bf16*)a.v_pool;
  p.bt = a.block_table;
  p.lens = a.seq_lens;
  p.o = (__bf16*)a.o;
  p.lse = a.lse;
  p.H = a.H;
  p.max_pages = a.max_pages;
  p.scale_log2 = a.scale * kLog2e;
  if (a.workspace == nullptr) {
    p.direct = 1;
    p.split_pages = a.max_pages;
    p.max_splits = 1;
    p.ws_acc = nullptr;
    p.ws_ml = nullptr;
    hipLaunchKernelGGL(decode_split_kernel<D>, dim3(1, a.H, a.S), dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  p.direct = 0;
  p.split_pages = kDecodeSplitPages;
  p.max_splits = split_count(a.max_pages);
  p.ws_acc = (float*)a.workspace;
  p.ws_ml = p.ws_acc + (size_t)a.S * a.H * p.max_splits * D;
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3(p.max_splits, a.H, a.S), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.S * a.H), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int S, int H, int d, int max_pages) {
  const size_t slots = (size_t)S * H * split_count(max_pages);
  return slots * ((size_t)d + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_decode_d<64>(a, stream) : launch_decode_d<128>(a, stream);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(a.max_pages, a.S), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
