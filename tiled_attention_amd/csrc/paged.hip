// Paged-KV decode and page gather on gfx950.
//
// Pool layout [num_pages, H, page, d] bf16 (page = 16 or 64 tokens) with a
// per-sequence block table ("Optimizing Triton kernels for custom attention
// patterns on H100", Pattern C, gather_pages). The decode walks 16-token
// units: a 64-token page is four of them, contiguous in its (page, head)
// slice. Decode is bound by HBM bandwidth: every cached
// K/V byte is read once, so the kernels are built around keeping enough bytes
// in flight, not around the matrix cores.
//
// decode_split: one wave per (sequence, head, range of 64 pages). The range's
//   page ids are loaded once, one per lane, and each is picked as a scalar
//   (it is uniform across the wave); the page gather is fused into the K/V
//   loads. Pattern C of that page recommends the two-stage route (gather,
//   then attend) for paged patterns; fusing the gather is this library's
//   measured departure from it for decode, where a separate gather would
//   write and read every cached byte once more. Load j of lane l reads the
//   16 bytes at 1024 j + 16 l of a (page, head) slice -- 4 KB contiguous for
//   d = 128 -- so the loads cover the slice exactly once, 1 KB per
//   instruction. q.k uses v_dot2_f32_bf16 on packed bf16; the online softmax
//   ("Flash MSA ...", "Understanding Flash MSA Core Mechanics") runs over two
//   pages per step. Each range writes its un-normalised state (m, l, acc) to
//   the workspace.
// decode_combine: merges the ranges of a (sequence, head) with the same
//   rescale algebra: m* = max m_i, l* = sum 2^(m_i - m*) l_i,
//   O = sum 2^(m_i - m*) acc_i / l*.
// With no workspace the whole sequence is one range and decode_split writes
// O directly.
#include <mutex>

#include "attn_common.h"
#include "launch.h"

// Device memory of attn_decode_paged_noalloc, for callers that cannot
// allocate: the split ranges' partial states (m, l, acc) go here instead of a
// caller workspace. Each GPU holds its own copy for the life of the process;
// host code must not pass `scratch` itself to a kernel (in host code the name
// stands for a host-side shadow), only the address hipGetSymbolAddress gives
// for the current device.
static __device__ __align__(256) unsigned char scratch[attn::kNoAllocScratchBytes];

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
  int H, max_pages, split_pages, max_splits, direct;   // max_pages: block-table row length
  int num_pages, len_max;   // page ids are clamped into [0, num_pages), lengths into [0, len_max]
  float scale_log2;
};

// x plus the value of the lane given by a DPP pattern within its row of 16
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over each group of G consecutive lanes (G = 8 or 16), left in every lane
// of the group: xor 1, xor 2, then the half-row and row mirrors.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x = dpp_add<0xB1>(x);    // quad_perm(1,0,3,2)
  x = dpp_add<0x4E>(x);    // quad_perm(2,3,0,1)
  x = dpp_add<0x141>(x);   // row_half_mirror
  if constexpr (G == 16) x = dpp_add<0x140>(x);   // row_mirror
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// A lane's moves of the reference beyond which its exponentials could grow
// past 2^16 trigger a rebase; below it P stays far inside fp32.
constexpr float kDecodeHeadroom = 16.f;

// SUB = 16-token units per page (1 or 4); "page" below means such a unit.
template <int D, int SUB>
__global__ __launch_bounds__(64) void decode_split_kernel(DecParams p) {
  // A unit of one head is 16 keys x D bf16, contiguous. Load j of a lane
  // reads 16 bytes at 1024 j + 16 lane: key j*KPJ + lane/LPK, dims
  // 8 (lane % LPK) .. +7. Every load instruction reads 1 KB contiguously.
  static_assert(SUB == 1 || SUB == 4, "16- or 64-token pages");
  constexpr int SLICE = PAGE * D * 2;
  constexpr int NJ = SLICE / 1024;   // loads per lane per page and tensor
  constexpr int LPK = D / 8;         // lanes per key
  constexpr int KPJ = 64 / LPK;      // keys per load
  const int h = blockIdx.x;
  const int split = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int H = p.H;
  const int len = min(max(p.lens[s], 0), p.len_max);
  const int npages = (len + PAGE - 1) / PAGE;
  const int pg0 = split * p.split_pages;
  if (pg0 >= npages) return;
  const int pg1 = min(pg0 + p.split_pages, npages);
  const int kq = lane / LPK;         // key within a load group
  const int dq = lane % LPK;         // 8-dim block

  uint32_t qw[4];
  {
    const u32x4 t = *(const u32x4*)(p.q + ((size_t)s * H + h) * D + 8 * dq);
    qw[0] = t[0];
    qw[1] = t[1];
    qw[2] = t[2];
    qw[3] = t[3];
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float m_ref = -INFINITY, l_lane = 0.f;
  const float c = p.scale_log2;
  const int32_t* bt = p.bt + (size_t)s * p.max_pages;
  const char* kbase = (const char*)p.kp + (size_t)h * SUB * SLICE + 16 * lane;
  const char* vbase = (const char*)p.vp + (size_t)h * SUB * SLICE + 16 * lane;
  const size_t page_stride = (size_t)H * SUB * SLICE;

  int pid_vec = 0, batch = pg0 - 64;
  for (int pg = pg0; pg < pg1; pg += 2) {
    if (pg - batch == 64) {
      // the page ids of the next 64 units of the range, one per lane (SUB
      // consecutive units share a page)
      batch = pg;
      pid_vec = pg + lane < pg1 ? min(max(bt[(pg + lane) / SUB], 0), p.num_pages - 1) : 0;
    }
    const int pid0 = __builtin_amdgcn_readlane(pid_vec, pg - batch);
    const bool two = pg + 1 < pg1;
    // a missing second unit reads the first again (its P is 0)
    const int pid1 = two ? __builtin_amdgcn_readlane(pid_vec, pg + 1 - batch) : pid0;
    const size_t off0 = pid0 * page_stride + (size_t)(pg % SUB) * SLICE;
    const size_t off1 = two ? pid1 * page_stride + (size_t)((pg + 1) % SUB) * SLICE : off0;
    u32x4 kr[2][NJ], vr[2][NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      kr[0][j] = __builtin_nontemporal_load((const u32x4*)(kbase + off0 + 1024 * j));
      kr[1][j] = __builtin_nontemporal_load((const u32x4*)(kbase + off1 + 1024 * j));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      vr[0][j] = __builtin_nontemporal_load((const u32x4*)(vbase + off0 + 1024 * j));
      vr[1][j] = __builtin_nontemporal_load((const u32x4*)(vbase + off1 + 1024 * j));
    }
    // scores (log2 units) of the lane's keys; -inf past the sequence or the range
    float sc[2][NJ];
    bool any_over = m_ref == -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        // the words go through a scalar array: a bit cast of a vector element
        // directly is lowered to one register for every index
        const uint32_t kw[4] = {kr[u][j][0], kr[u][j][1], kr[u][j][2], kr[u][j][3]};
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[w]), __builtin_bit_cast(bf16x2, kw[w]), d,
                                              false);
        d = group_sum<LPK>(d);
        const int t = (pg + u) * PAGE + j * KPJ + kq;
        const bool ok = (u == 0 || two) && t < len;
        sc[u][j] = ok ? d * c : -INFINITY;
        any_over |= sc[u][j] > m_ref + kDecodeHeadroom;
      }
    if (__builtin_expect(__any(any_over), 0)) {
      // slow path: the reference becomes the exact running max
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < NJ; ++j) mx = fmaxf(mx, sc[u][j]);
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == m_ref ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    // Only a step holding the sequence's last page (or no second page) has
    // keys past the end, whose rows may hold anything: their V words are
    // replaced by zeros there, since 0 * NaN would poison acc.
    const bool tail = !two || (pg + 2) * PAGE > len;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sc[u][j] - m_use);
        l_lane += pj;
        u32x4 vw = vr[u][j];
        if (tail) {
          const bool ok = sc[u][j] != -INFINITY;
#pragma unroll
          for (int w = 0; w < 4; ++w) vw[w] = ok ? vw[w] : 0u;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] = __builtin_fmaf(pj, bf16_lo(vw[w]), acc[2 * w]);
          acc[2 * w + 1] = __builtin_fmaf(pj, bf16_hi(vw[w]), acc[2 * w + 1]);
        }
      }
  }
  // sum over the lanes holding the same 8 dims (different keys); l_lane counts
  // each key once per group of LPK lanes, so l is summed the same way
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    l_lane += __shfl_xor(l_lane, o);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o);
  }
  if (lane >= LPK) return;   // lane dq < LPK holds dims 8 dq .. +7
  const size_t sh = (size_t)s * H + h;
  const float l_tot = l_lane;
  if (p.direct) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
    bf16x8v ov;
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(acc[i] * inv);
    *(bf16x8v*)(p.o + sh * D + 8 * dq) = ov;
    if (p.lse != nullptr && lane == 0)
      p.lse[sh] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const size_t slot = sh * p.max_splits + split;
    float* ap = p.ws_acc + slot * D + 8 * dq;
    *(float4*)ap = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(ap + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (lane == 0) *(float2*)(p.ws_ml + 2 * slot) = make_float2(m_ref, l_tot);
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecParams p) {
  const int sh = blockIdx.x;
  const int s = sh / p.H;
  const int len = min(max(p.lens[s], 0), p.len_max);
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
  const int page = a.page_size;
  const int len = a.seq_lens[s];
  if (slot * page >= len) return;
  const int rows = min(page, len - slot * page);
  const int pid = min(max(a.block_table[(size_t)s * a.max_pages + slot], 0), a.num_pages - 1);
  const int row_chunks = a.d * a.elem_bytes / 16;
  const int per_head = rows * row_chunks;
  const int total = a.H * per_head;
  const size_t row_bytes = (size_t)a.d * a.elem_bytes;
  for (int c = threadIdx.x; c < total; c += 256) {
    const int h = c / per_head;
    const int rem = c - h * per_head;
    const int r = rem / row_chunks;
    const int col = rem - r * row_chunks;
    const size_t src = (((size_t)pid * a.H + h) * page + r) * row_bytes + (size_t)col * 16;
    const size_t dst = (((size_t)s * a.H + h) * ((size_t)a.max_pages * page) + (size_t)slot * page + r) * row_bytes +
                       (size_t)col * 16;
    *(uint4*)((char*)a.k_out + dst) = *(const uint4*)((const char*)a.k_pool + src);
    *(uint4*)((char*)a.v_out + dst) = *(const uint4*)((const char*)a.v_pool + src);
  }
}

int split_count(int max_pages) { return (max_pages + kDecodeSplitPages - 1) / kDecodeSplitPages; }

template <int D, int SUB>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const int units = a.max_pages * SUB;   // 16-token units a table row can address
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
  p.num_pages = a.num_pages;
  p.len_max = a.max_pages * SUB * PAGE;
  p.scale_log2 = a.scale * kLog2e;
  if (a.workspace == nullptr) {
    p.direct = 1;
    p.split_pages = units;
    p.max_splits = 1;
    p.ws_acc = nullptr;
    p.ws_ml = nullptr;
    hipLaunchKernelGGL((decode_split_kernel<D, SUB>), dim3(a.H, 1, a.S), dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  p.direct = 0;
  p.split_pages = kDecodeSplitPages;
  p.max_splits = split_count(units);
  p.ws_acc = (float*)a.workspace;
  p.ws_ml = p.ws_acc + (size_t)a.S * a.H * p.max_splits * D;
  // heads innermost: the waves of one (sequence, range) run together, and the
  // slices they read of each page -- one per head -- are adjacent in the pool,
  // so the page's H * 4 KB are fetched as one contiguous run (measured 14%
  // faster than ranges innermost, whose concurrent reads are scattered 4 KB)
  hipLaunchKernelGGL((decode_split_kernel<D, SUB>), dim3(a.H, p.max_splits, a.S), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.S * a.H), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int S, int H, int d, int max_pages, int page_size) {
  const size_t slots = (size_t)S * H * split_count(max_pages * (page_size / PAGE));
  return slots * ((size_t)d + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.page_size == 64) return a.d == 64 ? launch_decode_d<64, 4>(a, stream) : launch_decode_d<128, 4>(a, stream);
  return a.d == 64 ? launch_decode_d<64, 1>(a, stream) : launch_decode_d<128, 1>(a, stream);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

// Device address of this GPU's `scratch`, looked up once per device (with the
// device current) and kept.
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_decode_noalloc(const DecodeArgs& a_in, hipStream_t stream) {
  DecodeArgs a = a_in;
  hipError_t e = scratch_address(&a.workspace);
  if (e != hipSuccess) return e;
  // every partial state the combine reads is written earlier in the same
  // call, so nothing needs clearing between calls
  return launch_decode(a, stream);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(a.max_pages, a.S), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
