// Per-128-row-block fp8 (OCP E4M3FN) quantisation of Q or K on gfx950.
//
// "FlashAttention-3: Warp Specialization ...", "FP8 Block Quantization": each
// block is divided by its own fp32 scale = absmax / 448 and cast to E4M3.
// One workgroup per (block, head): pass 1 finds the block's absmax, pass 2
// writes the codes. The power-of-two variant (for V in the all-fp8 path)
// rounds the scale up to 2^k, the smallest power of two with absmax / 2^k <=
// 448, so a matrix core can apply it as an exponent. Divisions are IEEE fp32 (correctly rounded), so the codes
// are a pure function of the fp32 input; the rounding to E4M3 is done on the
// fp32 bit pattern (nearest, ties to even, saturating at 448).
#include "attn_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int QB = 128;   // rows per block

// E4M3FN code of fp32 y. Normal range: keep the top 3 mantissa bits of y and
// round the remaining 20 to nearest-even (a carry bumps the exponent);
// below 2^-6 the grid is k * 2^-9, k = rint(|y| * 2^9). |y| > 448 -> 448.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  float a = fabsf(y);
  if (a != a) return 0x7Fu;
  a = fminf(a, 448.0f);
  uint32_t mag;
  if (a < 0.015625f) {                       // 2^-6
    mag = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8; 8 is 2^-6 = code 0x08
  } else {
    const uint32_t ab = __float_as_uint(a);
    const int e = (int)(ab >> 23) - 127;     // -6 .. 8
    uint32_t keep = (ab >> 20) & 7u;
    const uint32_t rem = ab & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    uint32_t ef = (uint32_t)(e + 7);
    if (keep == 8u) {
      keep = 0;
      ++ef;
    }
    mag = (ef << 3) | keep;
    if (mag > 0x7Eu) mag = 0x7Eu;
  }
  return sign | mag;
}

__global__ __launch_bounds__(256) void quant_fp8_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int N, int D, int nb, int pow2) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int bh = blockIdx.y;
  const int r0 = b * QB;
  const int r1 = min(r0 + QB, N);
  const size_t off = ((size_t)bh * N + r0) * D;
  const int cnt4 = (r1 - r0) * D / 4;
  const float4* xb = (const float4*)(x + off);
  float amax = 0.f;
  for (int i = threadIdx.x; i < cnt4; i += 256) {
    const float4 v = xb[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = amax == 0.f ? 1.0f : amax / 448.0f;
  if (pow2 && amax != 0.f) {
    // amax = m * 2^e with m in [0.5, 1) and 448 = 0.875 * 2^9: the exact
    // comparison of mantissas picks 2^(e-9) or 2^(e-8)
    int e;
    const float m = frexpf(amax, &e);
    s = ldexpf(1.0f, max(m <= 0.875f ? e - 9 : e - 8, -127));
  }
  uint32_t* cb = (uint32_t*)(codes + off);
  for (int i = threadIdx.x; i < cnt4; i += 256) {
    const float4 v = xb[i];
    cb[i] = e4m3_code(v.x / s) | (e4m3_code(v.y / s) << 8) | (e4m3_code(v.z / s) << 16) |
            (e4m3_code(v.w / s) << 24);
  }
  if (threadIdx.x == 0) scales[(size_t)bh * nb + b] = s;
}

}  // namespace

hipError_t launch_quant_fp8(const float* x, uint8_t* codes, float* scales, int BH, int N, int d, bool pow2,
                            hipStream_t stream) {
  const int nb = (N + QB - 1) / QB;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(nb, BH), dim3(256), 0, stream, x, codes, scales, N, d, nb,
                     pow2 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace attn
