// NVFP4 quantiser on gfx950: fp32 matrix -> e2m1 codes, e4m3 block scales
// (one per 16 consecutive elements along K) and an fp32 per-tensor scale.
// The format is the one the al-engr.com Kimi-K3 plan describes for the
// NVFP4 checkpoint (section "What has to be built - and the discovery that
// changed it") and the Geodesic post contrasts with MXFP4 ("Number formats
// on Blackwell").  The pages give no rounding rule; the one used here (all
// steps fp32, divisions correctly rounded):
//   gs     = amax / 2688, or 1 when the matrix is all zero (2688 = 6 * 448)
//   sf_b   = e4m3_rne((blockmax_b / 6) / gs), saturating at 448
//   d_b    = e4m3(sf_b) * gs
//   code   = e2m1_rne(|w| / d_b), ties to the even code, saturating at 6;
//            sign only for w < 0 with a non-zero code; d_b = 0 -> code 0.
#include "internal.h"

namespace moe {
namespace {

__global__ void zero_word_kernel(uint32_t* p) { p[0] = 0u; }

// amax as the largest bit pattern of |w| (order-preserving for non-negative
// floats), so the integer atomic max is exact and deterministic.
__global__ __launch_bounds__(256) void amax_kernel(const float* __restrict__ w, long long n4,
                                                  uint32_t* __restrict__ amax_bits) {
  uint32_t m = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const float4 v = reinterpret_cast<const float4*>(w)[i];
    m = max(m, __float_as_uint(fabsf(v.x)));
    m = max(m, __float_as_uint(fabsf(v.y)));
    m = max(m, __float_as_uint(fabsf(v.z)));
    m = max(m, __float_as_uint(fabsf(v.w)));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, WAVE));
  __shared__ uint32_t wmax[256 / WAVE];
  if (threadIdx.x % WAVE == 0) wmax[threadIdx.x / WAVE] = m;
  __syncthreads();
  if (threadIdx.x == 0) {  // one atomic per block
    for (int i = 1; i < 256 / WAVE; i++) m = max(m, wmax[i]);
    atomicMax(amax_bits, m);
  }
}

// Nearest non-negative finite e4m3 code to t >= 0, ties to the even code;
// t >= 448 gives 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_code_rne(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);  // subnormals m * 2^-9; 8 -> 2^-6
  const uint32_t u = __float_as_uint(t);
  int ex = (int)(u >> 23) - 127;
  uint32_t m3 = (u >> 20) & 7u;
  const uint32_t rest = u & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) m3++;
  if (m3 == 8u) {
    m3 = 0u;
    ex++;
  }
  const uint32_t code = ((uint32_t)(ex + 7) << 3) | m3;
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  if (code < 8u) return (float)code * (1.0f / 512.0f);
  return __uint_as_float((((code >> 3) + 120u) << 23) | ((code & 7u) << 20));
}

// Magnitude code of the nearest e2m1 value {0,.5,1,1.5,2,3,4,6} to r >= 0.
// At a midpoint the even code wins: strict '>' where the lower neighbour's
// code is even, '>=' where the upper one's is.
__device__ __forceinline__ uint32_t e2m1_code_rne(float r) {
  return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) + (uint32_t)(r >= 1.75f) +
         (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) + (uint32_t)(r > 5.0f);
}

// One thread per 16-element block; blocks are contiguous in w, q (8 bytes
// each) and sf (1 byte each) because all three are row-major.
__global__ __launch_bounds__(256) void quant_kernel(const float* __restrict__ w, long long nblk,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                                                   float* __restrict__ gs_out,
                                                   const uint32_t* __restrict__ amax_bits) {
  const float amax = __uint_as_float(*amax_bits);
  const float gs = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  const long long first = (long long)blockIdx.x * 256 + threadIdx.x;
  if (first == 0) *gs_out = gs;
  for (long long b = first; b < nblk; b += (long long)gridDim.x * 256) {
    const float4* src = reinterpret_cast<const float4*>(w) + 4 * b;
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float4 t = src[i];
      v[4 * i] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) bmax = fmaxf(bmax, fabsf(v[i]));
    const uint32_t sc = e4m3_code_rne(__fdiv_rn(__fdiv_rn(bmax, 6.0f), gs));
    const float d = __fmul_rn(e4m3_value(sc), gs);
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      uint32_t c = 0u;
      if (d > 0.0f) {
        c = e2m1_code_rne(__fdiv_rn(fabsf(v[i]), d));
        if (v[i] < 0.0f && c != 0u) c |= 8u;
      }
      if (i < 8)
        lo |= c << (4 * i);
      else
        hi |= c << (4 * (i - 8));
    }
    reinterpret_cast<uint2*>(q)[b] = make_uint2(lo, hi);
    sf[b] = (uint8_t)sc;
  }
}

// ---- MXFP4 (OCP microscaling: e8m0 power-of-two scale per 32 elements) -------
// floor(log2(a)) of a finite a > 0, subnormals included.
__device__ __forceinline__ int floor_log2(float a) { return __builtin_amdgcn_frexp_expf(a) - 1; }

// One thread per 32-element block: scale byte s = floor(log2(blockmax)) - 2
// + 127 clamped to 0..254 (a zero block: 0), codes = e2m1_rne(|w| / 2^(s-127))
// clamped to 6 (the division by a power of two is exact); the first thread
// also writes gs = 2^(smax - 135) from the matrix's largest |w|.
__global__ __launch_bounds__(256) void quant_mx_kernel(const float* __restrict__ w, long long nblk,
                                                      uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                                                      float* __restrict__ gs_out,
                                                      const uint32_t* __restrict__ amax_bits) {
  const long long first = (long long)blockIdx.x * 256 + threadIdx.x;
  if (first == 0) {
    const float amax = __uint_as_float(*amax_bits);
    const int smax = amax > 0.0f ? min(max(floor_log2(amax) - 2 + 127, 0), 254) : 0;
    *gs_out = __builtin_ldexpf(1.0f, smax - 135);
  }
  for (long long b = first; b < nblk; b += (long long)gridDim.x * 256) {
    const float4* src = reinterpret_cast<const float4*>(w) + 8 * b;
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float4 t = src[i];
      v[4 * i] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) bmax = fmaxf(bmax, fabsf(v[i]));
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    int s = 0;
    if (bmax > 0.0f) {
      s = min(max(floor_log2(bmax) - 2 + 127, 0), 254);
      const float inv = __builtin_ldexpf(1.0f, 127 - s);  // 1 / X, a power of two
#pragma unroll
      for (int i = 0; i < 32; i++) {
        uint32_t c = e2m1_code_rne(fabsf(v[i]) * inv);
        if (v[i] < 0.0f && c != 0u) c |= 8u;
        words[i / 8] |= c << (4 * (i % 8));
      }
    }
    reinterpret_cast<uint4*>(q)[b] = make_uint4(words[0], words[1], words[2], words[3]);
    sf[b] = (uint8_t)s;
  }
}

unsigned grid_for(long long n) {
  long long g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, uint32_t* ws,
                           hipStream_t s) {
  const long long n = (long long)N * K;
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, ws);
  long long ga = (n / 4 + 4095) / 4096;  // >= 16 float4 per thread
  if (ga > 1024) ga = 1024;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)(ga > 0 ? ga : 1)), dim3(256), 0, s, w, n / 4, ws);
  hipLaunchKernelGGL(quant_kernel, dim3(grid_for(n / 16)), dim3(256), 0, s, w, n / 16, q, sf, gs, ws);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, uint32_t* ws,
                              hipStream_t s) {
  const long long n = (long long)N * K;
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, ws);
  long long ga = (n / 4 + 4095) / 4096;
  if (ga > 1024) ga = 1024;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)(ga > 0 ? ga : 1)), dim3(256), 0, s, w, n / 4, ws);
  hipLaunchKernelGGL(quant_mx_kernel, dim3(grid_for(n / 32)), dim3(256), 0, s, w, n / 32, q, sf, gs, ws);
  return hipGetLastError();
}

}  // namespace moe
