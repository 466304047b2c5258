// HBM read calibration: reads a buffer once, as plainly as a streaming read
// can be written, so that the expert GEMMs' achieved bandwidth can be set
// against what this GPU delivers to a kernel (not only against the
// datasheet figure).  Block b reads a contiguous segment; wavefront w of the
// block reads the segment's 1 KB pieces w, w+4, w+8, ... (one 16-byte load
// per lane, a whole 1 KB per instruction), four pieces in flight; each block
// folds what it read into one word (XOR), so no load can be dropped.  The
// loads are non-temporal, like the expert GEMMs' code loads: on a cold
// 252 MiB read they reach about 6.0 TB/s against 5.2-5.4 TB/s cached.
// The matrix-core calibration below does the same for the prefill GEMMs.
#include "internal.h"

namespace moe {
namespace {

constexpr int STREAM_THREADS = 256;
constexpr int STREAM_U = 4;  // pieces in flight per wavefront

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* q) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(q));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__global__ __launch_bounds__(STREAM_THREADS) void stream_read_kernel(const uint4* __restrict__ p, long long n16,
                                                                   long long per16, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const long long begin = (long long)blockIdx.x * per16;
  const long long end = min(begin + per16, n16);
  uint32_t acc = 0;
  for (long long piece = begin / WAVE + w; piece * WAVE < end; piece += 4 * STREAM_U) {
    uint4 v[STREAM_U];
#pragma unroll
    for (int u = 0; u < STREAM_U; u++) {
      const long long i = (piece + 4 * u) * WAVE + lane;
      v[u] = i < end ? load_nt(p + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < STREAM_U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, WAVE);
  __shared__ uint32_t part[STREAM_THREADS / WAVE];
  if (lane == 0) part[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < STREAM_THREADS / WAVE; i++) r ^= part[i];
    sink[blockIdx.x] = r;
  }
}

// ---- matrix-core calibration ------------------------------------------------
// Sustained v_mfma_f32_32x32x16_f16 on operands with the expert GEMMs' value
// patterns: activations are bf16 values (an approximately normal variate,
// the sum of four uniforms, rounded to bf16 and held in fp16), weights are
// e2m1 values times an e4m3 block scale (3 mantissa bits, a few binades).
// Each wavefront keeps four accumulators and four A / two B fragments in
// registers and rotates them every round, so every MFMA sees new operands.
// On the power-limited chip the flop rate depends on how much the operands
// toggle, which is why the values, not just the instruction, are modelled.
typedef float f32x16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {  // a 32-bit integer hash (lowbias32)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ f16 activation_like(uint32_t h) {
  float u = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) u += (float)((h >> (8 * i)) & 0xFFu) * (1.0f / 255.0f);
  const float v = (u - 2.0f) * 1.7320508f;  // variance 1
  return (f16)bf16_to_f32(f32_to_bf16(v));
}

__device__ __forceinline__ f16 weight_like(uint32_t h) {
  const float e2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float sig = (1.0f + (float)((h >> 3) & 7u) * 0.125f) * __builtin_ldexpf(1.0f, -(int)((h >> 6) & 3u));
  const float v = e2m1[h & 7u] * sig;
  return (f16)((h >> 8) & 1u ? -v : v);
}

__global__ __launch_bounds__(512, 1) void mfma_rate_kernel(int iters, float* __restrict__ sink) {
  const uint32_t g = blockIdx.x * 512u + threadIdx.x;
  f16x8 a[4], b[2];
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int i = 0; i < 8; i++) a[f][i] = activation_like(mix32(g * 64u + f * 8u + i));
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int i = 0; i < 8; i++) b[f][i] = weight_like(mix32(0x9e3779b9u ^ (g * 64u + f * 8u + i)));
  f32x16v c[4] = {};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int f = 0; f < 4; f++) c[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[f], b[f / 2], c[f], 0, 0, 0);
    const f16x8 t = a[0];
    a[0] = a[1];
    a[1] = a[2];
    a[2] = a[3];
    a[3] = t;
    const f16x8 u = b[0];
    b[0] = b[1];
    b[1] = u;
  }
  float s = 0.0f;
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int i = 0; i < 16; i++) s += c[f][i];
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, WAVE);
  __shared__ float part[8];
  if (threadIdx.x % WAVE == 0) part[threadIdx.x / WAVE] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.0f;
    for (int i = 0; i < 8; i++) r += part[i];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_mfma_rate(int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(MOE_MFMA_RATE_BLOCKS), dim3(512), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, long long bytes, uint32_t* sink, hipStream_t s) {
  const long long n16 = bytes / 16;
  // segments of whole 1 KB pieces; at most STREAM_SINK_WORDS blocks
  long long per16 = (n16 + STREAM_SINK_WORDS - 1) / STREAM_SINK_WORDS;
  per16 = (per16 + WAVE - 1) / WAVE * WAVE;
  if (per16 < 16 * WAVE) per16 = 16 * WAVE;
  const long long blocks = (n16 + per16 - 1) / per16;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(STREAM_THREADS), 0, s,
                     static_cast<const uint4*>(buf), n16, per16, sink);
  return hipGetLastError();
}

}  // namespace moe
