// HBM read calibration: reads a buffer once, as plainly as a streaming read
// can be written, so that the expert GEMMs' achieved bandwidth can be set
// against what this GPU delivers to a kernel (not only against the
// datasheet figure).  Block b reads a contiguous segment; wavefront w of the
// block reads the segment's 1 KB pieces w, w+4, w+8, ... (one 16-byte load
// per lane, a whole 1 KB per instruction), four pieces in flight; each block
// folds what it read into one word (XOR), so no load can be dropped.  The
// loads are non-temporal, like the expert GEMMs' code loads: on a cold
// 252 MiB read they reach about 6.0 TB/s against 5.2-5.4 TB/s cached.
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

}  // namespace

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
