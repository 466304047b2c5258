// GPU implementation of the seeded synthetic inputs (see synth_def.h); the
// values are bit-identical to the CPU implementation in synth.c.
#include <hip/hip_runtime.h>
#include "synth.h"
#include "synth_def.h"

namespace {

__global__ void k_x(uint64_t key, int64_t t0, int64_t T, int H, uint16_t* out) {
  int64_t n = T * H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t t = i / H, h = i - t * H;
    out[i] = synth_bf16_rne(synth_normal(key, (uint64_t)(t0 + t) * (uint64_t)H + (uint64_t)h));
  }
}

__global__ void k_router(uint64_t key, int64_t n, float std, uint16_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = synth_bf16_rne(std * synth_normal(key, (uint64_t)i));
}

__global__ void k_expert(uint64_t key, int64_t n, float std, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = std * synth_normal(key, (uint64_t)i);
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" int synth_gpu_x_bf16(uint64_t seed, int64_t t0, int T, int H, uint16_t* out, void* stream) {
  if (T <= 0 || H <= 0) return 0;
  int64_t n = (int64_t)T * H;
  hipLaunchKernelGGL(k_x, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, synth_key(seed, SYNTH_STREAM_X), t0,
                     (int64_t)T, H, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int synth_gpu_router_bf16(uint64_t seed, int H, int E, float std, uint16_t* out, void* stream) {
  int64_t n = (int64_t)H * E;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_router, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, synth_key(seed, SYNTH_STREAM_WR), n,
                     std, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int synth_gpu_proj_bf16(uint64_t seed, int which, int K, int N, float std, uint16_t* out, void* stream) {
  int64_t n = (int64_t)K * N;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_router, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     synth_key(seed, (uint64_t)SYNTH_STREAM_PROJ_DOWN + (uint64_t)which), n, std, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int synth_gpu_expert_f32(uint64_t seed, int e, int m, int N, int K, float std, float* out, void* stream) {
  int64_t n = (int64_t)N * K;
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_expert, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     synth_key(seed, synth_expert_stream((uint32_t)e, (uint32_t)m)), n, std, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
