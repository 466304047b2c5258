// Dense bf16 work around the routed experts: the shared experts, and the
// projections of the latent routed-expert block.
//
// Shared experts (wpnews.pro, "Serving Kimi K3 End to End", section 3.3:
// every token uses the 2 shared experts, whose output joins the MoE sum;
// "Serving Kimi-K3 ... with 8xB300 GPUs", "Precision: what is stored in
// which format": they are bf16).  For shared expert s with intermediate
// width I: g, u = x . Wgu (columns 2sI.. and 2sI+I..), h = bf16(SiLU(g) * u),
// and h . Wd (rows sI..) is added to the routed sum by the combine.
//
// Projections of the latent block (K3's LatentMoE):
// the routed-down projection of the hidden state into the routed latent
// before the experts, and the routed-up projection of their combined output
// back to the hidden width (lightseek.org, "Kimi K3 optimization on GB300",
// part I, sections "Routed-down projection: column sharding and latent
// assembly" and "Routed-up projection: sharding the post-expert tail").
//
// out[T][N] = bf16(x[T][K] . W[K][N]) with W stored input-major, the layout
// of the router weight: the router's GEMV (small T) and bf16 matrix-core GEMM
// (large T) compute the K-slab partial sums in fp32, and one more kernel adds
// the slabs in a fixed order and rounds to bf16 (and, for the latent that
// feeds the experts, also writes its exact fp16 copy).
#include "internal.h"

namespace moe {
namespace {

constexpr int PROJ_THREADS = 256;

// Four consecutive outputs per thread.
__global__ __launch_bounds__(PROJ_THREADS) void proj_reduce_kernel(const float* __restrict__ part, int slabs,
                                                                   long long n4, long long stride,
                                                                   uint16_t* __restrict__ out,
                                                                   f16* __restrict__ out16) {
  const long long i = (long long)blockIdx.x * PROJ_THREADS + threadIdx.x;
  if (i >= n4) return;
  float4 acc = reinterpret_cast<const float4*>(part)[i];
  add_slab_partials4(acc, part + 4 * i, stride, 1, slabs);
  const uint16_t b0 = f32_to_bf16(acc.x), b1 = f32_to_bf16(acc.y), b2 = f32_to_bf16(acc.z), b3 = f32_to_bf16(acc.w);
  uint2 o;
  o.x = (uint32_t)b0 | ((uint32_t)b1 << 16);
  o.y = (uint32_t)b2 | ((uint32_t)b3 << 16);
  reinterpret_cast<uint2*>(out)[i] = o;
  if (out16) {
    // bf16 values of 2^-17 <= |v| < 65504 (and zero) are exact in fp16;
    // smaller ones fall in fp16's subnormal range and round to a multiple
    // of 2^-24 (an error of at most 2^-25)
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 h;
    h[0] = (f16)bf16_to_f32(b0);
    h[1] = (f16)bf16_to_f32(b1);
    h[2] = (f16)bf16_to_f32(b2);
    h[3] = (f16)bf16_to_f32(b3);
    reinterpret_cast<h4*>(out16)[i] = h;
  }
}

// h[t][c] = bf16(SiLU(g) * u) for shared-expert column c (expert s = c / I,
// i = c % I): g = column 2sI + i, u = column 2sI + I + i of the gate/up
// product, each the fixed-order sum of its slab partials.  Four columns per
// thread (I % 4 == 0).
__global__ __launch_bounds__(PROJ_THREADS) void swiglu_reduce_kernel(const float* __restrict__ part, int slabs, int T,
                                                                     int I, int width, uint16_t* __restrict__ h) {
  const long long q = (long long)blockIdx.x * PROJ_THREADS + threadIdx.x;  // group of four columns
  const long long n4 = (long long)T * width / 4;
  if (q >= n4) return;
  const int t = (int)(q / (width / 4)), c = (int)(q % (width / 4)) * 4;
  const int s = c / I, i = c % I;
  const long long stride = (long long)T * 2 * width;
  const float* gp = part + (size_t)t * 2 * width + 2 * s * I + i;
  float4 g = *reinterpret_cast<const float4*>(gp), u = *reinterpret_cast<const float4*>(gp + I);
  add_slab_partials4(g, gp, stride, 1, slabs);
  add_slab_partials4(u, gp + I, stride, 1, slabs);
  const float v0 = g.x / (1.0f + expf(-g.x)) * u.x, v1 = g.y / (1.0f + expf(-g.y)) * u.y;
  const float v2 = g.z / (1.0f + expf(-g.z)) * u.z, v3 = g.w / (1.0f + expf(-g.w)) * u.w;
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  o.y = (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16);
  *reinterpret_cast<uint2*>(h + (size_t)t * width + c) = o;
}

}  // namespace

hipError_t launch_shared_hidden(const uint16_t* x, const uint16_t* w_gate_up, float* part, int T, int H, int count,
                                int I, const RouterPlan& rp, uint16_t* h, hipStream_t s) {
  const int width = count * I;
  hipError_t e = launch_router(x, w_gate_up, part, T, H, 2 * width, rp, s);
  if (e != hipSuccess) return e;
  const long long n4 = (long long)T * width / 4;
  hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((n4 + PROJ_THREADS - 1) / PROJ_THREADS)),
                     dim3(PROJ_THREADS), 0, s, part, rp.slabs, T, I, width, h);
  return hipGetLastError();
}

hipError_t launch_projection(const uint16_t* x, const uint16_t* w, float* part, int T, int K, int N,
                             const RouterPlan& rp, uint16_t* out, f16* out16, hipStream_t s) {
  hipError_t e = launch_router(x, w, part, T, K, N, rp, s);
  if (e != hipSuccess) return e;
  const long long n4 = (long long)T * N / 4;
  const long long blocks = (n4 + PROJ_THREADS - 1) / PROJ_THREADS;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)blocks), dim3(PROJ_THREADS), 0, s, part, rp.slabs, n4,
                     (long long)T * N, out, out16);
  return hipGetLastError();
}

}  // namespace moe
