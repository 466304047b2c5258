// Routing on gfx950: router logits, softmax + top-k at one wavefront per
// token, and the token-to-expert permutation built from a histogram and a
// prefix scan.
//
// What is computed follows "Computation and Data Movement for Inference"
// (section 3.4 "Decode experts": the router, a small tensor, picks a few
// experts per token; section 4: route records are sorted by expert id so one
// weight load serves a bucket; section 15: counts, permutation and the
// restore to token order are part of the work) and the al-engr.com Kimi-K3
// plan (table "What we verified today": 16 of 896 experts per token).
#include "internal.h"

namespace moe {
namespace {

// ---- router logits: partial sums over slabs of H ---------------------------
// logits[t][e] = sum_h x[t][h] * W_r[h][e] with W_r stored [H][E] (E
// contiguous).  Each lane owns 8 consecutive experts (one 16-byte load per
// row h) and TT tokens; the four waves of a block take interleaved rows of
// the block's slab and are summed through LDS, then each slab writes its
// partial [slab][T][E].  bf16 x bf16 products are exact in fp32, so only the
// summation order differs from an exact dot product.
constexpr int RT_THREADS = 256;
constexpr int RT_E_PER_BLOCK = WAVE * 8;  // 512 experts per block

template <int TT>
__global__ __launch_bounds__(RT_THREADS) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ wr,
                                                                   float* __restrict__ part, int T, int H, int E,
                                                                   int slab_rows) {
  __shared__ float red[4][WAVE][TT * 8];
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int e0 = blockIdx.x * RT_E_PER_BLOCK + lane * 8;
  const int t0 = blockIdx.y * TT;
  const int h0 = blockIdx.z * slab_rows;
  const int h1 = min(H, h0 + slab_rows);
  float acc[TT][8];
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int i = 0; i < 8; i++) acc[a][i] = 0.0f;
  if (e0 < E) {
    for (int h = h0 + wv; h < h1; h += 4) {
      uint4 wv8 = *reinterpret_cast<const uint4*>(wr + (size_t)h * E + e0);
      float wf[8];
      wf[0] = __uint_as_float(wv8.x << 16); wf[1] = __uint_as_float(wv8.x & 0xFFFF0000u);
      wf[2] = __uint_as_float(wv8.y << 16); wf[3] = __uint_as_float(wv8.y & 0xFFFF0000u);
      wf[4] = __uint_as_float(wv8.z << 16); wf[5] = __uint_as_float(wv8.z & 0xFFFF0000u);
      wf[6] = __uint_as_float(wv8.w << 16); wf[7] = __uint_as_float(wv8.w & 0xFFFF0000u);
#pragma unroll
      for (int a = 0; a < TT; a++) {
        if (t0 + a < T) {
          float xv = bf16_to_f32(x[(size_t)(t0 + a) * H + h]);
#pragma unroll
          for (int i = 0; i < 8; i++) acc[a][i] = fmaf(xv, wf[i], acc[a][i]);
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int i = 0; i < 8; i++) red[wv][lane][a * 8 + i] = acc[a][i];
  __syncthreads();
  // Sum the four waves in a fixed order; thread -> (token a, expert i).
  for (int q = threadIdx.x; q < WAVE * TT * 8; q += RT_THREADS) {
    int ln = q / (TT * 8), ai = q % (TT * 8), a = ai / 8, i = ai % 8;
    int e = blockIdx.x * RT_E_PER_BLOCK + ln * 8 + i;
    if (e < E && t0 + a < T) {
      float s = ((red[0][ln][ai] + red[1][ln][ai]) + red[2][ln][ai]) + red[3][ln][ai];
      part[((size_t)blockIdx.z * T + (t0 + a)) * E + e] = s;
    }
  }
}

// logits[t][e] = (sum over slabs, ascending) + bias[e].
__global__ __launch_bounds__(256) void logits_reduce_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T, int E, int slabs) {
  const int t = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float s = 0.0f;
  for (int z = 0; z < slabs; z++) s += part[((size_t)z * T + t) * E + e];
  if (bias) s += bias[e];
  logits[(size_t)t * E + e] = s;
}

// ---- softmax + top-k: one wavefront per token ------------------------------
// Selection key: a 64-bit integer whose order is (logit descending, expert
// index ascending): the high word maps the fp32 logit to an order-preserving
// unsigned integer (with -0 folded onto +0), the low word is ~index.
constexpr int TOPK_MAX_PER_LANE = 16;  // E <= 1024

__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, WAVE);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ ids, float* __restrict__ wout) {
  const int lane = threadIdx.x % WAVE;
  const int t = blockIdx.x * 4 + threadIdx.x / WAVE;
  if (t >= T) return;  // whole wavefront leaves together
  const float* row = logits + (size_t)t * E;
  uint64_t key[TOPK_MAX_PER_LANE];
#pragma unroll
  for (int i = 0; i < TOPK_MAX_PER_LANE; i++) {
    int e = lane + WAVE * i;
    key[i] = 0;  // below every real key
    if (e < E) key[i] = ((uint64_t)float_order(row[e]) << 32) | (uint32_t)~(uint32_t)e;
  }
  int my_id = 0;
  float my_logit = 0.0f, top = 0.0f;
  for (int j = 0; j < k; j++) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < TOPK_MAX_PER_LANE; i++) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)~(uint32_t)best;
    const float l = order_float((uint32_t)(best >> 32));
    if (j == 0) top = l;
    if (lane == (e % WAVE)) {
#pragma unroll
      for (int i = 0; i < TOPK_MAX_PER_LANE; i++)
        if (i == e / WAVE) key[i] = 0;
    }
    if (lane == j) {
      my_id = e;
      my_logit = l;
    }
  }
  // w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0): softmax restricted to the
  // selected logits, identical to the full softmax renormalised over them.
  float ex = lane < k ? expf(my_logit - top) : 0.0f;
  float sum = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wout[(size_t)t * k + lane] = ex / sum;
  }
}

// ---- permutation: histogram, scan, stable scatter ----------------------------
// Tokens are processed in blocks of 64 (one per lane).  For block b and
// expert e, mask[b][e] has bit l set when token 64b+l selected e.  The
// records of expert e are ordered by token, so the position of record
// (t, j) is offsets[e] + (records of e in earlier blocks) + popcount of the
// mask bits below lane l.  Integer work only: exact and deterministic.
constexpr int PERM_MAX_E = 1024;

__global__ __launch_bounds__(WAVE) void perm_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         uint64_t* __restrict__ masks, int32_t* __restrict__ counts) {
  __shared__ unsigned long long m[PERM_MAX_E];
  const int lane = threadIdx.x, b = blockIdx.x;
  for (int e = lane; e < E; e += WAVE) m[e] = 0ull;
  __syncthreads();
  const int t = b * WAVE + lane;
  if (t < T)
    for (int j = 0; j < k; j++) atomicOr(&m[ids[(size_t)t * k + j]], 1ull << lane);
  __syncthreads();
  for (int e = lane; e < E; e += WAVE) {
    masks[(size_t)b * E + e] = m[e];
    counts[(size_t)b * E + e] = __popcll(m[e]);
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan(int v, int* lds /*[1024/64]*/, int* total) {
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  int incl = v;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    int o = __shfl_up(incl, off, WAVE);
    if (lane >= off) incl += o;
  }
  if (lane == WAVE - 1) lds[wv] = incl;
  __syncthreads();
  int wave_base = 0, all = 0;
  for (int i = 0; i < (int)(blockDim.x / WAVE); i++) {
    if (i < wv) wave_base += lds[i];
    all += lds[i];
  }
  __syncthreads();
  *total = all;
  return wave_base + incl - v;
}

// One block of 1024 threads, thread e = expert.  Turns per-block counts into
// absolute bases, writes offsets and the list of experts with work.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ counts, int nblocks, int E,
                                                        int P, int32_t* __restrict__ base,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                                        int32_t* __restrict__ n_active) {
  __shared__ int lds[1024 / WAVE];
  const int e = threadIdx.x;
  int running = 0;
  if (e < E)
    for (int b = 0; b < nblocks; b++) {
      base[(size_t)b * E + e] = running;
      running += counts[(size_t)b * E + e];
    }
  int total;
  const int off = block_exclusive_scan(e < E ? running : 0, lds, &total);
  const int flag = (e < E && running > 0) ? 1 : 0;
  int nact;
  const int slot = block_exclusive_scan(flag, lds, &nact);
  if (e < E) {
    offsets[e] = off;
    for (int b = 0; b < nblocks; b++) base[(size_t)b * E + e] += off;
    if (flag) active[slot] = e;
  }
  if (e == 0) {
    offsets[E] = P;
    *n_active = nact;
  }
}

__global__ __launch_bounds__(WAVE) void perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const uint64_t* __restrict__ masks,
                                                           const int32_t* __restrict__ base,
                                                           int32_t* __restrict__ sorted_pairs,
                                                           int32_t* __restrict__ pair_pos) {
  const int lane = threadIdx.x, b = blockIdx.x;
  const int t = b * WAVE + lane;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; j++) {
    const int f = t * k + j;
    const int e = ids[f];
    const int pos = base[(size_t)b * E + e] + __popcll(masks[(size_t)b * E + e] & below);
    sorted_pairs[pos] = f;
    pair_pos[f] = pos;
  }
}

// Experts with work, from offsets alone (when the permutation comes from
// the caller).
__global__ __launch_bounds__(1024) void active_list_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active) {
  __shared__ int lds[1024 / WAVE];
  const int e = threadIdx.x;
  const int flag = (e < E && offsets[e + 1] > offsets[e]) ? 1 : 0;
  int nact;
  const int slot = block_exclusive_scan(flag, lds, &nact);
  if (flag) active[slot] = e;
  if (e == 0) *n_active = nact;
}

// ---- activations bf16 -> fp16 (exact for |x| < 65504 above 2^-14) --------
__global__ __launch_bounds__(256) void cast_kernel(const uint16_t* __restrict__ x, f16* __restrict__ x16,
                                                  long long n8) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    uint4 v = reinterpret_cast<const uint4*>(x)[i];
    f16x8 o;
    o[0] = (f16)__uint_as_float(v.x << 16); o[1] = (f16)__uint_as_float(v.x & 0xFFFF0000u);
    o[2] = (f16)__uint_as_float(v.y << 16); o[3] = (f16)__uint_as_float(v.y & 0xFFFF0000u);
    o[4] = (f16)__uint_as_float(v.z << 16); o[5] = (f16)__uint_as_float(v.z & 0xFFFF0000u);
    o[6] = (f16)__uint_as_float(v.w << 16); o[7] = (f16)__uint_as_float(v.w & 0xFFFF0000u);
    reinterpret_cast<f16x8*>(x16)[i] = o;
  }
}

}  // namespace

int router_slabs(int T, int H, int E) {
  const int tt = T <= 1 ? 1 : 8;
  const long long tiles = (long long)((E + RT_E_PER_BLOCK - 1) / RT_E_PER_BLOCK) * ((T + tt - 1) / tt);
  long long s = 512 / (tiles > 0 ? tiles : 1);
  const int max_s = H / 16;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, float* part, int T, int H, int E, int slabs,
                         hipStream_t s) {
  const int slab_rows = (H + slabs - 1) / slabs;
  const int gx = (E + RT_E_PER_BLOCK - 1) / RT_E_PER_BLOCK;
  if (T <= 1)
    hipLaunchKernelGGL((router_partial_kernel<1>), dim3(gx, T, slabs), dim3(RT_THREADS), 0, s, x, wr, part, T, H, E,
                       slab_rows);
  else
    hipLaunchKernelGGL((router_partial_kernel<8>), dim3(gx, (T + 7) / 8, slabs), dim3(RT_THREADS), 0, s, x, wr, part,
                       T, H, E, slab_rows);
  return hipGetLastError();
}

hipError_t launch_logits_reduce(const float* part, const float* bias, float* logits, int T, int E, int slabs,
                                hipStream_t s) {
  hipLaunchKernelGGL(logits_reduce_kernel, dim3((E + 255) / 256, T), dim3(256), 0, s, part, bias, logits, T, E,
                     slabs);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, uint64_t* masks, int32_t* counts, int32_t* base,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active,
                          int32_t* n_active, hipStream_t s) {
  const int nb = perm_blocks(T);
  hipLaunchKernelGGL(perm_count_kernel, dim3(nb), dim3(WAVE), 0, s, ids, T, E, k, masks, counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, counts, nb, E, T * k, base, offsets, active,
                     n_active);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(WAVE), 0, s, ids, T, E, k, masks, base, sorted_pairs,
                     pair_pos);
  return hipGetLastError();
}

hipError_t launch_active_list(const int32_t* offsets, int E, int32_t* active, int32_t* n_active, hipStream_t s) {
  hipLaunchKernelGGL(active_list_kernel, dim3(1), dim3(1024), 0, s, offsets, E, active, n_active);
  return hipGetLastError();
}

hipError_t launch_cast(const uint16_t* x, f16* x16, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  long long g = (n8 + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(cast_kernel, dim3((unsigned)g), dim3(256), 0, s, x, x16, n8);
  return hipGetLastError();
}

}  // namespace moe
