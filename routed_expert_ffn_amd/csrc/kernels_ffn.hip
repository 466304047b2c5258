// Grouped expert FFN on gfx950: gate/up GEMM fused with SiLU*mul, the down
// GEMM, and the weighted un-permute + combine.
//
// Each expert is three matrices ("Serving Kimi-K3 ... with 8xB300 GPUs",
// section "The model, as the serving system sees it"), stored as NVFP4
// (al-engr.com Kimi-K3 plan, section "What has to be built - and the
// discovery that changed it").  The grouped kernels walk the active experts
// in expert order so each expert's weights are streamed once for its whole
// bucket of tokens ("Computation and Data Movement for Inference", sections
// 4 and 15); at decode sizes all selected experts of the layer run in one
// launch, the point the Geodesic post makes in "Number formats on
// Blackwell".  The combine restores token order, weights and sums (essay,
// sections 4 and 5).
//
// Matrix-core mapping.  v_mfma_f32_16x16x32_f16: lane l holds A[l%16][8g..8g+7]
// and B[8g..8g+7][l%16] with g = l/16, and D[4g..4g+3][l%16].  A = tokens
// (fp16 activations), B = one expert's weight rows, dequantised in registers:
// the conversion instruction turns e2m1 codes into fp16 and a packed fp16
// multiply applies the e4m3 block scale (exact, see common.h).  The fp32
// per-tensor scale is applied once per output.
//
// Loads.  A block owns 64 weight rows (4 groups of 16).  Per 256-k chunk,
// lane (r = l%16, g = l/16) reads 32 bytes (64 codes) of row r at k offset
// 64g and the 4 scale bytes of those 64 codes, so each row's 128-byte span
// of the chunk is read whole by one wavefront.  Code dword s (k = 64g+8s..)
// is exactly the B fragment of MFMA step s, so the k order inside an MFMA is
// permuted consistently for A and B.  The four wavefronts of a block take
// interleaved chunks of K and are reduced through LDS in a fixed order.
#include "internal.h"

namespace moe {
namespace {

constexpr int FFN_THREADS = 256;
constexpr int KCHUNK = 256;
constexpr int GU_COLS = 32;    // h columns per gate/up block (32 gate + 32 up rows)
constexpr int DN_COLS = 64;    // output columns per down block

struct GroupedParams {
  int H, I, k;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* active;
  const int32_t* n_active;
  const f16* a;        // gate/up: x16 [T][H]; down: h [P][I]
  const uint8_t* q0;   // gate/up: gate codes; down: down codes
  const uint8_t* sf0;
  const float* gs0;
  const uint8_t* q1;   // gate/up: up codes; down: unused
  const uint8_t* sf1;
  const float* gs1;
  f16* h;              // gate/up output [P][I]
  float* rows;         // down output [P][H]
};

// K loop shared by both GEMMs: accumulate the block's 64 weight rows
// (qrow[ng] / srow[ng] point at row r of group ng) against MF 16-token
// fragments of A rows arow[f] (nvalid rows are real), over chunks
// c = wv, wv+4, ... of K.
template <int MF>
__device__ __forceinline__ void kloop(f32x4 (&acc)[MF][4], const uint8_t* const (&qrow)[4],
                                      const uint8_t* const (&srow)[4], const f16* const (&arow)[MF], int K, int wv,
                                      int g, int nvalid) {
  const int nchunks = K / KCHUNK;
  for (int c = wv; c < nchunks; c += 4) {
    const int kb = c * KCHUNK + 64 * g;
    uint4 qa[4], qb[4];
    uint32_t sc[4];
#pragma unroll
    for (int ng = 0; ng < 4; ng++) {
      qa[ng] = *reinterpret_cast<const uint4*>(qrow[ng] + kb / 2);
      qb[ng] = *reinterpret_cast<const uint4*>(qrow[ng] + kb / 2 + 16);
      sc[ng] = *reinterpret_cast<const uint32_t*>(srow[ng] + kb / 16);
    }
#pragma unroll
    for (int s = 0; s < 8; s++) {
      f16x8 bf[4];
#pragma unroll
      for (int ng = 0; ng < 4; ng++) {
        const uint32_t codes = s < 4 ? (&qa[ng].x)[s] : (&qb[ng].x)[s - 4];
        const f16 sig = e4m3_to_f16((sc[ng] >> (8 * (s / 2))) & 0xFFu);
        f16x2 sig2;
        sig2[0] = sig;
        sig2[1] = sig;
        bf[ng] = dequant8(codes, sig2);
      }
#pragma unroll
      for (int f = 0; f < MF; f++) {
        if (f * 16 < nvalid) {
          const f16x8 av = load_f16x8(arow[f] + kb + 8 * s);
#pragma unroll
          for (int ng = 0; ng < 4; ng++) acc[f][ng] = mfma16x16x32(av, bf[ng], acc[f][ng]);
        }
      }
    }
  }
}

template <int MF>
__device__ __forceinline__ void spill_partials(float (*red)[WAVE][MF * 16], f32x4 (&acc)[MF][4], int wv, int lane) {
#pragma unroll
  for (int f = 0; f < MF; f++)
#pragma unroll
    for (int ng = 0; ng < 4; ng++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[wv][lane][(f * 4 + ng) * 4 + i] = acc[f][ng][i];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// h[p][i] = SiLU(gs_g * (x.Wg)[i]) * (gs_u * (x.Wu)[i]) for the pairs p of
// expert active[blockIdx.y], columns i in [32*blockIdx.x, +32).
template <int MF>
__global__ __launch_bounds__(FFN_THREADS) void gateup_kernel(GroupedParams p) {
  __shared__ float red[4][WAVE][MF * 16];
  if ((int)blockIdx.y >= *p.n_active) return;
  const int e = p.active[blockIdx.y];
  const int begin = p.offsets[e], end = p.offsets[e + 1];
  const int H = p.H, I = p.I;
  const int i0 = blockIdx.x * GU_COLS;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, r = lane % 16, g = lane / 16;
  const uint8_t* qrow[4];
  const uint8_t* srow[4];
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    const size_t row = (size_t)e * I + i0 + 16 * (ng & 1) + r;
    qrow[ng] = (ng < 2 ? p.q0 : p.q1) + row * (H / 2);
    srow[ng] = (ng < 2 ? p.sf0 : p.sf1) + row * (H / 16);
  }
  const float gsg = p.gs0[e], gsu = p.gs1[e];
  for (int mb = begin; mb < end; mb += MF * 16) {
    const int nvalid = end - mb;
    const f16* arow[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) {
      const int pp = min(mb + f * 16 + r, end - 1);
      arow[f] = p.a + (size_t)(p.sorted_pairs[pp] / p.k) * H;
    }
    f32x4 acc[MF][4];
#pragma unroll
    for (int f = 0; f < MF; f++)
#pragma unroll
      for (int ng = 0; ng < 4; ng++) acc[f][ng] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    kloop<MF>(acc, qrow, srow, arow, H, wv, g, nvalid);
    spill_partials<MF>(red, acc, wv, lane);
    __syncthreads();
    // Outputs (f, column pair cp, lane ln, i): gate in group cp, up in cp+2.
    for (int q = threadIdx.x; q < MF * 2 * WAVE * 4; q += FFN_THREADS) {
      const int i = q % 4, ln = (q / 4) % WAVE, cp = (q / (4 * WAVE)) % 2, f = q / (8 * WAVE);
      const int m = f * 16 + 4 * (ln / 16) + i;
      if (m < nvalid) {
        const int gi = (f * 4 + cp) * 4 + i, ui = (f * 4 + cp + 2) * 4 + i;
        const float G = ((red[0][ln][gi] + red[1][ln][gi]) + red[2][ln][gi]) + red[3][ln][gi];
        const float U = ((red[0][ln][ui] + red[1][ln][ui]) + red[2][ln][ui]) + red[3][ln][ui];
        const float hv = silu(gsg * G) * (gsu * U);
        p.h[(size_t)(mb + m) * I + i0 + cp * 16 + ln % 16] = (f16)hv;
      }
    }
    __syncthreads();
  }
}

// rows[p][n] = gs_d * (h[p].Wd)[n] for the pairs p of expert
// active[blockIdx.y], columns n in [64*blockIdx.x, +64).
template <int MF>
__global__ __launch_bounds__(FFN_THREADS) void down_kernel(GroupedParams p) {
  __shared__ float red[4][WAVE][MF * 16];
  if ((int)blockIdx.y >= *p.n_active) return;
  const int e = p.active[blockIdx.y];
  const int begin = p.offsets[e], end = p.offsets[e + 1];
  const int H = p.H, I = p.I;
  const int n0 = blockIdx.x * DN_COLS;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, r = lane % 16, g = lane / 16;
  const uint8_t* qrow[4];
  const uint8_t* srow[4];
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    const size_t row = (size_t)e * H + n0 + 16 * ng + r;
    qrow[ng] = p.q0 + row * (I / 2);
    srow[ng] = p.sf0 + row * (I / 16);
  }
  const float gsd = p.gs0[e];
  for (int mb = begin; mb < end; mb += MF * 16) {
    const int nvalid = end - mb;
    const f16* arow[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) arow[f] = p.a + (size_t)min(mb + f * 16 + r, end - 1) * I;
    f32x4 acc[MF][4];
#pragma unroll
    for (int f = 0; f < MF; f++)
#pragma unroll
      for (int ng = 0; ng < 4; ng++) acc[f][ng] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    kloop<MF>(acc, qrow, srow, arow, I, wv, g, nvalid);
    spill_partials<MF>(red, acc, wv, lane);
    __syncthreads();
    for (int q = threadIdx.x; q < MF * 4 * WAVE * 4; q += FFN_THREADS) {
      const int i = q % 4, ln = (q / 4) % WAVE, ng = (q / (4 * WAVE)) % 4, f = q / (16 * WAVE);
      const int m = f * 16 + 4 * (ln / 16) + i;
      if (m < nvalid) {
        const int xi = (f * 4 + ng) * 4 + i;
        const float v = ((red[0][ln][xi] + red[1][ln][xi]) + red[2][ln][xi]) + red[3][ln][xi];
        p.rows[(size_t)(mb + m) * H + n0 + 16 * ng + ln % 16] = gsd * v;
      }
    }
    __syncthreads();
  }
}

// y[t][n] = bf16( sum_j w[t][j] * rows[pair_pos[t*k+j]][n] ), fp32 sum over
// ascending j.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows,
                                                     const int32_t* __restrict__ pair_pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     uint16_t* __restrict__ y) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  for (int j = 0; j < k; j++) {
    const int pos = pair_pos[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(rows + (size_t)pos * H + n);
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
  o.y = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + n) = o;
}

// Fragments per pass: an expert never has more pairs than there are tokens.
int pick_mf(int T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

GroupedParams base_params(const FfnArgs& a) {
  GroupedParams p{};
  p.H = a.H;
  p.I = a.I;
  p.k = a.k;
  p.offsets = a.offsets;
  p.sorted_pairs = a.sorted_pairs;
  p.active = a.active;
  p.n_active = a.n_active;
  p.h = a.h;
  p.rows = a.rows;
  return p;
}

}  // namespace

hipError_t launch_gateup(const FfnArgs& a, hipStream_t s) {
  GroupedParams p = base_params(a);
  p.a = a.x16;
  p.q0 = a.w->gate.q;
  p.sf0 = a.w->gate.sf;
  p.gs0 = a.w->gate.gs;
  p.q1 = a.w->up.q;
  p.sf1 = a.w->up.sf;
  p.gs1 = a.w->up.gs;
  const dim3 grid(a.I / GU_COLS, a.max_active);
  switch (pick_mf(a.T)) {
    case 1: hipLaunchKernelGGL((gateup_kernel<1>), grid, dim3(FFN_THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gateup_kernel<2>), grid, dim3(FFN_THREADS), 0, s, p); break;
    default: hipLaunchKernelGGL((gateup_kernel<4>), grid, dim3(FFN_THREADS), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  GroupedParams p = base_params(a);
  p.a = a.h;
  p.q0 = a.w->down.q;
  p.sf0 = a.w->down.sf;
  p.gs0 = a.w->down.gs;
  const dim3 grid(a.H / DN_COLS, a.max_active);
  switch (pick_mf(a.T)) {
    case 1: hipLaunchKernelGGL((down_kernel<1>), grid, dim3(FFN_THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((down_kernel<2>), grid, dim3(FFN_THREADS), 0, s, p); break;
    default: hipLaunchKernelGGL((down_kernel<4>), grid, dim3(FFN_THREADS), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const float* rows, const int32_t* pair_pos, const float* w, int T, int H, int k,
                          uint16_t* y, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, rows, pair_pos, w, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
