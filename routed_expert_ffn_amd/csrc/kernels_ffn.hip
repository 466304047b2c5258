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

// One 256-k chunk of a wavefront's operands: per weight row group ng, 32
// NVFP4 code bytes (64 consecutive k) and their 4 scale bytes; per token
// fragment f, the eight A fragments of the chunk.  All of a chunk's loads are
// issued together so the wavefront waits once per chunk, not once per MFMA.
template <int MF>
struct Chunk {
  uint4 qa[4], qb[4];
  uint32_t sc[4];
  f16x8 a[MF][8];
};

template <int MF>
__device__ __forceinline__ void load_b(Chunk<MF>& ch, const uint8_t* const (&qrow)[4],
                                       const uint8_t* const (&srow)[4], int kb) {
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    ch.qa[ng] = *reinterpret_cast<const uint4*>(qrow[ng] + kb / 2);
    ch.qb[ng] = *reinterpret_cast<const uint4*>(qrow[ng] + kb / 2 + 16);
    ch.sc[ng] = *reinterpret_cast<const uint32_t*>(srow[ng] + kb / 16);
  }
}

template <int MF>
__device__ __forceinline__ void load_a(Chunk<MF>& ch, const f16* const (&arow)[MF], int kb, int nvalid) {
#pragma unroll
  for (int f = 0; f < MF; f++)
    if (f * 16 < nvalid)
#pragma unroll
      for (int s = 0; s < 8; s++) ch.a[f][s] = load_f16x8(arow[f] + kb + 8 * s);
}

// acc[f][ng] += A fragments x dequantised weights of one chunk.  Each row
// group is dequantised and multiplied in turn, so one B fragment is live.
template <int MF>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[MF][4], const Chunk<MF>& ch, int nvalid) {
#pragma unroll
  for (int s = 0; s < 8; s++) {
#pragma unroll
    for (int ng = 0; ng < 4; ng++) {
      const uint32_t codes = s < 4 ? (&ch.qa[ng].x)[s] : (&ch.qb[ng].x)[s - 4];
      const f16 sig = e4m3_to_f16((ch.sc[ng] >> (8 * (s / 2))) & 0xFFu);
      f16x2 sig2;
      sig2[0] = sig;
      sig2[1] = sig;
      const f16x8 bf = dequant8(codes, sig2);
#pragma unroll
      for (int f = 0; f < MF; f++)
        if (f * 16 < nvalid) acc[f][ng] = mfma16x16x32(ch.a[f][s], bf, acc[f][ng]);
    }
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// One grouped NVFP4 GEMM over the active experts (blockIdx.y indexes the
// active list).  A block is four wavefronts; KSPLIT consecutive wavefronts
// share one 64-row tile and take interleaved 256-k chunks of K, so a block
// covers 4/KSPLIT row tiles.
//   GATEUP: a row tile is 32 columns of h: gate rows (groups 0, 1) and the
//           same up rows (groups 2, 3); the epilogue applies the per-tensor
//           scales and SiLU(gate) * up and stores h in fp16.
//   down:   a row tile is 64 output columns; rows = gs_d * (h . Wd).
// The first chunk's weight loads are issued before the token rows are
// looked up, and each later chunk is loaded while the previous one is
// multiplied.  Partial sums of the KSPLIT wavefronts meet in LDS and are
// added in a fixed order.
template <int MF, int KSPLIT, bool GATEUP, bool DB, int WAVES_PER_EU>
__global__ __launch_bounds__(FFN_THREADS, WAVES_PER_EU) void expert_gemm_kernel(GroupedParams p) {
  constexpr int RT = 4 / KSPLIT;
  __shared__ float red[KSPLIT > 1 ? 4 : 1][WAVE][MF * 16];
  if ((int)blockIdx.y >= *p.n_active) return;
  const int e = p.active[blockIdx.y];
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, r = lane % 16, g = lane / 16;
  const int rt = wv / KSPLIT, ks = wv % KSPLIT;
  const int K = GATEUP ? p.H : p.I;
  const int N = GATEUP ? p.I : p.H;
  const int tile = blockIdx.x * RT + rt;
  const uint8_t* qrow[4];
  const uint8_t* srow[4];
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    size_t row;
    const uint8_t* qb;
    const uint8_t* sb;
    if (GATEUP) {
      row = (size_t)e * N + tile * 32 + 16 * (ng & 1) + r;
      qb = ng < 2 ? p.q0 : p.q1;
      sb = ng < 2 ? p.sf0 : p.sf1;
    } else {
      row = (size_t)e * N + tile * 64 + 16 * ng + r;
      qb = p.q0;
      sb = p.sf0;
    }
    qrow[ng] = qb + row * (K / 2);
    srow[ng] = sb + row * (K / 16);
  }
  const int nchunks = K / KCHUNK;
  Chunk<MF> cur;
  if (ks < nchunks) load_b(cur, qrow, srow, ks * KCHUNK + 64 * g);  // before the token lookups
  const int begin = p.offsets[e], end = p.offsets[e + 1];
  const float gsa = p.gs0[e], gsb = GATEUP ? p.gs1[e] : 0.0f;
  bool first_pass = true;
  for (int mb = begin; mb < end; mb += MF * 16) {
    const int nvalid = end - mb;
    const f16* arow[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) {
      const int pp = min(mb + f * 16 + r, end - 1);
      arow[f] = GATEUP ? p.a + (size_t)(p.sorted_pairs[pp] / p.k) * K : p.a + (size_t)pp * K;
    }
    f32x4 acc[MF][4];
#pragma unroll
    for (int f = 0; f < MF; f++)
#pragma unroll
      for (int ng = 0; ng < 4; ng++) acc[f][ng] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (ks < nchunks) {
      if (!first_pass) load_b(cur, qrow, srow, ks * KCHUNK + 64 * g);
      load_a(cur, arow, ks * KCHUNK + 64 * g, nvalid);
    }
    first_pass = false;
    for (int c = ks; c < nchunks; c += KSPLIT) {
      const int kb = c * KCHUNK + 64 * g;
      const bool more = c + KSPLIT < nchunks;
      if (DB) {  // load the next chunk while this one is multiplied
        Chunk<MF> nxt;
        if (more) {
          load_b(nxt, qrow, srow, kb + KSPLIT * KCHUNK);
          load_a(nxt, arow, kb + KSPLIT * KCHUNK, nvalid);
        }
        mma_chunk<MF>(acc, cur, nvalid);
        if (more) cur = nxt;
      } else {
        mma_chunk<MF>(acc, cur, nvalid);
        if (more) {
          load_b(cur, qrow, srow, kb + KSPLIT * KCHUNK);
          load_a(cur, arow, kb + KSPLIT * KCHUNK, nvalid);
        }
      }
    }
    if (KSPLIT > 1) {
#pragma unroll
      for (int f = 0; f < MF; f++)
#pragma unroll
        for (int ng = 0; ng < 4; ng++)
#pragma unroll
          for (int i = 0; i < 4; i++) red[wv][lane][(f * 4 + ng) * 4 + i] = acc[f][ng][i];
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int f = 0; f < MF; f++)
#pragma unroll
          for (int ng = 0; ng < 4; ng++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              float v = red[wv][lane][(f * 4 + ng) * 4 + i];
#pragma unroll
              for (int s2 = 1; s2 < KSPLIT; s2++) v += red[wv + s2][lane][(f * 4 + ng) * 4 + i];
              acc[f][ng][i] = v;
            }
      }
    }
    if (ks == 0) {
#pragma unroll
      for (int f = 0; f < MF; f++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = f * 16 + 4 * g + i;
          if (m < nvalid) {
            if (GATEUP) {
#pragma unroll
              for (int cp = 0; cp < 2; cp++) {
                const float hv = silu(gsa * acc[f][cp][i]) * (gsb * acc[f][cp + 2][i]);
                p.h[(size_t)(mb + m) * N + tile * 32 + 16 * cp + r] = (f16)hv;
              }
            } else {
#pragma unroll
              for (int ng = 0; ng < 4; ng++) p.rows[(size_t)(mb + m) * N + tile * 64 + 16 * ng + r] = gsa * acc[f][ng][i];
            }
          }
        }
    }
    if (KSPLIT > 1) __syncthreads();
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
// At decode sizes one 16-token fragment per pass keeps two wavefronts per
// SIMD resident; an expert with more tokens takes several passes, the later
// ones re-reading its weights from the caches.  Large batches use four.
int pick_mf(int T) { return T <= 1024 ? 1 : 4; }

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

// Row tiles per block: gate/up splits K over all four wavefronts (one
// 32-column tile per block), down over two (two 64-column tiles per block).
constexpr int GU_KSPLIT = 4;
constexpr int DN_KSPLIT = 2;

// Measured on MI355X at T = 1, 64 and 256: no register double buffer and a
// two-wavefronts-per-SIMD register budget stream fastest.
constexpr bool GEMM_DB = false;
constexpr int GEMM_WAVES = 2;

template <int KSPLIT, bool GATEUP>
hipError_t launch_gemm(const GroupedParams& p, int mf, dim3 grid, hipStream_t s) {
  switch (mf) {
    case 1:
      hipLaunchKernelGGL((expert_gemm_kernel<1, KSPLIT, GATEUP, GEMM_DB, GEMM_WAVES>), grid, dim3(FFN_THREADS),
                         0, s, p);
      break;
    case 2:
      hipLaunchKernelGGL((expert_gemm_kernel<2, KSPLIT, GATEUP, GEMM_DB, GEMM_WAVES>), grid, dim3(FFN_THREADS),
                         0, s, p);
      break;
    default:
      hipLaunchKernelGGL((expert_gemm_kernel<4, KSPLIT, GATEUP, GEMM_DB, 1>), grid, dim3(FFN_THREADS), 0, s, p);
      break;
  }
  return hipGetLastError();
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
  const dim3 grid(a.I / (32 * (4 / GU_KSPLIT)), a.max_active);
  return launch_gemm<GU_KSPLIT, true>(p, pick_mf(a.T), grid, s);
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  GroupedParams p = base_params(a);
  p.a = a.h;
  p.q0 = a.w->down.q;
  p.sf0 = a.w->down.sf;
  p.gs0 = a.w->down.gs;
  const dim3 grid(a.H / (64 * (4 / DN_KSPLIT)), a.max_active);
  return launch_gemm<DN_KSPLIT, false>(p, pick_mf(a.T), grid, s);
}

hipError_t launch_combine(const float* rows, const int32_t* pair_pos, const float* w, int T, int H, int k,
                          uint16_t* y, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, rows, pair_pos, w, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
