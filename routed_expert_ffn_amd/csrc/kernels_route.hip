// Routing on gfx950: router logits, softmax + top-k, and the token-to-expert
// permutation built from a histogram and a prefix scan.
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

// ---- router logits: 2-D tiled GEMV with slab partial sums ---------------------
// logits[t][e] = sum_h x[t][h] * W_r[h][e], W_r stored [H][E] (E contiguous).
// A block owns ET experts (ET/8 lanes x 8 experts, one 16-byte load per row)
// and a slab of rows; lane l reads row (64/(ET/8)) * wave + l/(ET/8) of each
// step, so one wavefront load covers whole 2*ET-byte row segments.  The
// lanes that share a column group are summed with butterfly steps and then
// across the four waves through LDS, in a fixed order, and the block writes
// one partial per (slab, token, expert).  bf16 x bf16 products are exact in
// fp32.  ET = 128 for wide outputs; ET = 64 for a router's few hundred
// experts, where twice the column tiles let half the K slabs fill the chip
// (fewer partials for the single-block routing to add).
constexpr int RT_THREADS = 256;
constexpr int ROUTER_MAX_SLABS = 32;  // K slabs of the router, at most
constexpr int RT_E_TILE = 128;
constexpr int RT_E_TILE_NARROW = 64;
constexpr int RT_NARROW_MAX_E = 1024;  // outputs up to this width take the narrow tile
constexpr int RT_BATCH = 16;  // weight rows per thread in flight
// rows of W_r one step of a block covers (four wavefronts)
constexpr int rt_rows_per_step(int et) { return 4 * (WAVE / (et / 8)); }

template <int TT, int ET>
__global__ __launch_bounds__(RT_THREADS) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wr,
                                                                float* __restrict__ part, int T, int H, int E,
                                                                int slab_rows, f16* __restrict__ x16) {
  constexpr int CG = ET / 8;                   // column groups: lanes per row
  constexpr int RPW = WAVE / CG;               // rows of a wavefront per step
  constexpr int RPS = rt_rows_per_step(ET);    // rows of the block per step
  extern __shared__ float smem[];
  float* xs = smem;                               // [TT][slab_rows]
  float* red = smem + TT * slab_rows;             // [4 waves][CG groups][TT * 8]
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int cg = lane % CG, rr = lane / CG;
  const int e0 = blockIdx.x * ET + cg * 8;
  const int h0 = blockIdx.y * slab_rows;
  const int t0 = blockIdx.z * TT;
  const int rows = min(slab_rows, H - h0);
  // Rows in batches of RT_BATCH loads in flight, then their FMAs in row
  // order.  The first batch is issued before the activations are staged (it
  // does not depend on them), so a slab of up to RT_BATCH * 16 rows costs
  // one memory round trip for the weights, overlapped with the one for x.
  uint4 w8[RT_BATCH];
  const bool active = e0 < E;
  auto load_batch = [&](int r0) {
#pragma unroll
    for (int b = 0; b < RT_BATCH; b++) {
      const int r = r0 + b * RPS;
      w8[b] = r < rows ? *reinterpret_cast<const uint4*>(wr + (size_t)(h0 + r) * E + e0) : make_uint4(0, 0, 0, 0);
    }
  };
  if (active) load_batch(RPW * wv + rr);
  // the blocks of the first expert tile also write the fp16 copy of their
  // slab of x (bf16 -> fp32 exact, then the fp16 rounding)
  const bool cast = x16 != nullptr && blockIdx.x == 0;
  for (int i = threadIdx.x; i < TT * slab_rows; i += RT_THREADS) {
    const int a = i / slab_rows, r = i % slab_rows;
    const bool in = t0 + a < T && r < rows;
    xs[i] = in ? bf16_to_f32(x[(size_t)(t0 + a) * H + h0 + r]) : 0.0f;
    if (cast && in) x16[(size_t)(t0 + a) * H + h0 + r] = (f16)xs[i];
  }
  __syncthreads();
  float acc[TT][8];
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int i = 0; i < 8; i++) acc[a][i] = 0.0f;
  if (active) {
    for (int r0 = RPW * wv + rr; r0 < rows; r0 += RT_BATCH * RPS) {
      if (r0 != RPW * wv + rr) load_batch(r0);
#pragma unroll
      for (int b = 0; b < RT_BATCH; b++) {
        const int r = r0 + b * RPS;
        if (r < rows) {
          float wf[8];
          wf[0] = __uint_as_float(w8[b].x << 16); wf[1] = __uint_as_float(w8[b].x & 0xFFFF0000u);
          wf[2] = __uint_as_float(w8[b].y << 16); wf[3] = __uint_as_float(w8[b].y & 0xFFFF0000u);
          wf[4] = __uint_as_float(w8[b].z << 16); wf[5] = __uint_as_float(w8[b].z & 0xFFFF0000u);
          wf[6] = __uint_as_float(w8[b].w << 16); wf[7] = __uint_as_float(w8[b].w & 0xFFFF0000u);
#pragma unroll
          for (int a = 0; a < TT; a++) {
            const float xv = xs[a * slab_rows + r];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[a][i] = fmaf(xv, wf[i], acc[a][i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float v = acc[a][i];
#pragma unroll
      for (int o = CG; o < WAVE; o *= 2) v += __shfl_xor(v, o, WAVE);
      if (rr == 0) red[(wv * CG + cg) * (TT * 8) + a * 8 + i] = v;
    }
  __syncthreads();
  for (int q = threadIdx.x; q < CG * TT * 8; q += RT_THREADS) {
    const int g = q / (TT * 8), ai = q % (TT * 8), a = ai / 8, i = ai % 8;
    const int e = blockIdx.x * ET + g * 8 + i;
    if (e < E && t0 + a < T) {
      const float s = ((red[(0 * CG + g) * (TT * 8) + ai] + red[(1 * CG + g) * (TT * 8) + ai]) +
                       red[(2 * CG + g) * (TT * 8) + ai]) +
                      red[(3 * CG + g) * (TT * 8) + ai];
      part[((size_t)blockIdx.y * T + (t0 + a)) * E + e] = s;
    }
  }
}

// ---- router logits on bf16 matrix cores (T >= 32) --------------------------------
// v_mfma_f32_16x16x32_bf16 with A = 16 tokens x 32 k (x is K-contiguous) and
// B = 32 k x 16 experts.  W_r is stored [H][E] (experts contiguous), so each
// lane (c = l%16, g = l/16) loads rows k0+8g .. k0+8g+7 of experts
// e0+8c .. e0+8c+7 (eight 16-byte loads) and transposes them in registers
// into eight 8-element k-runs, one per expert: B fragment j of MFMA j holds
// expert e0 + 8*(l%16) + j, so eight MFMAs cover 128 experts.  One wavefront
// computes 64 tokens x 128 experts over one slab of K; slabs write partials
// [slab][T][E] that the top-k kernel adds in a fixed order.  bf16 products
// are exact in fp32.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int RM_TOKENS = 64;
constexpr int RM_EXPERTS = 128;

__global__ __launch_bounds__(WAVE) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          float* __restrict__ part, int T, int H, int E,
                                                          int kslab, f16* __restrict__ x16) {
  const int lane = threadIdx.x, c = lane % 16, g = lane / 16;
  const int e0 = blockIdx.x * RM_EXPERTS, t0 = blockIdx.y * RM_TOKENS;
  const int k_begin = blockIdx.z * kslab, k_end = min(H, k_begin + kslab);
  const int ec = e0 + 8 * c;  // this lane's 8 experts
  const bool e_ok = ec < E;
  const uint16_t* arow[4];
#pragma unroll
  for (int f = 0; f < 4; f++) arow[f] = x + (size_t)min(t0 + 16 * f + c, T - 1) * H;
  f32x4 acc[4][8];
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[f][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    uint4 rw[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      rw[i] = e_ok ? *reinterpret_cast<const uint4*>(wr + (size_t)(k0 + 8 * g + i) * E + ec) : make_uint4(0, 0, 0, 0);
    uint4 av[4];
#pragma unroll
    for (int f = 0; f < 4; f++) av[f] = *reinterpret_cast<const uint4*>(arow[f] + k0 + 8 * g);
    // the fp16 copy of x: each 32-k step of a (token tile, slab) is written
    // by one of its expert tiles, in turn
    if (x16 != nullptr && ((k0 - k_begin) / 32) % gridDim.x == blockIdx.x) {
#pragma unroll
      for (int f = 0; f < 4; f++)
        if (t0 + 16 * f + c < T) {
          const uint4 v = av[f];
          f16x8 o;
          o[0] = (f16)__uint_as_float(v.x << 16); o[1] = (f16)__uint_as_float(v.x & 0xFFFF0000u);
          o[2] = (f16)__uint_as_float(v.y << 16); o[3] = (f16)__uint_as_float(v.y & 0xFFFF0000u);
          o[4] = (f16)__uint_as_float(v.z << 16); o[5] = (f16)__uint_as_float(v.z & 0xFFFF0000u);
          o[6] = (f16)__uint_as_float(v.w << 16); o[7] = (f16)__uint_as_float(v.w & 0xFFFF0000u);
          *reinterpret_cast<f16x8*>(x16 + (size_t)(t0 + 16 * f + c) * H + k0 + 8 * g) = o;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      // column j: (w[0][j], ..., w[7][j]); w[i][j] is half j%2 of dword j/2 of row i
      uint32_t col[4];
#pragma unroll
      for (int p2 = 0; p2 < 4; p2++) {
        const uint32_t lo = (&rw[2 * p2].x)[j / 2], hi = (&rw[2 * p2 + 1].x)[j / 2];
        col[p2] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const bf16x8 bfrag = __builtin_bit_cast(bf16x8, make_uint4(col[0], col[1], col[2], col[3]));
#pragma unroll
      for (int f = 0; f < 4; f++)
        acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[f]), bfrag, acc[f][j], 0,
                                                            0, 0);
    }
  }
  // D[4g+i][c] of MFMA (f, j): token t0+16f+4g+i, expert e0+8c+j.
  if (!e_ok) return;
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int t = t0 + 16 * f + 4 * g + i;
      if (t < T) {
        float* dst = part + ((size_t)blockIdx.z * T + t) * E + ec;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[f][0][i], acc[f][1][i], acc[f][2][i], acc[f][3][i]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[f][4][i], acc[f][5][i], acc[f][6][i], acc[f][7][i]);
      }
    }
}

// ---- logits reduction + softmax + top-k ------------------------------------------
// A block takes one or more tokens.  All its threads first sum the slab
// partials of those tokens' logits (a fixed order), add the bias and store
// the logits; then wavefront w selects the top k of token w (wave_topk).
// Selection key: a 64-bit integer ordered as (logit descending, expert index
// ascending): the high word maps the fp32 logit to an order-preserving
// unsigned integer (-0 folded onto +0), the low word is ~index.  wave_topk
// filters the keys down to a few candidates and ranks them; its fallback
// (select_topk) sorts each lane's (up to) 16 keys and takes k rounds of the
// wavefront maximum of the lanes' heads, popping it from the winning lane.
constexpr int TOPK_KEYS = 16;  // E <= 1024

__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Wavefront maximum of an unsigned 32-bit value with DPP lane moves:
// quad_perm [1,0,3,2] and [2,3,0,1], row_ror 4 and 8 leave every lane of a
// row with the row maximum; row_bcast 15 and 31 carry it across rows, so
// lane 63 ends with the maximum of all 64 lanes.  Lanes without a source
// read 0, the identity of the maximum.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_move<0xb1>(v));
  v = max(v, dpp_move<0x4e>(v));
  v = max(v, dpp_move<0x124>(v));
  v = max(v, dpp_move<0x128>(v));
  v = max(v, dpp_move<0x142>(v));
  v = max(v, dpp_move<0x143>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Maximum 64-bit key: the high words first, then the low words among the
// lanes holding the high-word maximum.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}
// Wavefront sum in a fixed order with the same DPP moves (lanes without a
// source add 0): quads, then rows of 16, then across rows into lane 63,
// whose value is the result.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_float(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                               false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_float<0xb1>(v);
  v += dpp_float<0x4e>(v);
  v += dpp_float<0x124>(v);
  v += dpp_float<0x128>(v);
  v += dpp_float<0x142, 0xa>(v);
  v += dpp_float<0x143, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive scan over the 64 lanes with DPP lane moves: three row shifts
// (1, 2, 3) of the input give each lane the sum of its quad-aligned run of
// four; shifts by 4 and 8 (upper banks only) complete each row of 16; row
// broadcasts 15 and 31 carry the row totals into the rows above.  Lanes
// without a source add 0.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  int v = x + dpp_int<0x111>(x);
  v += dpp_int<0x112>(x);
  v += dpp_int<0x113>(x);
  v += dpp_int<0x114, 0xf, 0xe>(v);
  v += dpp_int<0x118, 0xf, 0xc>(v);
  v += dpp_int<0x142, 0xa, 0xf>(v);
  v += dpp_int<0x143, 0xc, 0xf>(v);
  return v;
}

__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Bitonic sort of 16 keys, descending.
__device__ __forceinline__ void sort16_desc(uint64_t (&k)[TOPK_KEYS]) {
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0)
            cas_desc(k[i], k[j]);
          else
            cas_desc(k[j], k[i]);
        }
      }
}

constexpr int TOPK_THREADS = 1024;

// One wavefront: the top k of E logits (LDS) and their renormalised softmax
// weights, written to ids[0..k) / w[0..k) (and ids_copy, if given).
// Returns lane j's id (j < k), -1 in the other lanes.
__device__ __forceinline__ int select_topk(const float* ls, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids_copy) {
  const int lane = threadIdx.x % WAVE;
  uint64_t key[TOPK_KEYS];
#pragma unroll
  for (int i = 0; i < TOPK_KEYS; i++) {
    const int e = lane + WAVE * i;
    key[i] = e < E ? (((uint64_t)float_order(ls[e]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
  }
  sort16_desc(key);
  int my_id = 0;
  float my_logit = 0.0f, top = 0.0f;
  for (int j = 0; j < k; j++) {
    const uint64_t best = wave_max_u64(key[0]);
    const int e = (int)~(uint32_t)best;
    const float l = order_float((uint32_t)(best >> 32));
    if (j == 0) top = l;
    if (lane == j) {
      my_id = e;
      my_logit = l;
    }
    const bool pop = key[0] == best;  // keys are unique: only the owner pops
#pragma unroll
    for (int i = 0; i < TOPK_KEYS - 1; i++) key[i] = pop ? key[i + 1] : key[i];
    key[TOPK_KEYS - 1] = pop ? 0ull : key[TOPK_KEYS - 1];
  }
  // w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0): the softmax restricted to
  // the selected logits, equal to the full softmax renormalised over them.
  const float ex = lane < k ? expf(my_logit - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = ex / sum;
    if (ids_copy) ids_copy[lane] = my_id;
  }
  return lane < k ? my_id : -1;
}

// ---- top-k of one token by one wavefront, by filtering ---------------------------
// Lane l owns the experts e = l + 64 i; hi(e) = float_order(logit e), and the
// full key is (hi << 32 | ~e).
//   1. m_l = the largest hi of lane l's experts (0 for a lane without any:
//      every finite logit maps above 0);
//   2. tau = the k-th largest of the 64 lane maxima, found as the smallest
//      maximum that fewer than k maxima exceed.  At least k lanes hold a key
//      with hi >= tau, so at least k keys have hi >= tau, and since a larger
//      hi means a larger key, every key of the top k has hi >= tau;
//   3. the keys with hi >= tau (the candidates, a few more than k for
//      ordinary logits) are gathered in LDS: each lane counts its own, a
//      wavefront prefix sum of the counts gives each lane its first slot,
//      and every key is written, a non-candidate to a spare slot of its lane
//      (no branch);
//   4. a candidate's rank is the number of larger candidates (keys are
//      unique: the index is part of the key).
// Winners are placed at lane = rank and weighted as in select_topk, so the
// results are the same bit for bit.  More than 64 candidates (heavy ties)
// fall back to select_topk.  No block barrier is involved: the lanes of a
// wavefront exchange values through LDS, whose operations complete in issue
// order for one wavefront.  The reads of the 64 maxima and of the
// candidates go eight at a time, with one wait.
struct WaveTopkLds {
  uint64_t cand[2 * WAVE];  // slots 0..63 candidates, 64 + l lane l's spare
  uint32_t m[WAVE];
  float out_l[WAVE];
  int out_e[WAVE];
};

// Keeps the compiler from moving this wavefront's LDS accesses across.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }
// Eight 16-byte LDS reads of p[0..128) issued back to back, and one wait
// for all of them in the same block (the compiler would otherwise issue two
// at a time, waiting between).
typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_read8(const void* p, u32x4n (&q)[8]) {
  const uint32_t a = (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:16\n\t"
      "ds_read_b128 %2, %8 offset:32\n\t"
      "ds_read_b128 %3, %8 offset:48\n\t"
      "ds_read_b128 %4, %8 offset:64\n\t"
      "ds_read_b128 %5, %8 offset:80\n\t"
      "ds_read_b128 %6, %8 offset:96\n\t"
      "ds_read_b128 %7, %8 offset:112\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]), "=&v"(q[7])
      : "v"(a)
      : "memory");
}

// Returns lane j's id (j < k), -1 in the other lanes.
__device__ __forceinline__ int wave_topk(const float* ls, int E, int k, int32_t* __restrict__ ids,
                                         float* __restrict__ w, int32_t* ids_copy, WaveTopkLds& S) {
  const int lane = threadIdx.x % WAVE;
  const int n = (E + WAVE - 1) / WAVE;
  // ls holds 1024 entries: all reads are issued together, the ones past E
  // are discarded
  float lv[TOPK_KEYS];
#pragma unroll
  for (int i = 0; i < TOPK_KEYS; i++) lv[i] = ls[lane + WAVE * i];
  uint32_t hi[TOPK_KEYS];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < TOPK_KEYS; i++) {
    hi[i] = (i < n && lane + WAVE * i < E) ? float_order(lv[i]) : 0u;
    m = max(m, hi[i]);
  }
  S.m[lane] = m;
  wave_lds_order();
  int above = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    u32x4n q[8];
    lds_read8(&S.m[32 * h], q);
#pragma unroll
    for (int u = 0; u < 8; u++)
      above += (q[u][0] > m ? 1 : 0) + (q[u][1] > m ? 1 : 0) + (q[u][2] > m ? 1 : 0) + (q[u][3] > m ? 1 : 0);
  }
  // smallest maximum with fewer than k maxima above it (a max of inverted values)
  const uint32_t tau = ~wave_max_u32(above < k ? ~m : 0u);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < TOPK_KEYS; i++) cnt += (i < n && hi[i] >= tau) ? 1 : 0;
  const int incl = wave_inclusive_scan(cnt);
  const int total = __builtin_amdgcn_readlane(incl, WAVE - 1);
  if (total > WAVE) return select_topk(ls, E, k, ids, w, ids_copy);
  int slot = incl - cnt;
#pragma unroll
  for (int i = 0; i < TOPK_KEYS; i++) {
    const bool c = i < n && hi[i] >= tau;
    S.cand[c ? slot : WAVE + lane] = ((uint64_t)hi[i] << 32) | (uint32_t)~(uint32_t)(lane + WAVE * i);
    slot += c ? 1 : 0;
  }
  wave_lds_order();
  const uint64_t mine = lane < total ? S.cand[lane] : 0ull;
  int rank = 0;
  for (int j0 = 0; j0 < total; j0 += 16) {  // 16 keys (8 reads) at a time, all 64 slots in bounds
    u32x4n q[8];
    lds_read8(&S.cand[j0], q);
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const uint64_t a = ((uint64_t)q[u][1] << 32) | q[u][0], b = ((uint64_t)q[u][3] << 32) | q[u][2];
      rank += (j0 + 2 * u < total && a > mine ? 1 : 0) + (j0 + 2 * u + 1 < total && b > mine ? 1 : 0);
    }
  }
  if (lane < total && rank < k) {
    S.out_l[rank] = order_float((uint32_t)(mine >> 32));
    S.out_e[rank] = (int)~(uint32_t)mine;
  }
  wave_lds_order();
  const float l = lane < k ? S.out_l[lane] : 0.0f;
  const float top = S.out_l[0];
  const int e = lane < k ? S.out_e[lane] : -1;
  const float ex = lane < k ? expf(l - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[lane] = e;
    w[lane] = ex / sum;
    if (ids_copy) ids_copy[lane] = e;
  }
  return e;
}

// Logits of the consecutive tokens row0 .. row0+nrows-1 (a contiguous run of
// [T][E]) into LDS rows of 1024 (and out to `logits`): each thread takes
// float4 pieces u = 0..U-1 (a block-stride apart) and issues the loads of
// ZB slabs for all of them before adding; slabs are added in ascending
// order.  With part == NULL the logits are an input.
template <int U, int ZB>
__device__ __forceinline__ void logits_rows(const float* __restrict__ part, int slabs, size_t slab_stride,
                                            const float* __restrict__ bias, float* __restrict__ logits, float* ls,
                                            int row0, int nrows, int E) {
  const int n4 = nrows * E / 4;  // E % 8 == 0
  const size_t base = (size_t)row0 * E;
  for (int q0 = threadIdx.x; q0 < n4; q0 += U * blockDim.x) {
    float4 acc[U];
#pragma unroll
    for (int u = 0; u < U; u++) acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (part) {
      for (int z0 = 0; z0 < slabs; z0 += ZB) {
        float4 b[U][ZB];
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
          for (int z = 0; z < ZB; z++) {
            const int q = q0 + u * blockDim.x;
            b[u][z] = (q < n4 && z0 + z < slabs)
                          ? *reinterpret_cast<const float4*>(part + (size_t)(z0 + z) * slab_stride + base + 4 * q)
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
          for (int z = 0; z < ZB; z++)
            if (z0 + z < slabs) {
              acc[u].x += b[u][z].x;
              acc[u].y += b[u][z].y;
              acc[u].z += b[u][z].z;
              acc[u].w += b[u][z].w;
            }
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int q = q0 + u * blockDim.x;
      if (q >= n4) continue;
      const int a = 4 * q / E, e = 4 * q % E;
      float4 v = acc[u];
      if (part) {
        if (bias) {
          const float4 bb = *reinterpret_cast<const float4*>(bias + e);
          v.x += bb.x;
          v.y += bb.y;
          v.z += bb.z;
          v.w += bb.w;
        }
        *reinterpret_cast<float4*>(logits + base + 4 * q) = v;
      } else {
        v = *reinterpret_cast<const float4*>(logits + base + 4 * q);  // logits given by the caller
      }
      *reinterpret_cast<float4*>(ls + a * 1024 + e) = v;
    }
  }
}

// Logits of the first `nrows` rows of [T][E] (rows row0 ..) into LDS rows of
// 1024, for a block of 1024 threads: thread (g, q) = (tid / 256, tid % 256)
// adds slab group g (a quarter of the slabs, at most eight, their loads
// issued together) for float4 piece q; the four group sums meet in LDS
// (gsum, 256 float4) and are added in group order.  One round of loads for
// up to 256 pieces (one token at E = 1024) and 32 slabs.
__device__ __forceinline__ void logits_rows_grouped(const float* __restrict__ part, int slabs, size_t slab_stride,
                                                    const float* __restrict__ bias, float* __restrict__ logits,
                                                    float* ls, int row0, int nrows, int E, float4* gsum,
                                                    bool store_logits = true) {
  const int n4 = nrows * E / 4;  // E % 8 == 0
  const size_t base = (size_t)row0 * E;
  const int g = threadIdx.x / 256, ql = threadIdx.x % 256;
  const int zper = (slabs + 3) / 4;  // <= ROUTER_MAX_SLABS / 4
  for (int q0 = 0; q0 < n4; q0 += 256) {
    const int q = q0 + ql;
    if (part) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (q < n4) {
        float4 b[ROUTER_MAX_SLABS / 4];
#pragma unroll
        for (int z = 0; z < ROUTER_MAX_SLABS / 4; z++) {
          const int zz = g * zper + z;
          b[z] = (z < zper && zz < slabs) ? *reinterpret_cast<const float4*>(part + (size_t)zz * slab_stride + base + 4 * q)
                                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int z = 0; z < ROUTER_MAX_SLABS / 4; z++)
          if (z < zper && g * zper + z < slabs) {
            acc.x += b[z].x;
            acc.y += b[z].y;
            acc.z += b[z].z;
            acc.w += b[z].w;
          }
      }
      gsum[threadIdx.x] = acc;
      __syncthreads();
      if (g == 0 && q < n4) {
        float4 v = gsum[ql];
#pragma unroll
        for (int h = 1; h < 4; h++) {
          const float4 o = gsum[h * 256 + ql];
          v.x += o.x;
          v.y += o.y;
          v.z += o.z;
          v.w += o.w;
        }
        const int e = 4 * q % E;
        if (bias) {
          const float4 bb = *reinterpret_cast<const float4*>(bias + e);
          v.x += bb.x;
          v.y += bb.y;
          v.z += bb.z;
          v.w += bb.w;
        }
        if (store_logits) *reinterpret_cast<float4*>(logits + base + 4 * q) = v;
        *reinterpret_cast<float4*>(ls + (4 * q / E) * 1024 + e) = v;
      }
      __syncthreads();
    } else if (g == 0 && q < n4) {  // logits given by the caller
      const int e = 4 * q % E;
      *reinterpret_cast<float4*>(ls + (4 * q / E) * 1024 + e) = *reinterpret_cast<const float4*>(logits + base + 4 * q);
    }
  }
}

template <int TB>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const float* __restrict__ part, int slabs,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T, int E, int k,
                                                           int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ __attribute__((aligned(16))) float ls[TB * 1024];
  __shared__ __attribute__((aligned(16))) WaveTopkLds tk[TB];
  const int t0 = blockIdx.x * TB;
  // Phase 1: logits of this block's tokens (slab partials added in ascending
  // slab order, or the caller's logits), with many loads in flight: four
  // pieces of four slabs when there are few slabs, else sixteen slabs.
  const int nrows = min(TB, T - t0);
  if (slabs <= 4)
    logits_rows<4, 4>(part, slabs, (size_t)T * E, bias, logits, ls, t0, nrows, E);
  else
    logits_rows<1, 16>(part, slabs, (size_t)T * E, bias, logits, ls, t0, nrows, E);
  __syncthreads();
  // Phase 2: wavefront w selects for token t0 + w.
  const int wv = threadIdx.x / WAVE;
  const int t = t0 + wv;
  if (wv >= TB || t >= T) return;
  wave_topk(ls + wv * 1024, E, k, ids + (size_t)t * k, wout + (size_t)t * k, nullptr, tk[wv]);
}

// ---- permutation ---------------------------------------------------------------
// For a block of up to 64 tokens and expert e, mask[e] has bit l set when
// token 64b+l selected e.  The records of expert e are ordered by token, so
// record (t, j) goes to offsets[e] + (records of e in earlier blocks) +
// popcount of the mask bits below l.  Integer work only: exact and
// deterministic.
constexpr int PERM_MAX_E = 1024;

// Block-wide exclusive scan of one int per thread (blockDim.x = 1024, lds
// 16-byte aligned).
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds /*[16]*/, int* total) {
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int incl = wave_inclusive_scan(v);
  if (lane == WAVE - 1) lds[wv] = incl;
  __syncthreads();
  int4 q[4];
#pragma unroll
  for (int u = 0; u < 4; u++) q[u] = reinterpret_cast<const int4*>(lds)[u];
  int base = 0, all = 0;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int t[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
    for (int r = 0; r < 4; r++) {
      base += 4 * u + r < wv ? t[r] : 0;
      all += t[r];
    }
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

// One token per block: the logits (grouped slab sums), then wave_topk by
// wavefront 0.
__global__ __launch_bounds__(TOPK_THREADS) void topk_block_kernel(const float* __restrict__ part, int slabs,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ logits, int T, int E, int k,
                                                                 int32_t* __restrict__ ids,
                                                                 float* __restrict__ wout) {
  __shared__ __attribute__((aligned(16))) float ls[1024];
  __shared__ __attribute__((aligned(16))) WaveTopkLds tk;
  __shared__ float4 gsum[1024];
  const int t = blockIdx.x;
  logits_rows_grouped(part, slabs, (size_t)T * E, bias, logits, ls, t, 1, E, gsum);
  __syncthreads();
  if (threadIdx.x < WAVE) wave_topk(ls, E, k, ids + (size_t)t * k, wout + (size_t)t * k, nullptr, tk);
}

__device__ __forceinline__ void cast_rows(const uint16_t* __restrict__ x, f16* __restrict__ x16, size_t first8,
                                         size_t n8, int tid, int nthreads) {
  for (size_t i = first8 + tid; i < first8 + n8; i += nthreads) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    f16x8 o;
    o[0] = (f16)__uint_as_float(v.x << 16); o[1] = (f16)__uint_as_float(v.x & 0xFFFF0000u);
    o[2] = (f16)__uint_as_float(v.y << 16); o[3] = (f16)__uint_as_float(v.y & 0xFFFF0000u);
    o[4] = (f16)__uint_as_float(v.z << 16); o[5] = (f16)__uint_as_float(v.z & 0xFFFF0000u);
    o[6] = (f16)__uint_as_float(v.w << 16); o[7] = (f16)__uint_as_float(v.w & 0xFFFF0000u);
    reinterpret_cast<f16x8*>(x16)[i] = o;
  }
}

// A record is served here when its expert id lies in [0, E); any other id
// (by convention -1: an expert another device serves) is masked, takes no
// position and is not counted.
__device__ __forceinline__ bool served_id(int e, int E) { return (unsigned)e < (unsigned)E; }

// The permutation of up to 64 * NWD tokens in one block of 1024 threads
// (thread e = expert e for the counts): m holds NWD 64-bit token masks per
// expert ([E][NWD], word w bit l = token 64w + l selected e) and off_s E
// ints, LDS arrays with m zeroed by the caller before a barrier.  A
// record's position is its expert's offset plus the bits set in the words
// before its own and below it in its own.  Also writes the active-expert
// list.
template <int NWD>
__device__ __forceinline__ void permute_block(const int32_t* ids, int T, int E, int k, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                              int32_t* __restrict__ active, int32_t* __restrict__ n_active, unsigned long long* m,
                              int* off_s, int* lds) {
  const int tid = threadIdx.x;
  for (int f = tid; f < T * k; f += 1024) {
    const int e = ids[f], t = f / k;
    if (served_id(e, E)) atomicOr(&m[e * NWD + t / 64], 1ull << (t % 64));
  }
  __syncthreads();
  int cnt = 0;
  if (tid < E)
#pragma unroll
    for (int w = 0; w < NWD; w++) cnt += __popcll(m[tid * NWD + w]);
  // offsets (< T k <= 64 NWD * 64 <= 2^16) and active slots (< E <= 1024) in one scan
  int packed_total;
  const int packed = block_exclusive_scan(cnt + (cnt > 0 ? 1 << 16 : 0), lds, &packed_total);
  const int off = packed & 0xFFFF, slot = packed >> 16, nact = packed_total >> 16;
  if (tid < E) {
    off_s[tid] = off;
    offsets[tid] = off;
    if (cnt > 0) active[slot] = tid;
  }
  if (tid == 0) {
    offsets[E] = packed_total & 0xFFFF;  // the served records (T k when none is masked)
    *n_active = nact;
  }
  __syncthreads();
  for (int f = tid; f < T * k; f += 1024) {
    const int t = f / k, e = ids[f];
    if (!served_id(e, E)) {
      pair_pos[f] = -1;
      continue;
    }
    const int w = t / 64;
    int pos = off_s[e] + __popcll(m[e * NWD + w] & ((1ull << (t % 64)) - 1ull));
#pragma unroll
    for (int w2 = 0; w2 < NWD - 1; w2++)
      if (w2 < w) pos += __popcll(m[e * NWD + w2]);
    sorted_pairs[pos] = f;
    pair_pos[f] = pos;
  }
}

// T <= 64 * NWD: the whole permutation and the active-expert list, in one
// block of 1024 threads.
template <int NWD>
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_pairs,
                                                         int32_t* __restrict__ pair_pos,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ n_active) {
  __shared__ unsigned long long m[PERM_MAX_E * NWD];
  __shared__ int off_s[PERM_MAX_E];
  __shared__ __attribute__((aligned(16))) int lds[16];
  for (int i = threadIdx.x; i < E * NWD; i += 1024) m[i] = 0ull;
  __syncthreads();
  permute_block<NWD>(ids, T, E, k, offsets, sorted_pairs, pair_pos, active, n_active, m, off_s, lds);
}
// Largest batch of the single-block permutation (four mask words per expert).
constexpr int PERM_ONE_BLOCK_T = 256;

// T <= ROUTE_SMALL_T: the whole routing in one block of 1024 threads (one
// launch instead of three): logits from the slab partials (or the caller's
// logits), top-k and weights (wave_topk, wavefront t for token t), then the
// permutation and the active-expert list.  The logits reach memory from
// wavefronts that select nothing (wavefront 0 never waits on those stores).
// One token: its k experts are distinct, so a record's sorted position is
// the number of selected ids below its own, and offsets[e] the number below
// e; wavefront 0 places the records right after selecting them, and a
// single barrier later every thread writes its experts' offsets.
constexpr int ROUTE_SMALL_T = 8;

__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ part, int slabs,
                                                          const float* __restrict__ bias, float* __restrict__ logits,
                                                          int T, int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ wout, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_pos,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active) {
  __shared__ __attribute__((aligned(16))) float ls[ROUTE_SMALL_T * PERM_MAX_E];
  __shared__ __attribute__((aligned(16))) int ids_s[ROUTE_SMALL_T * 64];
  __shared__ unsigned long long m[PERM_MAX_E];
  __shared__ int off_s[PERM_MAX_E];
  __shared__ __attribute__((aligned(16))) int lds[16];
  __shared__ __attribute__((aligned(16))) WaveTopkLds tk[ROUTE_SMALL_T];
  __shared__ float4 gsum[1024];
  const int tid = threadIdx.x;
  if (T > 1 && tid < E) m[tid] = 0ull;
  logits_rows_grouped(part, slabs, (size_t)T * E, bias, logits, ls, 0, T, E, gsum, false);
  __syncthreads();
  const int wv = tid / WAVE, lane = tid % WAVE;
  if (part && wv >= ROUTE_SMALL_T)  // the logits out to memory (E % 8 == 0)
    for (int q = tid - ROUTE_SMALL_T * WAVE; q < T * E / 4; q += 1024 - ROUTE_SMALL_T * WAVE)
      reinterpret_cast<float4*>(logits)[q] = *reinterpret_cast<const float4*>(ls + (4 * q / E) * PERM_MAX_E + 4 * q % E);
  if (T == 1) {
    if (wv == 0) {
      const int e = wave_topk(ls, E, k, ids, wout, ids_s, tk[0]);
      wave_lds_order();
      int pos = 0;
      for (int j0 = 0; j0 < k; j0 += 4) {  // ids_s holds 64 entries: reads past k are discarded
        const int4 v = *reinterpret_cast<const int4*>(ids_s + j0);
        pos += (v.x < e ? 1 : 0) + (j0 + 1 < k && v.y < e ? 1 : 0) + (j0 + 2 < k && v.z < e ? 1 : 0) +
               (j0 + 3 < k && v.w < e ? 1 : 0);
      }
      if (lane < k) {
        sorted_pairs[pos] = lane;
        pair_pos[lane] = pos;
        active[pos] = e;
      }
      if (lane == 0) {
        *n_active = k;
        offsets[E] = k;
      }
    }
    __syncthreads();
    if (tid < E) {
      int below = 0;
      for (int j0 = 0; j0 < k; j0 += 4) {
        const int4 v = *reinterpret_cast<const int4*>(ids_s + j0);
        below += (v.x < tid ? 1 : 0) + (j0 + 1 < k && v.y < tid ? 1 : 0) + (j0 + 2 < k && v.z < tid ? 1 : 0) +
                 (j0 + 3 < k && v.w < tid ? 1 : 0);
      }
      offsets[tid] = below;
    }
    return;
  }
  if (wv < T)
    wave_topk(ls + wv * PERM_MAX_E, E, k, ids + (size_t)wv * k, wout + (size_t)wv * k, ids_s + wv * k, tk[wv]);
  __syncthreads();
  permute_block<1>(ids_s, T, E, k, offsets, sorted_pairs, pair_pos, active, n_active, m, off_s, lds);
}

__global__ __launch_bounds__(WAVE) void perm_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         uint64_t* __restrict__ masks, int32_t* __restrict__ counts) {
  __shared__ unsigned long long m[PERM_MAX_E];
  const int lane = threadIdx.x, b = blockIdx.x;
  for (int e = lane; e < E; e += WAVE) m[e] = 0ull;
  __syncthreads();
  const int t = b * WAVE + lane;
  if (t < T)
    for (int j = 0; j < k; j++) {
      const int e = ids[(size_t)t * k + j];
      if (served_id(e, E)) atomicOr(&m[e], 1ull << lane);
    }
  __syncthreads();
  for (int e = lane; e < E; e += WAVE) {
    masks[(size_t)b * E + e] = m[e];
    counts[(size_t)b * E + e] = __popcll(m[e]);
  }
}

// One block of 1024 threads, thread e = expert: per-block counts become
// absolute bases; writes offsets and the list of experts with work.
// Entries (expert, token tile) for the large-batch GEMMs: expert e with c
// records has ceil(c / MTILE) entries e * 65536 + tile, in expert order.
__device__ __forceinline__ void write_mtiles(int e, int cnt, int* lds, int32_t* __restrict__ mtiles,
                             int32_t* __restrict__ n_mtiles) {
  const int nt = (cnt + MTILE - 1) / MTILE;
  int total;
  const int first = block_exclusive_scan(nt, lds, &total);
  for (int m = 0; m < nt; m++) mtiles[first + m] = e * 65536 + m;
  if (threadIdx.x == 0) *n_mtiles = total;
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ counts, int nblocks, int E,
                                                        int P, int32_t* __restrict__ base,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                                        int32_t* __restrict__ n_active, int32_t* __restrict__ mtiles,
                                                        int32_t* __restrict__ n_mtiles) {
  __shared__ __attribute__((aligned(16))) int lds[16];
  const int e = threadIdx.x;
  int running = 0;
  if (e < E)
    for (int b0 = 0; b0 < nblocks; b0 += 16) {  // 16 loads in flight
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; u++) c[u] = b0 + u < nblocks ? counts[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; u++)
        if (b0 + u < nblocks) {
          base[(size_t)(b0 + u) * E + e] = running;
          running += c[u];
        }
    }
  int total;
  const int off = block_exclusive_scan(e < E ? running : 0, lds, &total);
  const int flag = (e < E && running > 0) ? 1 : 0;
  int nact;
  const int slot = block_exclusive_scan(flag, lds, &nact);
  if (e < E) {
    offsets[e] = off;
    if (flag) active[slot] = e;
  }
  if (e == 0) {
    offsets[E] = total;  // the served records (P when none is masked)
    *n_active = nact;
  }
  write_mtiles(e, e < E ? running : 0, lds, mtiles, n_mtiles);
}

__global__ __launch_bounds__(WAVE) void perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                          const uint64_t* __restrict__ masks,
                                                          const int32_t* __restrict__ base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_pos) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int t = b * WAVE + lane;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < k; j0 += 16) {  // 16 records' loads in flight
    int e[16];
    bool in[16];
#pragma unroll
    for (int u = 0; u < 16; u++) {
      e[u] = j0 + u < k ? ids[(size_t)t * k + j0 + u] : 0;
      in[u] = served_id(e[u], E);
      if (!in[u]) e[u] = 0;  // (masked: no lookups of its own)
    }
    int pos[16];
#pragma unroll
    for (int u = 0; u < 16; u++)
      pos[u] = offsets[e[u]] + base[(size_t)b * E + e[u]] + __popcll(masks[(size_t)b * E + e[u]] & below);
#pragma unroll
    for (int u = 0; u < 16; u++)
      if (j0 + u < k) {
        const int f = t * k + j0 + u;
        if (in[u]) sorted_pairs[pos[u]] = f;
        pair_pos[f] = in[u] ? pos[u] : -1;
      }
  }
}

// Experts in [lo, hi) with work and their (expert, token tile) entries,
// from offsets alone (when the permutation comes from the caller, or when
// only one share of the experts runs here).
__global__ __launch_bounds__(1024) void active_list_kernel(const int32_t* __restrict__ offsets, int E, int lo, int hi,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active,
                                                          int32_t* __restrict__ mtiles,
                                                          int32_t* __restrict__ n_mtiles) {
  __shared__ __attribute__((aligned(16))) int lds[16];
  const int e = threadIdx.x;
  const int cnt = (e < E && e >= lo && e < hi) ? offsets[e + 1] - offsets[e] : 0;
  const int flag = cnt > 0 ? 1 : 0;
  int nact;
  const int slot = block_exclusive_scan(flag, lds, &nact);
  if (flag) active[slot] = e;
  if (e == 0) *n_active = nact;
  write_mtiles(e, cnt, lds, mtiles, n_mtiles);
}

__global__ __launch_bounds__(256) void cast_kernel(const uint16_t* __restrict__ x, f16* __restrict__ x16,
                                                  long long n8) {
  const size_t per = 256 * 8;
  const size_t first = (size_t)blockIdx.x * per;
  if (first < (size_t)n8) cast_rows(x, x16, first, min((size_t)n8 - first, per), threadIdx.x, 256);
}

// local[f] = map[ids[f]]: the router's global expert ids as slots of this
// device's store, -1 where the map says the expert is served elsewhere (a
// map entry outside [0, n_local) counts as -1).
__global__ __launch_bounds__(256) void remap_ids_kernel(const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ map, int E, int n_local,
                                                       long long n, int32_t* __restrict__ local) {
  const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
  if (f >= n) return;
  const int e = ids[f];
  const int l = served_id(e, E) ? map[e] : -1;
  local[f] = served_id(l, n_local) ? l : -1;
}

int router_tt(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8)); }
constexpr int ROUTER_MFMA_MIN_T = 32;

}  // namespace

RouterPlan router_plan(int T, int H, int E) {
  RouterPlan p;
  p.tiled = false;
  p.e_tile = RT_E_TILE;
  {
    const DensePlan d = dense_plan(T, H, E);
    if (d.tiled) {
      p.mfma = true;
      p.tiled = true;
      p.slabs = d.slabs;
      p.slab_rows = d.kslab;
      return p;
    }
  }
  if (T >= ROUTER_MFMA_MIN_T) {
    // one wavefront per (128 experts, 64 tokens, K slab); aim for >= 2048
    // (eight per CU)
    const int tiles = ((E + RM_EXPERTS - 1) / RM_EXPERTS) * ((T + RM_TOKENS - 1) / RM_TOKENS);
    int s = (2048 + tiles - 1) / tiles;
    if (s > ROUTER_MAX_SLABS) s = ROUTER_MAX_SLABS;
    const int steps = H / 32;
    if (s > steps) s = steps;
    if (s < 1) s = 1;
    const int steps_per_slab = (steps + s - 1) / s;
    p.mfma = true;
    p.slab_rows = steps_per_slab * 32;
    p.slabs = (H + p.slab_rows - 1) / p.slab_rows;
    return p;
  }
  const int tt = router_tt(T);
  // wide tiles: blocks for up to 512 (in practice the 32-slab cap); narrow
  // tiles: up to 256 blocks, one round of loads each, about half the slabs
  const int et = E <= RT_NARROW_MAX_E ? RT_E_TILE_NARROW : RT_E_TILE, rps = rt_rows_per_step(et);
  const int tiles = ((E + et - 1) / et) * ((T + tt - 1) / tt);
  int s = (et == RT_E_TILE ? 512 : 256) / (tiles > 0 ? tiles : 1);  // (narrow: at most one block per CU)
  if (s > ROUTER_MAX_SLABS) s = ROUTER_MAX_SLABS;
  const int steps = H / rps;
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  int steps_per_slab = (steps + s - 1) / s;
  // the block's activations slab lives in LDS: at most 64 KB
  const int max_steps = 16384 / (tt * rps);
  if (steps_per_slab > max_steps) steps_per_slab = max_steps;
  p.mfma = false;
  p.e_tile = et;
  p.slab_rows = steps_per_slab * rps;
  p.slabs = (H + p.slab_rows - 1) / p.slab_rows;
  return p;
}

template <int ET>
hipError_t launch_gemv(const uint16_t* x, const uint16_t* wr, float* part, int T, int H, int E, const RouterPlan& rp,
                       hipStream_t s, f16* x16) {
  const int tt = router_tt(T);
  const dim3 grid((E + ET - 1) / ET, rp.slabs, (T + tt - 1) / tt);
  const size_t lds = sizeof(float) * ((size_t)tt * rp.slab_rows + 4 * (ET / 8) * tt * 8);
  switch (tt) {
    case 1: hipLaunchKernelGGL((router_gemv_kernel<1, ET>), grid, dim3(RT_THREADS), lds, s, x, wr, part, T, H, E, rp.slab_rows, x16); break;
    case 2: hipLaunchKernelGGL((router_gemv_kernel<2, ET>), grid, dim3(RT_THREADS), lds, s, x, wr, part, T, H, E, rp.slab_rows, x16); break;
    case 4: hipLaunchKernelGGL((router_gemv_kernel<4, ET>), grid, dim3(RT_THREADS), lds, s, x, wr, part, T, H, E, rp.slab_rows, x16); break;
    default: hipLaunchKernelGGL((router_gemv_kernel<8, ET>), grid, dim3(RT_THREADS), lds, s, x, wr, part, T, H, E, rp.slab_rows, x16); break;
  }
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, float* part, int T, int H, int E,
                         const RouterPlan& rp, hipStream_t s, f16* x16) {
  if (rp.tiled) {
    DensePlan dp;
    dp.tiled = true;
    dp.slabs = rp.slabs;
    dp.kslab = rp.slab_rows;
    return launch_dense_tiled(x, wr, T, H, E, dp, part, nullptr, nullptr, x16, s);
  }
  if (rp.mfma) {
    const dim3 grid((E + RM_EXPERTS - 1) / RM_EXPERTS, (T + RM_TOKENS - 1) / RM_TOKENS, rp.slabs);
    hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(WAVE), 0, s, x, wr, part, T, H, E, rp.slab_rows, x16);
    return hipGetLastError();
  }
  return rp.e_tile == RT_E_TILE_NARROW ? launch_gemv<RT_E_TILE_NARROW>(x, wr, part, T, H, E, rp, s, x16)
                                        : launch_gemv<RT_E_TILE>(x, wr, part, T, H, E, rp, s, x16);
}

hipError_t launch_topk(const float* part, int slabs, const float* bias, float* logits, int T, int E, int k,
                       int32_t* ids, float* w, hipStream_t s) {
  if (T <= 64)
    hipLaunchKernelGGL(topk_block_kernel, dim3(T), dim3(TOPK_THREADS), 0, s, part, slabs, bias, logits, T, E, k, ids,
                       w);
  else if (T < 2048)  // four tokens a block: at least 17 blocks
    hipLaunchKernelGGL((topk_kernel<4>), dim3((T + 3) / 4), dim3(TOPK_THREADS), 0, s, part, slabs, bias, logits, T,
                       E, k, ids, w);
  else  // sixteen: one per wavefront, at least 128 blocks
    hipLaunchKernelGGL((topk_kernel<16>), dim3((T + 15) / 16), dim3(TOPK_THREADS), 0, s, part, slabs, bias, logits, T,
                       E, k, ids, w);
  return hipGetLastError();
}

bool route_fused(int T) { return T <= ROUTE_SMALL_T; }

hipError_t launch_route_small(const float* part, int slabs, const float* bias, float* logits, int T, int E, int k,
                              int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                              int32_t* active, int32_t* n_active, hipStream_t s) {
  hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(1024), 0, s, part, slabs, bias, logits, T, E, k, ids, w,
                     offsets, sorted_pairs, pair_pos, active, n_active);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, uint64_t* masks, int32_t* counts, int32_t* base,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active,
                          int32_t* n_active, int32_t* mtiles, int32_t* n_mtiles, hipStream_t s) {
  if (T <= 64) {
    hipLaunchKernelGGL(perm_small_kernel<1>, dim3(1), dim3(1024), 0, s, ids, T, E, k, offsets, sorted_pairs, pair_pos,
                       active, n_active);
    return hipGetLastError();
  }
  if (T <= PERM_ONE_BLOCK_T) {  // (no token-tile list: it serves only the large-tile GEMMs, T >= 1024)
    hipLaunchKernelGGL(perm_small_kernel<PERM_ONE_BLOCK_T / 64>, dim3(1), dim3(1024), 0, s, ids, T, E, k, offsets,
                       sorted_pairs, pair_pos, active, n_active);
    return hipGetLastError();
  }
  const int nb = perm_blocks(T);
  hipLaunchKernelGGL(perm_count_kernel, dim3(nb), dim3(WAVE), 0, s, ids, T, E, k, masks, counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, counts, nb, E, T * k, base, offsets, active,
                     n_active, mtiles, n_mtiles);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(WAVE), 0, s, ids, T, E, k, masks, base, offsets,
                     sorted_pairs, pair_pos);
  return hipGetLastError();
}

hipError_t launch_active_list(const int32_t* offsets, int E, int lo, int hi, int32_t* active, int32_t* n_active,
                              int32_t* mtiles, int32_t* n_mtiles, hipStream_t s) {
  hipLaunchKernelGGL(active_list_kernel, dim3(1), dim3(1024), 0, s, offsets, E, lo, hi, active, n_active, mtiles,
                     n_mtiles);
  return hipGetLastError();
}

hipError_t launch_remap_ids(const int32_t* ids, const int32_t* map, int E, int n_local, long long n, int32_t* local,
                            hipStream_t s) {
  const long long g = (n + 255) / 256;
  hipLaunchKernelGGL(remap_ids_kernel, dim3((unsigned)(g > 0 ? g : 1)), dim3(256), 0, s, ids, map, E, n_local, n,
                     local);
  return hipGetLastError();
}

hipError_t launch_cast(const uint16_t* x, f16* x16, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  const long long g = (n8 + 2047) / 2048;
  hipLaunchKernelGGL(cast_kernel, dim3((unsigned)(g > 0 ? g : 1)), dim3(256), 0, s, x, x16, n8);
  return hipGetLastError();
}

}  // namespace moe
