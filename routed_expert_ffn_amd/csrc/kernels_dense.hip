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
// of the router weight.  Small batches: the router's GEMV or its one-wave
// bf16 matrix-core GEMM compute K-slab partial sums in fp32, and one more
// kernel adds the slabs in a fixed order and rounds to bf16 (and, for the
// latent that feeds the experts, also writes its exact fp16 copy).  Large
// batches (and the router itself there): the LDS-tiled GEMM below, which
// writes the rounded output directly when one K slab fills the chip.
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


// ---- LDS-tiled bf16 GEMM of large batches ----------------------------------------
// A block computes a tile of DT_M tokens x DT_N output columns over one K
// slab.  Each 64-k chunk of both operands reaches LDS by LDS DMA into one of
// two stages, two chunks ahead (the software pipeline is described at the K
// loop):
//   tokens: 128 bytes (64 k) of each of the tile's rows of x, a row being 8
//           pieces of 16 bytes, piece q of row r in slot q ^ ((r/2) % 8), so
//           that the 16 rows one fragment read touches cover all banks;
//   weights: the chunk's 64 rows of W [K][N] as stored, DT_N columns each
//           (448 bytes a row).  The matrix cores want 8 consecutive k of one
//           column per lane: ds_read_b64_tr_b16 gives them, since among 16
//           lanes, lane 4r + c passing the address of row k0 + r, columns
//           n0 + 4c .. n0 + 4c + 3 hands lane i the values of rows
//           k0 .. k0 + 3 in column n0 + i; two such reads make a fragment.
//           So W is never transposed in memory.  LDS serves such reads 32
//           lanes at a time, and lanes 16 apart read rows 8 apart, which
//           fall on the same banks (a row is 112 dwords): rows r with
//           (r/8) odd hold their two 112-column halves swapped, which puts
//           those rows' reads on the other half of the banks.
//
// Eight wavefronts, 4 (tokens, 64 each) x 2 (columns, 112 each); wavefront
// products are v_mfma_f32_16x16x32_bf16 with the weight columns as the A
// operand and the tokens as B, so a lane's four accumulators are four
// consecutive output columns of one token.  Inside a chunk, step s (32 k) of
// lane group g = lane/16 covers k = 32s + 8g .. + 7 of both operands.
//
// Tiles: DT_N = 224 divides the widths of a K3-shaped layer (896 router
// columns, 3584 latent, 7168 hidden), and a prefill chunk of 8192 tokens
// fills whole waves of 256 blocks.  Items are laid out (slab, column group,
// token tile, column tile in group) and dealt to the eight XCDs in
// contiguous runs, so the 32 blocks an XCD runs at once share a few token
// tiles and a group of column tiles in its L2.
constexpr int DT_M = 256;
constexpr int DT_N = 224;
constexpr int DT_KC = 64;
constexpr int DT_WAVES = 8;
constexpr int DT_ROWB = DT_KC * 2;                 // bytes of a row's chunk
constexpr int DT_X_BYTES = DT_M * DT_ROWB;         // token rows of one chunk
constexpr int DT_W_ROWB = DT_N * 2;                // bytes of a weight row (k) of one chunk
constexpr int DT_W_BYTES = DT_KC * DT_W_ROWB;      // weight rows of one chunk
constexpr int DT_STAGE = DT_X_BYTES + DT_W_BYTES;
constexpr int DT_LDS = 2 * DT_STAGE;
constexpr int DT_X_INSTR = DT_M / 8;  // DMA instructions (8 rows each) per chunk
constexpr int DT_W_INSTR = DT_W_BYTES / 1024;
constexpr int DT_MIN_T = 1024;
constexpr int DT_MAX_SLABS = 16;
static_assert(DT_LDS <= 160 * 1024, "LDS budget of one CU");
static_assert(DT_W_BYTES % 1024 == 0 && DT_W_ROWB % 16 == 0, "weight chunk of whole DMA instructions and pieces");
static_assert(DT_X_INSTR == 4 * DT_WAVES && DT_W_INSTR <= 4 * DT_WAVES, "DMA instructions per wavefront");
static_assert(DT_N == 2 * 112 && DT_W_ROWB % 32 == 0, "two column halves of 112, swapped as whole 16-byte pieces");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct DenseParams {
  const unsigned char* x;   // [T][K] bf16
  const unsigned char* w;   // [K][N] bf16
  float* part;              // [slabs][T][N] fp32, or NULL
  uint16_t* out;            // [T][N] bf16 (one slab, part NULL)
  f16* out16;               // fp16 copy of out, or NULL
  f16* x16;                 // fp16 copy of x, or NULL
  int T, K, N, kslab;
  int n_tt, n_ct, cg, n_items;
};

__device__ __forceinline__ uint32_t dt_lds_addr(const unsigned char* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// LDS DMA of 16 bytes per lane from gbase + voff to LDS address lds + 16 *
// lane.  Written as an instruction of our own, so the compiler does not count
// it as outstanding LDS work (it would wait for it before every fragment
// read); the only wait for it is the vmcnt(0) of dt_barrier.
__device__ __forceinline__ void dt_dma16(const unsigned char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// All of this wavefront's vector-memory work (its DMA copies included) and
// LDS reads are complete, then the block meets.  Builtins rather than inline
// asm, so the compiler's own wait counting knows that every earlier LDS read
// has landed (after an opaque asm wait it re-waits for them later, behind
// newer reads).  The callers fence it with scheduling barriers.
__device__ __forceinline__ void dt_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__global__ __launch_bounds__(DT_WAVES * WAVE, 1) void dense_tile_kernel(DenseParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dt_smem[];
  const int per_xcd = (p.n_items + 7) / 8;
  const int slot = blockIdx.x / 8, item = (blockIdx.x % 8) * per_xcd + slot;
  if (slot >= per_xcd || item >= p.n_items) return;
  int r = item / p.cg;
  const int ci = item % p.cg;
  const int tt = r % p.n_tt;
  r /= p.n_tt;
  const int n_grp = p.n_ct / p.cg;
  const int ct = (r % n_grp) * p.cg + ci, slab = r / n_grp;
  const int t0 = tt * DT_M, n0 = ct * DT_N;
  const int k_begin = slab * p.kslab;
  const int nchunks = (min(p.K, k_begin + p.kslab) - k_begin) / DT_KC;

  const int lane = threadIdx.x % WAVE, w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const size_t row_bytes = (size_t)p.K * 2;
  // DMA: instruction i of wavefront w is i = w + 8m.  Tokens: rows 8i ..
  // 8i+7, lane l copying row 8i + l/8, piece (l%8) ^ ((row/2)%8) into slot
  // l%8 (rows past T repeat the last one).  Weights: bytes 1024i .. of the
  // [64][DT_N] chunk, lane l the 16 bytes at 1024i + 16l (columns past N
  // repeat the last eight).
  const unsigned char* xb = p.x + (size_t)t0 * row_bytes + 2 * (size_t)k_begin;
  const size_t wrow_bytes = (size_t)p.N * 2;
  const unsigned char* wb = p.w + (size_t)k_begin * wrow_bytes + 2 * (size_t)n0;
  uint32_t xoff[4], woff[4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const int row = 8 * (w + 8 * m) + lane / 8;
    const uint32_t piece = (uint32_t)((lane % 8) ^ ((row / 2) % 8));
    xoff[m] = (uint32_t)(min(t0 + row, p.T - 1) - t0) * (uint32_t)row_bytes + 16 * piece;
    const int off = 1024 * (w + 8 * m) + 16 * lane, krow = off / DT_W_ROWB;
    const int slot = (off % DT_W_ROWB) / 16;                                       // 16-byte slot in the row
    const int wpiece = (krow / 8) % 2 ? (slot + DT_W_ROWB / 32) % (DT_W_ROWB / 16) : slot;  // the halves swapped
    woff[m] = (uint32_t)krow * (uint32_t)wrow_bytes + 2u * (uint32_t)(min(n0 + 8 * wpiece, p.N - 8) - n0);
  }
  const uint32_t lds0 = dt_lds_addr(dt_smem);
  auto issue = [&](int c) {
    const uint32_t st = lds0 + (uint32_t)((c % 2) * DT_STAGE);
    const unsigned char* xc = xb + (size_t)c * DT_ROWB;
    const unsigned char* wc = wb + (size_t)c * DT_KC * wrow_bytes;
#pragma unroll
    for (int m = 0; m < 4; m++) dt_dma16(xc, xoff[m], st + 1024 * (w + 8 * m));
#pragma unroll
    for (int m = 0; m < 4; m++)
      if (w + 8 * m < DT_W_INSTR) dt_dma16(wc, woff[m], st + DT_X_BYTES + 1024 * (w + 8 * m));
  };

  // fragment reads: tokens, row 16 f + l%16 of a 16-row group, piece
  // 4s + l/16; weights, two transposing reads of rows 32s + 8g + 4h + r
  // (h = 0, 1), columns 16 j + 4c .. of this wavefront's (r = (l%16)/4,
  // c = l%4), whose half is swapped where (row/8) = g is odd
  const int rl = lane % 16, g = lane / 16;
  const int wr = w % 4, wc = w / 4;
  const int xrow0 = 64 * wr, wrow0 = 112 * wc;
  const int half_swap = (g % 2) ? (wc ? -DT_W_ROWB / 2 : DT_W_ROWB / 2) : 0;
  int roff[2], wtro[2][2];
#pragma unroll
  for (int s = 0; s < 2; s++) {
    roff[s] = rl * DT_ROWB + 16 * ((4 * s + g) ^ (rl / 2));
#pragma unroll
    for (int h = 0; h < 2; h++)
      wtro[s][h] = (32 * s + 8 * g + 4 * h + rl / 4) * DT_W_ROWB + 2 * 4 * (rl % 4) + half_swap;
  }

  f32x4 acc[7][4];
#pragma unroll
  for (int j = 0; j < 7; j++)
#pragma unroll
    for (int f = 0; f < 4; f++) acc[j][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // the fp16 copy of x: chunk c of a (token tile, slab) by column tile c % n_ct
  auto copy_x16 = [&](int c) {
    const unsigned char* S = dt_smem + (c % 2) * DT_STAGE;
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const int row = threadIdx.x / 2, q = 4 * (threadIdx.x % 2) + h;
      const uint4 v = *reinterpret_cast<const uint4*>(S + row * DT_ROWB + 16 * (q ^ ((row / 2) % 8)));
      if (t0 + row < p.T) {
        f16x8 o;
        o[0] = (f16)__uint_as_float(v.x << 16); o[1] = (f16)__uint_as_float(v.x & 0xFFFF0000u);
        o[2] = (f16)__uint_as_float(v.y << 16); o[3] = (f16)__uint_as_float(v.y & 0xFFFF0000u);
        o[4] = (f16)__uint_as_float(v.z << 16); o[5] = (f16)__uint_as_float(v.z & 0xFFFF0000u);
        o[6] = (f16)__uint_as_float(v.w << 16); o[7] = (f16)__uint_as_float(v.w & 0xFFFF0000u);
        *reinterpret_cast<f16x8*>(p.x16 + (size_t)(t0 + row) * p.K + k_begin + c * DT_KC + 8 * q) = o;
      }
    }
  };
  // (fragments are held as integer vectors: as __bf16 vectors the compiler
  // repacks their halves when they cross the loop's back edge)
  auto read_step = [&](int c, int s, u32x4v (&xa)[4], u32x4v (&wa)[7]) {
    const unsigned char* S = dt_smem + (c % 2) * DT_STAGE;
#pragma unroll
    for (int f = 0; f < 4; f++) xa[f] = *reinterpret_cast<const u32x4v*>(S + (xrow0 + 16 * f) * DT_ROWB + roff[s]);
#pragma unroll
    for (int j = 0; j < 7; j++) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const unsigned char* base = S + DT_X_BYTES + 2 * (wrow0 + 16 * j);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + wtro[s][0]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + wtro[s][1]));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      wa[j] = u32x4v{l2.x, l2.y, h2.x, h2.y};
    }
  };
  auto mma_step = [&](const u32x4v (&xa)[4], const u32x4v (&wa)[7]) {
#pragma unroll
    for (int j = 0; j < 7; j++)
#pragma unroll
      for (int f = 0; f < 4; f++)
        acc[j][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[j]),
                                                            __builtin_bit_cast(bf16x8, xa[f]), acc[j][f], 0, 0, 0);
  };

  // Software pipeline over chunks: the barrier of chunk c sits between its
  // two steps.  Before it the wavefront has read all of chunk c (step 1's
  // fragments are in registers), so after it chunk c's stage takes the
  // copies of chunk c+2, and the wavefront reads chunk c+1's first
  // fragments while step 1's MFMAs run; the copies of a chunk have one
  // chunk's time to land.
  issue(0);
  if (nchunks > 1) issue(1);
  __builtin_amdgcn_sched_barrier(0);
  dt_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (p.x16 != nullptr && ct == 0) copy_x16(0);
  u32x4v xa0[4], wa0[7], xa1[4], wa1[7];
  read_step(0, 0, xa0, wa0);
  for (int c = 0; c < nchunks; c++) {
    read_step(c, 1, xa1, wa1);
    mma_step(xa0, wa0);
    // (the compiler would otherwise move the MFMAs, which touch no memory,
    // past the barrier)
    __builtin_amdgcn_sched_barrier(0);
    dt_barrier();  // all reads of chunk c are done; chunk c+1 is in its stage
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < nchunks) issue(c + 2);
    if (c + 1 < nchunks) {
      if (p.x16 != nullptr && (c + 1) % p.n_ct == ct) copy_x16(c + 1);
      read_step(c + 1, 0, xa0, wa0);
    }
    mma_step(xa1, wa1);
  }

  // D[4g+i][l%16] of product (j, f): column n0 + 112 wc + 16 j + 4 g + i of
  // token t0 + 64 wr + 16 f + l%16
#pragma unroll
  for (int f = 0; f < 4; f++) {
    const int t = t0 + xrow0 + 16 * f + rl;
    if (t >= p.T) continue;
#pragma unroll
    for (int j = 0; j < 7; j++) {
      const int n = n0 + wrow0 + 16 * j + 4 * g;
      if (n >= p.N) continue;
      const f32x4 v = acc[j][f];
      if (p.part != nullptr) {
        *reinterpret_cast<float4*>(p.part + ((size_t)slab * p.T + t) * p.N + n) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        const uint16_t b0 = f32_to_bf16(v[0]), b1 = f32_to_bf16(v[1]), b2 = f32_to_bf16(v[2]), b3 = f32_to_bf16(v[3]);
        uint2 o;
        o.x = (uint32_t)b0 | ((uint32_t)b1 << 16);
        o.y = (uint32_t)b2 | ((uint32_t)b3 << 16);
        *reinterpret_cast<uint2*>(p.out + (size_t)t * p.N + n) = o;
        if (p.out16 != nullptr) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          h4 h;
          h[0] = (f16)bf16_to_f32(b0);
          h[1] = (f16)bf16_to_f32(b1);
          h[2] = (f16)bf16_to_f32(b2);
          h[3] = (f16)bf16_to_f32(b3);
          *reinterpret_cast<h4*>(p.out16 + (size_t)t * p.N + n) = h;
        }
      }
    }
  }
}

}  // namespace

DensePlan dense_plan(int T, int K, int N) {
  DensePlan d;
  d.tiled = T >= DT_MIN_T && K >= DT_KC && K % DT_KC == 0 && N >= 8 && N % 8 == 0;
  d.slabs = 1;
  d.kslab = K;
  if (!d.tiled) return d;
  const long long tiles = (long long)((T + DT_M - 1) / DT_M) * ((N + DT_N - 1) / DT_N);
  const int chunks = K / DT_KC;
  int s = (int)((256 + tiles - 1) / tiles);  // at least one wave of 256 blocks
  if (s > DT_MAX_SLABS) s = DT_MAX_SLABS;
  if (s > chunks) s = chunks;
  if (s < 1) s = 1;
  const int per = (chunks + s - 1) / s;
  d.kslab = per * DT_KC;
  d.slabs = (chunks + per - 1) / per;
  return d;
}

hipError_t launch_dense_tiled(const uint16_t* x, const uint16_t* w, int T, int K, int N, const DensePlan& dp,
                              float* part, uint16_t* out, f16* out16, f16* x16, hipStream_t s) {
  if (!dp.tiled || (part == nullptr && (dp.slabs != 1 || out == nullptr))) return hipErrorInvalidValue;
  DenseParams p;
  p.x = reinterpret_cast<const unsigned char*>(x);
  p.w = reinterpret_cast<const unsigned char*>(w);
  p.part = part;
  p.out = out;
  p.out16 = out16;
  p.x16 = x16;
  p.T = T;
  p.K = K;
  p.N = N;
  p.kslab = dp.kslab;
  p.n_tt = (T + DT_M - 1) / DT_M;
  p.n_ct = (N + DT_N - 1) / DT_N;
  p.cg = 1;
  for (int c = 8; c >= 1; c--)
    if (p.n_ct % c == 0) {
      p.cg = c;
      break;
    }
  const long long items = (long long)dp.slabs * p.n_ct * p.n_tt;
  if (items > (1LL << 30)) return hipErrorInvalidValue;
  p.n_items = (int)items;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_tile_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, DT_LDS);
  if (e != hipSuccess) return e;
  const long long per_xcd = (items + 7) / 8;
  hipLaunchKernelGGL(dense_tile_kernel, dim3((unsigned)(8 * per_xcd)), dim3(DT_WAVES * WAVE), DT_LDS, s, p);
  return hipGetLastError();
}

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
  if (rp.tiled && rp.slabs == 1) {  // the tile writes the rounded output itself
    DensePlan dp;
    dp.tiled = true;
    dp.slabs = 1;
    dp.kslab = rp.slab_rows;
    return launch_dense_tiled(x, w, T, K, N, dp, nullptr, out, out16, nullptr, s);
  }
  hipError_t e = launch_router(x, w, part, T, K, N, rp, s);
  if (e != hipSuccess) return e;
  const long long n4 = (long long)T * N / 4;
  const long long blocks = (n4 + PROJ_THREADS - 1) / PROJ_THREADS;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)blocks), dim3(PROJ_THREADS), 0, s, part, rp.slabs, n4,
                     (long long)T * N, out, out16);
  return hipGetLastError();
}

}  // namespace moe
