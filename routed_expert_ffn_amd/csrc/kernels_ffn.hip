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
// Loads.  A wavefront owns 64 weight rows (4 groups of 16).  Per 256-k
// chunk, lane (r = l%16, g = l/16) reads 32 bytes (64 codes) of row r at k
// offset 64g and uses the 4 scale bytes of those 64 codes, so each row's
// 128-byte span of the chunk is read whole by one wavefront.  Code dword s
// (k = 64g+8s..) is exactly the B fragment of MFMA step s, so the k order
// inside an MFMA is permuted consistently for A and B.  The wavefronts that
// share rows split K into contiguous ranges and are reduced through LDS in a
// fixed order; the block scales of all the block's rows are staged in LDS
// once.
#include "internal.h"

namespace moe {
namespace {

constexpr int KCHUNK = 256;

struct GroupedParams {
  int T, H, I, k;
  int e_base;          // expert e's weights are entry e - e_base of the store
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
  float* rows;         // down output [P][H], fp32 unweighted (when rows16 is NULL)
  f16* rows16;         // or: down output [P][H] fp16, each row times its routing weight, in record order (row
                       //     t*k+j; small-batch kernel) or in sorted order (row p; large-tile kernel)
  const float* pair_w; //     the routing weights [T*k], indexed by record (sorted_pairs[p])
};

// Barrier for LDS hand-off: this wavefront's LDS accesses and all but its
// last N vector-memory instructions have completed when it arrives (N = 63:
// no vector-memory wait at all).  The memory clobber keeps the compiler from
// moving memory accesses across it, and unlike __syncthreads() it adds no
// fence of its own.
template <int N>
__device__ __forceinline__ void lds_barrier_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS DMA of 16 (4) bytes per lane from gbase + voff to LDS address lds +
// 16 (4) * lane, written as instructions of our own: the compiler would
// otherwise count the copies as outstanding LDS work and wait for all LDS
// traffic (lgkmcnt(0)) before every use of an LDS read, serialising the
// fragment reads with the MFMAs.  Every wait for these copies is explicit
// (lds_barrier_vm).  gbase and lds are wave-uniform (scalar registers).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
__device__ __forceinline__ void dma16(const unsigned char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const unsigned char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// One 256-k chunk of a wavefront's operands: per weight row group ng, 32
// NVFP4 code bytes (64 consecutive k); per token fragment f, the eight A
// fragments of the chunk.  All of a chunk's loads are issued together so the
// wavefront waits once per chunk, not once per MFMA.
template <int MF>
struct Chunk {
  uint4 qa[4], qb[4];
  f16x8 a[MF][8];
};

// Weight formats: NVFP4 (e4m3 scale per 16 k, 4 scale bytes per 64 codes)
// and MXFP4 (e8m0 power-of-two scale per 32 k, 2 bytes per 64 codes).
enum WeightFmt { FMT_NV = 0, FMT_MX = 1 };

// Codes of chunk c.  The MFMA wants lane (r, g) = (l%16, l/16) to hold
// pieces 2g and 2g+1 (16 bytes each) of row r of its 16-row group, but
// loads in that shape cover half of each 128-byte line per instruction.
// Instead each instruction covers 8 whole lines: lane l loads piece l/8 of
// row l%8 (qa) and of row 8 + l%8 (qb), as non-temporal loads (the codes
// are read once).  Measured on a cold 252 MiB read: 6.1 TB/s this way
// against 5.2-5.4 TB/s for any half-line or cached pattern.
// codes_to_fragments then moves the pieces into place.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// R8 = false keeps the fragment shape (lane (r, g) loads bytes 32g .. 32g+31
// of row r), which stays faster for the down GEMM when experts take several
// 16-token passes over their weights (measured at 64 and 256 tokens).
template <int MF, bool R8>
__device__ __forceinline__ void load_b(Chunk<MF>& ch, const uint8_t* const (&grp)[4], int c, size_t row_bytes) {
  const int lane = threadIdx.x % WAVE;
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    if (R8) {
      const uint8_t* p = grp[ng] + (size_t)(lane % 8) * row_bytes + 128 * (size_t)c + 16 * (lane / 8);
      ch.qa[ng] = load_nt16(p);
      ch.qb[ng] = load_nt16(p + 8 * row_bytes);
    } else {
      const uint8_t* p = grp[ng] + (size_t)(lane % 16) * row_bytes + 128 * (size_t)c + 32 * (lane / 16);
      ch.qa[ng] = *reinterpret_cast<const uint4*>(p);
      ch.qb[ng] = *reinterpret_cast<const uint4*>(p + 16);
    }
  }
}

// Lane l = r + 16g holds in qa piece l/8 of row l%8: for r < 8 that is its
// own piece 2g of row r, for r >= 8 piece 2g+1 of row r-8, which lane l-8
// needs; in qb piece l/8 of row 8 + l%8: for r >= 8 its own piece 2g+1 of
// row r, for r < 8 piece 2g of row r+8, which lane l+8 needs.  One exchange
// between lanes 8 apart in each row of 16 puts piece 2g in qa and piece
// 2g+1 in qb everywhere: a DPP row rotation by 8 whose bank mask writes only
// the lanes that take the moved word (banks 0-1 = lanes 0-7 of a row, banks
// 2-3 = lanes 8-15), two instructions per word, both reading the words as
// loaded.
template <int BANKS>
__device__ __forceinline__ uint32_t from_lane8_apart(uint32_t keep, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xF, BANKS, false);  // row_ror:8
}
__device__ __forceinline__ void codes_to_fragments(uint4& qa, uint4& qb) {
  uint32_t* a = &qa.x;
  uint32_t* b = &qb.x;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    const uint32_t na = from_lane8_apart<0xC>(a[d], b[d]);  // lanes 8-15: qb of lane - 8
    const uint32_t nb = from_lane8_apart<0x3>(b[d], a[d]);  // lanes 0-7: qa of lane + 8
    a[d] = na;
    b[d] = nb;
  }
}

// Block scales of a group of four consecutive chunks c .. c+3 (c a multiple
// of 4, so that a row's scale bytes of the group are one aligned 64-byte
// (MXFP4: 32-byte) piece whichever wavefront loads them).  Lane (r, g)
// of the wavefront (r = lane % 16, g = lane / 16) needs, in each chunk, the
// scale word of its own 64-k quarter g (NVFP4: 4 bytes, MXFP4: 2) for its row
// of every row group.  Loading those words one chunk at a time costs one
// cache-line request per row for 4 (2) bytes, which was measured to slow the
// decode GEMMs by a fifth; instead lane (r, g) loads all 16 (8) scale bytes
// of chunk c + g in one go, and a 4 x 4 transpose across the wavefront's four
// rows of 16 lanes hands each lane its quarter of each of the four chunks.
// Chunks past the end of K load the last chunk's bytes and are never used.
template <int FMT>
__device__ __forceinline__ void load_sq(uint32_t (&sq)[4][4], const uint8_t* const (&srow)[4], int c, int nchunks,
                                        int g) {
  const int cg = min(c + g, nchunks - 1);
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    if (FMT == FMT_MX) {
      const uint2 v = *reinterpret_cast<const uint2*>(srow[ng] + 8 * cg);
      sq[ng][0] = v.x;
      sq[ng][1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(srow[ng] + 16 * cg);
      sq[ng][0] = v.x;
      sq[ng][1] = v.y;
      sq[ng][2] = v.z;
      sq[ng][3] = v.w;
    }
  }
}

// Word j of lane row R (lanes 16R .. 16R+15) becomes word R of lane row j:
// the upper and lower 32 lanes swap the off-diagonal 2 x 2 blocks, then odd
// and even rows of 16 lanes swap the off-diagonal words inside each block.
__device__ __forceinline__ void transpose_rows4(uint32_t (&v)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// After load_sq's data has arrived: sq[ng][i] = this lane's scale word of
// chunk c + i (MXFP4 words are zero-extended 16-bit pairs).
template <int FMT>
__device__ __forceinline__ void sq_transpose(uint32_t (&sq)[4][4]) {
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    if (FMT == FMT_MX) {
      const uint32_t x = sq[ng][0], y = sq[ng][1];
      sq[ng][0] = x & 0xFFFFu;
      sq[ng][1] = x >> 16;
      sq[ng][2] = y & 0xFFFFu;
      sq[ng][3] = y >> 16;
    }
    transpose_rows4(sq[ng]);
  }
}

// This lane's scale words of chunk c (of the group loaded for c & ~3).
__device__ __forceinline__ void sq_pick(uint32_t (&w)[4], const uint32_t (&sq)[4][4], int c) {
  const int i = c & 3;
#pragma unroll
  for (int ng = 0; ng < 4; ng++) w[ng] = i == 0 ? sq[ng][0] : i == 1 ? sq[ng][1] : i == 2 ? sq[ng][2] : sq[ng][3];
}

// Scales staged in LDS.  A block's weight rows are consecutive in each
// matrix, so the block scales of all of them are one contiguous piece per
// matrix (gate/up: the gate rows and the same up rows; down: the rows).  The
// block copies these pieces into LDS once, as 16-byte-per-lane LDS DMA over
// whole lines, and each wavefront then reads its words chunk by chunk.  Read
// from memory in 64-byte pieces per row and group of four chunks instead,
// every 128-byte line was fetched twice: its two halves are read some
// microseconds apart, and by then the L2 no longer holds it.
template <int NW>
__device__ __forceinline__ void stage_scales(unsigned char* lds, const uint8_t* src, int bytes, int wv, int lane) {
  // src is the same in every lane (one block's piece); the DMA takes it in scalar registers
  const uint64_t sa = (uint64_t)(size_t)src;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sa), hi = __builtin_amdgcn_readfirstlane((uint32_t)(sa >> 32));
  src = reinterpret_cast<const uint8_t*>((size_t)(((uint64_t)hi << 32) | lo));
  const uint32_t dst = lds_addr(lds);
  for (int i = __builtin_amdgcn_readfirstlane(wv); i * 1024 < bytes; i += NW)
    if (i * 1024 + 16 * lane < bytes) dma16(src, (uint32_t)(i * 1024 + 16 * lane), dst + (uint32_t)(i * 1024));
}

// This lane's scale words of chunk c from the staged rows (byte offsets lsrow).
template <int FMT>
__device__ __forceinline__ void staged_words(uint32_t (&w)[4], const unsigned char* lds, const int (&lsrow)[4], int c,
                                             int g) {
#pragma unroll
  for (int ng = 0; ng < 4; ng++)
    w[ng] = FMT == FMT_MX ? (uint32_t)*reinterpret_cast<const uint16_t*>(lds + lsrow[ng] + 8 * c + 2 * g)
                          : *reinterpret_cast<const uint32_t*>(lds + lsrow[ng] + 16 * c + 4 * g);
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
// MXFP4: step s's codes share the scale byte s/4; the conversion applies
// 2^(scale - 127 - roff[ng]) itself (roff: the matrix's per-tensor power of
// two, applied back in fp32 with gs).
template <int MF, int FMT, bool R8>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[MF][4], Chunk<MF>& ch, const uint32_t (&sw)[4],
                                          int nvalid, const int (&roff)[4]) {
  if (R8)
#pragma unroll
    for (int ng = 0; ng < 4; ng++) codes_to_fragments(ch.qa[ng], ch.qb[ng]);
#pragma unroll
  for (int s = 0; s < 8; s++) {
#pragma unroll
    for (int ng = 0; ng < 4; ng++) {
      const uint32_t codes = s < 4 ? (&ch.qa[ng].x)[s] : (&ch.qb[ng].x)[s - 4];
      f16x8 bf;
      if (FMT == FMT_MX) {
        const int sb = (int)((sw[ng] >> (8 * (s / 4))) & 0xFFu);
        bf = dequant8_pow2(codes, __builtin_ldexpf(1.0f, sb - 127 - roff[ng]));
      } else {
        const f16 sig = e4m3_to_f16((sw[ng] >> (8 * (s / 2))) & 0xFFu);
        f16x2 sig2;
        sig2[0] = sig;
        sig2[1] = sig;
        bf = dequant8(codes, sig2);
      }
#pragma unroll
      for (int f = 0; f < MF; f++)
        if (f * 16 < nvalid) acc[f][ng] = mfma16x16x32(ch.a[f][s], bf, acc[f][ng]);
    }
  }
}

// SiLU(z) = z / (1 + e^-z) with the hardware base-2 exponential and
// reciprocal (each within about one fp32 ulp); h is rounded to fp16 (2^-11)
// right after, so their error does not show.  e^-z overflows to infinity
// for z below about -88, giving z * 0 = -0, within fp16 rounding of the
// true value there.
__device__ __forceinline__ float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// One grouped NVFP4 GEMM over the active experts (blockIdx.y indexes the
// active list).  A block is four wavefronts; KSPLIT consecutive wavefronts
// share one 64-row tile and each takes a contiguous range of its 256-k
// chunks, so a block covers 4/KSPLIT row tiles.  (Contiguous ranges let one
// grouped scale load serve four chunks; they read about 3% slower than
// interleaved chunks, far less than per-chunk scale loads cost.)  SLDS: the
// block scales are staged in LDS (dynamic shared memory) at the start.
//   GATEUP: a row tile is 32 columns of h: gate rows (groups 0, 1) and the
//           same up rows (groups 2, 3); the epilogue applies the per-tensor
//           scales and SiLU(gate) * up and stores h in fp16.
//   down:   a row tile is 64 output columns; rows = gs_d * (h . Wd).
// The first chunk's weight loads are issued before the token rows are
// looked up; each later chunk's loads are issued once the previous chunk has
// been multiplied.  Partial sums of the KSPLIT wavefronts meet in LDS and
// are added in a fixed order.
template <int MF, int KSPLIT, bool GATEUP, int WAVES_PER_EU, int FMT, bool SLDS, bool R8, int NW = 4>
__global__ __launch_bounds__(NW * WAVE, WAVES_PER_EU) void expert_gemm_kernel(GroupedParams p) {
  constexpr int RT = NW / KSPLIT;
  static_assert(NW % KSPLIT == 0, "whole row tiles per block");
  __shared__ float red[KSPLIT > 1 ? NW : 1][WAVE][MF * 16];
  extern __shared__ __align__(16) unsigned char staged[];
  // both loads issued before either is waited for (the empty asm takes the
  // id before the test; the compiler would otherwise load it only after);
  // active has gridDim.y entries, and an id past n_active is never used
  const int n_act = *p.n_active;
  const int e = p.active[blockIdx.y];
  asm volatile("" ::"s"(e));
  if ((int)blockIdx.y >= n_act) return;
  const int el = e - p.e_base;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, r = lane % 16, g = lane / 16;
  const int rt = wv / KSPLIT, ks = wv % KSPLIT;
  const int K = GATEUP ? p.H : p.I;
  const int N = GATEUP ? p.I : p.H;
  const int tile = blockIdx.x * RT + rt;
  const uint8_t* qrow[4];  // codes: first row of each 16-row group
  const uint8_t* srow[4];  // scales: this lane's row
#pragma unroll
  for (int ng = 0; ng < 4; ng++) {
    size_t row;
    const uint8_t* qb;
    const uint8_t* sb;
    if (GATEUP) {
      row = (size_t)el * N + tile * 32 + 16 * (ng & 1) + r;
      qb = ng < 2 ? p.q0 : p.q1;
      sb = ng < 2 ? p.sf0 : p.sf1;
    } else {
      row = (size_t)el * N + tile * 64 + 16 * ng + r;
      qb = p.q0;
      sb = p.sf0;
    }
    qrow[ng] = qb + (row - r) * (K / 2);  // row 0 of the lane's 16-row group
    srow[ng] = sb + row * (K / (FMT == FMT_MX ? 32 : 16));
  }
  const size_t row_bytes = (size_t)(K / 2);
  const int nchunks = K / KCHUNK;
  const int per = (nchunks + KSPLIT - 1) / KSPLIT;
  const int c_lo = min(ks * per, nchunks), c_hi = min(c_lo + per, nchunks);
  // staged scales: this lane's rows within the block's pieces
  const int SB = K / (FMT == FMT_MX ? 32 : 16);
  int lsrow[4];
  if (SLDS) {
    const size_t r0 = (size_t)el * N + (size_t)blockIdx.x * RT * (GATEUP ? 32 : 64);
    if (GATEUP) {
      stage_scales<NW>(staged, p.sf0 + r0 * SB, RT * 32 * SB, wv, lane);
      stage_scales<NW>(staged + RT * 32 * SB, p.sf1 + r0 * SB, RT * 32 * SB, wv, lane);
    } else {
      stage_scales<NW>(staged, p.sf0 + r0 * SB, RT * 64 * SB, wv, lane);
    }
#pragma unroll
    for (int ng = 0; ng < 4; ng++)
      lsrow[ng] = GATEUP ? ((ng >> 1) * RT * 32 + rt * 32 + 16 * (ng & 1) + r) * SB : (rt * 64 + 16 * ng + r) * SB;
  }
  Chunk<MF> cur;
  uint32_t sq[4][4];
  if (c_lo < c_hi) {  // before the token lookups
    load_b<MF, R8>(cur, qrow, c_lo, row_bytes);
    if (!SLDS) load_sq<FMT>(sq, srow, c_lo & ~3, nchunks, g);
  }
  const int begin = p.offsets[e], end = p.offsets[e + 1];
  const float gsa = p.gs0[el], gsb = GATEUP ? p.gs1[el] : 0.0f;
  // MXFP4: gs = 2^r (frexp exponent r + 1); the block scales are divided by it
  int roff[4];
  {
    const int r0 = FMT == FMT_MX ? __builtin_amdgcn_frexp_expf(gsa) - 1 : 0;
    const int r1 = FMT == FMT_MX && GATEUP ? __builtin_amdgcn_frexp_expf(gsb) - 1 : 0;
#pragma unroll
    for (int ng = 0; ng < 4; ng++) roff[ng] = GATEUP && ng >= 2 ? r1 : r0;
  }
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
    if (c_lo < c_hi) {
      if (!first_pass) {
        load_b<MF, R8>(cur, qrow, c_lo, row_bytes);
        if (!SLDS) load_sq<FMT>(sq, srow, c_lo & ~3, nchunks, g);
      }
      load_a(cur, arow, c_lo * KCHUNK + 64 * g, nvalid);
    }
    // weighted fp16 rows: each output row's record and its routing weight,
    // loaded here so that their two dependent round trips overlap the K loop
    // (in the epilogue they stalled every block for both)
    int rec_pf[MF][4];
    float w_pf[MF][4];
    if (!GATEUP && p.rows16)
#pragma unroll
      for (int f = 0; f < MF; f++)
#pragma unroll
        for (int i = 0; i < 4; i++) rec_pf[f][i] = p.sorted_pairs[mb + min(f * 16 + 4 * g + i, nvalid - 1)];
    uint32_t sw[4];
    if (SLDS) {
      if (first_pass) lds_barrier_vm<0>();  // the staged scales (and chunk c_lo) have landed
      if (c_lo < c_hi) staged_words<FMT>(sw, staged, lsrow, c_lo, g);
    }
    first_pass = false;
    if (!GATEUP && p.rows16)
#pragma unroll
      for (int f = 0; f < MF; f++)
#pragma unroll
        for (int i = 0; i < 4; i++) w_pf[f][i] = p.pair_w[rec_pf[f][i]];
    for (int c = c_lo; c < c_hi; c++) {
      if (!SLDS) {
        if (c == c_lo || (c & 3) == 0) sq_transpose<FMT>(sq);
        sq_pick(sw, sq, c);
      }
      mma_chunk<MF, FMT, R8>(acc, cur, sw, nvalid, roff);
      if (c + 1 < c_hi) {
        const int kb = (c + 1) * KCHUNK + 64 * g;
        load_b<MF, R8>(cur, qrow, c + 1, row_bytes);
        if (SLDS)
          staged_words<FMT>(sw, staged, lsrow, c + 1, g);
        else if (((c + 1) & 3) == 0)
          load_sq<FMT>(sq, srow, c + 1, nchunks, g);
        load_a(cur, arow, kb, nvalid);
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
            } else if (p.rows16) {
              const int rec = rec_pf[f][i];  // stored at its record's row
              const float ws = w_pf[f][i] * gsa;
#pragma unroll
              for (int ng = 0; ng < 4; ng++)
                p.rows16[(size_t)rec * N + tile * 64 + 16 * ng + r] = (f16)(ws * acc[f][ng][i]);
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

// ---- large batches: 224-token x 256-row tiles on 32x32x16 matrix cores ---------
// Work items are (expert, token tile) entries of a list built with the
// permutation (mtiles), times the row tiles of the matrix; an expert's
// records are split evenly over ceil(n / 224) tiles.  A block of eight
// wavefronts, two per SIMD, computes a tile of up to 224 tokens (NF =
// ceil(n / 32) token fragments, a template parameter so the inner loop is
// straight-line code) against 256 weight rows: wavefronts w and w + 4 share
// one SIMD and its 64 weight rows (two fragments) and take the even and the
// odd token fragments, as v_mfma_f32_32x32x16_f16 (lane l holds
// A[l%32][8(l/32)..+7], B[8(l/32)..+7][l%32] and D[8(i/4) + 4(l/32) +
// i%4][l%32]).  Each SIMD thus multiplies every token fragment against its
// rows once; the two wavefronts each dequantise the rows (at most 128
// accumulator registers each, so two fit a SIMD), and one's LDS reads and
// barrier waits overlap the other's matrix-core work.
//
// K runs in chunks of 64.  Inside a chunk the sum is taken in a permuted
// order: lane half g = l/32 in step s covers the chunk's k = 32g + 8s .. +7,
// the same for both operands, so one lane's codes for all four steps are 16
// contiguous bytes of the weight row.  All operands reach LDS by LDS DMA
// (global_load_lds), which is limited by the number of cache-line requests
// a CU keeps in flight, so every request fetches whole lines where it can:
//   tokens:  fp16 rows of one chunk (128 bytes a row), three buffers, copied
//            two chunks ahead;
//   weights: the raw NVFP4 bytes of four chunks ("a span": 128 code bytes
//            and 16 scale bytes a row), two slots, copied while the previous
//            span is in use.
// A 128-byte row is 8 pieces of 16 bytes, piece q of row m stored in slot
// q ^ ((m/2) % 8), so the 16 rows that one read phase touches cover all 64
// banks.  Each wavefront turns the raw bytes of its own weight rows into
// exact fp16 in registers (e2m1 code times e4m3 block scale) step by step.
//
// DMA and waits: pair A = wavefronts 0, 1 and pair B = 2, 3.  In chunk c
// pair A (c even) or B (c odd) copies the tokens of chunk c+2 (wavefront w
// the token groups g with g % 2 == w % 2); in the span's chunks 1 and 2
// pairs B and A also copy the two halves (128 rows each) of the next span.
// A pair waits for all of its copies (vmcnt(0)) at the end of the chunk
// after the one it issued in, when nothing else of its own is in flight; a
// partial vmcnt wait that leaves newer DMA in flight was measured not to
// guarantee that older DMA writes are visible in LDS, so only vmcnt(0) is
// used.  Wavefronts 4-7 copy nothing; they only meet the others at the
// chunk barriers.
//
// Gate/up tiles pair 128 gate rows with the same 128 up rows (wavefronts w
// and w + 4: gate rows 32w .. and up rows 128 + 32w ..), so SiLU * up
// happens in registers.  Items are mapped to blocks so that the row tiles of one
// (expert, token tile) run back to back on one XCD (blocks are dealt to the
// eight XCDs round robin): its activations stay in that XCD's L2 while the
// weights stream once.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int BIG_M = MTILE;    // tokens per tile (7 fragments of 32)
constexpr int BIG_MF = BIG_M / 32;
constexpr int BIG_N = 256;      // weight rows per tile (8 fragments of 32)
constexpr int BIG_KC = 64;      // k per chunk: 8 pieces of 8 halves per token row
constexpr int BIG_SPAN = 4;     // chunks per raw weight span
constexpr int BIG_WAVES = 8;    // two wavefronts per SIMD
static_assert(BIG_M % 32 == 0 && BIG_MF <= 8, "token tile of whole fragments");
// LDS layout (bytes)
constexpr int BIG_TILE_BYTES = BIG_M * BIG_KC * 2;                  // tokens of one chunk
constexpr int BIG_SPANQ_BYTES = BIG_N * BIG_SPAN * BIG_KC / 2;      // codes of one span [256][128]
constexpr int BIG_SPANS_BYTES = BIG_N * BIG_SPAN * BIG_KC / 16;     // scales of one span [256][16]
constexpr int BIG_OFF_A = 0;                                        // [3][224][64] fp16
constexpr int BIG_OFF_RQ = BIG_OFF_A + 3 * BIG_TILE_BYTES;          // [2][256][128] u8
constexpr int BIG_OFF_RS = BIG_OFF_RQ + 2 * BIG_SPANQ_BYTES;        // [2][256][16] u8
constexpr int BIG_OFF_ROW = BIG_OFF_RS + 2 * BIG_SPANS_BYTES;       // [224] i32
constexpr int BIG_OFF_RW = BIG_OFF_ROW + BIG_M * 4;                 // [224] f32 routing weights (down, fp16 rows)
constexpr int BIG_LDS = BIG_OFF_RW + BIG_M * 4;
static_assert(BIG_LDS <= 160 * 1024, "LDS budget of one CU");

struct BigParams {
  GroupedParams g;
  const int32_t* mtiles;    // entries e * 65536 + tile
  const int32_t* n_mtiles;  // [1]
  int n_row_tiles;          // row tiles of BIG_N weight rows per expert
};

struct BigTile {
  int e, mb, nvalid, rtile, K, N;
};

// Per-thread state of one tile.  DMA addresses are a wave-uniform base plus
// a 32-bit per-lane byte offset, the form the DMA instruction takes directly.
struct BigLane {
  const unsigned char* a;  // token operand rows (x or h), uniform
  uint32_t toff[16];       // this lane's source (row, piece): group 2j + w%2, instruction i -> 4j + i
  int ngrp;                // token groups this wavefront copies
  const uint8_t* q[2];     // raw codes of tile rows 0 / 128 (uniform, k = 0)
  const uint8_t* sc[2];    // raw scales of tile rows 0 / 128
  uint32_t qlane;          // per-lane code source offset (this wavefront's instructions)
  uint32_t slane;          // per-lane scale source offset
  uint32_t sstep;          // MXFP4: scale bytes of 32 rows (the second scale instruction)
  int roff[2];             // MXFP4: power of two r of gs for fragment nf's matrix
  uint32_t qstep;          // code bytes of 16 rows: two instructions of one wavefront apart
  int aoff[4];             // per step: LDS byte offset of token row m32 in a token buffer
  int qrow[2], srow[2];    // LDS byte offsets of this lane's weight row (fragment nf) in a span slot
  int K;
};

// Token rows of chunk kc, groups 2j + p (j < ngrp, p = w % 2), into token
// buffer buf.  Instruction i of group g fills rows R = 32g + 8i .. R+7; lane
// l writes row R + l/8, slot l%8.
__device__ __forceinline__ void dma_tokens(const BigLane& L, unsigned char* smem, int buf, int kc, int p) {
  const unsigned char* base = L.a + 2 * (size_t)kc;
  const uint32_t dst = lds_addr(smem + BIG_OFF_A + buf * BIG_TILE_BYTES + 32 * p * BIG_KC * 2);
#pragma unroll
  for (int j = 0; j < 4; j++)
    if (j < L.ngrp) {
#pragma unroll
      for (int i = 0; i < 4; i++) dma16(base, L.toff[4 * j + i], dst + (64 * j + 8 * i) * BIG_KC * 2);
    }
}

// Half h (tile rows 128h .. 128h+127) of the raw span starting at k = k0
// into span slot `slot`, by the wavefront of parity p of the issuing pair:
// code instructions i = p, p+2, .. < 16 cover rows 128h + 8i .. +7 (lane l:
// row + l/8, slot l%8, the swizzled piece), scale instruction p rows
// 128h + 64p + l (16 bytes each).  MXFP4 has 8 scale bytes per row and span,
// stored [256][8]: two 4-byte instructions, rows 128h + 64p + 32i + l/2,
// bytes 4(l%2).
template <int FMT>
__device__ __forceinline__ void dma_span_half(const BigLane& L, unsigned char* smem, int slot, int k0, int h, int p) {
  const uint32_t rq = lds_addr(smem + BIG_OFF_RQ + slot * BIG_SPANQ_BYTES + 128 * h * 128 + 8 * p * 128);
  const unsigned char* qb = L.q[h] + k0 / 2;
#pragma unroll
  for (int ii = 0; ii < 8; ii++) dma16(qb, L.qlane + ii * L.qstep, rq + 16 * ii * 128);
  if (FMT == FMT_MX) {
    const uint32_t rs = lds_addr(smem + BIG_OFF_RS + slot * BIG_SPANS_BYTES + 128 * h * 8 + 64 * p * 8);
    dma4(L.sc[h] + k0 / 32, L.slane, rs);
    dma4(L.sc[h] + k0 / 32, L.slane + L.sstep, rs + 32 * 8);
  } else {
    const uint32_t rs = lds_addr(smem + BIG_OFF_RS + slot * BIG_SPANS_BYTES + 128 * h * 16 + 64 * p * 16);
    dma16(L.sc[h] + k0 / 16, L.slane, rs);
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Step s of one chunk: the two weight fragments, dequantised from this
// lane's raw codes (word s) and block scale (NVFP4: element s/2 of the pair
// in sig; MXFP4: the one power of two in pw, the lane's 32 k being one block).
template <int FMT>
__device__ __forceinline__ void dequant_step(f16x8 (&bv)[2], const u32x4 (&q)[2], const f16x2 (&sig)[2],
                                             const float (&pw)[2], int s) {
#pragma unroll
  for (int nf = 0; nf < 2; nf++) {
    if (FMT == FMT_MX) {
      bv[nf] = dequant8_pow2(q[nf][s], pw[nf]);
    } else {
      f16x2 s2;
      s2[0] = sig[nf][s / 2];
      s2[1] = sig[nf][s / 2];
      bv[nf] = dequant8(q[nf][s], s2);
    }
  }
}

// Token fragments a wavefront multiplies: of the tile's NF, the even ones
// (HALF 0, wavefronts 0-3) or the odd ones (HALF 1, wavefronts 4-7).
template <int NF, int HALF>
struct Frags {
  static constexpr int n = (NF + 1 - HALF) / 2;            // this wavefront's count
  static constexpr int at(int f) { return 2 * f + HALF; }  // its f-th, in the tile
};

template <int NF, int HALF>
__device__ __forceinline__ void read_a(f16x8 (&av)[8], const unsigned char* Ab, int aoff) {
#pragma unroll
  for (int f = 0; f < Frags<NF, HALF>::n; f++)
    av[f] = *reinterpret_cast<const f16x8*>(Ab + aoff + 32 * Frags<NF, HALF>::at(f) * BIG_KC * 2);
}

template <int NF>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[8][2], const f16x8 (&av)[8], const f16x8 (&bv)[2]) {
#pragma unroll
  for (int f = 0; f < NF; f++)
#pragma unroll
    for (int nf = 0; nf < 2; nf++) acc[f][nf] = mfma32x32x16(av[f], bv[nf], acc[f][nf]);
}

// A wavefront issues in order, and an MFMA blocks its issue until the matrix
// core takes it, so a wavefront's vector work only overlaps the matrix core
// when it sits between its MFMAs: a step's 2 NF MFMAs are spread over the
// next step's dequantisation (about 18 vector instructions), the first LEAD
// of them with no vector work between them (time for LDS reads to land).
// The next step's NDS token-fragment reads are spread over the first MFMAs
// as well, one after each, rather than issued in a burst that can fill the
// LDS command queue and hold up the next MFMA's issue.  (This order was
// tuned with one wavefront per SIMD; with two, the other wavefront fills the
// gaps as well, and the hints neither help nor hurt measurably.)
template <int NF, int LEAD = 0, int NDS = 0>
__device__ __forceinline__ void interleave_mfma_valu() {
  if constexpr (NF == 0) return;
  constexpr int rest = 2 * NF - LEAD > 0 ? 2 * NF - LEAD : 1;
  constexpr int per = (20 + rest - 1) / rest;
#pragma unroll
  for (int i = 0; i < 2 * NF; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // one MFMA
    if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    if (i >= LEAD) __builtin_amdgcn_sched_group_barrier(0x002, per, 0);  // vector ALU
  }
}

// What a wavefront carries from one chunk into the next: step 0's token
// fragments (a) and dequantised weights (b), and the chunk's raw codes (q)
// and block scales (sp raw, sig / pw converted) for the later steps.
struct BigStep {
  f16x8 a[8];
  f16x8 b[2];
  u32x4 q[2];
  uint32_t sp[2];
  f16x2 sig[2];
  float pw[2];
};

// LDS reads of chunk J (of the span in slot `slot`): this lane's 16 code
// bytes of each weight fragment and their scale bytes.
template <int J, int FMT>
__device__ __forceinline__ void read_chunk_b(const BigLane& L, const unsigned char* smem, int slot, BigStep& st) {
  const unsigned char* rq = smem + BIG_OFF_RQ + slot * BIG_SPANQ_BYTES;
  const unsigned char* rs = smem + BIG_OFF_RS + slot * BIG_SPANS_BYTES;
  const int g2 = (threadIdx.x % WAVE) / 32, m32 = threadIdx.x % 32;
  const int qslot = (2 * J + g2) ^ ((m32 / 2) % 8);  // piece 2J + g of the lane's row
#pragma unroll
  for (int nf = 0; nf < 2; nf++) {
    st.q[nf] = *reinterpret_cast<const u32x4*>(rq + L.qrow[nf] + 16 * qslot);
    if (FMT == FMT_MX)
      st.sp[nf] = *(rs + L.srow[nf] + 2 * J + g2);  // the block of k = 64J + 32g2 ..
    else
      st.sp[nf] = *reinterpret_cast<const uint16_t*>(rs + L.srow[nf] + 4 * J + 2 * g2);
  }
}

// The scale bytes as the dequantisation takes them.
template <int FMT>
__device__ __forceinline__ void convert_scales(const BigLane& L, BigStep& st) {
#pragma unroll
  for (int nf = 0; nf < 2; nf++) {
    if (FMT == FMT_MX)
      st.pw[nf] = __builtin_ldexpf(1.0f, (int)st.sp[nf] - 127 - L.roff[nf]);
    else
      st.sig[nf] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(st.sp[nf], 1.0f, false);
  }
}

// Chunk c = 4 s + J of the tile.  TOK: a chunk c+2 exists (its tokens are
// copied by pair J % 2); SPAN: a span s+1 exists (its halves are copied in
// J = 1 by pair B and J = 2 by pair A); NEXT: a chunk c+1 exists.  On entry
// st holds step 0 of chunk c (token fragments read, weights dequantised)
// and chunk c's codes and scales; on return the same for chunk c+1.  Token
// fragments are read and weights dequantised one step ahead.  The barrier,
// at which the pair that issued in chunk c-1 waits for its DMA, sits between
// steps 2 and 3: after it the wavefront reads chunk c+1's codes, scales and
// first token fragments, and dequantises its first weights, while step 3's
// MFMAs run, so the matrix cores do not idle at the chunk boundary.  (Every
// read of chunk c's token buffer has completed at the barrier, which is what
// lets the next chunk's DMA overwrite it.)
template <int NF, int HALF, int J, bool TOK_, bool SPAN_, bool NEXT, int FMT>
__device__ __forceinline__ void big_chunk(const BigLane& L, f32x16 (&acc)[8][2], unsigned char* smem, int c, int wv,
                                          BigStep& st) {
  // (only the first four wavefronts, HALF 0, copy)
  constexpr bool TOK = TOK_ && HALF == 0, SPAN = SPAN_ && HALF == 0;
  constexpr int NW = Frags<NF, HALF>::n;
  const int pair = wv >> 1, par = wv & 1;
  const int span = c / BIG_SPAN, slot = span & 1;
  const bool tok_issuer = pair == (J & 1);
  const bool span_issuer = (J == 1 && pair == 1) || (J == 2 && pair == 0);
  if (TOK && tok_issuer) dma_tokens(L, smem, (c + 2) % 3, (c + 2) * BIG_KC, par);
  if (SPAN && span_issuer)
    dma_span_half<FMT>(L, smem, slot ^ 1, (span + 1) * BIG_SPAN * BIG_KC, J == 1 ? 0 : 1, par);
  asm volatile("" ::: "memory");
  const unsigned char* Ab = smem + BIG_OFF_A + (c % 3) * BIG_TILE_BYTES;
  // Steps, each fenced so that the compiler keeps the order.
  f16x8 a1[8], b1[2];
  mma_step<NW>(acc, st.a, st.b);
  read_a<NF, HALF>(a1, Ab, L.aoff[1]);
  dequant_step<FMT>(b1, st.q, st.sig, st.pw, 1);
  interleave_mfma_valu<NW, 0, NW>();
  __builtin_amdgcn_sched_barrier(0);
  mma_step<NW>(acc, a1, b1);
  read_a<NF, HALF>(st.a, Ab, L.aoff[2]);
  dequant_step<FMT>(st.b, st.q, st.sig, st.pw, 2);
  interleave_mfma_valu<NW, 0, NW>();
  __builtin_amdgcn_sched_barrier(0);
  mma_step<NW>(acc, st.a, st.b);
  read_a<NF, HALF>(a1, Ab, L.aoff[3]);
  dequant_step<FMT>(b1, st.q, st.sig, st.pw, 3);
  interleave_mfma_valu<NW, 0, NW>();
  __builtin_amdgcn_sched_barrier(0);
  // (step 3's weights are computed here, beside step 2's MFMAs; without this
  // the compiler sinks them past the barrier's branch)
  asm volatile("" : "+v"(b1[0]), "+v"(b1[1]));
  const bool issued = (TOK && tok_issuer) || (SPAN && span_issuer);
  if (issued)
    lds_barrier_vm<63>();  // its copies stay in flight one more chunk
  else
    lds_barrier_vm<0>();
  if (NEXT) {
    constexpr int JN = (J + 1) % BIG_SPAN;
    read_chunk_b<JN, FMT>(L, smem, JN == 0 ? slot ^ 1 : slot, st);
    __builtin_amdgcn_sched_barrier(0);
    mma_step<NW>(acc, a1, b1);
    read_a<NF, HALF>(st.a, smem + BIG_OFF_A + ((c + 1) % 3) * BIG_TILE_BYTES, L.aoff[0]);
    convert_scales<FMT>(L, st);
    dequant_step<FMT>(st.b, st.q, st.sig, st.pw, 0);
    interleave_mfma_valu<NW, NW, NW>();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(st.b[0]), "+v"(st.b[1]));  // (kept beside step 3's MFMAs)
  } else {
    mma_step<NW>(acc, a1, b1);
  }
}

template <int NF, int HALF, bool TOK, bool SPAN, int FMT>
__device__ __forceinline__ void big_span(const BigLane& L, f32x16 (&acc)[8][2], unsigned char* smem, int c, int wv,
                                         BigStep& st) {
  big_chunk<NF, HALF, 0, TOK, SPAN, true, FMT>(L, acc, smem, c, wv, st);
  big_chunk<NF, HALF, 1, TOK, SPAN, true, FMT>(L, acc, smem, c + 1, wv, st);
  big_chunk<NF, HALF, 2, TOK, SPAN, true, FMT>(L, acc, smem, c + 2, wv, st);
  big_chunk<NF, HALF, 3, TOK, SPAN, true, FMT>(L, acc, smem, c + 3, wv, st);
}

// 4x4 transpose across the four lanes of a quad: lane j's v[r] becomes lane
// r's v[j].  Two exchange rounds: lanes two apart swap register pairs
// (lane j < 2 takes registers 0, 1 of lane j + 2 into its registers 2, 3),
// then neighbouring lanes swap single registers (even lane j takes register
// 0 of lane j + 1 into register 1, register 2 into register 3), each a
// quad permutation followed by a per-lane select.
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ void quad_transpose(float (&v)[4]) {
  constexpr int XOR2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // lane j reads lane j ^ 2
  constexpr int XOR1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // lane j reads lane j ^ 1
  const int j = threadIdx.x & 3;
  {
    const float x0 = dpp_quad<XOR2>(v[0]), x1 = dpp_quad<XOR2>(v[1]);
    const float x2 = dpp_quad<XOR2>(v[2]), x3 = dpp_quad<XOR2>(v[3]);
    const bool lo = j < 2;
    v[0] = lo ? v[0] : x2;
    v[1] = lo ? v[1] : x3;
    v[2] = lo ? x0 : v[2];
    v[3] = lo ? x1 : v[3];
  }
  {
    const float x0 = dpp_quad<XOR1>(v[0]), x1 = dpp_quad<XOR1>(v[1]);
    const float x2 = dpp_quad<XOR1>(v[2]), x3 = dpp_quad<XOR1>(v[3]);
    const bool even = (j & 1) == 0;
    v[0] = even ? v[0] : x1;
    v[1] = even ? x0 : v[1];
    v[2] = even ? v[2] : x3;
    v[3] = even ? x2 : v[3];
  }
}

// Wavefronts w and w + 4 (one SIMD) take the same 64 weight rows (w % 4) and
// the even (HALF 0) and odd (HALF 1) token fragments; only the first four
// copy.
template <int NF, bool GATEUP, int FMT, int HALF>
__device__ __forceinline__ void big_tile(const GroupedParams& p, const BigTile& t, unsigned char* smem) {
  constexpr int NW = Frags<NF, HALF>::n;
  const int lane = threadIdx.x % WAVE, m32 = lane % 32, g2 = lane / 32;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), par = wv & 1;
  const int wr = wv & 3;  // weight rows 64 wr ..  (gate/up: 32 wr .. of each matrix)
  const int K = t.K, nch = K / BIG_KC;
  const int32_t* rowoff = reinterpret_cast<const int32_t*>(smem + BIG_OFF_ROW);
  BigLane L;
  L.K = K;
  // token DMA: groups 2j + par; row R + l/8 of instruction (g, i) holds
  // piece (l%8) ^ ((row/2) % 8) = (l%8) ^ (4(i%2) + l/16) in slot l%8
  {
    L.a = reinterpret_cast<const unsigned char*>(p.a);
    L.ngrp = (NF - par + 1) / 2;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t piece = (uint32_t)((lane % 8) ^ (4 * (i % 2) + lane / 16));
        const int r = min(32 * (2 * j + par) + 8 * i + lane / 8, BIG_M - 1);
        L.toff[4 * j + i] = 2u * ((uint32_t)rowoff[r] * (uint32_t)K + 8u * piece);
      }
  }
  // raw weight spans: tile row r is gate row rtile*128 + r (r < 128) or the
  // same up row (r >= 128) for gate/up, row rtile*256 + r for down; a code
  // instruction's lane l reads its row's piece (l%8) ^ (4(i%2) + l/16)
  {
    const size_t qrow = (size_t)(K / 2), srow = (size_t)(K / (FMT == FMT_MX ? 32 : 16));
    if (GATEUP) {
      const size_t r0 = (size_t)(t.e - p.e_base) * t.N + t.rtile * (BIG_N / 2);
      L.q[0] = p.q0 + r0 * qrow;
      L.q[1] = p.q1 + r0 * qrow;
      L.sc[0] = p.sf0 + r0 * srow;
      L.sc[1] = p.sf1 + r0 * srow;
    } else {
      const size_t r0 = (size_t)(t.e - p.e_base) * t.N + t.rtile * BIG_N;
      L.q[0] = p.q0 + r0 * qrow;
      L.q[1] = L.q[0] + 128 * qrow;
      L.sc[0] = p.sf0 + r0 * srow;
      L.sc[1] = L.sc[0] + 128 * srow;
    }
    // this wavefront's code instructions i = par, par+2, ..: rows 8i + l/8
    L.qlane = (uint32_t)((8 * par + lane / 8) * qrow + 16 * ((lane % 8) ^ (4 * par + lane / 16)));
    L.qstep = (uint32_t)(16 * qrow);
    if (FMT == FMT_MX) {
      L.slane = (uint32_t)((64 * par + lane / 2) * srow + 4 * (lane % 2));
      L.sstep = (uint32_t)(32 * srow);
      const float g0 = p.gs0[t.e - p.e_base], g1 = GATEUP ? p.gs1[t.e - p.e_base] : g0;
      L.roff[0] = __builtin_amdgcn_frexp_expf(g0) - 1;  // fragment 0: gate rows (gate/up) or rows 64w..
      L.roff[1] = __builtin_amdgcn_frexp_expf(GATEUP ? g1 : g0) - 1;
    } else {
      L.slane = (uint32_t)((64 * par + lane) * srow);
      L.sstep = 0;
      L.roff[0] = L.roff[1] = 0;
    }
  }
  // LDS read offsets: token row 32f + m32 (f a compile-time offset); weight
  // fragment nf = tile rows 32w + 128nf (gate/up) or 64w + 32nf (down)
  {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int slot = (4 * g2 + s) ^ ((m32 / 2) % 8);
      L.aoff[s] = (m32 * BIG_KC + 8 * slot) * 2;
    }
#pragma unroll
    for (int nf = 0; nf < 2; nf++) {
      const int row = (GATEUP ? 32 * wr + 128 * nf : 64 * wr + 32 * nf) + m32;
      L.qrow[nf] = row * 128;
      L.srow[nf] = row * (FMT == FMT_MX ? 8 : 16);
    }
  }
  f32x16 acc[8][2];
#pragma unroll
  for (int f = 0; f < 8; f++)
#pragma unroll
    for (int nf = 0; nf < 2; nf++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[f][nf][i] = 0.0f;
  // prologue: pair A copies the tokens of chunk 0 and all of span 0 and
  // waits for them; pair B copies the tokens of chunk 1 (as if issued in
  // chunk -1) and waits at the end of chunk 0.  nch % 4 == 0, nch >= 4.
  {
    const int pair = wv >> 1;
    if (HALF > 0) {
      lds_barrier_vm<0>();  // nothing of its own in flight
    } else if (pair == 0) {
      dma_tokens(L, smem, 0, 0, par);
      dma_span_half<FMT>(L, smem, 0, 0, 0, par);
      dma_span_half<FMT>(L, smem, 0, 0, 1, par);
      lds_barrier_vm<0>();
    } else {
      dma_tokens(L, smem, 1, BIG_KC, par);
      lds_barrier_vm<63>();
    }
  }
  // chunk 0's codes, scales and step 0
  BigStep st;
  read_chunk_b<0, FMT>(L, smem, 0, st);
  read_a<NF, HALF>(st.a, smem + BIG_OFF_A, L.aoff[0]);
  convert_scales<FMT>(L, st);
  dequant_step<FMT>(st.b, st.q, st.sig, st.pw, 0);
  int c = 0;
  for (; c + BIG_SPAN < nch; c += BIG_SPAN) big_span<NF, HALF, true, true, FMT>(L, acc, smem, c, wv, st);
  // the last span: tokens of chunks c+2, c+3 still to copy, no next span
  big_chunk<NF, HALF, 0, true, false, true, FMT>(L, acc, smem, c, wv, st);
  big_chunk<NF, HALF, 1, true, false, true, FMT>(L, acc, smem, c + 1, wv, st);
  big_chunk<NF, HALF, 2, false, false, true, FMT>(L, acc, smem, c + 2, wv, st);
  big_chunk<NF, HALF, 3, false, false, false, FMT>(L, acc, smem, c + 3, wv, st);
  // Epilogue.  Accumulator registers 4q .. 4q+3 of a lane hold rows
  // 8q + 4 g2 + 0..3 of its column m32; a quad transpose turns them into
  // four consecutive columns (m32 & ~3 ..) of row 8q + 4 g2 + (lane & 3), so
  // each lane stores 16 (h: 8) contiguous bytes and one store instruction
  // covers eight row segments.
  const float gsa = p.gs0[t.e - p.e_base], gsb = GATEUP ? p.gs1[t.e - p.e_base] : 0.0f;
  const int n4 = m32 & ~3, j4 = lane & 3;
#pragma unroll
  for (int f = 0; f < NW; f++)
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const int m = 32 * Frags<NF, HALF>::at(f) + 8 * q4 + 4 * g2 + j4;
      if (GATEUP) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; r++) hv[r] = silu(gsa * acc[f][0][4 * q4 + r]) * (gsb * acc[f][1][4 * q4 + r]);
        quad_transpose(hv);
        if (m < t.nvalid) {
          f16x4 o;
#pragma unroll
          for (int r = 0; r < 4; r++) o[r] = (f16)hv[r];
          *reinterpret_cast<f16x4*>(p.h + (size_t)(t.mb + m) * t.N + t.rtile * (BIG_N / 2) + 32 * wr + n4) = o;
        }
      } else {
        // fp16 rows carry the routing weight of their record and are stored
        // in sorted order: a tile's rows are then one contiguous region.
        // (Stored at their records' rows, t*k+j, the 224 rows of a tile are
        // spread over the whole buffer, which made this kernel 20% slower at
        // 8192 tokens, in the K loop as well as in the stores.)
        const float ws = p.rows16 ? reinterpret_cast<const float*>(smem + BIG_OFF_RW)[min(m, BIG_M - 1)] : 1.0f;
#pragma unroll
        for (int nf = 0; nf < 2; nf++) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; r++) v[r] = gsa * acc[f][nf][4 * q4 + r];
          quad_transpose(v);
          if (m < t.nvalid) {
            const size_t col = (size_t)t.rtile * BIG_N + 64 * wr + 32 * nf + n4;
            if (p.rows16) {
              f16x4 o;
#pragma unroll
              for (int r = 0; r < 4; r++) o[r] = (f16)(ws * v[r]);
              *reinterpret_cast<f16x4*>(p.rows16 + (size_t)(t.mb + m) * t.N + col) = o;
            } else {
              *reinterpret_cast<float4*>(p.rows + (size_t)(t.mb + m) * t.N + col) = make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
      }
    }
}

template <bool GATEUP, int FMT>
__global__ __launch_bounds__(BIG_WAVES * WAVE, 1) void expert_gemm_big_kernel(BigParams bp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char big_smem[];
  int32_t* rowoff = reinterpret_cast<int32_t*>(big_smem + BIG_OFF_ROW);
  const GroupedParams& p = bp.g;
  const int n_items = *bp.n_mtiles * bp.n_row_tiles;
  const int per_xcd = (n_items + 7) / 8;
  const int slot = blockIdx.x / 8, item = (blockIdx.x % 8) * per_xcd + slot;
  if (slot >= per_xcd || item >= n_items) return;
  const int mt = bp.mtiles[item / bp.n_row_tiles];
  BigTile t;
  t.rtile = item % bp.n_row_tiles;
  t.e = mt >> 16;
  const int mtile = mt & 0xFFFF;
  // an expert's n records are split evenly over ceil(n / BIG_M) tiles
  const int n_e = p.offsets[t.e + 1] - p.offsets[t.e];
  const int tiles = (n_e + BIG_M - 1) / BIG_M;
  const int ts = (n_e + tiles - 1) / tiles;
  t.mb = p.offsets[t.e] + mtile * ts;
  t.nvalid = min(ts, n_e - mtile * ts);
  t.K = GATEUP ? p.H : p.I;
  t.N = GATEUP ? p.I : p.H;
  // source row (in units of K elements) of every token row of the tile;
  // rows past the count take the zero row after the last token row (x16 row
  // T, h row T k): the padding MFMAs then multiply zeros, which costs the
  // power-limited chip far less energy than real values
  for (int m = threadIdx.x; m < BIG_M; m += BIG_WAVES * WAVE) {
    const int pp = t.mb + min(m, t.nvalid - 1);
    rowoff[m] = m < t.nvalid ? (GATEUP ? p.sorted_pairs[pp] / p.k : pp) : (GATEUP ? p.T : p.T * p.k);
    if (!GATEUP && p.rows16) reinterpret_cast<float*>(big_smem + BIG_OFF_RW)[m] = p.pair_w[p.sorted_pairs[pp]];
  }
  __syncthreads();
  const int nf = (t.nvalid + 31) / 32;  // token fragments, 1 .. 7
  if (threadIdx.x < 4 * WAVE) {
    switch (nf) {
      case 1: big_tile<1, GATEUP, FMT, 0>(p, t, big_smem); break;
      case 2: big_tile<2, GATEUP, FMT, 0>(p, t, big_smem); break;
      case 3: big_tile<3, GATEUP, FMT, 0>(p, t, big_smem); break;
      case 4: big_tile<4, GATEUP, FMT, 0>(p, t, big_smem); break;
      case 5: big_tile<5, GATEUP, FMT, 0>(p, t, big_smem); break;
      case 6: big_tile<6, GATEUP, FMT, 0>(p, t, big_smem); break;
      default: big_tile<BIG_MF, GATEUP, FMT, 0>(p, t, big_smem); break;
    }
  } else {
    switch (nf) {
      case 1: big_tile<1, GATEUP, FMT, 1>(p, t, big_smem); break;
      case 2: big_tile<2, GATEUP, FMT, 1>(p, t, big_smem); break;
      case 3: big_tile<3, GATEUP, FMT, 1>(p, t, big_smem); break;
      case 4: big_tile<4, GATEUP, FMT, 1>(p, t, big_smem); break;
      case 5: big_tile<5, GATEUP, FMT, 1>(p, t, big_smem); break;
      case 6: big_tile<6, GATEUP, FMT, 1>(p, t, big_smem); break;
      default: big_tile<BIG_MF, GATEUP, FMT, 1>(p, t, big_smem); break;
    }
  }
}

// Token batches from this size use the large-tile kernels.  Their tiles
// divide the matrices because the C ABI takes H and I in multiples of 256
// (row tiles of 256 and 128 rows, multiples of four chunks of 64 for the DMA
// rotation), and it bounds T max(H, k I) below 2^31, so that token rows
// (2 T H bytes of x, 2 T k I of h) have 32-bit byte offsets.
constexpr int BIG_MIN_T = 1024;
bool use_big(const FfnArgs& a) { return a.T >= BIG_MIN_T; }

template <bool GATEUP, int FMT>
hipError_t launch_big_fmt(const FfnArgs& a, const GroupedParams& p, hipStream_t s) {
  BigParams bp;
  bp.g = p;
  bp.mtiles = a.mtiles;
  bp.n_mtiles = a.n_mtiles;
  bp.n_row_tiles = GATEUP ? a.I / (BIG_N / 2) : a.H / BIG_N;
  const size_t lds = BIG_LDS;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_gemm_big_kernel<GATEUP, FMT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const long long items = (long long)a.max_mtiles * bp.n_row_tiles;
  const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
  hipLaunchKernelGGL((expert_gemm_big_kernel<GATEUP, FMT>), dim3(grid), dim3(BIG_WAVES * WAVE), lds, s, bp);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_big(const FfnArgs& a, const GroupedParams& p, hipStream_t s) {
  return a.w->format == MOE_FMT_MXFP4 ? launch_big_fmt<GATEUP, FMT_MX>(a, p, s) : launch_big_fmt<GATEUP, FMT_NV>(a, p, s);
}

// Combine: the positions (and weights) of 16 records, then their 16 row
// loads, are issued together before the sums.
constexpr int COMBINE_JB = 16;

// y[t][n] = bf16( sum_j rows16[row(t, j)][n] (+ add) ): the rows already
// carry their routing weights and sit at their records' rows (row(t, j) =
// t*k+j, pos NULL) or at their sorted positions (row(t, j) = pos[t*k+j]);
// fp32 sum over ascending j, then the add_slabs partials in order.  Four
// columns per thread; 16 records' positions, then their 16 row loads, are
// issued together.
__global__ __launch_bounds__(256) void combine16_kernel(const f16* __restrict__ rows,
                                                       const int32_t* __restrict__ pos, int H, int k,
                                                       uint16_t* __restrict__ y,
                                                       const float* __restrict__ add, int add_slabs,
                                                       long long add_stride) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const int t = blockIdx.y;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= H) return;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  for (int j0 = 0; j0 < k; j0 += COMBINE_JB) {
    size_t row[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++) {
      const size_t f = (size_t)t * k + j0 + u;
      row[u] = j0 + u < k ? (pos ? (size_t)pos[f] : f) : 0;
    }
    h4 v[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      v[u] = j0 + u < k ? *reinterpret_cast<const h4*>(rows + row[u] * H + n) : h4{};
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      if (j0 + u < k) {
        a0 += (float)v[u][0];
        a1 += (float)v[u][1];
        a2 += (float)v[u][2];
        a3 += (float)v[u][3];
      }
  }
  if (add) {
    float4 acc = make_float4(a0, a1, a2, a3);
    add_slab_partials4(acc, add + (size_t)t * H + n, add_stride, 0, add_slabs);
    a0 = acc.x;
    a1 = acc.y;
    a2 = acc.z;
    a3 = acc.w;
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
  o.y = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + n) = o;
}

// The same combine for large batches (rows in sorted order, gathered through
// pos): eight columns per thread, each row's 16-byte piece loaded
// non-temporally (the rows are read once, and one wavefront load covers
// eight whole lines), the same fp32 sums in the same order.
__global__ __launch_bounds__(128) void combine16_wide_kernel(const f16* __restrict__ rows,
                                                            const int32_t* __restrict__ pos, int H, int k,
                                                            uint16_t* __restrict__ y, const float* __restrict__ add,
                                                            int add_slabs, long long add_stride) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int t = blockIdx.y;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (n >= H) return;
  float a[8];
#pragma unroll
  for (int c = 0; c < 8; c++) a[c] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += COMBINE_JB) {
    size_t row[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++) row[u] = j0 + u < k ? (size_t)pos[(size_t)t * k + j0 + u] : 0;
    h8 v[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      v[u] = j0 + u < k ? __builtin_bit_cast(h8, load_nt16(reinterpret_cast<const uint8_t*>(rows + row[u] * H + n)))
                        : h8{};
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      if (j0 + u < k)
#pragma unroll
        for (int c = 0; c < 8; c++) a[c] += (float)v[u][c];
  }
  if (add) {
    float4 lo = make_float4(a[0], a[1], a[2], a[3]), hi = make_float4(a[4], a[5], a[6], a[7]);
    add_slab_partials4(lo, add + (size_t)t * H + n, add_stride, 0, add_slabs);
    add_slab_partials4(hi, add + (size_t)t * H + n + 4, add_stride, 0, add_slabs);
    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
    a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(a[4]) | ((uint32_t)f32_to_bf16(a[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(a[6]) | ((uint32_t)f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(y + (size_t)t * H + n) = o;
}

// One share of the experts ([lo, hi)): fp32 unweighted rows; only records
// whose expert lies in the share are summed, in ascending j, into fp32
// partial outputs, and block 0 of each token writes which records it
// served.  The partials of shares that partition the experts add up to the
// whole layer's sum.
__global__ __launch_bounds__(256) void combine_share_kernel(const float* __restrict__ rows,
                                                           const int32_t* __restrict__ pair_pos,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ ids, int lo, int hi, int H,
                                                           int k, float* __restrict__ y,
                                                           uint8_t* __restrict__ served) {
  const int t = blockIdx.y;
  if (served && blockIdx.x == 0)
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
      const int e = ids[(size_t)t * k + j];
      served[(size_t)t * k + j] = (e >= lo && e < hi) ? 1 : 0;
    }
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= H) return;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // 16 records at a time: their ids, weights and positions, then their row
  // loads, are issued together; the sum stays in ascending j
  for (int j0 = 0; j0 < k; j0 += COMBINE_JB) {
    bool in[COMBINE_JB];
    float wj[COMBINE_JB];
    int pos[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++) {
      const int j = j0 + u;
      const int e = j < k ? ids[(size_t)t * k + j] : -1;
      in[u] = e >= lo && e < hi;
      wj[u] = j < k ? w[(size_t)t * k + j] : 0.0f;
      pos[u] = j < k ? pair_pos[(size_t)t * k + j] : 0;
    }
    float4 v[COMBINE_JB];
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      v[u] = in[u] ? *reinterpret_cast<const float4*>(rows + (size_t)pos[u] * H + n) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < COMBINE_JB; u++)
      if (in[u]) {
        a.x = fmaf(wj[u], v[u].x, a.x);
        a.y = fmaf(wj[u], v[u].y, a.y);
        a.z = fmaf(wj[u], v[u].z, a.z);
        a.w = fmaf(wj[u], v[u].w, a.w);
      }
  }
  *reinterpret_cast<float4*>(y + (size_t)t * H + n) = a;
}

GroupedParams base_params(const FfnArgs& a) {
  GroupedParams p{};
  p.T = a.T;
  p.H = a.H;
  p.I = a.I;
  p.k = a.k;
  p.e_base = a.e_base;
  p.offsets = a.offsets;
  p.sorted_pairs = a.sorted_pairs;
  p.active = a.active;
  p.n_active = a.n_active;
  p.h = a.h;
  p.rows = a.rows;
  p.rows16 = a.rows16;
  p.pair_w = a.pair_w;
  return p;
}

// Row tiles per block: gate/up splits K over two wavefronts (two 32-column
// tiles per block); down does not split K (four 64-column tiles per block).
// Measured on MI355X at T = 1, 64 and 256 against splits of 1, 2 and 4.
constexpr int GU_KSPLIT = 2;
constexpr int DN_KSPLIT = 1;

// Measured on MI355X at T = 1, 64 and 256: a two-wavefronts-per-SIMD
// register budget streams fastest.
constexpr int GEMM_WAVES = 2;

// Block scales are staged in LDS when a block's piece (4/KSPLIT row tiles of
// 64 rows) fits in STAGE_MAX bytes: K up to 8192 for gate/up and 4096 for
// down with NVFP4.  Larger K reads them from memory in groups of four chunks.
constexpr int STAGE_MAX = 64 * 1024;

template <int MF, int KSPLIT, bool GATEUP, int WAVES, int FMT, bool R8, int NW = 4>
hipError_t launch_gemm_stage(const GroupedParams& p, dim3 grid, hipStream_t s) {
  const int K = GATEUP ? p.H : p.I;
  const int bytes = (NW / KSPLIT) * 64 * (K / (FMT == FMT_MX ? 32 : 16));
  if (bytes <= STAGE_MAX) {
    const void* f = reinterpret_cast<const void*>(&expert_gemm_kernel<MF, KSPLIT, GATEUP, WAVES, FMT, true, R8, NW>);
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, STAGE_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((expert_gemm_kernel<MF, KSPLIT, GATEUP, WAVES, FMT, true, R8, NW>), grid, dim3(NW * WAVE),
                       bytes, s, p);
  } else {
    hipLaunchKernelGGL((expert_gemm_kernel<MF, KSPLIT, GATEUP, WAVES, FMT, false, R8, NW>), grid, dim3(NW * WAVE), 0,
                       s, p);
  }
  return hipGetLastError();
}

// Small batches (below BIG_MIN_T tokens) take tokens in passes of one
// 16-token fragment, which keeps two wavefronts per SIMD resident; an expert
// with more tokens takes several passes, the later ones re-reading its
// weights from the caches.  Code loads in whole lines (R8) for gate/up at
// every small batch, and for down while every expert has at most 16 records
// (one token pass): T <= 16.
template <int KSPLIT, bool GATEUP, int FMT>
hipError_t launch_gemm_fmt(const GroupedParams& p, int T, dim3 grid, hipStream_t s) {
  return GATEUP || T <= 16 ? launch_gemm_stage<1, KSPLIT, GATEUP, GEMM_WAVES, FMT, true>(p, grid, s)
                           : launch_gemm_stage<1, KSPLIT, GATEUP, GEMM_WAVES, FMT, false>(p, grid, s);
}

template <int KSPLIT, bool GATEUP>
hipError_t launch_gemm(const GroupedParams& p, int T, dim3 grid, hipStream_t s, int fmt) {
  return fmt == MOE_FMT_MXFP4 ? launch_gemm_fmt<KSPLIT, GATEUP, FMT_MX>(p, T, grid, s)
                              : launch_gemm_fmt<KSPLIT, GATEUP, FMT_NV>(p, T, grid, s);
}

// Down GEMM of a single-pass batch (T <= 16) whose k <= 16 experts' H rows
// split into 7 row tiles of 64 per block: blocks of seven wavefronts, H / 448
// blocks per expert.  At 16 active experts and H = 7168 that is 256 blocks,
// one per CU, each streaming the same bytes; blocks of four wavefronts (448
// of them) leave 64 CUs with half the work of the others.
// Only where the block's scales fit the LDS staging (I up to 2304 for NVFP4):
// reading them from memory instead costs more than the balance gains.
constexpr int DN_WIDE_NW = 7;
bool down_wide(const FfnArgs& a) {
  const int scale_bytes = DN_WIDE_NW * 64 * (a.I / (a.w->format == MOE_FMT_MXFP4 ? 32 : 16));
  return a.T <= 16 && a.H % (64 * DN_WIDE_NW) == 0 && (long long)a.max_active * (a.H / (64 * DN_WIDE_NW)) <= 256 &&
         scale_bytes <= STAGE_MAX;
}

// The zero rows that the large-tile GEMMs' padding rows read: x16 row T
// (H halves) and h row T k (I halves).
__global__ __launch_bounds__(256) void zero_rows_kernel(f16* __restrict__ x_row, int H, f16* __restrict__ h_row,
                                                       int I) {
  for (int i = threadIdx.x; i < H / 8; i += 256) reinterpret_cast<uint4*>(x_row)[i] = make_uint4(0, 0, 0, 0);
  for (int i = threadIdx.x; i < I / 8; i += 256) reinterpret_cast<uint4*>(h_row)[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

bool pads_with_zero_rows(const FfnArgs& a) { return use_big(a); }

hipError_t launch_zero_pad_rows(const FfnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(zero_rows_kernel, dim3(1), dim3(256), 0, s, const_cast<f16*>(a.x16) + (size_t)a.T * a.H, a.H,
                     a.h + (size_t)a.T * a.k * a.I, a.I);
  return hipGetLastError();
}

hipError_t launch_gateup(const FfnArgs& a, hipStream_t s) {
  GroupedParams p = base_params(a);
  p.a = a.x16;
  p.q0 = a.w->gate.q;
  p.sf0 = a.w->gate.sf;
  p.gs0 = a.w->gate.gs;
  p.q1 = a.w->up.q;
  p.sf1 = a.w->up.sf;
  p.gs1 = a.w->up.gs;
  if (use_big(a)) return launch_big<true>(a, p, s);
  const dim3 grid(a.I / (32 * (4 / GU_KSPLIT)), a.max_active);
  return launch_gemm<GU_KSPLIT, true>(p, a.T, grid, s, a.w->format);
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  GroupedParams p = base_params(a);
  p.a = a.h;
  p.q0 = a.w->down.q;
  p.sf0 = a.w->down.sf;
  p.gs0 = a.w->down.gs;
  if (use_big(a)) return launch_big<false>(a, p, s);
  if (down_wide(a)) {
    const dim3 grid(a.H / (64 * DN_WIDE_NW), a.max_active);
    return a.w->format == MOE_FMT_MXFP4
               ? launch_gemm_stage<1, 1, false, GEMM_WAVES, FMT_MX, true, DN_WIDE_NW>(p, grid, s)
               : launch_gemm_stage<1, 1, false, GEMM_WAVES, FMT_NV, true, DN_WIDE_NW>(p, grid, s);
  }
  const dim3 grid(a.H / (64 * (4 / DN_KSPLIT)), a.max_active);
  return launch_gemm<DN_KSPLIT, false>(p, a.T, grid, s, a.w->format);
}

bool rows16_sorted(int T) { return T >= BIG_MIN_T; }

hipError_t launch_combine16(const f16* rows, const int32_t* pair_pos, int T, int H, int k, uint16_t* y,
                            hipStream_t s, const float* add, int add_slabs) {
  const int32_t* pos = rows16_sorted(T) ? pair_pos : nullptr;
  if (pos && H % 8 == 0) {
    hipLaunchKernelGGL(combine16_wide_kernel, dim3((H / 8 + 127) / 128, T), dim3(128), 0, s, rows, pos, H, k, y, add,
                       add_slabs, (long long)T * H);
    return hipGetLastError();
  }
  const int threads = T < 64 ? 64 : 256;
  hipLaunchKernelGGL(combine16_kernel, dim3((H / 4 + threads - 1) / threads, T), dim3(threads), 0, s, rows, pos, H,
                     k, y, add, add_slabs, (long long)T * H);
  return hipGetLastError();
}

hipError_t launch_combine_share(const float* rows, const int32_t* pair_pos, const float* w, const int32_t* ids,
                                int lo, int hi, int T, int H, int k, float* y, uint8_t* served, hipStream_t s) {
  const int threads = T < 64 ? 64 : 256;
  hipLaunchKernelGGL(combine_share_kernel, dim3((H / 4 + threads - 1) / threads, T), dim3(threads), 0, s, rows,
                     pair_pos, w, ids, lo, hi, H, k, y, served);
  return hipGetLastError();
}


}  // namespace moe
