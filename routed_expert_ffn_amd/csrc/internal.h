// Host-side interface between the C ABI (api.hip) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "moe.h"

namespace moe {

// The router's partial sums over H: slabs of slab_rows rows each.
struct RouterPlan {
  bool mfma;   // bf16 matrix-core GEMM (larger T) or the VALU GEMV
  bool tiled;  // the LDS-tiled GEMM of large batches
  int slabs, slab_rows;
  int e_tile;  // the GEMV's outputs per block
};
RouterPlan router_plan(int T, int H, int E);

// The LDS-tiled bf16 GEMM of large batches: x [T][K] . w [K][N] (w
// input-major, read as stored) over `slabs` K slabs of kslab rows.  Writes
// the fp32 slab partials part [slab][T][N]; or, with part NULL and one slab,
// out [T][N] bf16 and, when non-NULL, its fp16 copy out16.  x16, when
// non-NULL, receives the fp16 copy of x.
struct DensePlan {
  bool tiled;
  int slabs, kslab;
};
DensePlan dense_plan(int T, int K, int N);
hipError_t launch_dense_tiled(const uint16_t* x, const uint16_t* w, int T, int K, int N, const DensePlan& dp,
                              float* part, uint16_t* out, f16* out16, f16* x16, hipStream_t s);
// The permutation works on blocks of 64 tokens (one wavefront each).
inline int perm_blocks(int T) { return (T + 63) / 64; }
// Largest number of distinct experts that T tokens can select.
inline int max_active(const moe_dims& d) {
  long long p = (long long)d.T * d.k;
  return (int)(p < d.E ? p : d.E);
}

// Kernel-timing hook (see moe_profile_arm).
void prof_before(moe_kernel k, hipStream_t s);
void prof_after(moe_kernel k, hipStream_t s);

// Launchers.  Each enqueues on `s` and returns hipGetLastError().
// With x16 non-NULL the router also writes the fp16 copy of x [T][H].
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, float* part, int T, int H, int E,
                         const RouterPlan& rp, hipStream_t s, f16* x16 = nullptr);
// Sums the slab partials (part may be NULL: logits are then an input), adds
// the bias, and selects the top k with their softmax weights.
hipError_t launch_topk(const float* part, int slabs, const float* bias, float* logits, int T, int E, int k,
                       int32_t* ids, float* w, hipStream_t s);
// Offsets, permutation, active-expert list and (for T > 64) the list of
// (expert, token tile) entries.
// T small enough for the single-launch routing kernel.
bool route_fused(int T);
// Logits reduction, top-k, permutation and active list in one launch (T <=
// the fused limit).
hipError_t launch_route_small(const float* part, int slabs, const float* bias, float* logits, int T, int E, int k,
                              int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                              int32_t* active, int32_t* n_active, hipStream_t s);
// Ids outside [0, E) (by convention -1) are masked: not counted, no
// position (pair_pos -1), offsets[E] = the served records.
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, uint64_t* masks, int32_t* counts, int32_t* base,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active,
                          int32_t* n_active, int32_t* mtiles, int32_t* n_mtiles, hipStream_t s);
// Active list and (expert, token tile) entries of the experts in [lo, hi).
hipError_t launch_active_list(const int32_t* offsets, int E, int lo, int hi, int32_t* active, int32_t* n_active,
                              int32_t* mtiles, int32_t* n_mtiles, hipStream_t s);
// Token tile of the large-batch expert GEMMs: an expert's records are split
// evenly over ceil(n / MTILE) tiles.
constexpr int MTILE = 224;

// Upper bound on the (expert, token tile) entries of T tokens.
inline int max_mtiles(const moe_dims& d) { return max_active(d) + (int)(((long long)d.T * d.k) / MTILE) + 1; }
hipError_t launch_cast(const uint16_t* x, f16* x16, long long n, hipStream_t s);
// local[f] = map[ids[f]] for the n records (-1 where the expert is served
// elsewhere, or the map entry is outside [0, n_local)).
hipError_t launch_remap_ids(const int32_t* ids, const int32_t* map, int E, int n_local, long long n, int32_t* local,
                            hipStream_t s);

struct FfnArgs {
  int T, H, I, E, k;
  int e_base;                     // first expert of the store (weights of e at e - e_base)
  // x16 holds T + 1 rows and h P + 1: the last row of each is zeroed before
  // the large-tile GEMMs (pads_with_zero_rows), whose token tiles fill their
  // padding rows from it
  int max_active;                 // grid bound on the number of active experts
  const f16* x16;                 // [T][H]
  const int32_t* offsets;         // [E+1]
  const int32_t* sorted_pairs;    // [P]
  const int32_t* active;          // [max_active] expert ids with work
  const int32_t* n_active;        // [1]
  const int32_t* mtiles;          // (expert, token tile) entries
  const int32_t* n_mtiles;        // [1]
  int max_mtiles;                 // grid bound on the entries
  const moe_experts* w;
  f16* h;                         // [P][I]
  float* rows;                    // [P][H] fp32, unweighted (when rows16 is NULL)
  f16* rows16;                    // or [P][H] fp16 times its routing weight, at rows16_sorted(T) ? sorted position
                                  // : record (t*k+j)
  const float* pair_w;            // routing weights [T*k] for rows16
};
bool pads_with_zero_rows(const FfnArgs& a);
hipError_t launch_zero_pad_rows(const FfnArgs& a, hipStream_t s);
hipError_t launch_gateup(const FfnArgs& a, hipStream_t s);
hipError_t launch_down(const FfnArgs& a, hipStream_t s);
// The down GEMM's weighted fp16 rows of T tokens are in sorted order (row p)
// when this holds (the large-tile kernel), else in record order (row t*k+j).
bool rows16_sorted(int T);
// Combine of the weighted fp16 rows: y = bf16(sum_j rows16[row(t, j)] (+
// add)), row(t, j) = pair_pos[t*k+j] or t*k+j as rows16_sorted(T) says, add
// (may be NULL) being add_slabs fp32 partials [T][H] summed after the records
// (the shared experts' output).
hipError_t launch_combine16(const f16* rows, const int32_t* pair_pos, int T, int H, int k, uint16_t* y,
                            hipStream_t s, const float* add = nullptr, int add_slabs = 0);
// One share of the experts: only records whose expert is in [lo, hi) are
// summed, into fp32 partial outputs; served[t*k+j] (may be NULL) = 1 for
// those records, 0 for the others.
hipError_t launch_combine_share(const float* rows, const int32_t* pair_pos, const float* w, const int32_t* ids,
                                int lo, int hi, int T, int H, int k, float* y, uint8_t* served, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16) into at most
// STREAM_SINK_WORDS per-block XOR words.
constexpr int STREAM_SINK_WORDS = MOE_STREAM_SINK_WORDS;
hipError_t launch_stream_read(const void* buf, long long bytes, uint32_t* sink, hipStream_t s);
// Sustained fp16 MFMA on the expert GEMMs' value patterns: MOE_MFMA_RATE_BLOCKS
// blocks of eight wavefronts, `iters` rounds of four MFMAs each.
hipError_t launch_mfma_rate(int iters, float* sink, hipStream_t s);

// x [T][K] . w [K][N] (bf16, input-major) into out [T][N] bf16 and, if
// out16 is non-NULL, its fp16 copy; part holds rp.slabs * T * N fp32 (unused
// by a tiled plan of one slab).
hipError_t launch_projection(const uint16_t* x, const uint16_t* w, float* part, int T, int K, int N,
                             const RouterPlan& rp, uint16_t* out, f16* out16, hipStream_t s);

// Shared experts' hidden layer: h [T][count*I] bf16 from x [T][H] and the
// gate/up weights [H][count*2I]; part holds rp.slabs * T * 2*count*I fp32.
hipError_t launch_shared_hidden(const uint16_t* x, const uint16_t* w_gate_up, float* part, int T, int H, int count,
                                int I, const RouterPlan& rp, uint16_t* h, hipStream_t s);

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, uint32_t* ws,
                           hipStream_t s);
hipError_t launch_quantize_mx(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, uint32_t* ws,
                              hipStream_t s);

}  // namespace moe
