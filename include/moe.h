/* moe.h - C ABI of libmoe.so: the routed mixture-of-experts layer with NVFP4
 * experts on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (the pages this follows):
 *   - a router scores every token against E experts and picks k of them
 *     (16 of 896 in Kimi-K3: al-engr.com Kimi-K3 NVFP4 plan, table "What we
 *     verified today"; "Computation and Data Movement for Inference",
 *     section 3.4 "Decode experts");
 *   - the route records are sorted by expert so that one load of an
 *     expert's weights serves its whole bucket (same essay, section 4 "The
 *     flow of an MoE prefill layer" and section 15 "Prefill and midfill
 *     turn sparse routing into dense expert batches");
 *   - each selected expert runs its three matrices (gate, up, down:
 *     "Serving Kimi-K3 ... with 8xB300 GPUs", section "The model, as the
 *     serving system sees it") as a SwiGLU FFN on NVFP4 weights (e2m1
 *     values, an e4m3 scale per 16 values, a per-expert fp32 global scale:
 *     al-engr.com plan, section "What has to be built - and the discovery
 *     that changed it"; "Serving Kimi-K3", section "Number formats on
 *     Blackwell");
 *   - the expert outputs go back to token order, weighted and summed
 *     (essay, sections 4 and 5).
 * The entry points mirror that statement of the problem: prepare
 * (moe_route), compute (moe_expert_ffn), and the whole layer (moe_layer).
 * The al-engr.com plan splits its expert call the same way, into a prepare
 * step, the expert compute and a finalize step (section "What has to be
 * built - and the discovery that changed it"), and its expert workers are
 * handed a token's global expert ids and send back one row per expert
 * (section "Track A - the Spark tier, starting now").
 *
 * Conventions for every entry point:
 *   - Pointers named d_* or documented as device pointers point to device
 *     memory that the caller owns and keeps alive until the enqueued work
 *     has finished; the library never allocates device memory, frees it
 *     or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream).  Calls are asynchronous and may be captured in a
 *     HIP graph.  moe_layer_shared runs the shared experts, which do not
 *     depend on the routing, on a second stream of the library, which waits
 *     for what was enqueued on `stream` before the call and which `stream`
 *     waits for before their result is read, so ordering towards the caller
 *     is as if everything ran on `stream`.  That stream and its two events are
 *     created once per device, with default priority, by the first such
 *     call whose stream is not being captured, and live until the process
 *     ends; a call before that, or one whose `stream` belongs to another
 *     device than the current one, runs everything on `stream`.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK return nothing was launched and moe_last_error() says why.  A
 *     launch failure returns MOE_ERR_HIP; outputs are then undefined.
 *   - No C++ exception crosses this boundary.
 *   - Same inputs on the same GPU give bit-identical outputs: there are no
 *     floating-point atomics.
 *   - Shape limits: 1 <= k <= 64, k <= E <= 1024 with E a multiple of 8,
 *     H and I multiples of 256, 0 <= T <= 65535 and T * max(H, k*I) < 2^31
 *     (at H = 7168, I = 2048, k = 16: T <= 65535).  moe_permute,
 *     moe_expert_ffn and moe_workspace_bytes, which take expert ids rather
 *     than route, accept any 1 <= E <= 1024 (e.g. one device's experts).  T = 0 is a no-op
 *     returning MOE_OK once the dimensions are valid (pointers are then not
 *     examined).
 *   - Pointers must be 16-byte aligned, except the per-tensor scales gs
 *     of moe_nvfp4 (4-byte aligned, so that a share of a store can point
 *     into it) and the uint8 outputs.
 *   - Activations (x) must be finite with |x| < 65504, and so must the
 *     intermediate h = SiLU(x.W_gate)*(x.W_up): the expert GEMMs run on
 *     fp16 matrix cores (the NVFP4 products are exact in fp16; see the
 *     design notes).  Outside that range results are inf/NaN, not silently
 *     wrong.  x's bf16 values are exact in fp16 from 2^-17 up; smaller
 *     magnitudes fall in fp16's subnormal range and are rounded to a
 *     multiple of 2^-24 (an error of at most 2^-25 each). */
#ifndef MOE_H
#define MOE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,       /* NULL pointer where one is required, bad enum */
  MOE_ERR_SHAPE = 2,     /* dimensions outside the limits above          */
  MOE_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned             */
  MOE_ERR_WORKSPACE = 4, /* ws_bytes smaller than the size required      */
  MOE_ERR_HIP = 5        /* a HIP launch failed                          */
} moe_status;

/* T tokens, H hidden size, I expert intermediate size, E experts, k experts
 * per token. */
typedef struct {
  int32_t T, H, I, E, k;
} moe_dims;

/* One NVFP4 matrix per expert, stacked over the E experts.  For a logical
 * weight W[N][K] (N outputs, K the reduction axis):
 *   q  [E][N][K/2]  e2m1 codes, two per byte, element k even in the low
 *                   nibble; code = sign(bit 3) | exponent(bits 2:1, bias 1)
 *                   | mantissa(bit 0): magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
 *   sf [E][N][K/16] OCP e4m3 (E4M3FN) scale of 16 consecutive k of a row
 *   gs [E]          fp32 per-tensor global scale
 * Dequantised weight: W[n][k] = e2m1(q) * e4m3(sf) * gs. */
typedef struct {
  const uint8_t* q;
  const uint8_t* sf;
  const float* gs;
} moe_nvfp4;

/* Weight formats of a store.  MXFP4 (the OCP microscaling format; [p2]
 * "Number formats on Blackwell": K3's experts were trained in it) uses the
 * same moe_nvfp4 fields with
 *   sf [E][N][K/32] e8m0 scale 2^(sf - 127) of 32 consecutive k of a row
 *                   (255, NaN, is out of contract),
 *   gs [E]          a power of two 2^r per matrix: the fp16 dequantisation
 *                   computes e2m1 * 2^(sf - 127 - r), exact for block scales
 *                   within 2^8 .. 2^-23 of 2^r, and gs is multiplied back in
 *                   fp32.  moe_quantize_mxfp4 sets r = smax - 135 (smax the
 *                   largest scale byte), which keeps every block within 31
 *                   binades of the largest exact.
 * Dequantised weight: W[n][k] = e2m1(q) * 2^(sf - 127).  Every entry point
 * and GEMM variant takes either format. */
typedef enum { MOE_FMT_NVFP4 = 0, MOE_FMT_MXFP4 = 1 } moe_weight_format;

/* gate and up: N = I, K = H.  down: N = H, K = I.  All device pointers.
 * format: a moe_weight_format (0, NVFP4, when left zero). */
typedef struct {
  moe_nvfp4 gate, up, down;
  int32_t format;
} moe_experts;

/* Bytes of device workspace that moe_route, moe_expert_ffn and moe_layer
 * need for dims d (the same figure serves all three; 0 if d is invalid). */
size_t moe_workspace_bytes(moe_dims d);

/* Quantise one fp32 matrix w[N][K] (device) to NVFP4 (device outputs q
 * [N][K/2], sf [N][K/16], gs [1]), the weight store the FFN reads.
 * Rule (fp32, divisions correctly rounded): amax = max|w|; gs = amax/2688
 * (= 6 * 448; 1 if amax = 0); per 16-element block along K:
 * sf = e4m3_rne((blockmax / 6) / gs), saturating at 448; d = e4m3(sf) * gs;
 * code = nearest e2m1 to |w|/d, ties to the even code, saturating at 6;
 * sign bit only for w < 0 with a non-zero code; sf = 0 gives zero codes.
 * The pages give the format but not the rounding rule; this is the reading
 * taken.  Needs K % 16 == 0, N >= 1 and a workspace of at least
 * moe_quantize_workspace_bytes() bytes. */
size_t moe_quantize_workspace_bytes(void);
moe_status moe_quantize_nvfp4(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, void* ws,
                              size_t ws_bytes, void* stream);

/* Quantise one fp32 matrix w[N][K] (device) to MXFP4 (device outputs q
 * [N][K/2], sf [N][K/32], gs [1]), following the OCP MX specification's
 * conversion: per 32-element block along K, with blockmax the largest |w|,
 * sf = floor(log2(blockmax)) - 2 + 127 clamped to 0 .. 254 (X = 2^(sf-127));
 * code = nearest e2m1 to |w| / X, ties to the even code, clamped to 6; a
 * zero block gets sf = 0 and zero codes.  gs = 2^(smax - 135), smax the
 * scale of the matrix's largest |w| (see moe_weight_format).  Needs
 * K % 32 == 0, N >= 1 and a workspace as moe_quantize_nvfp4. */
moe_status moe_quantize_mxfp4(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, void* ws,
                              size_t ws_bytes, void* stream);

/* Route T tokens (device pointers):
 *   x              [T][H] bf16 activations, or NULL: then `logits` is an
 *                  input (fp32 [T][E]) and the router GEMM is skipped;
 *   w_router       [H][E] bf16 router weight (ignored when x is NULL);
 *   bias           [E] fp32 added to the logits, or NULL (ignored when x
 *                  is NULL: given logits are used as they are);
 *   logits         [T][E] fp32: logits = x.W_r + bias (fp32 accumulation);
 *   topk_ids       [T][k] int32: the k largest logits in the order (logit
 *                  descending, expert index ascending), so ties go to the
 *                  lower index;
 *   topk_w         [T][k] fp32: softmax over the k selected logits, which
 *                  equals softmax over all E then renormalising the k;
 *   expert_offsets [E+1] int32: exclusive prefix sum of per-expert counts;
 *   sorted_pairs   [T*k] int32: route records f = t*k + j in (expert,
 *                  token) order;
 *   pair_pos       [T*k] int32: inverse of sorted_pairs.
 * ids, offsets and the permutation are exact functions of the fp32
 * logits. */
moe_status moe_route(moe_dims d, const void* x, const void* w_router, const float* bias, float* logits,
                     int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                     int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream);

/* Build the expert-order permutation from ids the caller holds (device
 * pointers): topk_ids [T][k] int32, each an expert id in [0, E) or masked.
 * al-engr.com Kimi-K3 plan, section "What has to be built - and the
 * discovery that changed it": splitting one model's experts across devices
 * takes a mask on the router's chosen ids, an id of -1 standing for an
 * expert that another device serves.  A record whose id lies outside
 * [0, E) (by convention -1) is masked: it is not counted and takes no
 * position.  Outputs:
 *   expert_offsets [E+1]: exclusive prefix sum of the per-expert counts of
 *                  the served records (expert_offsets[E] = the number of
 *                  served records, T*k when none is masked);
 *   sorted_pairs   [T*k]: the served records f = t*k + j in (expert, token)
 *                  order, positions 0 .. expert_offsets[E]-1; the entries
 *                  from expert_offsets[E] on are left as they were;
 *   pair_pos       [T*k]: position of record f in sorted_pairs, -1 if masked.
 * The result is an exact function of the ids (moe_route builds the same
 * permutation from its own ids, none masked).  moe_expert_ffn takes it as it
 * is and computes only the served records.  Workspace as moe_route (dims d,
 * E being the size of the id space, e.g. a device's own experts). */
moe_status moe_permute(moe_dims d, const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pairs,
                       int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream);

/* Run every selected expert on its bucket (device pointers):
 *   x              [T][H] bf16 activations;
 *   expert_offsets [E+1], sorted_pairs [T*k]: as produced by moe_route or
 *                  moe_permute; only the records at positions
 *                  0 .. expert_offsets[E]-1 are computed (masked records
 *                  have none);
 *   w              NVFP4 experts (the struct itself is host memory, read
 *                  during the call only);
 *   rows           [T*k][H] fp32 output: rows[p] = SwiGLU FFN of expert e
 *                  on token sorted_pairs[p]/k, for p in e's bucket, i.e.
 *                  (SiLU(x.Wg) * (x.Wu)).Wd, unweighted, in sorted order. */
moe_status moe_expert_ffn(moe_dims d, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                          const moe_experts* w, float* rows, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: y[t] = sum_j topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t]):
 * each weighted term is stored in fp16 (|term| < 65504), the terms are
 * summed in fp32 over ascending j and the sum is rounded to bf16 (device
 * pointers):
 *   x [T][H] bf16, w_router [H][E] bf16, bias [E] fp32 or NULL,
 *   y [T][H] bf16 output,
 *   topk_ids_out [T][k] int32 / topk_w_out [T][k] fp32: optional copies of
 *   the routing (NULL to skip). */
moe_status moe_layer(moe_dims d, const void* x, const void* w_router, const float* bias, const moe_experts* w,
                     void* y, int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* ---- the layer without a caller workspace -----------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_layer
 * with its workspace taken from a scratch array of MOE_NOALLOC_SCRATCH_BYTES
 * that the library holds in device memory, one per device, until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); the caller still passes the inputs and outputs, as for
 * moe_layer, and gets the same results.
 *   - Limit: the layer's workspace without the fp32 rows of moe_expert_ffn
 *     (about half of moe_workspace_bytes) must fit the scratch; at H = 7168,
 *     I = 2048, E = 896, k = 16 that holds up to T = 156 tokens.  Larger
 *     calls return MOE_ERR_WORKSPACE before anything is enqueued.
 *   - The first call on a device looks up that device's scratch address
 *     (with the device current; `stream` must belong to the current device,
 *     else MOE_ERR_ARG); make that first call outside graph capture.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that
 *     overlap on one GPU (on different streams, or from several host threads
 *     without ordering) race and give undefined results.
 * Errors as moe_layer. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_noalloc(moe_dims d, const void* x, const void* w_router, const float* bias, const moe_experts* w,
                             void* y, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* ---- shared experts ------------------------------------------------------------
 * wpnews.pro, "Serving Kimi K3 End to End", section 3.3: every token also
 * uses the model's 2 shared experts, whose output joins the MoE layer's sum;
 * "Serving Kimi-K3 ... with 8xB300 GPUs", "Precision: what is stored in which
 * format": they are kept in bf16.  Each shared expert s is a dense SwiGLU
 * FFN of intermediate width I: g, u = x . Wgu (columns 2sI .. 2sI+I-1 and
 * 2sI+I .. 2sI+2I-1), h = bf16(SiLU(g) * u) (g, u accumulated in fp32),
 * out_s = h . Wd (rows sI .. sI+I-1), accumulated in fp32. */
typedef struct {
  int32_t count;          /* shared experts (K3: 2), >= 1 */
  int32_t I;              /* intermediate width of each: a positive multiple of 256 */
  const void* w_gate_up;  /* [H][count*2*I] bf16, device, input-major */
  const void* w_down;     /* [count*I][H] bf16, device, input-major */
} moe_shared;

/* Workspace of moe_layer_shared (0 for invalid dims or shared experts). */
size_t moe_layer_shared_workspace_bytes(moe_dims d, const moe_shared* shared);

/* moe_layer plus the shared experts (device pointers as moe_layer; shared
 * is host memory read during the call):
 *   y[t] = bf16( sum_j topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t]) + sum_s out_s(x[t]) ),
 * the routed sum in fp32 over ascending j, then the shared experts' fp32
 * output, rounded once.  MOE_KERNEL_SHARED times the shared experts' launches.
 * Errors as moe_layer, plus MOE_ERR_ARG (NULL shared or weights) and
 * MOE_ERR_SHAPE (count < 1 or I not a positive multiple of 256). */
moe_status moe_layer_shared(moe_dims d, const moe_shared* shared, const void* x, const void* w_router,
                            const float* bias, const moe_experts* w, void* y, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream);

/* ---- one share of the experts (expert parallelism) ---------------------------
 * al-engr.com Kimi-K3 plan, section "What has to be built - and the
 * discovery that changed it": splitting one model's experts across devices
 * takes a mask on the router's chosen ids and a routed kernel that takes a
 * local expert offset; section "Track A": an expert worker takes global
 * expert ids and returns rows plus the ids it actually served, so that every
 * token's experts are accounted for exactly once.  Here a share is the
 * contiguous range [base, base + count) of the E experts, and its store
 * holds those count experts only (store entry i is expert base + i).
 * Routing (moe_route, or the routing inside moe_layer_share) is over all E
 * experts, unchanged. */
typedef struct {
  int32_t base, count;
} moe_expert_share;

/* moe_expert_ffn for one share: rows[p] for the records p of the share's
 * experts, which are the contiguous range expert_offsets[base] ..
 * expert_offsets[base + count) of the sorted order; other rows are left as
 * they were.  w holds the share's count experts.  Errors as moe_expert_ffn,
 * plus MOE_ERR_SHAPE for a share that is empty or not inside [0, E). */
moe_status moe_expert_ffn_share(moe_dims d, moe_expert_share share, const void* x, const int32_t* expert_offsets,
                                const int32_t* sorted_pairs, const moe_experts* w, float* rows, void* ws,
                                size_t ws_bytes, void* stream);

/* moe_layer for one share: routing over all E experts, the share's experts
 * on their records, and (device pointers)
 *   y_partial [T][H] fp32: sum, over ascending j with topk_ids[t][j] in the
 *             share, of topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t]), in fp32;
 *   served    [T][k] uint8 or NULL: 1 where this share computed record
 *             (t, j), else 0 (summed over a partition of the experts: all 1).
 * The partials of shares that partition the experts add up to moe_layer's
 * sum; rounding that total to bf16 is left to the caller (after the
 * reduction across devices).  Workspace as moe_layer. */
moe_status moe_layer_share(moe_dims d, moe_expert_share share, const void* x, const void* w_router, const float* bias,
                           const moe_experts* w, float* y_partial, uint8_t* served, int32_t* topk_ids_out,
                           float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* moe_layer for the experts one device holds, in any placement: routing
 * over all E experts, then the mask on the chosen ids (al-engr.com plan,
 * section "What has to be built - and the discovery that changed it": the
 * split hook maps the router's global ids to this device's rows and masks
 * the rest to -1), the device's experts on their records, and its partial
 * output (device pointers):
 *   expert_map    [E] int32: slot in w of global expert e (0 .. n_local-1),
 *                 or -1 when another device serves e (an entry outside
 *                 [0, n_local) counts as -1); distinct experts should have
 *                 distinct slots;
 *   w             the n_local experts of this device, in slot order;
 *   y_partial     [T][H] fp32: sum, over ascending j with expert_map of
 *                 topk_ids[t][j] a slot, of topk_w[t][j] *
 *                 FFN_{topk_ids[t][j]}(x[t]), in fp32;
 *   served        [T][k] uint8 or NULL: 1 where this device computed record
 *                 (t, j), else 0;
 *   local_ids_out [T][k] int32 or NULL: the chosen ids as slots, -1 masked
 *                 ("Track A": a worker returns rows plus the ids it served).
 * Devices whose maps partition the experts produce partials that add up to
 * moe_layer's sum; rounding the total to bf16 is left to the caller.
 * moe_layer_share is the special case of a contiguous range.  Workspace as
 * moe_layer (dims d with the global E).  Errors as moe_layer, plus
 * MOE_ERR_SHAPE for n_local outside [1, E] and MOE_ERR_ARG for a NULL map. */
moe_status moe_layer_mapped(moe_dims d, const int32_t* expert_map, int32_t n_local, const void* x,
                            const void* w_router, const float* bias, const moe_experts* w, float* y_partial,
                            uint8_t* served, int32_t* topk_ids_out, float* topk_w_out, int32_t* local_ids_out,
                            void* ws, size_t ws_bytes, void* stream);

/* ---- the latent routed-expert block (K3's LatentMoE) -------------------------
 * lightseek.org, "Kimi K3 optimization on GB300" (part I), sections
 * "Routed-down projection: column sharding and latent assembly" and
 * "Routed-up projection: sharding the post-expert tail": each MoE block
 * projects the model's hidden state (width H_model, 7168 in K3) into the
 * routed latent (width d.H, 3584) with a bf16 weight, runs the routed
 * experts there (I = 3072), and projects their combined output back:
 *   z     = bf16(x . w_down)                      [T][d.H]
 *   route = top-k of the router on x              (the hidden state)
 *   y_lat = bf16(sum_j w_j * FFN_{id_j}(z))       as moe_layer, on z
 *   y     = bf16(y_lat . w_up)                    [T][H_model]
 * Projections accumulate in fp32.  Weights are stored input-major (the
 * transpose of a [out][in] linear weight), as w_router is.
 * MOE_KERNEL_PROJECT times each projection (its GEMM and the reduction). */
typedef struct {
  int32_t H_model;     /* hidden width: a positive multiple of 256 */
  const void* w_down;  /* [H_model][H] bf16, device */
  const void* w_up;    /* [H][H_model] bf16, device */
} moe_latent;

/* Workspace of moe_latent_layer (0 for invalid dims or H_model). */
size_t moe_latent_workspace_bytes(moe_dims d, int32_t H_model);

/* Device pointers: x [T][H_model] bf16; w_router [H_model][E] bf16; bias
 * [E] fp32 or NULL; y [T][H_model] bf16 output; z_out [T][H] bf16 copy of
 * the routed latent or NULL; topk_ids_out / topk_w_out as in moe_layer.
 * lat is host memory read during the call.  Errors as moe_layer, plus
 * MOE_ERR_ARG for a NULL lat or projection and MOE_ERR_SHAPE for H_model. */
moe_status moe_latent_layer(moe_dims d, const moe_latent* lat, const void* x, const void* w_router, const float* bias,
                            const moe_experts* w, void* y, void* z_out, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream);

const char* moe_status_string(moe_status s);
/* Detail of the last non-OK return on the calling thread. */
const char* moe_last_error(void);

/* ---- kernel timing for measurement ----------------------------------------
 * Kernels of the path, in launch order within moe_layer. */
typedef enum {
  MOE_KERNEL_ROUTER = 0,  /* router logits (slab partials + reduction)   */
  MOE_KERNEL_TOPK = 1,    /* softmax + top-k; for T <= 8 one launch that  */
                          /* also permutes (nothing is then PERMUTE)     */
  MOE_KERNEL_PERMUTE = 2, /* histogram, scan and scatter (three kernels) */
  MOE_KERNEL_CAST = 3,    /* activations bf16 -> fp16                    */
  MOE_KERNEL_GATEUP = 4,  /* grouped gate/up GEMM + SiLU*mul             */
  MOE_KERNEL_DOWN = 5,    /* grouped down GEMM                           */
  MOE_KERNEL_COMBINE = 6, /* weighted un-permute and sum                 */
  MOE_KERNEL_PROJECT = 7, /* latent block: one bf16 projection            */
  MOE_KERNEL_SHARED = 8,  /* shared experts: gate/up + SwiGLU, then down  */
  MOE_KERNEL_COUNT = 9
} moe_kernel;

/* Timing of one kernel's launches made by the calling thread.
 * moe_profile_arm creates n_pairs (1 .. 65536) pairs of HIP events on the
 * current device, with timing and without the system-scope fence (so that a
 * record costs the stream next to nothing), and arms: the i-th later launch
 * of `kernel` (i < n_pairs) records pair i around itself on its launch
 * stream.  Arming again first releases the events of a previous arming.
 * Returns MOE_OK, MOE_ERR_ARG (kernel or n_pairs out of range) or
 * MOE_ERR_HIP (event creation failed; nothing is armed).
 * moe_profile_read waits for the recorded pairs, writes the duration in
 * milliseconds of the first min(recorded, max) launches to ms (host
 * memory), releases the events, disarms, and returns the number written,
 * or minus the moe_status of a failure (ms NULL or max < 0: -MOE_ERR_ARG;
 * a HIP event call failed: -MOE_ERR_HIP). */
moe_status moe_profile_arm(moe_kernel kernel, int n_pairs);
int moe_profile_read(float* ms, int max);

/* ---- HBM read calibration ---------------------------------------------------
 * The decode configurations are bound by reading expert weights from HBM;
 * their achieved bandwidth is reported against the datasheet peak and
 * against what a plain streaming read reaches on the same GPU, measured with
 * this call.  It enqueues on `stream` one kernel that reads the `bytes`
 * bytes at device pointer buf (16-byte aligned, bytes a positive multiple of
 * 16) exactly once with coalesced 16-byte loads, and writes the XOR of the
 * 32-bit words each of its blocks read to sink[0 .. blocks-1] (device
 * memory, MOE_STREAM_SINK_WORDS words; words from `blocks` on are left
 * untouched), so the XOR of a zeroed sink equals the XOR of the buffer.
 * Returns MOE_OK, MOE_ERR_ARG (a NULL pointer or bytes not a positive
 * multiple of 16), MOE_ERR_ALIGN or MOE_ERR_HIP. */
#define MOE_STREAM_SINK_WORDS 4096
moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* ---- matrix-core calibration --------------------------------------------------
 * The prefill chunk is bound by the chip's power limit: at it the fp16
 * matrix cores run far below the datasheet peak, at a rate that depends on
 * how much the operand bits toggle.  This call measures what they sustain
 * on operands with the expert GEMMs' value patterns (bf16-valued
 * activations, e2m1 x e4m3 weights, generated in the kernel), so that
 * bench.py can set the prefill GEMMs' rate against it as well as against
 * the datasheet.  It enqueues on `stream` one kernel of MOE_MFMA_RATE_BLOCKS
 * blocks of eight wavefronts; each wavefront runs `iters` rounds of four
 * v_mfma_f32_32x32x16_f16 (32768 flops each) on operands held in registers,
 * so one call performs iters * MOE_MFMA_RATE_FLOPS_PER_ITER floating-point
 * operations, and writes one checksum per block to sink[0 ..
 * MOE_MFMA_RATE_BLOCKS-1] (fp32, device memory).  Returns MOE_OK,
 * MOE_ERR_ARG (NULL sink, iters outside [1, 10^7]), MOE_ERR_ALIGN or
 * MOE_ERR_HIP. */
#define MOE_MFMA_RATE_BLOCKS 1024
#define MOE_MFMA_RATE_FLOPS_PER_ITER (1024.0 * 8.0 * 4.0 * 32768.0)
moe_status moe_mfma_rate(int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
