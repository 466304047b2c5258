/* CPU oracle for the routed mixture-of-experts layer with NVFP4 experts.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never does, and
 * the two share no code.
 *
 * Floating point is fp64 unless stated.  Each function cites the passage of
 * the source pages it follows:
 *   [p2] "Serving Kimi-K3: a 2.8-trillion-parameter open agent model with
 *        8xB300 GPUs" (Geodesic, on Medium)
 *   [p3] al-engr.com, the plan for serving Kimi-K3's NVFP4 checkpoint from a
 *        GB300 Station plus eight DGX Sparks (the page prints no title)
 *   [p5] "Computation and Data Movement for Inference" (SemiAnalysis, in a
 *        Chinese translation)
 * Readings where the pages are silent are stated at each function. */
#ifndef ORACLE_H
#define ORACLE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* ---- element formats -------------------------------------------------- */
/* e2m1: sign bit 3, two exponent bits (bias 1), one mantissa bit.  [p2] "The
 * model, as the serving system sees it": 4-bit E2M1 values, two per byte. */
double oracle_e2m1_value(uint8_t code);
/* OCP E4M3FN: sign bit 7, four exponent bits (bias 7), three mantissa bits,
 * no infinities, 0x7F/0xFF are NaN, largest finite 448.  [p2] "Number formats
 * on Blackwell": NVFP4 carries an FP8 scale per 16 values. */
double oracle_e4m3_value(uint8_t code);
/* Nearest e2m1 magnitude code (0..7) to r >= 0; ties go to the even code;
 * r > 6 gives 6. */
uint8_t oracle_e2m1_round(double r);
/* Nearest non-negative finite e4m3 code to t >= 0; ties to the even code;
 * t > 448 gives 448. */
uint8_t oracle_e4m3_round(double t);

/* ---- NVFP4 weight store ------------------------------------------------ */
/* A logical matrix W[N][K] (N outputs, K the reduction axis) is stored as
 *   q [N][K/2]  e2m1 codes, element k even in the low nibble,
 *   sf[N][K/16] e4m3 scale of the 16 consecutive k of one row,
 *   gs          one fp32 per-tensor scale.
 * [p3] section "What has to be built - and the discovery that changed it":
 * the NVFP4 checkpoint has a scale per 16 values and a per-expert global
 * scale.  K must be a multiple of 16. */
size_t oracle_nvfp4_matrix_bytes(int64_t N, int64_t K);
/* Quantise.  The pages give no rounding rule; the reading taken (all steps
 * in fp32, divisions correctly rounded) puts the largest block scale at the
 * top of the e4m3 range and each block's largest element at the top of the
 * e2m1 range:
 *   amax = max|W|;  gs = amax / 2688 (6 * 448), or 1 when amax = 0
 *   per block b of row n: sigma_b = e4m3((amax_b / 6) / gs)
 *   d = sigma_b * gs;  code = e2m1(|w| / d), sign set only for w < 0 and a
 *   non-zero code; a block with sigma_b = 0 is all zero codes. */
void oracle_nvfp4_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs);
/* w[n][k] = e2m1(q) * sigma * gs, exact in fp64. */
void oracle_nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, float gs, int64_t N, int64_t K, double* w);

/* ---- MXFP4 weight store (the OCP microscaling format) ------------------------
 * [p2] "Number formats on Blackwell": MXFP4 carries an 8-bit power-of-two
 * scale per 32 values (Moonshot trained K3's experts in it); the OCP
 * Microscaling Formats (MX) v1.0 specification defines it: E8M0 scale byte
 * X = 2^(s - 127) (255 is NaN), elements e2m1.  Layout as NVFP4 but with
 *   sf [N][K/32]  e8m0 scale of the 32 consecutive k of one row,
 * and no per-tensor scale.  K must be a multiple of 32. */

/* E8M0 value: 2^(s - 127); s = 255 is NaN. */
double oracle_e8m0_value(uint8_t s);

/* Quantise, following the specification's conversion: per block, with
 * amax the largest |w| (fp32), the shared exponent is
 * floor(log2(amax)) - 2 (2 = the largest e2m1 exponent), clamped to the
 * E8M0 range; each element is the nearest e2m1 to w / X (ties to the even
 * code), clamped to 6; a block of zeros gets scale byte 0 and zero codes.
 * Division by the power of two X is exact. */
void oracle_mxfp4_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf);

/* w[n][k] = e2m1(q) * e8m0(sf), exact in fp64. */
void oracle_mxfp4_dequantize(const uint8_t* q, const uint8_t* sf, int64_t N, int64_t K, double* w);

/* ---- router -------------------------------------------------------------- */
/* logits[t][e] = fp32( sum_h x[t][h] * W_r[h][e] + bias[e] ), the sum in fp64
 * over ascending h.  x [T][H] and W_r [H][E] are bf16 bit patterns; bias may
 * be NULL.  [p5] section 3.4 "Decode experts": at the end of attention the
 * router, a small tensor, picks a few experts for every new token. */
void oracle_router_logits(const uint16_t* x, int64_t T, int64_t H, const uint16_t* wr, int64_t E, const float* bias,
                          float* logits);
/* Top-k selection and weights.  Selection: the k largest fp32 logits under
 * the order (logit descending, expert index ascending); slot j holds the
 * j-th in that order.  Weights: softmax over all E followed by renormalising
 * over the selected k, which equals the softmax of the k selected logits:
 * w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), in fp64.  [p3] "What we
 * verified today": 16 of 896 experts per token; [p5] section 4: the router
 * assigns several experts to every token. */
void oracle_topk_softmax(const float* logits, int64_t T, int64_t E, int k, int32_t* ids, double* w);
/* Expert-order permutation of the T*k route records f = t*k + j:
 *   offsets[e] = number of served records with expert < e (offsets[E] = the
 *   served records, T*k when none is masked),
 *   sorted_pairs[p] = the served records in (expert, token) order, p <
 *   offsets[E]; the entries from offsets[E] on are -1,
 *   pair_pos[f] = position of record f in sorted_pairs, -1 if masked.
 * A record whose id lies outside [0, E) (by convention -1) is masked: it is
 * served elsewhere and takes no position.
 * [p5] section 4: records are sorted by expert id so one load of an expert's
 * weights serves its whole bucket; section 15: expert e000 processes all of
 * its tokens, then e001, and so on; building counts and the permutation, and
 * restoring token order, are part of the cost.  [p3] "What has to be built -
 * and the discovery that changed it": splitting the experts across devices
 * takes a mask on the router's chosen ids, a masked id (-1) being one that
 * another device serves. */
void oracle_permute(const int32_t* ids, int64_t T, int64_t E, int k, int32_t* offsets, int32_t* sorted_pairs,
                    int32_t* pair_pos);

/* ---- expert FFN and the layer -------------------------------------------- */
/* NVFP4 tensors of one expert: gate and up are [I][H] logical (N = I,
 * K = H), down is [H][I] (N = H, K = I).  [p2] "The model, as the serving
 * system sees it": an expert is three matrices. */
typedef struct {
  const uint8_t* q[3];
  const uint8_t* sf[3];
  float gs[3];
  int32_t format; /* 0: NVFP4 (sf e4m3 per 16, gs used); 1: MXFP4 (sf e8m0 per 32, gs unused) */
} oracle_expert_nvfp4;

/* One token through one expert, weights already dequantised (fp64):
 *   g = x.W_gate, u = x.W_up, h = SiLU(g) * u, SiLU(z) = z / (1 + e^-z),
 *   out = h.W_down.
 * gate/up are [I][H], down [H][I]; x is [H] bf16 bits.  SwiGLU with SiLU is
 * the activation the workload configurations name; the pages do not. */
void oracle_swiglu_token(const double* gate, const double* up, const double* down, const uint16_t* x, int64_t H,
                         int64_t I, double* out);

/* The expert pass of the layer: for each expert e with a non-empty bucket
 * [offsets[e], offsets[e+1]) (as oracle_permute builds it), dequantise its
 * three matrices once and run every record of the bucket through them in
 * sorted order ([p5] sections 4 and 15):
 *   rows[p] = SwiGLU FFN of expert e on token sorted_pairs[p] / k,
 * unweighted, fp64, for p < offsets[E]; rows of other positions are not
 * written.  x [T][H] bf16 bits, rows [*][H].  nthreads > 1 spreads experts
 * over threads; results are bit-identical for any thread count.  Returns 0,
 * or -1 if an expert with records is NULL. */
int oracle_expert_ffn(const uint16_t* x, int64_t H, int64_t I, int64_t E, int k,
                      const oracle_expert_nvfp4* const* experts, const int32_t* offsets, const int32_t* sorted_pairs,
                      int nthreads, double* rows);

/* The whole layer.  If logits_in is non-NULL it is used in place of the
 * router (so the selection can be evaluated on another implementation's fp32
 * logits).  experts[e] may be NULL for experts that no token selects.  Each
 * active expert is dequantised once and serves its bucket in sorted order
 * ([p5] sections 4 and 15); outputs are restored to token order, weighted and
 * summed over ascending slot j ([p5] sections 4 and 5; [p3] "The number the
 * project hangs on": router, 16 experts, then a sum).  Routed scaling factor
 * 1, no capacity limit, no shared experts, no residual.
 * Outputs: ids/w [T][k], offsets [E+1], sorted_pairs/pair_pos [T*k],
 * rows [T*k][H] (per record in sorted order, unweighted; may be NULL) and
 * y [T][H].  nthreads > 1 spreads experts over threads; results are
 * bit-identical for any thread count.  Returns 0, or -1 if a selected
 * expert is NULL. */
int oracle_moe_layer(const uint16_t* x, int64_t T, int64_t H, int64_t I, const uint16_t* wr, const float* bias,
                     const float* logits_in, int64_t E, int k, const oracle_expert_nvfp4* const* experts,
                     int nthreads, float* logits_out, int32_t* ids, double* w, int32_t* offsets,
                     int32_t* sorted_pairs, int32_t* pair_pos, double* rows, double* y);

/* ---- latent routed-expert block (K3's LatentMoE) ----------------------------
 * [p4] lightseek.org, "Kimi K3 optimization on GB300" (part I), sections
 * "Routed-down projection: column sharding and latent assembly" and
 * "Routed-up projection: sharding the post-expert tail": every MoE block
 * projects the 7168-wide hidden state into the 3584-wide routed latent with
 * a bf16 weight, the experts work in the latent, and a second bf16
 * projection maps their combined output back.  [p2] "The model, as the
 * serving system sees it" gives the experts' 3584 x 3072 shape. */

/* Nearest bf16 to d (bit pattern), ties to the even pattern; a value half an
 * ulp or more above the largest finite bf16 gives infinity; NaN gives a
 * quiet NaN.  The two bf16 neighbours of |d| are found from its fp32
 * neighbour below, and the nearer one is chosen by exact fp64 distances. */
void oracle_round_bf16(const double* in, int64_t n, uint16_t* out);

/* out[t][c] = sum_r x[t][r] * W[r][c] in fp64 over ascending r, with x
 * [T][K] and W [K][N] bf16 bit patterns (W stored input-major, the
 * transpose of the pages' [out, in] weight). */
void oracle_bf16_matmul(const uint16_t* x, int64_t T, int64_t K, const uint16_t* W, int64_t N, double* out);

#ifdef __cplusplus
}
#endif
#endif
