/* Seeded synthetic inputs: C API of the CPU (libsynth.so) and GPU
 * (libsynth_gpu.so) generators.  Both produce bit-identical values.
 *
 * Layouts (all row-major):
 *   x      [T][H]  bf16 bits, N(0,1) approx.; token t uses index (t0+t)*H + h
 *   W_r    [H][E]  bf16 bits, std * N(0,1) rounded to bf16; index h*E + e
 *   P       [K][N] bf16 bits, std * N(0,1), index k*N + n, dense bf16
 *                  weights by `which`: 0 the latent routed-down projection
 *                  [Hm][H], 1 the routed-up projection [H][Hm], 2 the shared
 *                  experts' gate/up [H][count*2I], 3 their down [count*I][H]
 *   W_e,m  [N][K]  fp32, std * N(0,1); index n*K + k; m = 0 gate, 1 up, 2 down
 *                  (gate/up: N = I, K = H; down: N = H, K = I)
 *   bias   [E]     fp32 expert-popularity bias (CPU only, see synth_zipf_bias)
 * Buffers are caller-owned.  GPU functions take device pointers and a
 * hipStream_t passed as void*, and return 0 on success. */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

void synth_x_bf16(uint64_t seed, int64_t t0, int T, int H, uint16_t* out);
void synth_router_bf16(uint64_t seed, int H, int E, float std, uint16_t* out);
void synth_expert_f32(uint64_t seed, int e, int m, int N, int K, float std, float* out, int nthreads);
void synth_proj_bf16(uint64_t seed, int which, int K, int N, float std, uint16_t* out);
/* Zipf-style popularity bias: b[e] = -beta * s * ln(1 + pi(e)), where pi is a
 * seeded random permutation of 0..E-1 (Fisher-Yates on the PERM stream).
 * Adding it to the router logits makes expert popularity fall off as a power
 * law of exponent beta*s in rank. */
void synth_zipf_bias(uint64_t seed, int E, double beta, double s, float* out);
/* Raw normals number first .. first+n-1 of one stream (for checks). */
void synth_normals_f32(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, float* out);
/* Round fp32 to bf16 bits as the generators do (for checks). */
void synth_round_bf16(const float* in, int64_t n, uint16_t* out);
/* The popularity permutation itself (pi[e] = rank of expert e). */
void synth_popularity_perm(uint64_t seed, int E, int32_t* pi);

int synth_gpu_x_bf16(uint64_t seed, int64_t t0, int T, int H, uint16_t* out, void* stream);
int synth_gpu_router_bf16(uint64_t seed, int H, int E, float std, uint16_t* out, void* stream);
int synth_gpu_expert_f32(uint64_t seed, int e, int m, int N, int K, float std, float* out, void* stream);
int synth_gpu_proj_bf16(uint64_t seed, int which, int K, int N, float std, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif
