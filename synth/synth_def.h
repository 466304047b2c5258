/* Seeded synthetic inputs shared by the oracle tests and the GPU path.
 *
 * This header holds only the input generator: a counter-based SplitMix64
 * stream (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; the mixing constants are the published ones),
 * an approximately normal variate built from integer arithmetic alone, and
 * round-to-nearest-even narrowing to bfloat16.  None of the MoE layer's own
 * arithmetic (routing, quantisation, the FFN) lives here.
 *
 * Everything is integer arithmetic plus exactly representable float
 * conversions, so the CPU build (gcc) and the GPU build (hipcc) produce
 * bit-identical values for the same (seed, stream, index).
 *
 * Normal variate: the Irwin-Hall sum of twelve 16-bit uniforms, centred and
 * scaled by 2^-16.  Its mean is 0, its variance (65536^2-1)/65536^2, and its
 * support is bounded at +-6; the classic "sum of twelve uniforms" normal.
 * The result is an exact multiple of 2^-16 with |z| <= 6, so it is exact in
 * fp32. */
#ifndef SYNTH_DEF_H
#define SYNTH_DEF_H
#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN static inline __host__ __device__
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

/* Stream identifiers: one independent stream per input tensor. */
#define SYNTH_STREAM_X 1u          /* activations x[t][h]            */
#define SYNTH_STREAM_WR 2u         /* router weights W_r[h][e]       */
#define SYNTH_STREAM_PERM 3u       /* expert popularity permutation  */
#define SYNTH_STREAM_PROJ_DOWN 4u  /* routed-down projection [Hm][H] */
#define SYNTH_STREAM_PROJ_UP 5u    /* routed-up projection [H][Hm]   */
#define SYNTH_STREAM_SHARED_GU 6u  /* shared experts' gate/up [H][2cI] */
#define SYNTH_STREAM_SHARED_D 7u   /* shared experts' down [cI][H]    */
#define SYNTH_STREAM_EXPERT0 16u   /* expert e, matrix m: 16 + 3e + m */

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one stream of one seed. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed + SYNTH_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL));
}

/* i-th 64-bit word of a stream: SplitMix64 output for state key + (i+1)*gamma. */
SYNTH_FN uint64_t synth_word(uint64_t key, uint64_t i) {
  return synth_mix64(key + (i + 1u) * SYNTH_GAMMA);
}

/* Approximate standard normal number idx of a stream (three words). */
SYNTH_FN float synth_normal(uint64_t key, uint64_t idx) {
  int32_t s = 0;
  for (int w = 0; w < 3; w++) {
    uint64_t v = synth_word(key, 3u * idx + (uint64_t)w);
    s += (int32_t)(v & 0xFFFFu) + (int32_t)((v >> 16) & 0xFFFFu) +
         (int32_t)((v >> 32) & 0xFFFFu) + (int32_t)(v >> 48);
  }
  /* 12 * 32767.5 = 393210: centred sum, exact in fp32, times 2^-16. */
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
SYNTH_FN uint16_t synth_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

SYNTH_FN uint64_t synth_expert_stream(uint32_t e, uint32_t m) {
  return (uint64_t)SYNTH_STREAM_EXPERT0 + 3u * (uint64_t)e + m;
}

#endif
