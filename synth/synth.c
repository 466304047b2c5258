/* CPU implementation of the seeded synthetic inputs (see synth_def.h). */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include "synth.h"
#include "synth_def.h"

void synth_x_bf16(uint64_t seed, int64_t t0, int T, int H, uint16_t* out) {
  uint64_t key = synth_key(seed, SYNTH_STREAM_X);
  for (int64_t t = 0; t < T; t++)
    for (int h = 0; h < H; h++)
      out[t * H + h] = synth_bf16_rne(synth_normal(key, (uint64_t)(t0 + t) * (uint64_t)H + (uint64_t)h));
}

void synth_router_bf16(uint64_t seed, int H, int E, float std, uint16_t* out) {
  uint64_t key = synth_key(seed, SYNTH_STREAM_WR);
  for (int64_t i = 0; i < (int64_t)H * E; i++)
    out[i] = synth_bf16_rne(std * synth_normal(key, (uint64_t)i));
}

void synth_proj_bf16(uint64_t seed, int which, int K, int N, float std, uint16_t* out) {
  uint64_t key = synth_key(seed, (uint64_t)SYNTH_STREAM_PROJ_DOWN + (uint64_t)which);
  for (int64_t i = 0; i < (int64_t)K * N; i++)
    out[i] = synth_bf16_rne(std * synth_normal(key, (uint64_t)i));
}

typedef struct {
  uint64_t key;
  float std;
  float* out;
  int64_t begin, end;
} expert_job;

static void* expert_worker(void* arg) {
  expert_job* j = (expert_job*)arg;
  for (int64_t i = j->begin; i < j->end; i++) j->out[i] = j->std * synth_normal(j->key, (uint64_t)i);
  return NULL;
}

void synth_expert_f32(uint64_t seed, int e, int m, int N, int K, float std, float* out, int nthreads) {
  uint64_t key = synth_key(seed, synth_expert_stream((uint32_t)e, (uint32_t)m));
  int64_t n = (int64_t)N * K;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  pthread_t th[64];
  expert_job jobs[64];
  for (int i = 0; i < nthreads; i++) {
    jobs[i].key = key;
    jobs[i].std = std;
    jobs[i].out = out;
    jobs[i].begin = n * i / nthreads;
    jobs[i].end = n * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, expert_worker, &jobs[i]);
  expert_worker(&jobs[0]);
  for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
}

void synth_normals_f32(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, float* out) {
  uint64_t key = synth_key(seed, stream);
  for (int64_t i = 0; i < n; i++) out[i] = synth_normal(key, first + (uint64_t)i);
}

void synth_round_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = synth_bf16_rne(in[i]);
}

void synth_popularity_perm(uint64_t seed, int E, int32_t* pi) {
  uint64_t key = synth_key(seed, SYNTH_STREAM_PERM);
  for (int e = 0; e < E; e++) pi[e] = e;
  for (int i = E - 1; i > 0; i--) {
    int j = (int)(synth_word(key, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t tmp = pi[i];
    pi[i] = pi[j];
    pi[j] = tmp;
  }
}

void synth_zipf_bias(uint64_t seed, int E, double beta, double s, float* out) {
  int32_t* pi = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  synth_popularity_perm(seed, E, pi);
  for (int e = 0; e < E; e++) out[e] = (float)(-beta * s * log(1.0 + (double)pi[e]));
  free(pi);
}
