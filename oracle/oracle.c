/* CPU oracle for the routed MoE layer with NVFP4 experts: TEST
 * INFRASTRUCTURE ONLY (see oracle.h).  Plain C99, fp64 unless stated. */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- element formats -------------------------------------------------- */

double oracle_e2m1_value(uint8_t code) {
  int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

double oracle_e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* The value of every code, from the decoders above, tabulated once so the
 * searches below do not re-decode each candidate. */
static double g_e2m1_table[16], g_e4m3_table[256];
static pthread_once_t g_tables_once = PTHREAD_ONCE_INIT;
static void fill_tables(void) {
  for (int c = 0; c < 16; c++) g_e2m1_table[c] = oracle_e2m1_value((uint8_t)c);
  for (int c = 0; c < 256; c++) g_e4m3_table[c] = oracle_e4m3_value((uint8_t)c);
}

/* Nearest representable value by exhaustive search over the candidate
 * codes, ties to the even code.  Distances are exact in fp64 here. */
uint8_t oracle_e2m1_round(double r) {
  pthread_once(&g_tables_once, fill_tables);
  uint8_t best = 0;
  double bestd = fabs(r - g_e2m1_table[0]);
  for (uint8_t c = 1; c < 8; c++) {
    double d = fabs(r - g_e2m1_table[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

uint8_t oracle_e4m3_round(double t) {
  pthread_once(&g_tables_once, fill_tables);
  uint8_t best = 0;
  double bestd = fabs(t - g_e4m3_table[0]);
  for (uint8_t c = 1; c < 127; c++) { /* 0x7F is NaN */
    double d = fabs(t - g_e4m3_table[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* ---- NVFP4 weight store ------------------------------------------------ */

size_t oracle_nvfp4_matrix_bytes(int64_t N, int64_t K) {
  return (size_t)(N * (K / 2)) + (size_t)(N * (K / 16)) + sizeof(float);
}

void oracle_nvfp4_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < N * K; i++) {
    float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  volatile float gs = (amax > 0.0f) ? amax / 2688.0f : 1.0f;
  *gs_out = gs;
  memset(q, 0, (size_t)(N * (K / 2)));
  for (int64_t n = 0; n < N; n++) {
    for (int64_t b = 0; b < K / 16; b++) {
      const float* blk = w + n * K + 16 * b;
      float bmax = 0.0f;
      for (int i = 0; i < 16; i++) {
        float a = fabsf(blk[i]);
        if (a > bmax) bmax = a;
      }
      volatile float sixth = bmax / 6.0f;
      volatile float t = sixth / gs;
      uint8_t sc = oracle_e4m3_round((double)t);
      sf[n * (K / 16) + b] = sc;
      volatile float d = (float)oracle_e4m3_value(sc) * gs;
      for (int i = 0; i < 16; i++) {
        uint8_t code = 0;
        if (d > 0.0f) {
          volatile float r = fabsf(blk[i]) / d;
          code = oracle_e2m1_round((double)r);
          if (blk[i] < 0.0f && code != 0) code |= 8;
        }
        int64_t k = 16 * b + i;
        q[n * (K / 2) + k / 2] |= (uint8_t)(code << (4 * (k & 1)));
      }
    }
  }
}

void oracle_nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, float gs, int64_t N, int64_t K, double* w) {
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      uint8_t code = (q[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
      double sigma = oracle_e4m3_value(sf[n * (K / 16) + k / 16]);
      w[n * K + k] = oracle_e2m1_value(code) * sigma * (double)gs;
    }
}

/* ---- MXFP4 ---------------------------------------------------------------- */

double oracle_e8m0_value(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

void oracle_mxfp4_quantize(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf) {
  memset(q, 0, (size_t)(N * (K / 2)));
  for (int64_t n = 0; n < N; n++) {
    for (int64_t b = 0; b < K / 32; b++) {
      const float* blk = w + n * K + 32 * b;
      float bmax = 0.0f;
      for (int i = 0; i < 32; i++) {
        float a = fabsf(blk[i]);
        if (a > bmax) bmax = a;
      }
      if (bmax == 0.0f) {
        sf[n * (K / 32) + b] = 0;
        continue;
      }
      int e2;
      frexp((double)bmax, &e2); /* bmax = m * 2^e2, m in [0.5, 1): floor(log2) = e2 - 1 */
      int s = (e2 - 1) - 2 + 127;
      if (s < 0) s = 0;
      if (s > 254) s = 254;
      sf[n * (K / 32) + b] = (uint8_t)s;
      double x = oracle_e8m0_value((uint8_t)s);
      for (int i = 0; i < 32; i++) {
        uint8_t code = oracle_e2m1_round(fabs((double)blk[i]) / x);
        if (blk[i] < 0.0f && code != 0) code |= 8;
        int64_t k = 32 * b + i;
        q[n * (K / 2) + k / 2] |= (uint8_t)(code << (4 * (k & 1)));
      }
    }
  }
}

void oracle_mxfp4_dequantize(const uint8_t* q, const uint8_t* sf, int64_t N, int64_t K, double* w) {
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      uint8_t code = (q[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
      w[n * K + k] = oracle_e2m1_value(code) * oracle_e8m0_value(sf[n * (K / 32) + k / 32]);
    }
}

/* ---- router -------------------------------------------------------------- */

static double bf16_to_double(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

void oracle_router_logits(const uint16_t* x, int64_t T, int64_t H, const uint16_t* wr, int64_t E, const float* bias,
                          float* logits) {
  for (int64_t t = 0; t < T; t++)
    for (int64_t e = 0; e < E; e++) {
      double s = 0.0;
      for (int64_t h = 0; h < H; h++) s += bf16_to_double(x[t * H + h]) * bf16_to_double(wr[h * E + e]);
      if (bias) s += (double)bias[e];
      logits[t * E + e] = (float)s;
    }
}

/* Record a ranks before record b: logit descending, then index ascending.
 * The comparison is in fp32, so -0 equals +0 and the index decides. */
static int ranks_before(float la, int64_t ia, float lb, int64_t ib) {
  if (la != lb) return la > lb;
  return ia < ib;
}

void oracle_topk_softmax(const float* logits, int64_t T, int64_t E, int k, int32_t* ids, double* w) {
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; t++) {
    const float* row = logits + t * E;
    memset(taken, 0, (size_t)E);
    /* k rounds, each taking the best record not yet taken. */
    for (int j = 0; j < k; j++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++)
        if (!taken[e] && (best < 0 || ranks_before(row[e], e, row[best], best))) best = e;
      taken[best] = 1;
      ids[t * k + j] = (int32_t)best;
    }
    double top = (double)row[ids[t * k]], sum = 0.0;
    for (int j = 0; j < k; j++) sum += exp((double)row[ids[t * k + j]] - top);
    for (int j = 0; j < k; j++) w[t * k + j] = exp((double)row[ids[t * k + j]] - top) / sum;
  }
  free(taken);
}

void oracle_permute(const int32_t* ids, int64_t T, int64_t E, int k, int32_t* offsets, int32_t* sorted_pairs,
                    int32_t* pair_pos) {
  int64_t P = T * k;
  int32_t* cursor = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  for (int64_t f = 0; f < P; f++)
    if (ids[f] >= 0 && ids[f] < E) cursor[ids[f] + 1]++;
  for (int64_t e = 0; e < E; e++) cursor[e + 1] += cursor[e];
  memcpy(offsets, cursor, sizeof(int32_t) * ((size_t)E + 1));
  for (int64_t f = 0; f < P; f++) { /* ascending record = ascending token */
    if (ids[f] < 0 || ids[f] >= E) { /* masked: served elsewhere */
      pair_pos[f] = -1;
      continue;
    }
    int32_t p = cursor[ids[f]]++;
    sorted_pairs[p] = (int32_t)f;
    pair_pos[f] = p;
  }
  for (int64_t p = offsets[E]; p < P; p++) sorted_pairs[p] = -1;
  free(cursor);
}

/* ---- expert FFN and the layer -------------------------------------------- */

void oracle_swiglu_token(const double* gate, const double* up, const double* down, const uint16_t* x, int64_t H,
                         int64_t I, double* out) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  for (int64_t i = 0; i < H; i++) xd[i] = bf16_to_double(x[i]);
  for (int64_t i = 0; i < I; i++) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < H; c++) {
      g += xd[c] * gate[i * H + c];
      u += xd[c] * up[i * H + c];
    }
    h[i] = g / (1.0 + exp(-g)) * u;
  }
  for (int64_t n = 0; n < H; n++) {
    double s = 0.0;
    for (int64_t i = 0; i < I; i++) s += h[i] * down[n * I + i];
    out[n] = s;
  }
  free(h);
  free(xd);
}

typedef struct {
  const uint16_t* x;
  int64_t H, I, E;
  int k;
  const oracle_expert_nvfp4* const* experts;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  double* rows; /* [P][H] */
  int first_expert, stride;
  int status;
} layer_job;

static void* expert_bucket_worker(void* arg) {
  layer_job* j = (layer_job*)arg;
  int64_t H = j->H, I = j->I;
  double* g = NULL;
  double* u = NULL;
  double* d = NULL;
  for (int64_t e = j->first_expert; e < j->E; e += j->stride) {
    int32_t begin = j->offsets[e], end = j->offsets[e + 1];
    if (begin == end) continue;
    const oracle_expert_nvfp4* ex = j->experts[e];
    if (!ex) {
      j->status = -1;
      continue;
    }
    if (!g) {
      g = (double*)malloc(sizeof(double) * (size_t)(I * H));
      u = (double*)malloc(sizeof(double) * (size_t)(I * H));
      d = (double*)malloc(sizeof(double) * (size_t)(H * I));
    }
    if (ex->format == 1) {
      oracle_mxfp4_dequantize(ex->q[0], ex->sf[0], I, H, g);
      oracle_mxfp4_dequantize(ex->q[1], ex->sf[1], I, H, u);
      oracle_mxfp4_dequantize(ex->q[2], ex->sf[2], H, I, d);
    } else {
      oracle_nvfp4_dequantize(ex->q[0], ex->sf[0], ex->gs[0], I, H, g);
      oracle_nvfp4_dequantize(ex->q[1], ex->sf[1], ex->gs[1], I, H, u);
      oracle_nvfp4_dequantize(ex->q[2], ex->sf[2], ex->gs[2], H, I, d);
    }
    for (int32_t p = begin; p < end; p++) {
      int64_t t = j->sorted_pairs[p] / j->k;
      oracle_swiglu_token(g, u, d, j->x + t * H, H, I, j->rows + (int64_t)p * H);
    }
  }
  free(g);
  free(u);
  free(d);
  return NULL;
}

int oracle_expert_ffn(const uint16_t* x, int64_t H, int64_t I, int64_t E, int k,
                      const oracle_expert_nvfp4* const* experts, const int32_t* offsets, const int32_t* sorted_pairs,
                      int nthreads, double* rows) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  pthread_t th[64];
  layer_job jobs[64];
  for (int i = 0; i < nthreads; i++) {
    layer_job jb = {x, H, I, E, k, experts, offsets, sorted_pairs, rows, i, nthreads, 0};
    jobs[i] = jb;
  }
  for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, expert_bucket_worker, &jobs[i]);
  expert_bucket_worker(&jobs[0]);
  for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
  int status = 0;
  for (int i = 0; i < nthreads; i++)
    if (jobs[i].status) status = jobs[i].status;
  return status;
}

int oracle_moe_layer(const uint16_t* x, int64_t T, int64_t H, int64_t I, const uint16_t* wr, const float* bias,
                     const float* logits_in, int64_t E, int k, const oracle_expert_nvfp4* const* experts,
                     int nthreads, float* logits_out, int32_t* ids, double* w, int32_t* offsets,
                     int32_t* sorted_pairs, int32_t* pair_pos, double* rows, double* y) {
  int64_t P = T * k;
  float* logits = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)(T * E));
  if (logits_in)
    memcpy(logits, logits_in, sizeof(float) * (size_t)(T * E));
  else
    oracle_router_logits(x, T, H, wr, E, bias, logits);
  oracle_topk_softmax(logits, T, E, k, ids, w);
  oracle_permute(ids, T, E, k, offsets, sorted_pairs, pair_pos);

  double* r = rows ? rows : (double*)malloc(sizeof(double) * (size_t)(P * H));
  int status = oracle_expert_ffn(x, H, I, E, k, experts, offsets, sorted_pairs, nthreads, r);

  for (int64_t t = 0; t < T; t++)
    for (int64_t n = 0; n < H; n++) {
      double s = 0.0;
      for (int j = 0; j < k; j++) s += w[t * k + j] * r[(int64_t)pair_pos[t * k + j] * H + n];
      y[t * H + n] = s;
    }
  if (!rows) free(r);
  if (!logits_out) free(logits);
  return status;
}

/* ---- latent routed-expert block ---------------------------------------------- */

void oracle_round_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) {
    double d = in[i];
    if (isnan(d)) {
      out[i] = 0x7FC0;
      continue;
    }
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    /* largest fp32 <= a, then its bf16 truncation: the largest bf16 <= a */
    float f = (float)a;
    if ((double)f > a) f = nextafterf(f, 0.0f);
    uint32_t fb;
    memcpy(&fb, &f, 4);
    uint16_t lo = (uint16_t)(fb >> 16);
    if (lo >= 0x7F80) { /* a is at least 2^128: infinity */
      out[i] = sign | 0x7F80;
      continue;
    }
    uint16_t hi = (uint16_t)(lo + 1);
    double vlo = bf16_to_double(lo);
    /* the value above the largest finite bf16 is 2^128 for rounding */
    double vhi = (hi == 0x7F80) ? ldexp(1.0, 128) : bf16_to_double(hi);
    double dlo = a - vlo, dhi = vhi - a;
    uint16_t r;
    if (dlo < dhi)
      r = lo;
    else if (dhi < dlo)
      r = hi;
    else
      r = (lo & 1) ? hi : lo;
    out[i] = sign | r;
  }
}

void oracle_bf16_matmul(const uint16_t* x, int64_t T, int64_t K, const uint16_t* W, int64_t N, double* out) {
  for (int64_t t = 0; t < T; t++)
    for (int64_t c = 0; c < N; c++) {
      double s = 0.0;
      for (int64_t r = 0; r < K; r++) s += bf16_to_double(x[t * K + r]) * bf16_to_double(W[r * N + c]);
      out[t * N + c] = s;
    }
}
