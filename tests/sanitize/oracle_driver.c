/* Host sanitizer run of the oracle (test infrastructure checking test
 * infrastructure): oracle.c is compiled together with this driver under
 * AddressSanitizer and UndefinedBehaviorSanitizer, and every entry point runs
 * on small inputs -- every 16-bit and 8-bit code through the decoders, a sweep
 * through the fp8 encoder, decode and prefill over paged caches of each dtype
 * with 1 and 3 threads, the cache write with its skip and error rules.  Any
 * out-of-bounds access, use after free, leak or undefined operation ends the
 * run with a report; the checks below only catch gross wrong answers (the
 * numerical pins live in the Python tests). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_double(uint16_t h);
double oracle_bf16_to_double(uint16_t b);
double oracle_fp8_to_double(uint8_t c);
uint8_t oracle_float_to_fp8(float x);
int oracle_paged_decode(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                        int kv_dtype, const int32_t *block_tables, const int32_t *context_lens, int64_t num_seqs,
                        int64_t num_heads, int64_t num_kv_heads, int64_t head_dim, int64_t num_blocks,
                        int64_t block_size, int64_t max_blocks_per_seq, double scale, double k_scale, double v_scale,
                        const double *k_head_scale, const double *v_head_scale, const double *k_block_scale,
                        const double *v_block_scale, int nthreads);
int oracle_paged_prefill(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                         int kv_dtype, const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start_loc, int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads,
                         int64_t head_dim, int64_t num_blocks, int64_t block_size, int64_t max_blocks_per_seq,
                         double scale, double k_scale, double v_scale, const double *k_head_scale,
                         const double *v_head_scale, const double *k_block_scale, const double *v_block_scale,
                         int nthreads);
int oracle_cache_write(const void *k, const void *v, int in_dtype, void *k_cache, void *v_cache, int cache_dtype,
                       const int64_t *slot_mapping, int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
                       int64_t num_blocks, int64_t block_size, float k_scale, float v_scale,
                       const float *k_head_scale, const float *v_head_scale, const float *k_block_scale,
                       const float *v_block_scale);

static int fails = 0;
#define EXPECT(c)                                                          \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);         \
      ++fails;                                                             \
    }                                                                      \
  } while (0)

enum { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };
static const int kElem[4] = {4, 2, 2, 1};

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* a value of dtype dt near x, written at element i of buf */
static void put(void *buf, int dt, int64_t i, double x) {
  if (dt == F32) {
    ((float *)buf)[i] = (float)x;
  } else if (dt == FP8) {
    ((uint8_t *)buf)[i] = oracle_float_to_fp8((float)(x * 8.0));
  } else {
    /* a 16-bit code from the sign, a small exponent and random mantissa bits */
    const uint16_t sign = x < 0 ? 0x8000 : 0;
    const uint16_t code = dt == F16 ? (uint16_t)(sign | 0x3800 | (rng & 0x3FF)) : (uint16_t)(sign | 0x3F00 | (rng & 0x7F));
    ((uint16_t *)buf)[i] = code;
  }
}

static void decoders(void) {
  for (uint32_t c = 0; c < 65536; ++c) {
    const double f = oracle_f16_to_double((uint16_t)c), b = oracle_bf16_to_double((uint16_t)c);
    EXPECT(f == f || (c & 0x7C00) == 0x7C00);
    EXPECT(b == b || (c & 0x7F80) == 0x7F80);
  }
  int nans = 0;
  for (int c = 0; c < 256; ++c) {
    const double v = oracle_fp8_to_double((uint8_t)c);
    if (v != v) ++nans;
    else EXPECT(fabs(v) <= 448.0);
  }
  EXPECT(nans == 2);
  for (int i = -4000; i <= 4000; ++i) { /* the encoder round-trips its own grid within a half step */
    const float x = (float)i * 0.125f;
    const double back = oracle_fp8_to_double(oracle_float_to_fp8(x));
    EXPECT(fabs(back - (fabs(x) > 448.0f ? copysign(448.0, x) : x)) <= fmax(fabs(x) / 16.0, 1.0 / 512.0));
  }
  EXPECT(oracle_fp8_to_double(oracle_float_to_fp8(NAN)) != oracle_fp8_to_double(oracle_float_to_fp8(NAN)));
}

/* a paged layout: S sequences, blocks of bs tokens dealt in a scrambled order */
typedef struct {
  int64_t S, H, Hkv, D, bs, NB, W;
  int32_t *bt, *ctx;
} layout;

static layout make_layout(int64_t S, int64_t H, int64_t Hkv, int64_t D, int64_t bs, int64_t W) {
  layout L = {S, H, Hkv, D, bs, S * W + 3, W, NULL, NULL};
  L.bt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S * W));
  L.ctx = (int32_t *)malloc(sizeof(int32_t) * (size_t)S);
  for (int64_t s = 0; s < S; ++s) {
    L.ctx[s] = (int32_t)(s == 0 ? 0 : (s * 37) % (W * bs) + 1);
    for (int64_t j = 0; j < W; ++j) L.bt[s * W + j] = (int32_t)((s * W + j) * 7 % L.NB);
  }
  return L;
}

static void attention(int kv_dt, int q_dt, int heads_per_kv) {
  layout L = make_layout(5, 2 * heads_per_kv, 2, 16, 8, 6);
  const int64_t pool = L.NB * L.bs * L.Hkv * L.D;
  void *kc = malloc((size_t)(pool * kElem[kv_dt])), *vc = malloc((size_t)(pool * kElem[kv_dt]));
  for (int64_t i = 0; i < pool; ++i) {
    put(kc, kv_dt, i, urand());
    put(vc, kv_dt, i, urand());
  }
  void *q = malloc((size_t)(L.S * L.H * L.D * kElem[q_dt]));
  for (int64_t i = 0; i < L.S * L.H * L.D; ++i) put(q, q_dt, i, urand());
  double *o1 = (double *)malloc(sizeof(double) * (size_t)(L.S * L.H * L.D));
  double *o3 = (double *)malloc(sizeof(double) * (size_t)(L.S * L.H * L.D));
  double ks[2] = {0.5, 0.25}, vs[2] = {0.125, 2.0};
  const double *khs = kv_dt == FP8 ? ks : NULL, *vhs = kv_dt == FP8 ? vs : NULL;
  EXPECT(oracle_paged_decode(o1, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                             1.0, 1.0, khs, vhs, NULL, NULL, 1) == 0);
  EXPECT(oracle_paged_decode(o3, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                             1.0, 1.0, khs, vhs, NULL, NULL, 3) == 0);
  EXPECT(memcmp(o1, o3, sizeof(double) * (size_t)(L.S * L.H * L.D)) == 0);
  for (int64_t i = 0; i < L.S * L.H * L.D; ++i) EXPECT(isfinite(o1[i]));
  if (kv_dt == FP8) { /* one scale per (block, kv head); not together with per-head scales */
    double *kb = (double *)malloc(sizeof(double) * (size_t)(L.NB * L.Hkv));
    double *vb = (double *)malloc(sizeof(double) * (size_t)(L.NB * L.Hkv));
    for (int64_t i = 0; i < L.NB * L.Hkv; ++i) {
      kb[i] = 0.25 + 0.125 * (double)(i % 5);
      vb[i] = 2.0 - 0.25 * (double)(i % 7);
    }
    EXPECT(oracle_paged_decode(o3, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                               1.0, 1.0, NULL, NULL, kb, vb, 3) == 0);
    for (int64_t i = 0; i < L.S * L.H * L.D; ++i) EXPECT(isfinite(o3[i]));
    EXPECT(oracle_paged_decode(o3, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                               1.0, 1.0, khs, vhs, kb, vb, 3) != 0);
    int32_t qs1[6] = {0, 0, 1, 2, 3, 4};
    double *o4 = (double *)malloc(sizeof(double) * (size_t)(4 * L.H * L.D));
    EXPECT(oracle_paged_prefill(o4, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, qs1, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W,
                                0.25, 1.0, 1.0, NULL, NULL, kb, vb, 2) == 0);
    free(kb), free(vb), free(o4);
  }
  /* prefill: the last min(3, L) tokens of each sequence as queries */
  int32_t qsl[6] = {0};
  for (int64_t s = 0; s < L.S; ++s) qsl[s + 1] = qsl[s] + (L.ctx[s] < 3 ? L.ctx[s] : 3);
  const int64_t rows = qsl[L.S];
  void *qp = malloc((size_t)(rows * L.H * L.D * kElem[q_dt]));
  for (int64_t i = 0; i < rows * L.H * L.D; ++i) put(qp, q_dt, i, urand());
  double *op = (double *)malloc(sizeof(double) * (size_t)(rows * L.H * L.D));
  EXPECT(oracle_paged_prefill(op, qp, q_dt, kc, vc, kv_dt, L.bt, L.ctx, qsl, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W,
                              0.25, 1.0, 1.0, khs, vhs, NULL, NULL, 2) == 0);
  for (int64_t i = 0; i < rows * L.H * L.D; ++i) EXPECT(isfinite(op[i]));
  /* a table entry outside the pool and a context longer than its table are refused */
  L.bt[1 * L.W] = (int32_t)L.NB;
  EXPECT(oracle_paged_decode(o1, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                             1.0, 1.0, khs, vhs, NULL, NULL, 2) != 0);
  L.bt[1 * L.W] = 0;
  L.ctx[2] = (int32_t)(L.W * L.bs + 1);
  EXPECT(oracle_paged_decode(o1, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                             1.0, 1.0, khs, vhs, NULL, NULL, 2) != 0);
  EXPECT(oracle_paged_decode(NULL, q, q_dt, kc, vc, kv_dt, L.bt, L.ctx, L.S, L.H, L.Hkv, L.D, L.NB, L.bs, L.W, 0.25,
                             1.0, 1.0, khs, vhs, NULL, NULL, 1) != 0);
  free(kc), free(vc), free(q), free(o1), free(o3), free(qp), free(op), free(L.bt), free(L.ctx);
}

static void cache_write(int in_dt, int cache_dt) {
  const int64_t NB = 4, bs = 8, Hkv = 2, D = 16, N = 6;
  const int64_t pool = NB * bs * Hkv * D;
  void *kc = calloc((size_t)pool, (size_t)kElem[cache_dt]), *vc = calloc((size_t)pool, (size_t)kElem[cache_dt]);
  void *k = malloc((size_t)(N * Hkv * D * kElem[in_dt])), *v = malloc((size_t)(N * Hkv * D * kElem[in_dt]));
  for (int64_t i = 0; i < N * Hkv * D; ++i) {
    put(k, in_dt, i, urand());
    put(v, in_dt, i, urand());
  }
  int64_t slots[6] = {3, -1, 31, 0, 17, -5};
  const float hs[2] = {0.5f, 0.25f};
  const float *khs = cache_dt == FP8 ? hs : NULL;
  EXPECT(oracle_cache_write(k, v, in_dt, kc, vc, cache_dt, slots, N, Hkv, D, NB, bs, 1.0f, 1.0f, khs, khs, NULL, NULL) == 0);
  if (cache_dt == FP8) { /* one scale per (destination block, kv head) */
    float kb[8], vb[8];
    for (int i = 0; i < 8; ++i) kb[i] = 0.5f + 0.25f * (float)i, vb[i] = 4.0f / (float)(i + 1);
    EXPECT(oracle_cache_write(k, v, in_dt, kc, vc, cache_dt, slots, N, Hkv, D, NB, bs, 1.0f, 1.0f, NULL, NULL, kb,
                              vb) == 0);
    EXPECT(oracle_cache_write(k, v, in_dt, kc, vc, cache_dt, slots, N, Hkv, D, NB, bs, 1.0f, 1.0f, NULL, NULL, kb,
                              NULL) != 0);
  }
  if (in_dt == cache_dt) /* same dtype: the bytes of token 2 land at slot 31 */
    EXPECT(memcmp((char *)kc + 31 * Hkv * D * kElem[cache_dt], (char *)k + 2 * Hkv * D * kElem[in_dt],
                  (size_t)(Hkv * D * kElem[in_dt])) == 0);
  slots[1] = NB * bs; /* past the pool */
  EXPECT(oracle_cache_write(k, v, in_dt, kc, vc, cache_dt, slots, N, Hkv, D, NB, bs, 1.0f, 1.0f, khs, khs, NULL, NULL) != 0);
  slots[1] = 3; /* a duplicate */
  EXPECT(oracle_cache_write(k, v, in_dt, kc, vc, cache_dt, slots, N, Hkv, D, NB, bs, 1.0f, 1.0f, khs, khs, NULL, NULL) != 0);
  free(kc), free(vc), free(k), free(v);
}

int main(void) {
  decoders();
  const int kv[4] = {F32, F16, BF16, FP8};
  for (int i = 0; i < 4; ++i)
    for (int g = 1; g <= 4; g *= 2) attention(kv[i], kv[i] == F32 ? F32 : (kv[i] == BF16 ? BF16 : F16), g);
  for (int i = 0; i < 3; ++i) cache_write(kv[i], kv[i]);
  cache_write(F16, FP8);
  cache_write(BF16, FP8);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer run: all entry points clean\n");
  return 0;
}
