/*
 * Oracle for paged-KV decode -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow fp64 CPU reference that the tests, the smoke check and the
 * benchmark's CPU-baseline leg use to check the HIP path.  The product path
 * never calls it.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * What it computes (the plain definition; paging only changes where each
 * token's K/V rows live, never the result):
 *
 *   - Cache layout [num_blocks, block_size, num_kv_heads, head_dim], each
 *     block holding block_size tokens (page "vLLM推理引擎架构：PagedAttention机制与
 *     高吞吐推理", sections 2.1-2.2; block size in tokens per page
 *     "大模型推理KV Cache内存管理与PagedAttention分页显存实战").
 *   - A sequence's logical token t lives in physical block
 *     block_tables[seq][t / block_size] at offset t % block_size (page
 *     "Paged KVCache：大模型推理显存管理优化方案", section 2.3, address
 *     translation: page id = address / page size, offset = address % page size,
 *     physical = block id * page size + offset).
 *   - Each sequence's one query row per head attends over its first
 *     context_lens[seq] tokens (the kernel interface in section 2.3 of the first
 *     page named above): out = softmax(scale * q . K^T) V, the query head h
 *     reading KV head h / (num_heads / num_kv_heads).
 *   - fp8 KV holds OCP e4m3fn codes; a stored value is code_value * scale with
 *     one fp32 scale per tensor (page "大模型推理KV Cache内存管理与PagedAttention分页
 *     显存实战", closing paragraph on FP8 KV caches), or one per kv head: the
 *     scale of the head the element belongs to (precision set per attention
 *     head, page "vLLM框架中的KV cache优化与PagedAttention机制详解", section 8.2), or
 *     one per (physical block, kv head): the scale of the block that holds the
 *     token, for that head (the finer grain of the same section's per-head
 *     precision: a block's tokens share one scale, like a page's contents).
 *   - The cache write puts the K/V row of new token n at slot_mapping[n], slot
 *     = block * block_size + offset, and skips negative slots.
 *   - Prefill (several query tokens per sequence): the query rows of sequence
 *     s are rows query_start_loc[s] .. query_start_loc[s+1]-1 of q (the first
 *     page's kernel interface takes a num_tokens-long query), and they are the
 *     sequence's newest tokens, already in the cache: with q_len of them in a
 *     context of context_lens[s], query j sits at position context_lens[s] -
 *     q_len + j and attends to the tokens at positions 0 .. that position
 *     (causal order, as every token of an autoregressive prompt).
 *
 * Arithmetic: every stored value is decoded exactly to double; the gather,
 * dot products, softmax (two passes: max, then exp and sum) and the weighted
 * sum of V rows are all in double, in plain sequential loops.
 */

#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8 = 3 };

enum {
  ORC_OK = 0,
  ORC_BAD_ARG = 1,
  ORC_BAD_BLOCK = 2,     /* a table entry the sequence needs is outside the pool */
  ORC_CTX_TOO_LONG = 3,  /* context needs more blocks than the table row has */
  ORC_BAD_SLOT = 4,      /* a slot outside the pool */
  ORC_DUP_SLOT = 5,      /* two new tokens target one slot */
  ORC_NO_MEMORY = 6,
};

static int elem_size(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8: return 1;
  }
  return 0;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* OCP 8-bit e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN; exponent field 0 encodes subnormals
 * m * 2^-9; otherwise (1 + m/8) * 2^(e-7). */
double oracle_fp8_to_double(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return sign ? -v : v;
}

/* fp32 -> e4m3fn code, rounding to the nearest representable value with ties
 * going to the even code, saturating to +-448, NaN -> 0x7F with the sign.
 * Done by brute force over the 127 non-negative finite codes. */
uint8_t oracle_float_to_fp8(float x) {
  uint32_t bits;
  memcpy(&bits, &x, 4);
  uint8_t sign = (uint8_t)((bits >> 31) << 7);
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int best = 0;
  double best_err = a; /* code 0 is +0 */
  for (int c = 1; c <= 0x7E; ++c) {
    double err = fabs(oracle_fp8_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

static double load_elem(const void *base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_F32: {
      float f;
      memcpy(&f, (const char *)base + 4 * i, 4);
      return (double)f;
    }
    case ORC_F16: {
      uint16_t h;
      memcpy(&h, (const char *)base + 2 * i, 2);
      return oracle_f16_to_double(h);
    }
    case ORC_BF16: {
      uint16_t b;
      memcpy(&b, (const char *)base + 2 * i, 2);
      return oracle_bf16_to_double(b);
    }
    case ORC_FP8:
      return oracle_fp8_to_double(((const uint8_t *)base)[i]);
  }
  return NAN;
}

/* ------------------------------------------------------------------------------------ */
/* decode */

typedef struct {
  double *out;
  const void *q;
  int q_dtype;
  const void *k_cache, *v_cache;
  int kv_dtype;
  const int32_t *block_tables, *context_lens;
  int64_t num_seqs, num_heads, num_kv_heads, head_dim, num_blocks, block_size, max_blocks;
  double scale, k_scale, v_scale;
  const double *k_heads, *v_heads; /* fp8: one scale per kv head instead of k_scale / v_scale, or NULL */
  const double *k_blocks, *v_blocks; /* fp8: one scale per (block, kv head) [num_blocks][num_kv_heads], or NULL */
  /* work distribution */
  int64_t next_item;
  pthread_mutex_t lock;
  int status;
} decode_job;

/* One (sequence, kv head): gather that head's K and V rows in logical order,
 * then attend for each query head that reads it. */
static int decode_item(decode_job *J, int64_t seq, int64_t kvh, double *Kc, double *Vc, double *s) {
  const int64_t D = J->head_dim, H = J->num_heads, Hkv = J->num_kv_heads, bs = J->block_size;
  const int64_t G = H / Hkv;
  const int64_t L = J->context_lens[seq];
  if (L < 0) return ORC_BAD_ARG;
  if (L == 0) { /* nothing to attend to: the output is zero */
    for (int64_t g = 0; g < G; ++g)
      for (int64_t d = 0; d < D; ++d) J->out[(seq * H + kvh * G + g) * D + d] = 0.0;
    return ORC_OK;
  }
  if ((L + bs - 1) / bs > J->max_blocks) return ORC_CTX_TOO_LONG;
  double ks = 1.0, vs = 1.0;
  if (J->kv_dtype == ORC_FP8) {
    ks = J->k_heads ? J->k_heads[kvh] : J->k_scale;
    vs = J->v_heads ? J->v_heads[kvh] : J->v_scale;
  }

  for (int64_t t = 0; t < L; ++t) {
    int64_t blk = J->block_tables[seq * J->max_blocks + t / bs];
    int64_t off = t % bs;
    if (blk < 0 || blk >= J->num_blocks) return ORC_BAD_BLOCK;
    int64_t row = ((blk * bs + off) * Hkv + kvh) * D;
    const double kst = J->k_blocks ? J->k_blocks[blk * Hkv + kvh] : ks;
    const double vst = J->v_blocks ? J->v_blocks[blk * Hkv + kvh] : vs;
    for (int64_t d = 0; d < D; ++d) {
      Kc[t * D + d] = load_elem(J->k_cache, J->kv_dtype, row + d) * kst;
      Vc[t * D + d] = load_elem(J->v_cache, J->kv_dtype, row + d) * vst;
    }
  }

  for (int64_t g = 0; g < G; ++g) {
    const int64_t h = kvh * G + g;
    const int64_t qrow = (seq * H + h) * D;
    for (int64_t t = 0; t < L; ++t) {
      double dot = 0.0;
      for (int64_t d = 0; d < D; ++d) dot += load_elem(J->q, J->q_dtype, qrow + d) * Kc[t * D + d];
      s[t] = J->scale * dot;
    }
    double m = s[0];
    for (int64_t t = 1; t < L; ++t)
      if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t t = 0; t < L; ++t) {
      s[t] = exp(s[t] - m);
      l += s[t];
    }
    double *o = J->out + qrow;
    for (int64_t d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < L; ++t) acc += s[t] * Vc[t * D + d];
      o[d] = acc / l;
    }
  }
  return ORC_OK;
}

static void *decode_worker(void *arg) {
  decode_job *J = (decode_job *)arg;
  const int64_t cap = J->max_blocks * J->block_size;
  double *Kc = (double *)malloc(sizeof(double) * (size_t)(cap * J->head_dim + 1));
  double *Vc = (double *)malloc(sizeof(double) * (size_t)(cap * J->head_dim + 1));
  double *s = (double *)malloc(sizeof(double) * (size_t)(cap + 1));
  int err = (Kc && Vc && s) ? ORC_OK : ORC_NO_MEMORY;
  const int64_t n_items = J->num_seqs * J->num_kv_heads;
  while (!err) {
    pthread_mutex_lock(&J->lock);
    int64_t item = J->next_item++;
    int stop = J->status != ORC_OK;
    pthread_mutex_unlock(&J->lock);
    if (stop || item >= n_items) break;
    err = decode_item(J, item / J->num_kv_heads, item % J->num_kv_heads, Kc, Vc, s);
  }
  if (err) {
    pthread_mutex_lock(&J->lock);
    if (J->status == ORC_OK) J->status = err;
    pthread_mutex_unlock(&J->lock);
  }
  free(Kc);
  free(Vc);
  free(s);
  return NULL;
}

/* out: double [num_seqs, num_heads, head_dim]; every other array contiguous in
 * the layouts stated at the top of this file.  Work items (sequence, kv head)
 * are spread over nthreads threads; results do not depend on nthreads. */
int oracle_paged_decode(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                        int kv_dtype, const int32_t *block_tables, const int32_t *context_lens,
                        int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads, int64_t head_dim,
                        int64_t num_blocks, int64_t block_size, int64_t max_blocks_per_seq, double scale,
                        double k_scale, double v_scale, const double *k_head_scale, const double *v_head_scale,
                        const double *k_block_scale, const double *v_block_scale, int nthreads) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return ORC_BAD_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_heads % num_kv_heads != 0 || max_blocks_per_seq < 0)
    return ORC_BAD_ARG;
  if (!elem_size(q_dtype) || q_dtype == ORC_FP8 || !elem_size(kv_dtype)) return ORC_BAD_ARG;
  decode_job J;
  memset(&J, 0, sizeof J);
  J.out = out;
  J.q = q;
  J.q_dtype = q_dtype;
  J.k_cache = k_cache;
  J.v_cache = v_cache;
  J.kv_dtype = kv_dtype;
  J.block_tables = block_tables;
  J.context_lens = context_lens;
  J.num_seqs = num_seqs;
  J.num_heads = num_heads;
  J.num_kv_heads = num_kv_heads;
  J.head_dim = head_dim;
  J.num_blocks = num_blocks;
  J.block_size = block_size;
  J.max_blocks = max_blocks_per_seq;
  J.scale = scale;
  J.k_scale = k_scale;
  J.v_scale = v_scale;
  if ((k_head_scale == NULL) != (v_head_scale == NULL)) return ORC_BAD_ARG;
  if ((k_block_scale == NULL) != (v_block_scale == NULL) || (k_head_scale && k_block_scale)) return ORC_BAD_ARG;
  J.k_heads = k_head_scale;
  J.v_heads = v_head_scale;
  J.k_blocks = k_block_scale;
  J.v_blocks = v_block_scale;
  J.status = ORC_OK;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads == 1) {
    decode_worker(&J);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return ORC_NO_MEMORY;
    int started = 0;
    for (; started < nthreads; ++started)
      if (pthread_create(&th[started], NULL, decode_worker, &J) != 0) break;
    if (started == 0) decode_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
  return J.status;
}

/* ------------------------------------------------------------------------------------ */
/* prefill: several query tokens per sequence, causal */

typedef struct {
  double *out;
  const void *q;
  int q_dtype;
  const void *k_cache, *v_cache;
  int kv_dtype;
  const int32_t *block_tables, *context_lens, *query_start_loc;
  int64_t num_seqs, num_heads, num_kv_heads, head_dim, num_blocks, block_size, max_blocks;
  double scale, k_scale, v_scale;
  const double *k_heads, *v_heads; /* fp8: one scale per kv head instead of k_scale / v_scale, or NULL */
  const double *k_blocks, *v_blocks; /* fp8: one scale per (block, kv head) [num_blocks][num_kv_heads], or NULL */
  int64_t next_item;
  pthread_mutex_t lock;
  int status;
} prefill_job;

/* One (sequence, kv head): gather the context's K and V rows in logical order
 * once, then for every query token of the sequence and every query head that
 * reads this kv head, attend over the positions up to the token's own. */
static int prefill_item(prefill_job *J, int64_t seq, int64_t kvh, double *Kc, double *Vc, double *w) {
  const int64_t D = J->head_dim, H = J->num_heads, Hkv = J->num_kv_heads, bs = J->block_size;
  const int64_t G = H / Hkv;
  const int64_t L = J->context_lens[seq];
  const int64_t r0 = J->query_start_loc[seq], r1 = J->query_start_loc[seq + 1];
  const int64_t nq = r1 - r0;
  if (L < 0 || nq < 0 || nq > L) return ORC_BAD_ARG;
  if (nq == 0) return ORC_OK;
  if ((L + bs - 1) / bs > J->max_blocks) return ORC_CTX_TOO_LONG;
  double ks = 1.0, vs = 1.0;
  if (J->kv_dtype == ORC_FP8) {
    ks = J->k_heads ? J->k_heads[kvh] : J->k_scale;
    vs = J->v_heads ? J->v_heads[kvh] : J->v_scale;
  }
  for (int64_t t = 0; t < L; ++t) {
    const int64_t blk = J->block_tables[seq * J->max_blocks + t / bs];
    if (blk < 0 || blk >= J->num_blocks) return ORC_BAD_BLOCK;
    const int64_t src = ((blk * bs + t % bs) * Hkv + kvh) * D;
    const double kst = J->k_blocks ? J->k_blocks[blk * Hkv + kvh] : ks;
    const double vst = J->v_blocks ? J->v_blocks[blk * Hkv + kvh] : vs;
    for (int64_t d = 0; d < D; ++d) {
      Kc[t * D + d] = load_elem(J->k_cache, J->kv_dtype, src + d) * kst;
      Vc[t * D + d] = load_elem(J->v_cache, J->kv_dtype, src + d) * vst;
    }
  }
  for (int64_t j = 0; j < nq; ++j) {
    const int64_t pos = L - nq + j; /* this query token's own position */
    const int64_t n = pos + 1;      /* it sees positions 0 .. pos */
    for (int64_t g = 0; g < G; ++g) {
      const int64_t row = ((r0 + j) * H + kvh * G + g) * D;
      double mx = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += load_elem(J->q, J->q_dtype, row + d) * Kc[t * D + d];
        w[t] = J->scale * dot;
        if (w[t] > mx) mx = w[t];
      }
      double sum = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        w[t] = exp(w[t] - mx);
        sum += w[t];
      }
      for (int64_t d = 0; d < D; ++d) {
        double a = 0.0;
        for (int64_t t = 0; t < n; ++t) a += w[t] * Vc[t * D + d];
        J->out[row + d] = a / sum;
      }
    }
  }
  return ORC_OK;
}

static void *prefill_worker(void *arg) {
  prefill_job *J = (prefill_job *)arg;
  const int64_t cap = J->max_blocks * J->block_size;
  double *Kc = (double *)malloc(sizeof(double) * (size_t)(cap * J->head_dim + 1));
  double *Vc = (double *)malloc(sizeof(double) * (size_t)(cap * J->head_dim + 1));
  double *w = (double *)malloc(sizeof(double) * (size_t)(cap + 1));
  int err = (Kc && Vc && w) ? ORC_OK : ORC_NO_MEMORY;
  const int64_t n_items = J->num_seqs * J->num_kv_heads;
  while (!err) {
    pthread_mutex_lock(&J->lock);
    const int64_t item = J->next_item++;
    const int stop = J->status != ORC_OK;
    pthread_mutex_unlock(&J->lock);
    if (stop || item >= n_items) break;
    err = prefill_item(J, item / J->num_kv_heads, item % J->num_kv_heads, Kc, Vc, w);
  }
  if (err) {
    pthread_mutex_lock(&J->lock);
    if (J->status == ORC_OK) J->status = err;
    pthread_mutex_unlock(&J->lock);
  }
  free(Kc);
  free(Vc);
  free(w);
  return NULL;
}

/* out: double [query_start_loc[num_seqs], num_heads, head_dim]; q has the same
 * row count; query_start_loc: int32 [num_seqs + 1], non-decreasing from 0.
 * Other arrays as for the decode above. */
int oracle_paged_prefill(double *out, const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                         int kv_dtype, const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start_loc, int64_t num_seqs, int64_t num_heads,
                         int64_t num_kv_heads, int64_t head_dim, int64_t num_blocks, int64_t block_size,
                         int64_t max_blocks_per_seq, double scale, double k_scale, double v_scale,
                         const double *k_head_scale, const double *v_head_scale, const double *k_block_scale,
                         const double *v_block_scale, int nthreads) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc) return ORC_BAD_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_heads % num_kv_heads != 0 || max_blocks_per_seq < 0)
    return ORC_BAD_ARG;
  if (!elem_size(q_dtype) || q_dtype == ORC_FP8 || !elem_size(kv_dtype)) return ORC_BAD_ARG;
  if (query_start_loc[0] != 0) return ORC_BAD_ARG;
  for (int64_t s = 0; s < num_seqs; ++s)
    if (query_start_loc[s + 1] < query_start_loc[s]) return ORC_BAD_ARG;
  prefill_job J;
  memset(&J, 0, sizeof J);
  J.out = out;
  J.q = q;
  J.q_dtype = q_dtype;
  J.k_cache = k_cache;
  J.v_cache = v_cache;
  J.kv_dtype = kv_dtype;
  J.block_tables = block_tables;
  J.context_lens = context_lens;
  J.query_start_loc = query_start_loc;
  J.num_seqs = num_seqs;
  J.num_heads = num_heads;
  J.num_kv_heads = num_kv_heads;
  J.head_dim = head_dim;
  J.num_blocks = num_blocks;
  J.block_size = block_size;
  J.max_blocks = max_blocks_per_seq;
  J.scale = scale;
  J.k_scale = k_scale;
  J.v_scale = v_scale;
  if ((k_head_scale == NULL) != (v_head_scale == NULL)) return ORC_BAD_ARG;
  if ((k_block_scale == NULL) != (v_block_scale == NULL) || (k_head_scale && k_block_scale)) return ORC_BAD_ARG;
  J.k_heads = k_head_scale;
  J.v_heads = v_head_scale;
  J.k_blocks = k_block_scale;
  J.v_blocks = v_block_scale;
  J.status = ORC_OK;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads == 1) {
    prefill_worker(&J);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return ORC_NO_MEMORY;
    int started = 0;
    for (; started < nthreads; ++started)
      if (pthread_create(&th[started], NULL, prefill_worker, &J) != 0) break;
    if (started == 0) prefill_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
  return J.status;
}

/* ------------------------------------------------------------------------------------ */
/* cache write */

/* k, v: [num_tokens, num_kv_heads, head_dim] in in_dtype; caches as above in
 * cache_dtype.  Same dtype: the bytes are copied.  fp8 cache: each element is
 * converted to fp32, divided in fp32 by its scale -- the tensor's fp32 scale,
 * or its kv head's when k_head_scale / v_head_scale ([num_kv_heads]) are
 * given, or its (destination block, kv head)'s when k_block_scale /
 * v_block_scale ([num_blocks][num_kv_heads]) are -- and encoded with
 * oracle_float_to_fp8.  Validates every slot before writing anything. */
int oracle_cache_write(const void *k, const void *v, int in_dtype, void *k_cache, void *v_cache, int cache_dtype,
                       const int64_t *slot_mapping, int64_t num_tokens, int64_t num_kv_heads, int64_t head_dim,
                       int64_t num_blocks, int64_t block_size, float k_scale, float v_scale,
                       const float *k_head_scale, const float *v_head_scale, const float *k_block_scale,
                       const float *v_block_scale) {
  if ((k_head_scale == NULL) != (v_head_scale == NULL)) return ORC_BAD_ARG;
  if ((k_block_scale == NULL) != (v_block_scale == NULL) || (k_head_scale && k_block_scale)) return ORC_BAD_ARG;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return ORC_BAD_ARG;
  if (!elem_size(in_dtype) || !elem_size(cache_dtype)) return ORC_BAD_ARG;
  if (in_dtype != cache_dtype && !(cache_dtype == ORC_FP8 && in_dtype != ORC_FP8)) return ORC_BAD_ARG;
  const int64_t n_slots = num_blocks * block_size;
  for (int64_t n = 0; n < num_tokens; ++n) {
    if (slot_mapping[n] < 0) continue;
    if (slot_mapping[n] >= n_slots) return ORC_BAD_SLOT;
    for (int64_t j = 0; j < n; ++j)
      if (slot_mapping[j] == slot_mapping[n]) return ORC_DUP_SLOT;
  }
  const int64_t row = num_kv_heads * head_dim;
  const int es_in = elem_size(in_dtype), es_c = elem_size(cache_dtype);
  for (int64_t n = 0; n < num_tokens; ++n) {
    const int64_t slot = slot_mapping[n];
    if (slot < 0) continue;
    const int64_t blk = slot / block_size, off = slot % block_size;
    const int64_t dst = (blk * block_size + off) * row;
    for (int which = 0; which < 2; ++which) {
      const void *src = which ? v : k;
      char *cache = (char *)(which ? v_cache : k_cache);
      const float *heads = which ? v_head_scale : k_head_scale;
      const float *blocks = which ? v_block_scale : k_block_scale; /* the scales of block blk's heads */
      if (in_dtype == cache_dtype) {
        memcpy(cache + dst * es_c, (const char *)src + n * row * es_in, (size_t)(row * es_c));
      } else {
        for (int64_t i = 0; i < row; ++i) {
          const float sc = blocks ? blocks[blk * num_kv_heads + i / head_dim]
                                  : (heads ? heads[i / head_dim] : (which ? v_scale : k_scale));
          float x = (float)load_elem(src, in_dtype, n * row + i);
          ((uint8_t *)cache)[dst + i] = oracle_float_to_fp8(x / sc);
        }
      }
    }
  }
  return ORC_OK;
}
