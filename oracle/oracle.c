/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, obviously correct CPU reference that the GPU path is
 * checked against. Only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never does, and this file
 * shares no code, header or constant with the GPU library.
 *
 * What it computes (fp64 throughout, bf16/fp32 inputs widened exactly):
 *
 *  1. KV write. Each new token t whose slot s = slot_mapping[t] is >= 0 is
 *     copied bit for bit into block s / 16, row s % 16 of the pool: K into
 *     the block's first half, V into its second. ("Inside vLLM", section "Run
 *     forward pass", step 2 builds slot_mapping; the forward pass then fills
 *     the paged KV cache -- section "Prefix Caching".)
 *
 *  2. Gather. Key position j of sequence s lives in physical block
 *     block_tables[s][j / 16], row j % 16 (ngrok "Serving models at scale
 *     with vLLM", section "PagedAttention": a request's block table lists
 *     its blocks in order; 16 tokens per block).
 *
 *  3. Attention over the flattened super-sequence ("Inside vLLM", "Run
 *     forward pass", step 3: every sequence attends only to its own tokens).
 *     Query i of sequence s sits at position C_s + i, C_s = context_lens[s],
 *     and sees keys j <= C_s + i: all cached context plus the chunk's own
 *     earlier tokens (ngrok, section "Chunked prefill": a later chunk reads
 *     the earlier chunks' K/V from the cache; a token depends only on tokens
 *     before it). Query head h reads KV head h / (Hq / Hkv).
 *       x_j = scale * sum_d q[h][d] * K[j][d]
 *       o   = sum_j exp(x_j - max x) * V[j] / sum_j exp(x_j - max x)
 *     Two passes (max first, then weights), not an online recurrence.
 *
 * Pool layout: [num_blocks][2][16][Hkv][D], elements of `dtype`.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8 = 2 };
enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = 1,      /* null pointer, bad size or dtype */
  ORACLE_ERR_META = 2,     /* query_start_loc / lengths / block ids inconsistent */
  ORACLE_ERR_SLOT = 3,     /* slot out of range or used twice */
  ORACLE_ERR_NOMEM = 4
};

#define ORACLE_BLOCK 16

static size_t elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : dtype == ORACLE_BF16 ? 2 : 1; }

/*
 * 8-bit KV pool: OCP FP8 E4M3 ("FN": no infinities) codes with one scale for
 * all keys and one for all values. The pages name 8-bit KV quantization
 * without a format ("Serving models at scale with vLLM", section on
 * quantization); this is the reading taken.
 *   code: sign bit, 4 exponent bits e (bias 7), 3 mantissa bits m.
 *   e > 0: (-1)^s (1 + m/8) 2^(e-7);  e = 0: (-1)^s (m/8) 2^-6;
 *   e = 15, m = 7: NaN.  Largest finite magnitude: 448 (code 0x7E).
 * Stored code = encode(x / scale), the quotient rounded to fp32; the cache
 * holds code, and reading it back gives decode(code) * scale.
 */
double oracle_fp8_decode(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Nearest finite code to x, by search over all non-negative finite codes;
 * on a tie the code with the even mantissa (even code); magnitudes above the
 * largest finite value give it (saturation); NaN gives 0x7F. The sign is
 * x's sign bit (so -0 and negative values that round to zero give 0x80). */
uint8_t oracle_fp8_encode(double x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double err = fabs(oracle_fp8_decode((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* The value quantized: the input element divided by the scale in fp32. */
static uint8_t quantize(const void* base, int64_t idx, int in_dtype, float scale);

/* Exact widening of element idx of an fp32 or bf16 array to double. */
static double widen(const void* base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static uint8_t quantize(const void* base, int64_t idx, int in_dtype, float scale) {
  const float x = (float)widen(base, idx, in_dtype); /* exact */
  const float y = x / scale;                         /* IEEE fp32 division, rounded once */
  return oracle_fp8_encode((double)y);
}

/* Element idx of a pool of kv_dtype as a double: exact widening, and for
 * fp8 codes decode(code) * scale (exact: 4 x 24 significant bits). */
static double widen_kv(const void* base, int64_t idx, int kv_dtype, double scale) {
  if (kv_dtype == ORACLE_FP8) return oracle_fp8_decode(((const uint8_t*)base)[idx]) * scale;
  return widen(base, idx, kv_dtype);
}

/* Element offset of (block, kv, row, head, dim) in the pool. */
static int64_t pool_index(int64_t block, int kv, int64_t row, int64_t head, int64_t dim,
                          int64_t Hkv, int64_t D) {
  return (((block * 2 + kv) * ORACLE_BLOCK + row) * Hkv + head) * D + dim;
}

int oracle_reshape_and_cache(const void* k, const void* v, void* pool, const int64_t* slot_mapping,
                             int64_t T, int64_t num_blocks, int64_t Hkv, int64_t D, int dtype) {
  if (T < 0 || num_blocks < 1 || Hkv < 1 || D < 1) return ORACLE_ERR_ARG;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (T > 0 && (!k || !v || !pool || !slot_mapping)) return ORACLE_ERR_ARG;
  const size_t es = elem_size(dtype);
  const int64_t nslots = num_blocks * ORACLE_BLOCK;
  unsigned char* used = calloc((size_t)nslots, 1);
  if (!used) return ORACLE_ERR_NOMEM;
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= nslots || used[s]) {
      free(used);
      return ORACLE_ERR_SLOT;
    }
    used[s] = 1;
  }
  free(used);
  const size_t row_bytes = (size_t)(Hkv * D) * es;
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t block = s / ORACLE_BLOCK, row = s % ORACLE_BLOCK;
    memcpy((char*)pool + (size_t)pool_index(block, 0, row, 0, 0, Hkv, D) * es,
           (const char*)k + (size_t)t * row_bytes, row_bytes);
    memcpy((char*)pool + (size_t)pool_index(block, 1, row, 0, 0, Hkv, D) * es,
           (const char*)v + (size_t)t * row_bytes, row_bytes);
  }
  return ORACLE_OK;
}

/* KV write into an fp8 pool: like oracle_reshape_and_cache, but each element
 * of k (v) is stored as encode(element / k_scale (v_scale)). */
int oracle_reshape_and_cache_fp8(const void* k, const void* v, uint8_t* pool, const int64_t* slot_mapping,
                                 int64_t T, int64_t num_blocks, int64_t Hkv, int64_t D, int in_dtype,
                                 float k_scale, float v_scale) {
  if (T < 0 || num_blocks < 1 || Hkv < 1 || D < 1) return ORACLE_ERR_ARG;
  if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale)) return ORACLE_ERR_ARG;
  if (T > 0 && (!k || !v || !pool || !slot_mapping)) return ORACLE_ERR_ARG;
  const int64_t nslots = num_blocks * ORACLE_BLOCK;
  unsigned char* used = calloc((size_t)nslots, 1);
  if (!used) return ORACLE_ERR_NOMEM;
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= nslots || used[s]) {
      free(used);
      return ORACLE_ERR_SLOT;
    }
    used[s] = 1;
  }
  free(used);
  const int64_t row = Hkv * D;
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t block = s / ORACLE_BLOCK, r = s % ORACLE_BLOCK;
    for (int64_t e = 0; e < row; ++e) {
      pool[pool_index(block, 0, r, 0, 0, Hkv, D) + e] = quantize(k, t * row + e, in_dtype, k_scale);
      pool[pool_index(block, 1, r, 0, 0, Hkv, D) + e] = quantize(v, t * row + e, in_dtype, v_scale);
    }
  }
  return ORACLE_OK;
}

static int gather_kv(double* dst, const void* pool, const int32_t* table_row, int64_t L, int64_t num_blocks,
                     int64_t Hkv, int64_t D, int64_t head, int kv, int kv_dtype, double scale) {
  if (!dst || !pool || !table_row || L < 0 || head < 0 || head >= Hkv || (kv != 0 && kv != 1))
    return ORACLE_ERR_ARG;
  for (int64_t j = 0; j < L; ++j) {
    int64_t block = table_row[j / ORACLE_BLOCK];
    int64_t row = j % ORACLE_BLOCK;
    if (block < 0 || block >= num_blocks) return ORACLE_ERR_META;
    for (int64_t d = 0; d < D; ++d)
      dst[j * D + d] = widen_kv(pool, pool_index(block, kv, row, head, d, Hkv, D), kv_dtype, scale);
  }
  return ORACLE_OK;
}

/* Gather keys (kv = 0) or values (kv = 1) of one KV head of one sequence:
 * dst[j][d] for j < L, through that sequence's block-table row. */
int oracle_gather(double* dst, const void* pool, const int32_t* table_row, int64_t L,
                  int64_t num_blocks, int64_t Hkv, int64_t D, int64_t head, int kv, int dtype) {
  return gather_kv(dst, pool, table_row, L, num_blocks, Hkv, D, head, kv, dtype, 1.0);
}

static int check_metadata(const int32_t* block_tables, const int32_t* qsl, const int32_t* seq_lens,
                          const int32_t* ctx_lens, int64_t S, int64_t MB, int64_t NB) {
  if (qsl[0] != 0) return ORACLE_ERR_META;
  for (int64_t s = 0; s < S; ++s) {
    int64_t n = (int64_t)qsl[s + 1] - qsl[s];
    if (n < 1) return ORACLE_ERR_META;
    if (ctx_lens[s] < 0 || (int64_t)seq_lens[s] != (int64_t)ctx_lens[s] + n) return ORACLE_ERR_META;
    int64_t nblk = ((int64_t)seq_lens[s] + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    if (nblk > MB) return ORACLE_ERR_META;
    for (int64_t b = 0; b < nblk; ++b) {
      int32_t id = block_tables[s * MB + b];
      if (id < 0 || id >= NB) return ORACLE_ERR_META;
    }
  }
  return ORACLE_OK;
}

/* One (sequence, KV head) work item: all its queries, all G query heads. */
static int attend_one(double* out, const void* q, const void* pool, const int32_t* table_row,
                      int64_t q_begin, int64_t n, int64_t C, int64_t NB, int64_t Hq, int64_t Hkv,
                      int64_t D, int64_t g, int dtype, int kv_dtype, double k_scale, double v_scale,
                      double scale) {
  const int64_t L = C + n, G = Hq / Hkv;
  double* K = malloc(sizeof(double) * (size_t)(L * D));
  double* V = malloc(sizeof(double) * (size_t)(L * D));
  double* x = malloc(sizeof(double) * (size_t)L);
  double* o = malloc(sizeof(double) * (size_t)D);
  double* qv = malloc(sizeof(double) * (size_t)D);
  int rc = (K && V && x && o && qv) ? ORACLE_OK : ORACLE_ERR_NOMEM;
  if (rc == ORACLE_OK) rc = gather_kv(K, pool, table_row, L, NB, Hkv, D, g, 0, kv_dtype, k_scale);
  if (rc == ORACLE_OK) rc = gather_kv(V, pool, table_row, L, NB, Hkv, D, g, 1, kv_dtype, v_scale);
  for (int64_t i = 0; rc == ORACLE_OK && i < n; ++i) {
    const int64_t t = q_begin + i;
    const int64_t last = C + i; /* keys 0 .. last are visible */
    for (int64_t h = g * G; h < (g + 1) * G; ++h) {
      for (int64_t d = 0; d < D; ++d) qv[d] = widen(q, (t * Hq + h) * D + d, dtype);
      double m = -INFINITY;
      for (int64_t j = 0; j <= last; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qv[d] * K[j * D + d];
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
      }
      double l = 0.0;
      for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t j = 0; j <= last; ++j) {
        double w = exp(x[j] - m);
        l += w;
        for (int64_t d = 0; d < D; ++d) o[d] += w * V[j * D + d];
      }
      for (int64_t d = 0; d < D; ++d) out[(t * Hq + h) * D + d] = o[d] / l;
    }
  }
  free(K);
  free(V);
  free(x);
  free(o);
  free(qv);
  return rc;
}

/* Attention with q of dtype and a pool of kv_dtype (fp8 codes read back
 * as decode(code) * k_scale or * v_scale; other pools ignore the scales).
 * out: [T][Hq][D] doubles. Returns ORACLE_* ; *threads_used (if non-null)
 * receives the number of threads that ran. */
int oracle_attention_kv(double* out, const void* q, const void* pool, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* context_lens,
                        int64_t S, int64_t MB, int64_t NB, int64_t Hq, int64_t Hkv, int64_t D, int dtype,
                        int kv_dtype, float k_scale_f, float v_scale_f, double scale, int num_threads,
                        int* threads_used) {
  double k_scale = (double)k_scale_f, v_scale = (double)v_scale_f; /* scales are fp32 values */
  if (!out || !q || !pool || !block_tables || !query_start_loc || !seq_lens || !context_lens) return ORACLE_ERR_ARG;
  if (S < 0 || MB < 1 || NB < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return ORACLE_ERR_ARG;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (kv_dtype != dtype && kv_dtype != ORACLE_FP8) return ORACLE_ERR_ARG;
  if (kv_dtype != ORACLE_FP8) k_scale = v_scale = 1.0;
  int rc = check_metadata(block_tables, query_start_loc, seq_lens, context_lens, S, MB, NB);
  if (rc != ORACLE_OK) return rc;
  const int64_t items = S * Hkv;
  int failed = ORACLE_OK, used = 1;
#ifdef _OPENMP
  if (num_threads < 1) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (int64_t it = 0; it < items; ++it) {
    const int64_t s = it / Hkv, g = it % Hkv;
#ifdef _OPENMP
    if (it == 0) used = omp_get_num_threads();
#endif
    int r = attend_one(out, q, pool, block_tables + s * MB, query_start_loc[s],
                       (int64_t)query_start_loc[s + 1] - query_start_loc[s], context_lens[s], NB, Hq, Hkv, D,
                       g, dtype, kv_dtype, k_scale, v_scale, scale);
    if (r != ORACLE_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      failed = r;
    }
  }
  if (threads_used) *threads_used = used;
  return failed;
}

/* Attention with q and pool of the same dtype. */
int oracle_attention(double* out, const void* q, const void* pool, const int32_t* block_tables,
                     const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* context_lens,
                     int64_t S, int64_t MB, int64_t NB, int64_t Hq, int64_t Hkv, int64_t D, int dtype,
                     double scale, int num_threads, int* threads_used) {
  return oracle_attention_kv(out, q, pool, block_tables, query_start_loc, seq_lens, context_lens, S, MB, NB, Hq,
                             Hkv, D, dtype, dtype, 1.0f, 1.0f, scale, num_threads, threads_used);
}

/* Batch forms for the tests: out[i] = encode(x[i] / scale) with x of
 * in_dtype; and out[i] = decode(codes[i]). */
int oracle_fp8_quantize_array(const void* x, int in_dtype, float scale, uint8_t* out, int64_t n) {
  if ((n > 0 && (!x || !out)) || n < 0 || (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16)) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = quantize(x, i, in_dtype, scale);
  return ORACLE_OK;
}

int oracle_fp8_decode_array(const uint8_t* codes, double* out, int64_t n) {
  if ((n > 0 && (!codes || !out)) || n < 0) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_decode(codes[i]);
  return ORACLE_OK;
}
