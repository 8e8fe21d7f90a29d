/*
 * pa_oracle.c -- CPU reference for paged verify attention, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library. The GPU library never calls it, and the
 * two share no source, header, table or helper.
 *
 * What it computes (the plain definition, written out without blocking,
 * splitting or online rescaling):
 *
 *   For sequence b with context length L (the cache holds L tokens, the q new
 *   ones included), query length q, optional sliding window W and query
 *   offset t_b = sum of the earlier sequences' query lengths; for every query
 *   head h (KV head g = h / G, G = Hq / Hkv) and query row i in [0, q):
 *
 *     p      = L - q + i                 absolute position of row i
 *     lo     = W > 0 ? max(0, p - W + 1) : 0
 *     K_j    = dequant(Kpool[bt[b][j/16]][g][j%16][:])   for lo <= j <= p
 *     s_j    = sigma * sum_d Q[t_b+i][h][d] * K_j[d]
 *     z      = the sink logit of head h for sequence b (absent: -inf)
 *     M      = max(max_j s_j, z)
 *     Z      = sum_j exp(s_j - M) + exp(z - M)
 *     out    = sum_j exp(s_j - M) * V_j / Z,   lse = M + ln Z
 *
 * Sources (the pages never print the mathematics; the steps below are the
 * plainest reading of what they describe):
 *  - ATOM #2843 "keep MTP-5 decode on FlyDSL pa_decode past the gluon
 *    query-length limit", Motivation: a verify step has query length
 *    k + 1 = 6 at MTP-5; its rows are query length x GQA group; the KV cache
 *    may be FP8 with per-token scales (with a trailing singleton dimension,
 *    Tests section); sinks and a sliding window are layer properties (Change
 *    section).
 *  - ATOM #3091 "High-interactivity monokernel decode for DeepSeek-V4.1-Flash
 *    on MI355X", Summary and "How to reproduce": 16-token blocks reached
 *    through a block table, context up to 1 Mi tokens.
 *  - ATOM #3038 "[MiniMax-M3.1] P/D from a PP4 prefill into a TP4 decode
 *    (2/2: DSpark)", commit message on the KV export: pages are head-major
 *    (each page holds, per KV head, its 16 tokens).
 *
 * Readings where the pages are silent: "context length" includes the q new
 * tokens; the causal mask is aligned to the end of the context (row i sits at
 * L - q + i); query head h uses KV head h / G; a window of W keys counts the
 * row's own key; a sink adds exp(z) to the denominator and carries no value;
 * FP8 is OCP e4m3fn (bias 7, max 448, NaN 0x7F/0xFF, no infinities); a
 * dequantised value is code * scale of its token and KV head.
 *
 * Arithmetic: every product and sum is in double; bf16 inputs widen exactly,
 * e4m3 codes are decoded from the format definition and multiplied by their
 * fp32 scale in double. Two passes per row (max, then exponentials).
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PAGE_TOKENS 16

/* bf16 is the top half of an IEEE binary32: widening is exact. */
double pa_oracle_bf16_to_double(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN;
 * there is no infinity. */
double pa_oracle_e4m3_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

typedef struct {
  int B, Hq, Hkv, D;
  const int32_t *ctx_lens, *q_lens, *window; /* window may be NULL */
  const int64_t *q_off;                      /* [B] query row offsets */
  const uint16_t *q;                         /* [T][Hq][D] bf16 bits */
  const void *k_pool, *v_pool;               /* [NB][Hkv][16][D] */
  int kv_fp8;
  const float *k_scales, *v_scales; /* [NB][Hkv][16] (FP8 only) */
  const int32_t *block_table;       /* [B][max_blocks] */
  int max_blocks;
  const float *sinks; /* NULL, [Hq] (mode 1) or [B][Hq] (mode 2) */
  int sinks_mode;
  double sigma;
  const uint8_t *unit_mask; /* [B][Hq] or NULL: which (b, h) to compute */
  double *out;              /* [T][Hq][D] */
  double *lse;              /* [T][Hq] or NULL */
  atomic_int next;
} job_t;

/* Dequantised element d of key/value token j of sequence b, KV head g. */
static double kv_elem(const job_t *J, int is_v, int b, int g, int64_t j, int d) {
  int32_t blk = J->block_table[(int64_t)b * J->max_blocks + j / PAGE_TOKENS];
  int64_t slot = ((int64_t)blk * J->Hkv + g) * PAGE_TOKENS + (j % PAGE_TOKENS);
  int64_t idx = slot * J->D + d;
  if (J->kv_fp8) {
    const uint8_t *pool = (const uint8_t *)(is_v ? J->v_pool : J->k_pool);
    const float *sc = is_v ? J->v_scales : J->k_scales;
    return pa_oracle_e4m3_to_double(pool[idx]) * (double)sc[slot];
  }
  const uint16_t *pool = (const uint16_t *)(is_v ? J->v_pool : J->k_pool);
  return pa_oracle_bf16_to_double(pool[idx]);
}

static double sink_of(const job_t *J, int b, int h) {
  if (J->sinks_mode == 1) return (double)J->sinks[h];
  if (J->sinks_mode == 2) return (double)J->sinks[(int64_t)b * J->Hq + h];
  return -INFINITY;
}

/* One (sequence, query head): all its query rows. */
static void one_unit(const job_t *J, int b, int h, double *s, double *acc) {
  const int G = J->Hq / J->Hkv;
  const int g = h / G;
  const int64_t L = J->ctx_lens[b];
  const int q = J->q_lens[b];
  const int W = J->window ? J->window[b] : 0;
  const int D = J->D;
  for (int i = 0; i < q; ++i) {
    const int64_t row = J->q_off[b] + i;
    const uint16_t *qv = J->q + (row * J->Hq + h) * D;
    const int64_t p = L - q + i;
    const int64_t lo = (W > 0) ? (p - W + 1 > 0 ? p - W + 1 : 0) : 0;
    const int64_t n = p - lo + 1;
    /* pass 1: scores and their maximum (the sink counts as one more logit) */
    double M = sink_of(J, b, h);
    for (int64_t t = 0; t < n; ++t) {
      const int64_t j = lo + t;
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += pa_oracle_bf16_to_double(qv[d]) * kv_elem(J, 0, b, g, j, d);
      s[t] = J->sigma * dot;
      if (s[t] > M) M = s[t];
    }
    /* pass 2: exponentials, denominator and the weighted sum of values */
    const double z = sink_of(J, b, h);
    double Z = (z == -INFINITY) ? 0.0 : exp(z - M);
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      const int64_t j = lo + t;
      const double e = exp(s[t] - M);
      Z += e;
      for (int d = 0; d < D; ++d) acc[d] += e * kv_elem(J, 1, b, g, j, d);
    }
    double *o = J->out + (row * J->Hq + h) * D;
    for (int d = 0; d < D; ++d) o[d] = acc[d] / Z;
    if (J->lse) J->lse[row * J->Hq + h] = M + log(Z);
  }
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  const int units = J->B * J->Hq;
  int64_t max_n = 1;
  for (int b = 0; b < J->B; ++b)
    if (J->ctx_lens[b] > max_n) max_n = J->ctx_lens[b];
  double *s = (double *)malloc(sizeof(double) * (size_t)max_n);
  double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
  if (!s || !acc) {
    free(s);
    free(acc);
    return (void *)1;
  }
  for (;;) {
    int u = atomic_fetch_add(&J->next, 1);
    if (u >= units) break;
    int b = u / J->Hq, h = u % J->Hq;
    if (J->unit_mask && !J->unit_mask[u]) continue;
    one_unit(J, b, h, s, acc);
  }
  free(s);
  free(acc);
  return NULL;
}

/*
 * Returns 0 on success, -1 on an argument that cannot describe a valid call
 * (nothing is written then), -2 if a thread could not start or allocate.
 * Units not selected by unit_mask leave their outputs untouched.
 */
int pa_oracle_verify(int B, int Hq, int Hkv, int D, const int32_t *ctx_lens,
                     const int32_t *q_lens, const int32_t *window,
                     const uint16_t *q, const void *k_pool, const void *v_pool,
                     int kv_fp8, const float *k_scales, const float *v_scales,
                     const int32_t *block_table, int max_blocks,
                     const float *sinks, int sinks_mode, double sigma,
                     const uint8_t *unit_mask, double *out, double *lse,
                     int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return -1;
  if (!ctx_lens || !q_lens || !q || !k_pool || !v_pool || !block_table || !out) return -1;
  if (kv_fp8 && (!k_scales || !v_scales)) return -1;
  if (sinks_mode < 0 || sinks_mode > 2 || (sinks_mode != 0 && !sinks)) return -1;
  int64_t *q_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)B);
  if (!q_off) return -2;
  int64_t acc = 0;
  for (int b = 0; b < B; ++b) {
    if (q_lens[b] < 0 || ctx_lens[b] < q_lens[b] ||
        (int64_t)(ctx_lens[b] + PAGE_TOKENS - 1) / PAGE_TOKENS > max_blocks ||
        (window && window[b] < 0)) {
      free(q_off);
      return -1;
    }
    q_off[b] = acc;
    acc += q_lens[b];
  }
  job_t J;
  memset(&J, 0, sizeof J);
  J.B = B;
  J.Hq = Hq;
  J.Hkv = Hkv;
  J.D = D;
  J.ctx_lens = ctx_lens;
  J.q_lens = q_lens;
  J.window = window;
  J.q_off = q_off;
  J.q = q;
  J.k_pool = k_pool;
  J.v_pool = v_pool;
  J.kv_fp8 = kv_fp8;
  J.k_scales = k_scales;
  J.v_scales = v_scales;
  J.block_table = block_table;
  J.max_blocks = max_blocks;
  J.sinks = sinks;
  J.sinks_mode = sinks_mode;
  J.sigma = sigma;
  J.unit_mask = unit_mask;
  J.out = out;
  J.lse = lse;
  atomic_init(&J.next, 0);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &J) != 0) break;
    ++started;
  }
  if (started == 0) {
    rc = (worker(&J) == NULL) ? 0 : -2;
  }
  for (int t = 0; t < started; ++t) {
    void *r = NULL;
    pthread_join(th[t], &r);
    if (r != NULL) rc = -2;
  }
  free(q_off);
  return rc;
}

/*
 * Paged KV append with per-token FP8 quantisation: the step before verify
 * attention, which writes the q new tokens' K and V into their 16-token
 * slots through the block table.
 *
 * Sources: ATOM #3091 "High-interactivity monokernel decode for
 * DeepSeek-V4.1-Flash on MI355X", Summary (stores into the paged pool are
 * masked by row liveness: a padded slot, q = 0, stores nothing); ATOM #2843
 * Motivation (FP8 KV with one fp32 scale per token and KV head); the FP8
 * workload's scale rule, scale = amax / 448 of the token's values.
 *
 * For sequence b, new token i in [0, q) sits at position pos = L - q + i,
 * page = bt[b][pos / 16], slot = pos % 16, and arrives as row t_b + i of the
 * new K and V ([T][Hkv][D] bf16). For every KV head g:
 *   bf16 pool: pool[page][g][slot][:] = the row, bit for bit;
 *   FP8 pool:  x_d = the row's values (bf16, exact in fp32);
 *              amax = max_d |x_d|; scale = amax / 448 in fp32 (1 if amax is 0);
 *              code_d = the e4m3 value nearest to clamp(x_d / scale, -448, 448)
 *                       (the division in fp32), ties to the even mantissa;
 *              pool[page][g][slot][:] = the codes, scales[page][g][slot] = scale.
 * Reading: the division and the scale are fp32 (the scales are fp32 and the
 * FP8 workload quantises in fp32); amax = 0 gives scale 1 and zero codes.
 */

/* The e4m3 code nearest to v (|v| <= 448, not NaN), ties to the code with
 * the even mantissa: a brute-force search over the 127 non-negative finite
 * codes, decoded from the format definition above. The differences are exact
 * in double (v has 24 significant bits, a code at most 4, both in
 * [2^-9, 448]). */
uint8_t pa_oracle_e4m3_encode(float v) {
  const double a = fabs((double)v);
  int best = 0;
  double best_d = a; /* code 0 is +0 */
  for (int c = 1; c <= 0x7E; ++c) {
    const double d = fabs(a - pa_oracle_e4m3_to_double((uint8_t)c));
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

static uint8_t *pool_row8(void *pool, int64_t page, int Hkv, int g, int slot, int D) {
  return (uint8_t *)pool + ((page * Hkv + g) * PAGE_TOKENS + slot) * (int64_t)D;
}
static uint16_t *pool_row16(void *pool, int64_t page, int Hkv, int g, int slot, int D) {
  return (uint16_t *)pool + ((page * Hkv + g) * PAGE_TOKENS + slot) * (int64_t)D;
}

/* Quantise one row of D bf16 values: codes and the fp32 scale. */
static float quantise_row(const uint16_t *row, int D, uint8_t *codes) {
  float amax = 0.0f;
  for (int d = 0; d < D; ++d) {
    const float x = (float)pa_oracle_bf16_to_double(row[d]);
    if (fabsf(x) > amax) amax = fabsf(x);
  }
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int d = 0; d < D; ++d) {
    const float x = (float)pa_oracle_bf16_to_double(row[d]);
    float y = x / scale;
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    codes[d] = pa_oracle_e4m3_encode(y);
  }
  return scale;
}

/*
 * Writes the new tokens into the pools as described above. Returns 0, or -1
 * on arguments that cannot describe a valid call (nothing is written then).
 * The caller's block table must give every new position a page < num_blocks.
 */
int pa_oracle_kv_append(int B, int Hkv, int D, const int32_t *ctx_lens, const int32_t *q_lens,
                        const uint16_t *k_new, const uint16_t *v_new,
                        const int32_t *block_table, int max_blocks, int num_blocks, int kv_fp8,
                        void *k_pool, void *v_pool, float *k_scales, float *v_scales) {
  if (B < 1 || Hkv < 1 || D < 1 || !ctx_lens || !q_lens || !k_new || !v_new || !block_table ||
      !k_pool || !v_pool)
    return -1;
  if (kv_fp8 && (!k_scales || !v_scales)) return -1;
  for (int b = 0; b < B; ++b) {
    if (q_lens[b] < 0 || ctx_lens[b] < q_lens[b] ||
        (int64_t)(ctx_lens[b] + PAGE_TOKENS - 1) / PAGE_TOKENS > max_blocks)
      return -1;
    for (int i = 0; i < q_lens[b]; ++i) {
      const int pos = ctx_lens[b] - q_lens[b] + i;
      const int32_t page = block_table[(int64_t)b * max_blocks + pos / PAGE_TOKENS];
      if (page < 0 || page >= num_blocks) return -1;
    }
  }
  uint8_t *codes = (uint8_t *)malloc((size_t)D);
  if (!codes) return -1;
  int64_t t = 0;
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < q_lens[b]; ++i, ++t) {
      const int pos = ctx_lens[b] - q_lens[b] + i;
      const int64_t page = block_table[(int64_t)b * max_blocks + pos / PAGE_TOKENS];
      const int slot = pos % PAGE_TOKENS;
      for (int g = 0; g < Hkv; ++g) {
        const uint16_t *kr = k_new + (t * Hkv + g) * (int64_t)D;
        const uint16_t *vr = v_new + (t * Hkv + g) * (int64_t)D;
        const int64_t si = (page * Hkv + g) * PAGE_TOKENS + slot;
        if (kv_fp8) {
          k_scales[si] = quantise_row(kr, D, codes);
          memcpy(pool_row8(k_pool, page, Hkv, g, slot, D), codes, (size_t)D);
          v_scales[si] = quantise_row(vr, D, codes);
          memcpy(pool_row8(v_pool, page, Hkv, g, slot, D), codes, (size_t)D);
        } else {
          memcpy(pool_row16(k_pool, page, Hkv, g, slot, D), kr, (size_t)D * 2);
          memcpy(pool_row16(v_pool, page, Hkv, g, slot, D), vr, (size_t)D * 2);
        }
      }
    }
  }
  free(codes);
  return 0;
}

/* ------------------------------------------------------------------------
 * Greedy verify verdict.
 *
 * Sources: ATOM #3091 ("High-interactivity monokernel decode for
 * DeepSeek-V4.1-Flash on MI355X"): the verify head gives a step's output ids
 * and its verdict in one launch, greedy rows included (Engine hooks), and
 * the next step takes each request's next id from the output ids at the
 * verdict's accepted count (the review rounds on the head-served verify).
 *
 * For sequence b with q = q_b verify rows at t_b .. t_b + q - 1 (q = k + 1:
 * row 0's input is the last committed token, rows 1..k hold the k draft
 * tokens, so draft j is input_ids[t_b + 1 + j]):
 *   a_i      = argmax_v logits[t_b + i][v]      for every row i
 *   n        = the number of leading drafts the target agrees with:
 *              the largest n in [0, k] with input_ids[t_b + 1 + j] == a_j
 *              for all j < n
 *   out_ids[t_b + i] = a_i,  accepted[b] = n,  next_ids[b] = a_n
 * (the step emits a_0 .. a_n, the n accepted drafts and one target token).
 * A padded slot (q = 0) writes nothing.
 * Readings: argmax takes the lowest index among equal maxima; a NaN never
 * wins (it compares false); a row with no value above -inf gives index 0.
 * bf16 logits widen exactly.
 */
static double logit_at(const void *logits, int is_bf16, int64_t idx) {
  if (is_bf16) return pa_oracle_bf16_to_double(((const uint16_t *)logits)[idx]);
  return (double)((const float *)logits)[idx];
}

/* Returns 0, or -1 on arguments that cannot describe a call (nothing is
 * written then). */
int pa_oracle_greedy_verdict(int B, const int32_t *q_lens, int vocab, int64_t row_stride,
                             const void *logits, int logits_bf16, const int32_t *input_ids,
                             int32_t *out_ids, int32_t *accepted, int32_t *next_ids) {
  if (B < 1 || vocab < 1 || row_stride < vocab || !q_lens || !logits || !input_ids ||
      !out_ids || !accepted || !next_ids)
    return -1;
  for (int b = 0; b < B; ++b)
    if (q_lens[b] < 0) return -1;
  int64_t t = 0;
  for (int b = 0; b < B; ++b) {
    const int q = q_lens[b];
    if (q == 0) continue;
    for (int i = 0; i < q; ++i) {
      double best = -INFINITY;
      int arg = 0;
      for (int v = 0; v < vocab; ++v) {
        const double x = logit_at(logits, logits_bf16, (t + i) * row_stride + v);
        if (x > best) {
          best = x;
          arg = v;
        }
      }
      out_ids[t + i] = arg;
    }
    int n = 0;
    while (n < q - 1 && input_ids[t + 1 + n] == out_ids[t + n]) ++n;
    accepted[b] = n;
    next_ids[b] = out_ids[t + n];
    t += q;
  }
  return 0;
}
