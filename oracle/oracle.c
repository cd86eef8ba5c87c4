/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the paged KV
 * append + paged attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libpkv.so and its Python binding) never links, loads or calls it, and it
 * shares no source, header, table or helper with the HIP kernels.
 *
 * Everything here is the plain definition, written out step by step in
 * double precision (fp64), with no blocking, fusion or reordering:
 *
 *   - slot mapping: where each new token of a sequence lands in the pool
 *     (a sequence owns whole fixed 16-token blocks, listed in logical order
 *     by its block table; the new tokens sit on top of the ones already
 *     computed) -- deepconcepts.dev, "Continuous Batching Is Not a Bigger
 *     Batch", sections "What the scheduler does on one step" (each request
 *     carries num_computed_tokens and asks for num_new_tokens; the cache
 *     manager allocates slots for them) and "The allocator is the other
 *     half" (fixed 16-token blocks);
 *   - KV append: copy each new token's K and V rows into its slot
 *     ("Continuous Batching Is Not a Bigger Batch", introduction: every
 *     sequence carries one K/V pair per token per layer);
 *   - attention: gather a sequence's K/V rows through its block table into
 *     contiguous arrays, then softmax(scale * q K^T) V per query head, the
 *     query head h reading KV head h / (Hq / Hkv) (grouped-query attention,
 *     "Where the batch size actually comes from": the KV heads are fewer
 *     than the query heads by the group factor);
 *   - partial attention over a position range and the log-sum-exp merge of
 *     such partials, used to pin the split-KV algebra.
 *
 * Readings where the pages are silent (all listed with reasons in the
 * design notes): a context length includes this step's new tokens (append,
 * then attend); query k of a sequence with n new tokens sits at position
 * ctx - n + k and attends positions [0, pos] (causal); slot < 0 means
 * "skip" (padding).
 *
 * Parity status: every function below is pinned by the CPU test suite
 * (closed forms, invariants, a numpy dense brute force written without block
 * tables, and the pages' worked byte/block arithmetic).  Beyond those pins
 * the attention values rest on this plain fp64 definition alone: the pages
 * print no attention output for any input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_RANGE (-2)
#define ORACLE_ERR_NOMEM (-3)

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is
 * zero/subnormal (value = f * 2^-24), exponent 31 is inf/NaN. */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);
  }
  return sign ? -v : v;
}

void oracle_half_array_to_double(const uint16_t* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = oracle_half_to_double(src[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of new tokens of sequence i: query_start_loc[i+1] - query_start_loc[i],
 * or 1 for every sequence when query_start_loc is NULL (a pure decode step). */
static int32_t new_tokens_of(const int32_t* qsl, int32_t i) {
  return qsl ? qsl[i + 1] - qsl[i] : 1;
}
static int32_t first_row_of(const int32_t* qsl, int32_t i) {
  return qsl ? qsl[i] : i;
}

/*
 * Slot mapping.  Sequence i has ctx_i tokens after this step, the last n_i of
 * which are new.  New token k sits at logical position p = ctx_i - n_i + k;
 * logical position p lives in the sequence's (p / block_size)-th block,
 * at offset p % block_size inside it, so its pool slot is
 *     block_tables[i][p / block_size] * block_size + p % block_size.
 * Writes slot_mapping[first_row_i + k].  Returns ORACLE_ERR_RANGE when a
 * position falls outside the table row (ctx too large) or ctx < n.
 */
int oracle_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* query_start_loc,
                        int32_t num_seqs, int32_t block_size, int64_t* slot_mapping) {
  if (!block_tables || !context_lens || !slot_mapping || num_seqs < 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0)
    return ORACLE_ERR_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t n = new_tokens_of(query_start_loc, i);
    int32_t ctx = context_lens[i];
    if (n < 0 || ctx < n) return ORACLE_ERR_RANGE;
    for (int32_t k = 0; k < n; ++k) {
      int64_t p = (int64_t)ctx - n + k;
      int64_t logical_block = p / block_size;
      int64_t offset = p % block_size;
      if (logical_block >= max_blocks_per_seq) return ORACLE_ERR_RANGE;
      int64_t physical_block = block_tables[(int64_t)i * max_blocks_per_seq + logical_block];
      slot_mapping[first_row_of(query_start_loc, i) + k] = physical_block * block_size + offset;
    }
  }
  return ORACLE_OK;
}

/*
 * KV append.  Pools are [num_blocks][num_kv_heads][block_size][head_dim]
 * fp16 (stored as raw 16-bit patterns; the append moves bits, it does no
 * arithmetic).  New rows are [num_tokens][num_kv_heads][head_dim].
 * For every token t with slot >= 0: block = slot / block_size,
 * offset = slot % block_size, and for every KV head g the head_dim values of
 * k_new[t][g] go to k_pool[block][g][offset] (likewise V).
 */
int oracle_kv_append(uint16_t* k_pool, uint16_t* v_pool, int64_t num_blocks,
                     int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                     const uint16_t* k_new, const uint16_t* v_new,
                     const int64_t* slot_mapping, int32_t num_tokens) {
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping || num_tokens < 0)
    return ORACLE_ERR_ARG;
  for (int32_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue; /* padding token: nothing to write */
    int64_t block = slot / block_size;
    int64_t offset = slot % block_size;
    if (block >= num_blocks) return ORACLE_ERR_RANGE;
    for (int32_t g = 0; g < num_kv_heads; ++g) {
      for (int32_t e = 0; e < head_dim; ++e) {
        int64_t dst = ((block * num_kv_heads + g) * block_size + offset) * head_dim + e;
        int64_t src = ((int64_t)t * num_kv_heads + g) * head_dim + e;
        k_pool[dst] = k_new[src];
        v_pool[dst] = v_new[src];
      }
    }
  }
  return ORACLE_OK;
}

/*
 * Gather: copy the rows of positions [0, count) of KV head g of sequence i
 * from the pool into a contiguous [count][head_dim] fp64 array, following
 * the block table (position p is in block table entry p / block_size, at
 * offset p % block_size).  The pool is fp16 bits (pool) or, for a quantized
 * cache already dequantized, fp64 values (pool64); exactly one is non-NULL.
 */
static int gather_rows(const uint16_t* pool, const double* pool64, int64_t num_blocks,
                       int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                       const int32_t* table_row, int32_t max_blocks_per_seq, int32_t g,
                       int32_t count, double* out) {
  for (int32_t p = 0; p < count; ++p) {
    int32_t logical_block = p / block_size;
    if (logical_block >= max_blocks_per_seq) return ORACLE_ERR_RANGE;
    int64_t block = table_row[logical_block];
    if (block < 0 || block >= num_blocks) return ORACLE_ERR_RANGE;
    int64_t base = ((block * num_kv_heads + g) * block_size + p % block_size) * head_dim;
    for (int32_t e = 0; e < head_dim; ++e)
      out[(int64_t)p * head_dim + e] =
          pool ? oracle_half_to_double(pool[base + e]) : pool64[base + e];
  }
  return ORACLE_OK;
}

/*
 * Attention of one query vector q[head_dim] over contiguous K/V rows
 * [lo, hi):
 *   s_p = scale * sum_e q[e] K[p][e]
 *   m   = max_p s_p
 *   l   = sum_p exp(s_p - m)
 *   o   = sum_p exp(s_p - m) V[p] / l
 * Returns o in out[head_dim] and (m, l) in *m_out, *l_out (either may be
 * NULL).  An empty range gives o = 0, m = -inf, l = 0.
 */
static void attend_range(const double* q, const double* K, const double* V, int32_t lo,
                         int32_t hi, int32_t head_dim, double scale, double* s_scratch,
                         double* out, double* m_out, double* l_out) {
  double m = -INFINITY, l = 0.0;
  for (int32_t e = 0; e < head_dim; ++e) out[e] = 0.0;
  for (int32_t p = lo; p < hi; ++p) {
    double dot = 0.0;
    for (int32_t e = 0; e < head_dim; ++e) dot += q[e] * K[(int64_t)p * head_dim + e];
    s_scratch[p - lo] = scale * dot;
    if (s_scratch[p - lo] > m) m = s_scratch[p - lo];
  }
  for (int32_t p = lo; p < hi; ++p) {
    double w = exp(s_scratch[p - lo] - m);
    l += w;
    for (int32_t e = 0; e < head_dim; ++e) out[e] += w * V[(int64_t)p * head_dim + e];
  }
  if (hi > lo)
    for (int32_t e = 0; e < head_dim; ++e) out[e] /= l;
  if (m_out) *m_out = m;
  if (l_out) *l_out = l;
}

/*
 * Paged attention for a step.
 *   q:   [T][num_q_heads][head_dim] fp16 bits, rows ordered by sequence
 *        (sequence i owns rows first_row_i .. first_row_i + n_i - 1).
 *   out: [T][num_q_heads][head_dim] fp64.
 *   lse_out (optional): [T][num_q_heads] natural-log log-sum-exp m + ln(l).
 *   seq_subset (optional): if non-NULL, only these sequence indices are
 *        computed (others' rows of out are left untouched).
 * For every sequence, K and V rows of every KV head are first gathered
 * into contiguous arrays, then each query row k attends positions
 * [0, ctx - n + k] (decode: n = 1, the whole context including the token
 * just appended).
 */
static int paged_attention_impl(const uint16_t* q, const uint16_t* k_pool,
                                const uint16_t* v_pool, const double* k_pool64,
                                const double* v_pool64, int64_t num_blocks,
                                int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t num_q_heads, double scale,
                                double* out, double* lse_out, const int32_t* seq_subset,
                                int32_t num_subset) {
  if (!q || !(k_pool || k_pool64) || !(v_pool || v_pool64) || !block_tables || !context_lens ||
      !out)
    return ORACLE_ERR_ARG;
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      head_dim <= 0 || block_size <= 0)
    return ORACLE_ERR_ARG;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t count = seq_subset ? num_subset : num_seqs;
  int status = ORACLE_OK;

#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t it = 0; it < count * num_kv_heads; ++it) {
    int32_t i = seq_subset ? seq_subset[it / num_kv_heads] : it / num_kv_heads;
    int32_t g = it % num_kv_heads;
    if (i < 0 || i >= num_seqs) {
#pragma omp atomic write
      status = ORACLE_ERR_RANGE;
      continue;
    }
    int32_t ctx = context_lens[i];
    int32_t n = new_tokens_of(query_start_loc, i);
    if (ctx < n || ctx <= 0) {
#pragma omp atomic write
      status = ORACLE_ERR_RANGE;
      continue;
    }
    double* K = (double*)malloc(sizeof(double) * (size_t)ctx * head_dim);
    double* V = (double*)malloc(sizeof(double) * (size_t)ctx * head_dim);
    double* qd = (double*)malloc(sizeof(double) * (size_t)head_dim);
    double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
    if (!K || !V || !qd || !s) {
#pragma omp atomic write
      status = ORACLE_ERR_NOMEM;
      free(K); free(V); free(qd); free(s);
      continue;
    }
    const int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    int rc = gather_rows(k_pool, k_pool64, num_blocks, num_kv_heads, block_size, head_dim, row,
                         max_blocks_per_seq, g, ctx, K);
    if (rc == ORACLE_OK)
      rc = gather_rows(v_pool, v_pool64, num_blocks, num_kv_heads, block_size, head_dim, row,
                       max_blocks_per_seq, g, ctx, V);
    if (rc != ORACLE_OK) {
#pragma omp atomic write
      status = rc;
    } else {
      for (int32_t k = 0; k < n; ++k) {
        int64_t r = (int64_t)first_row_of(query_start_loc, i) + k;
        int32_t pos = ctx - n + k;
        for (int32_t h = g * group; h < (g + 1) * group; ++h) {
          const uint16_t* qh = q + (r * num_q_heads + h) * head_dim;
          for (int32_t e = 0; e < head_dim; ++e) qd[e] = oracle_half_to_double(qh[e]);
          double m, l;
          attend_range(qd, K, V, 0, pos + 1, head_dim, scale, s,
                       out + (r * num_q_heads + h) * head_dim, &m, &l);
          if (lse_out) lse_out[r * num_q_heads + h] = m + log(l);
        }
      }
    }
    free(K); free(V); free(qd); free(s);
  }
  return status;
}

int oracle_paged_attention(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                           int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                           int32_t head_dim, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int32_t num_q_heads, double scale, double* out, double* lse_out,
                           const int32_t* seq_subset, int32_t num_subset) {
  if (!k_pool || !v_pool) return ORACLE_ERR_ARG;
  return paged_attention_impl(q, k_pool, v_pool, NULL, NULL, num_blocks, num_kv_heads,
                              block_size, head_dim, block_tables, max_blocks_per_seq,
                              context_lens, query_start_loc, num_seqs, num_q_heads, scale, out,
                              lse_out, seq_subset, num_subset);
}

/*
 * The same over pools of fp64 values [num_blocks][num_kv_heads][block_size]
 * [head_dim]: a quantized (fp8) cache after dequantization (code value x
 * row scale, exact in fp64), so that attention over it is the plain
 * definition again.
 */
int oracle_paged_attention_f64(const uint16_t* q, const double* k_pool, const double* v_pool,
                               int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                               int32_t head_dim, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               const int32_t* query_start_loc, int32_t num_seqs,
                               int32_t num_q_heads, double scale, double* out,
                               const int32_t* seq_subset, int32_t num_subset) {
  if (!k_pool || !v_pool) return ORACLE_ERR_ARG;
  return paged_attention_impl(q, NULL, NULL, k_pool, v_pool, num_blocks, num_kv_heads,
                              block_size, head_dim, block_tables, max_blocks_per_seq,
                              context_lens, query_start_loc, num_seqs, num_q_heads, scale, out,
                              NULL, seq_subset, num_subset);
}

/*
 * Partial attention of one query row over positions [lo, hi) of contiguous
 * fp64 K/V arrays [ctx][head_dim]: returns the partition's normalised output
 * o_part, its running max m_part and its sum of exponentials l_part.
 */
void oracle_attention_partial(const double* q, const double* K, const double* V,
                              int32_t lo, int32_t hi, int32_t head_dim, double scale,
                              double* o_part, double* m_part, double* l_part) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(hi > lo ? hi - lo : 1));
  attend_range(q, K, V, lo, hi, head_dim, scale, s, o_part, m_part, l_part);
  free(s);
}

/*
 * Log-sum-exp merge of P partials of one query row:
 *   M   = max_p m_p
 *   w_p = l_p * exp(m_p - M)
 *   O   = sum_p w_p o_p / sum_p w_p
 * A partial with l_p = 0 (empty range) has weight 0 and is skipped, so
 * that its m_p = -inf never enters exp().
 */
void oracle_lse_merge(const double* o_parts, const double* m_parts, const double* l_parts,
                      int32_t num_parts, int32_t head_dim, double* out) {
  double M = -INFINITY, W = 0.0;
  for (int32_t p = 0; p < num_parts; ++p)
    if (l_parts[p] > 0.0 && m_parts[p] > M) M = m_parts[p];
  for (int32_t e = 0; e < head_dim; ++e) out[e] = 0.0;
  for (int32_t p = 0; p < num_parts; ++p) {
    if (!(l_parts[p] > 0.0)) continue;
    double w = l_parts[p] * exp(m_parts[p] - M);
    W += w;
    for (int32_t e = 0; e < head_dim; ++e) out[e] += w * o_parts[(int64_t)p * head_dim + e];
  }
  if (W > 0.0)
    for (int32_t e = 0; e < head_dim; ++e) out[e] /= W;
}

/*
 * Full-range attention of one query row over contiguous fp64 K/V, without
 * any paging: the reference the merge self-check compares against.
 */
void oracle_attention_contiguous(const double* q, const double* K, const double* V,
                                 int32_t count, int32_t head_dim, double scale, double* out) {
  double m, l;
  oracle_attention_partial(q, K, V, 0, count, head_dim, scale, out, &m, &l);
}
