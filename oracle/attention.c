/*
 * ORACLE -- test infrastructure only.  Nothing in the product path may link,
 * load or call this file; only the tests, the smoke check and the CPU leg of
 * the benchmark use it.
 *
 * Decode attention restricted to the selected entries, written as its
 * definition in double precision.  The AVSG abstract (arxivdaily 2609.37538,
 * abstract) states that the operator preserves the exact token selections of
 * dynamic sparse attention, so a step's output is plain softmax attention of
 * each query head over exactly the selected K/V rows, read here straight from
 * the host KV cache (never from a device buffer).  For query token j and
 * query head h of unit u = (request b, KV head g), with g = h / (Hq / Hkv):
 *   s_i  = scale * sum_d q[b][j][h][d] * K_i[d]   over the selected token rows i
 *   p_i  = exp(s_i - max_i s_i) / sum_i exp(s_i - max_i s_i)
 *   o[d] = sum_i p_i * V_i[d]
 * Row layouts (Spin summary, section 2B, head-wise pages): a split-layout
 * entry is K[tpe][dqk] followed by V[tpe][dv] and contributes all of its tpe
 * token rows; a latent entry is one vector whose dqk values are the key and
 * whose first dv values are the value.  With context lengths, token row t of
 * entry e is position e * tpe + t of its request, and rows at or past the
 * request's length are not attended (the last page of a context may be only
 * partly written; what its other rows hold never matters).  A unit whose
 * step failed (nonzero status) produces zeros.  The work is independent per
 * (unit, token, head) and shared over OpenMP threads on that index, nothing
 * else.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, n_kv_heads, n_q_heads, n_tokens;  /* B, Hkv, Hq, T */
  int32_t head_dim_qk, head_dim_v;                 /* dqk, dv */
  int32_t latent;                                  /* 1: latent rows */
  int32_t tokens_per_entry;                        /* tpe (split layout) */
  int32_t n_entries, k;                            /* N, selected entries per list */
  double scale;
} oracle_attn_cfg;

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 *   q        bf16 bits [B][T][Hq][dqk]
 *   host_kv  bf16 bits [units][N][row], row = tpe * (dqk + dv) or dqk (latent)
 *   sel      [units][T][k] selected entry ids
 *   len      [units][T] entries in use of each list (its first len ids), or
 *            NULL for k
 *   status   [units] or NULL (all 0)
 *   ctx_len  [B] context length of each request in tokens, or NULL (every
 *            row of a selected entry is attended)
 *   out      [B][T][Hq][dv] doubles, every element written
 */
void oracle_attend(const oracle_attn_cfg* c, const uint16_t* q, const uint16_t* host_kv,
                   const int32_t* sel, const int32_t* len, const int32_t* status,
                   const int32_t* ctx_len, double* out) {
  const int64_t Hkv = c->n_kv_heads, Hq = c->n_q_heads, T = c->n_tokens, k = c->k;
  const int64_t dqk = c->head_dim_qk, dv = c->head_dim_v, G = Hq / Hkv;
  const int64_t tpe = c->latent ? 1 : c->tokens_per_entry;
  const int64_t row = c->latent ? dqk : tpe * (dqk + dv);
  const int64_t units = (int64_t)c->batch * Hkv;
  const int64_t tasks = units * T * G;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < tasks; ++task) {
    const int64_t u = task / (T * G), j = (task / G) % T, hl = task % G;
    const int64_t b = u / Hkv, g = u % Hkv, h = g * G + hl;
    double* o = out + ((b * T + j) * Hq + h) * dv;
    for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
    if (status && status[u] != 0) continue;
    int64_t n_sel = len ? len[u * T + j] : k;
    if (n_sel < 1 || n_sel > k) continue;  /* a failed step (its status says so) */
    const int64_t n = n_sel * tpe;
    double* qd = (double*)malloc(sizeof(double) * (size_t)dqk);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    const uint16_t* qrow = q + ((b * T + j) * Hq + h) * dqk;
    for (int64_t d = 0; d < dqk; ++d) qd[d] = bf16_value(qrow[d]);
    const int32_t* ids = sel + (u * T + j) * k;
    /* token row t of entry e is attended iff its position is in the context */
    const int64_t lim = ctx_len ? ctx_len[b] : INT64_MAX;
#define IN_CONTEXT(e, t) ((int64_t)ids[e] * tpe + (t) < lim)
    /* scores, token rows in selection order (the tokens of a page in order) */
    int have = 0;
    double mx = 0.0;
    for (int64_t e = 0; e < n_sel; ++e) {
      const uint16_t* r = host_kv + (u * (int64_t)c->n_entries + ids[e]) * row;
      for (int64_t t = 0; t < tpe; ++t) {
        if (!IN_CONTEXT(e, t)) continue;
        const uint16_t* key = r + t * dqk;
        double acc = 0.0;
        for (int64_t d = 0; d < dqk; ++d) acc += qd[d] * bf16_value(key[d]);
        s[e * tpe + t] = c->scale * acc;
        if (!have || s[e * tpe + t] > mx) mx = s[e * tpe + t];
        have = 1;
      }
    }
    double sum = 0.0;
    for (int64_t e = 0; e < n_sel; ++e)
      for (int64_t t = 0; t < tpe; ++t) {
        if (!IN_CONTEXT(e, t)) continue;
        s[e * tpe + t] = exp(s[e * tpe + t] - mx);
        sum += s[e * tpe + t];
      }
    for (int64_t e = 0; e < n_sel; ++e) {
      const uint16_t* r = host_kv + (u * (int64_t)c->n_entries + ids[e]) * row;
      for (int64_t t = 0; t < tpe; ++t) {
        if (!IN_CONTEXT(e, t)) continue;
        const uint16_t* val = c->latent ? r : r + tpe * dqk + t * dv;
        const double p = s[e * tpe + t] / sum;
        for (int64_t d = 0; d < dv; ++d) o[d] += p * bf16_value(val[d]);
      }
    }
#undef IN_CONTEXT
    free(qd);
    free(s);
  }
}
