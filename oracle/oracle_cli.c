/*
 * ORACLE -- test infrastructure only.  A command-line front end of the
 * oracle's C functions (avsg_oracle.c, attention.c), so that the oracle can
 * be built as a standalone program with the address and undefined-behaviour
 * sanitizers and driven by a test through plain text.
 *
 * Input on stdin, whitespace-separated integers, one command per run:
 *
 *   state S N T k policy L B steps
 *     then per step: t cap ids[T*k]            (cap -1: all S slots)
 *   prints per step:
 *     status n_hit n_miss n_evict n_union
 *     flags[T*k]
 *     slots[T*k]
 *     tok[S]
 *     life[S]
 *
 *   attn B Hkv Hq T dqk dv latent tpe N k scale_bits_hi scale_bits_lo
 *     then q[B*T*Hq*dqk] (bf16 bits), host[units*N*row] (bf16 bits),
 *     ids[units*T*k], status[units]
 *   prints out[B*T*Hq*dv] as %.17g
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t n_slots, n_entries, n_tokens, k, policy, lifetime_L, n_buckets, bucket_width;
} oracle_cfg;
typedef struct {
  int32_t batch, n_kv_heads, n_q_heads, n_tokens, head_dim_qk, head_dim_v, latent,
      tokens_per_entry, n_entries, k;
  double scale;
} oracle_attn_cfg;

int oracle_unit_step(const oracle_cfg* c, int64_t t, const int32_t* sel, const int32_t* len,
                     int32_t cap, int32_t* slot_tok, int32_t* life, uint8_t* hit_flag,
                     int32_t* sel_slot, int32_t* fill_slot, int32_t* fill_id, int32_t* counts,
                     const uint8_t* mapped, int32_t n_ctx);
void oracle_attend(const oracle_attn_cfg* c, const uint16_t* q, const uint16_t* host_kv,
                   const int32_t* sel, const int32_t* len, const int32_t* status,
                   const int32_t* ctx_len, double* out);

static long long rd(void) {
  long long v;
  if (scanf("%lld", &v) != 1) {
    fprintf(stderr, "oracle_cli: truncated input\n");
    exit(2);
  }
  return v;
}

static void print_i32(const int32_t* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i) printf(i ? " %d" : "%d", a[i]);
  printf("\n");
}

static int run_state(void) {
  oracle_cfg c;
  c.n_slots = (int32_t)rd();
  c.n_entries = (int32_t)rd();
  c.n_tokens = (int32_t)rd();
  c.k = (int32_t)rd();
  c.policy = (int32_t)rd();
  c.lifetime_L = (int32_t)rd();
  c.n_buckets = (int32_t)rd();
  c.bucket_width = 1;
  const int64_t steps = rd();
  const int64_t S = c.n_slots, tk = (int64_t)c.n_tokens * c.k;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* life = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)tk);
  uint8_t* flags = (uint8_t*)malloc((size_t)tk);
  int32_t* slots = (int32_t*)malloc(sizeof(int32_t) * (size_t)tk);
  int32_t* fs = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* fi = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* fl = (int32_t*)malloc(sizeof(int32_t) * (size_t)tk);
  int32_t counts[4];
  for (int64_t s = 0; s < S; ++s) {
    tok[s] = -1;
    life[s] = c.policy == 1 ? -1 : 0;
  }
  for (int64_t i = 0; i < steps; ++i) {
    const int64_t t = rd();
    const int32_t cap = (int32_t)rd();
    for (int64_t e = 0; e < tk; ++e) sel[e] = (int32_t)rd();
    const int st = oracle_unit_step(&c, t, sel, NULL, cap < 0 ? c.n_slots : cap, tok, life, flags,
                                    slots, fs, fi, counts, NULL, c.n_entries);
    printf("%d %d %d %d %d\n", st, counts[0], counts[1], counts[2], counts[3]);
    for (int64_t e = 0; e < tk; ++e) fl[e] = flags[e];
    print_i32(fl, tk);
    print_i32(slots, tk);
    print_i32(tok, S);
    print_i32(life, S);
  }
  free(tok); free(life); free(sel); free(flags); free(slots); free(fs); free(fi); free(fl);
  return 0;
}

static int run_attn(void) {
  oracle_attn_cfg c;
  c.batch = (int32_t)rd();
  c.n_kv_heads = (int32_t)rd();
  c.n_q_heads = (int32_t)rd();
  c.n_tokens = (int32_t)rd();
  c.head_dim_qk = (int32_t)rd();
  c.head_dim_v = (int32_t)rd();
  c.latent = (int32_t)rd();
  c.tokens_per_entry = (int32_t)rd();
  c.n_entries = (int32_t)rd();
  c.k = (int32_t)rd();
  const uint64_t hi = (uint64_t)rd(), lo = (uint64_t)rd();
  const uint64_t bits = hi << 32 | lo;
  memcpy(&c.scale, &bits, sizeof c.scale);
  const int64_t units = (int64_t)c.batch * c.n_kv_heads;
  const int64_t row = c.latent ? c.head_dim_qk
                               : (int64_t)c.tokens_per_entry * (c.head_dim_qk + c.head_dim_v);
  const int64_t nq = (int64_t)c.batch * c.n_tokens * c.n_q_heads * c.head_dim_qk;
  const int64_t nh = units * c.n_entries * row, ns = units * c.n_tokens * c.k;
  const int64_t no = (int64_t)c.batch * c.n_tokens * c.n_q_heads * c.head_dim_v;
  uint16_t* q = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nq);
  uint16_t* host = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nh);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)ns);
  int32_t* status = (int32_t*)malloc(sizeof(int32_t) * (size_t)units);
  double* out = (double*)malloc(sizeof(double) * (size_t)no);
  for (int64_t i = 0; i < nq; ++i) q[i] = (uint16_t)rd();
  for (int64_t i = 0; i < nh; ++i) host[i] = (uint16_t)rd();
  for (int64_t i = 0; i < ns; ++i) sel[i] = (int32_t)rd();
  for (int64_t i = 0; i < units; ++i) status[i] = (int32_t)rd();
  oracle_attend(&c, q, host, sel, NULL, status, NULL, out);
  for (int64_t i = 0; i < no; ++i) printf(i ? " %.17g" : "%.17g", out[i]);
  printf("\n");
  free(q); free(host); free(sel); free(status); free(out);
  return 0;
}

int main(void) {
  char cmd[16];
  if (scanf("%15s", cmd) != 1) return 2;
  if (strcmp(cmd, "state") == 0) return run_state();
  if (strcmp(cmd, "attn") == 0) return run_attn();
  fprintf(stderr, "oracle_cli: unknown command %s\n", cmd);
  return 2;
}
