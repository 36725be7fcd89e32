/*
 * ORACLE -- test infrastructure only.  Nothing in the product path may link,
 * load or call this file; only the tests, the smoke check and the CPU leg of
 * the benchmark use it.
 *
 * A plain, slow CPU model of one decode step of HBM slot-buffer management for
 * dynamic sparse attention over a host-offloaded KV cache, as the AVSG
 * abstract describes it (arxivdaily 2609.37538, abstract: selected entries are
 * matched against the entries retained in a device buffer, slots are reserved
 * for the entries that need a host-to-device transfer, lifetime-based
 * management keeps frequently selected entries resident across steps, and one
 * reservation is shared by the query tokens of a multi-token-prediction
 * iteration), with the bucketed-LRU alternative of the Spin summary
 * (gist.science 2604.26837, section 2B, "Bucketed LRU-beleid": recency
 * buckets, e.g. 64, instead of a global LRU order).
 *
 * The pages give no formulas; the readings taken here are:
 *  - an entry is matched by its position id within its (request, KV head)
 *    unit (a page id when entries are pages);
 *  - the selection of an iteration is the sorted union U of its query
 *    tokens' lists; |U| larger than the buffer is an error (selections stay
 *    exact, AVSG abstract);
 *  - lifetime policy: every slot whose entry is in U is set to L; every other
 *    occupied slot loses one (never below 0); a slot at 0 is still resident
 *    and can still hit;
 *  - LRU policy: a slot's stamp is the step it was last selected; its bucket
 *    is min(floor((t - stamp - 1) / W), B - 1) for buckets W steps wide (1
 *    unless configured), larger buckets are older;
 *  - victims are the m slots not holding an entry of U that come first in
 *    the order (occupied?, lifetime or minus bucket, slot index): empty slots
 *    first, then the least-recently/least-often kept, then the lowest index;
 *  - the r-th miss in ascending id order takes the r-th victim.
 * Each step is written out in that order, with a library sort (qsort) where
 * the reading asks for an order and a two-pointer merge for the match.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status codes (numeric values fixed by the library's documented ABI) */
enum {
  OR_OK = 0,
  OR_ERR_UNSORTED = 16,
  OR_ERR_RANGE = 17,
  OR_ERR_CAPACITY = 18,
  OR_ERR_STATE = 19,
};
enum { OR_LIFETIME = 0, OR_LRU = 1 };

typedef struct {
  int32_t n_slots;     /* S */
  int32_t n_entries;   /* N */
  int32_t n_tokens;    /* T query tokens sharing one reservation */
  int32_t k;           /* selected entries per query token */
  int32_t policy;      /* OR_LIFETIME or OR_LRU */
  int32_t lifetime_L;
  int32_t n_buckets;   /* B */
  int32_t bucket_width; /* W: steps per LRU bucket */
} oracle_cfg;

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

typedef struct { int32_t tok, slot; } resident_t;
static int cmp_resident(const void* a, const void* b) {
  const resident_t *x = (const resident_t*)a, *y = (const resident_t*)b;
  if (x->tok != y->tok) return (x->tok > y->tok) - (x->tok < y->tok);
  return (x->slot > y->slot) - (x->slot < y->slot);
}

typedef struct { int32_t occupied, key, slot; } cand_t;
static int cmp_cand(const void* a, const void* b) {
  const cand_t *x = (const cand_t*)a, *y = (const cand_t*)b;
  if (x->occupied != y->occupied) return x->occupied - y->occupied;
  if (x->key != y->key) return (x->key > y->key) - (x->key < y->key);
  return (x->slot > y->slot) - (x->slot < y->slot);
}

/* position of x in the sorted array a[0..n), or -1 */
static int32_t find_sorted(const int32_t* a, int32_t n, int32_t x) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = lo + (hi - lo) / 2;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return (lo < n && a[lo] == x) ? lo : -1;
}

/*
 * One decode step t of one unit.
 *   sel        [T][k]  selected ids of each query token
 *   len        [T]     entries of each token's list in use (its first len[j]
 *                      ids; the rest is ignored), or NULL for k each.  A
 *                      length outside [1, k] is a range error.
 *   cap                slots this unit may use, [0, cap) (Spin summary,
 *                      section 2B: the buffer of each request is sized
 *                      dynamically); slots at or past cap take no part in
 *                      the step and are emptied once every check has passed
 *                      (a shrink drops what they held; an error, which
 *                      leaves the whole state unchanged, takes precedence).
 *                      A cap outside [1, S] is a range error; |U| > cap is
 *                      a capacity error.
 *   slot_tok   [S]     in/out: id held by each slot, -1 = empty
 *   life       [S]     in/out: lifetime (lifetime policy) or last-selected
 *                      step (LRU policy; -1 for a slot never filled)
 *   hit_flag   [T][k]  out: entry was resident before this step
 *   sel_slot   [T][k]  out: slot that holds the entry after this step
 *   fill_slot, fill_id [S] out: the m reservations, in miss order
 *   counts     [4]     out: n_hit, n_miss, n_evict, |U|
 *   mapped     [N]     1 if entry x has a row in host memory (a host KV
 *                      reached through a directory, Spin summary section
 *                      2C), or NULL: every entry has one.  A miss without a
 *                      row cannot be transferred: a range error, found
 *                      after every other check.
 *   n_ctx              entries that hold tokens of the request's context
 *                      (page e holds positions [e P, (e + 1) P); it is in
 *                      the context when e P < the context length): an id in
 *                      use at or past n_ctx is out of range like one past N.
 *                      n_ctx < 1 (a context length outside [1, N P]) is a
 *                      range error.
 * Returns a status; on error the state is unchanged, flags are 0, slots -1.
 */
int oracle_unit_step(const oracle_cfg* c, int64_t t, const int32_t* sel, const int32_t* len,
                     int32_t cap, int32_t* slot_tok, int32_t* life, uint8_t* hit_flag,
                     int32_t* sel_slot, int32_t* fill_slot, int32_t* fill_id, int32_t* counts,
                     const uint8_t* mapped, int32_t n_ctx) {
  const int32_t S_all = c->n_slots, N = c->n_entries, T = c->n_tokens, k = c->k;
  /* the slots in use: [0, S) */
  const int32_t S = cap;
  const int32_t L = c->lifetime_L, B = c->n_buckets;
  const int32_t tk = T * k;
  int status = OR_OK;
  for (int32_t i = 0; i < tk; ++i) { hit_flag[i] = 0; sel_slot[i] = -1; }
  for (int32_t i = 0; i < 4; ++i) counts[i] = 0;

  /* 1. validate the selection and form the union U of the lists in use */
  int range_bad = 0, order_bad = 0;
  int32_t n_used = 0;
  for (int32_t j = 0; j < T; ++j) {
    const int32_t nj = len ? len[j] : k;
    if (nj < 1 || nj > k) { range_bad = 1; continue; }
    for (int32_t i = 0; i < nj; ++i) {
      int32_t x = sel[j * k + i];
      if (x < 0 || x >= N || x >= n_ctx) range_bad = 1;
      if (i > 0 && x <= sel[j * k + i - 1]) order_bad = 1;
    }
    n_used += nj;
  }
  if (cap < 1 || cap > S_all || n_ctx < 1) range_bad = 1;
  if (range_bad) return OR_ERR_RANGE;
  if (order_bad) return OR_ERR_UNSORTED;
  int32_t* U = (int32_t*)malloc(sizeof(int32_t) * (size_t)(tk > 0 ? tk : 1));
  n_used = 0;
  for (int32_t j = 0; j < T; ++j) {
    const int32_t nj = len ? len[j] : k;
    memcpy(U + n_used, sel + j * k, sizeof(int32_t) * (size_t)nj);
    n_used += nj;
  }
  qsort(U, (size_t)n_used, sizeof(int32_t), cmp_i32);
  int32_t nu = 0;
  for (int32_t i = 0; i < n_used; ++i)
    if (nu == 0 || U[i] != U[nu - 1]) U[nu++] = U[i];
  if (nu > S) { free(U); return OR_ERR_CAPACITY; }

  /* the buffer state must be well formed: ids in range, counters in range */
  for (int32_t s = 0; s < S; ++s) {
    int32_t x = slot_tok[s];
    if (x < -1 || x >= N) status = OR_ERR_STATE;
    if (x >= 0) {
      if (c->policy == OR_LIFETIME && (life[s] < 0 || life[s] > L)) status = OR_ERR_STATE;
      if (c->policy == OR_LRU && (life[s] < 0 || (int64_t)life[s] >= t)) status = OR_ERR_STATE;
    }
  }
  if (status != OR_OK) { free(U); return status; }

  /* 2. match U against the resident ids of the slots in use: two-pointer
   *    merge of two sorted lists.  Nothing is written to the state until
   *    this last check has passed. */
  resident_t* R = (resident_t*)malloc(sizeof(resident_t) * (size_t)S);
  int32_t nr = 0;
  for (int32_t s = 0; s < S; ++s)
    if (slot_tok[s] >= 0) { R[nr].tok = slot_tok[s]; R[nr].slot = s; ++nr; }
  qsort(R, (size_t)nr, sizeof(resident_t), cmp_resident);
  int32_t* uslot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nu > 0 ? nu : 1));
  uint8_t* uhit = (uint8_t*)malloc((size_t)(nu > 0 ? nu : 1));
  uint8_t* selected_slot = (uint8_t*)calloc((size_t)S, 1);
  {
    int32_t a = 0, b = 0;
    for (a = 0; a < nu; ++a) { uslot[a] = -1; uhit[a] = 0; }
    a = 0;
    while (a < nu && b < nr) {
      if (U[a] < R[b].tok) ++a;
      else if (U[a] > R[b].tok) ++b;
      else {
        /* an id of U held by two slots is a corrupted state */
        if (b + 1 < nr && R[b + 1].tok == U[a]) status = OR_ERR_STATE;
        uslot[a] = R[b].slot;
        uhit[a] = 1;
        selected_slot[R[b].slot] = 1;
        ++a; ++b;
      }
    }
  }
  free(R);
  if (status != OR_OK) { free(U); free(uslot); free(uhit); free(selected_slot); return status; }

  int32_t n_hit = 0;
  for (int32_t a = 0; a < nu; ++a) n_hit += uhit[a];
  const int32_t m = nu - n_hit;

  /* every miss must have a row to transfer */
  if (mapped)
    for (int32_t a = 0; a < nu; ++a)
      if (!uhit[a] && !mapped[U[a]]) status = OR_ERR_RANGE;
  if (status != OR_OK) { free(U); free(uslot); free(uhit); free(selected_slot); return status; }

  /* every check has passed: the slots past the capacity are emptied (they
   * take no part in the match above, and are never candidates below) */
  for (int32_t s = S; s < S_all; ++s) {
    slot_tok[s] = -1;
    life[s] = c->policy == OR_LRU ? -1 : 0;
  }

  /* 3. policy update of the slots (all slots; the caller's arrays) */
  for (int32_t s = 0; s < S; ++s) {
    if (c->policy == OR_LIFETIME) {
      if (selected_slot[s]) life[s] = L;
      else if (slot_tok[s] >= 0) life[s] = life[s] > 0 ? life[s] - 1 : 0;
    } else {
      if (selected_slot[s]) life[s] = (int32_t)t;
    }
  }

  /* 4. candidates (slots not holding an id of U) in eviction order */
  cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)S);
  int32_t nc = 0;
  for (int32_t s = 0; s < S; ++s) {
    if (selected_slot[s]) continue;
    cand[nc].slot = s;
    cand[nc].occupied = slot_tok[s] >= 0;
    if (!cand[nc].occupied) cand[nc].key = 0;
    else if (c->policy == OR_LIFETIME) cand[nc].key = life[s];
    else {
      int64_t bucket = (t - (int64_t)life[s] - 1) / c->bucket_width;
      if (bucket > B - 1) bucket = B - 1;
      cand[nc].key = -(int32_t)bucket;
    }
    ++nc;
  }
  qsort(cand, (size_t)nc, sizeof(cand_t), cmp_cand);

  /* 5. reserve: the r-th miss (ascending id) takes the r-th victim */
  int32_t r = 0, n_evict = 0;
  for (int32_t a = 0; a < nu; ++a) {
    if (uhit[a]) continue;
    int32_t s = cand[r].slot;
    if (slot_tok[s] >= 0) ++n_evict;
    slot_tok[s] = U[a];
    life[s] = c->policy == OR_LIFETIME ? L : (int32_t)t;
    uslot[a] = s;
    fill_slot[r] = s;
    fill_id[r] = U[a];
    ++r;
  }

  /* 6. per-(token, entry) outputs read off the union (entries past a list's
   *    length keep slot -1 and flag 0) */
  for (int32_t j = 0; j < T; ++j) {
    const int32_t nj = len ? len[j] : k;
    for (int32_t i = j * k; i < j * k + nj; ++i) {
      int32_t a = find_sorted(U, nu, sel[i]);
      sel_slot[i] = uslot[a];
      hit_flag[i] = uhit[a];
    }
  }
  counts[0] = n_hit;
  counts[1] = m;
  counts[2] = n_evict;
  counts[3] = nu;
  free(U); free(uslot); free(uhit); free(selected_slot); free(cand);
  return OR_OK;
}

/* All units of one step (units are independent; OpenMP over units).  len is
 * [units][T] or NULL, cap [units] or NULL (every unit uses all S slots),
 * mapped [units][N] or NULL (every entry has a host row), n_ctx [units] or
 * NULL (every entry is in the context). */
void oracle_step(const oracle_cfg* c, int64_t units, int64_t t, const int32_t* sel,
                 const int32_t* len, const int32_t* cap, int32_t* slot_tok, int32_t* life,
                 uint8_t* hit_flag, int32_t* sel_slot, int32_t* fill_slot, int32_t* fill_id,
                 int32_t* counts, int32_t* status, const uint8_t* mapped, const int32_t* n_ctx) {
  const int64_t tk = (int64_t)c->n_tokens * c->k, S = c->n_slots;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u)
    status[u] = oracle_unit_step(c, t, sel + u * tk, len ? len + u * c->n_tokens : NULL,
                                 cap ? cap[u] : c->n_slots,
                                 slot_tok + u * S, life + u * S, hit_flag + u * tk,
                                 sel_slot + u * tk, fill_slot + u * S, fill_id + u * S,
                                 counts + u * 4, mapped ? mapped + u * c->n_entries : NULL,
                                 n_ctx ? n_ctx[u] : c->n_entries);
}

/* Threads used by oracle_step's loop over units. */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
