/* Host-only exercise of the C ABI for the sanitizer build: random trees are
 * planned, exported and grown through tree_attn_plan_extend; every documented
 * error code and every allocation step of ta_plan_opts.fail_alloc_after is
 * hit; every plan is destroyed. Built and run with the address and
 * undefined-behaviour sanitizers (leak checking on) by
 * tests/test_sanitized_host.py. Prints "ok <plans>" and exits 0 when every
 * check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tree_attn.h"

static uint64_t rng_state = 88172645463325252ull;
static uint32_t rnd(uint32_t n) { /* xorshift64 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state % n);
}

static int failures = 0;
#define CHECK(cond, ...)                            \
  do {                                              \
    if (!(cond)) {                                  \
      fprintf(stderr, "check failed: " __VA_ARGS__); \
      fprintf(stderr, " (%s)\n", tree_attn_last_error()); \
      ++failures;                                   \
    }                                               \
  } while (0)

typedef struct {
  int32_t n, ps, qpl, hq, hk, d;
  int32_t parent[64], len[64], ptr[65], ids[40 * 400];
} tree;

static void random_tree(tree* t) {
  t->n = 1 + (int32_t)rnd(40);
  t->ps = (int32_t[]){1, 8, 16, 32}[rnd(4)];
  t->qpl = 1 + (int32_t)rnd(4);
  t->hk = 1 + (int32_t)rnd(4);
  t->hq = t->hk * (int32_t[]){1, 2, 4, 16}[rnd(4)];
  t->d = rnd(2) ? 128 : 64;
  int has_child[64] = {0};
  t->parent[0] = -1;
  for (int v = 1; v < t->n; ++v) {
    t->parent[v] = (int32_t)rnd((uint32_t)v);
    has_child[t->parent[v]] = 1;
  }
  int32_t pages = 0;
  for (int v = 0; v < t->n; ++v) {
    int32_t l = 1 + (int32_t)rnd(400);
    if (!has_child[v] && l < t->qpl) l = t->qpl;
    t->len[v] = l;
    t->ptr[v] = pages;
    pages += (l + t->ps - 1) / t->ps;
  }
  t->ptr[t->n] = pages;
  for (int32_t x = 0; x < pages; ++x) t->ids[x] = x;
}

static ta_status plan_tree(const tree* t, ta_plan_opts* o, ta_plan** p) {
  return tree_attn_plan(t->parent, t->n, t->len, t->ptr, t->ids, t->ps, t->qpl, t->hq, t->hk, t->d, o, p);
}

static void export_all(const ta_plan* p) {
  int64_t none = 0;  /* host-only plans have no device tables to read back */
  CHECK(tree_attn_plan_export(p, TA_T_DEVICE_TABLES, NULL, &none) == TA_EINVAL, "device tables of a host-only plan");
  for (int32_t id = 0; id < TA_T_COUNT; ++id) {
    if (id == TA_T_DEVICE_TABLES) continue;
    int64_t len = 0;
    CHECK(tree_attn_plan_export(p, id, NULL, &len) == TA_OK, "export len %d", id);
    int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)(len ? len : 1));
    CHECK(tree_attn_plan_export(p, id, buf, &len) == TA_OK, "export %d", id);
    free(buf);
  }
}

/* grow every leaf by 1..qpl tokens, with fresh page ids after the tree's */
static ta_status grow(ta_plan* p, const tree* t, int32_t* lens, int32_t* next_page) {
  int32_t n_leaves = 0, leaf_len[64], add[64], pages[512], n_pages = 0;
  int has_child[64] = {0};
  for (int v = 1; v < t->n; ++v) has_child[t->parent[v]] = 1;
  for (int v = 0; v < t->n; ++v)
    if (!has_child[v]) leaf_len[n_leaves++] = v;
  for (int r = 0; r < n_leaves; ++r) {
    const int v = leaf_len[r];
    add[r] = 1 + (int32_t)rnd((uint32_t)t->qpl);
    const int32_t need = (lens[v] + add[r] + t->ps - 1) / t->ps - (lens[v] + t->ps - 1) / t->ps;
    for (int32_t x = 0; x < need; ++x) pages[n_pages++] = (*next_page)++;
  }
  const ta_status s = tree_attn_plan_extend(p, add, pages, n_pages, NULL, NULL);
  if (s == TA_OK)
    for (int r = 0; r < n_leaves; ++r) lens[leaf_len[r]] += add[r];
  return s;
}

int main(void) {
  int plans = 0;
  tree t;
  for (int iter = 0; iter < 300; ++iter) {
    random_tree(&t);
    ta_plan_opts o;
    memset(&o, 0, sizeof o);
    o.host_only = 1;
    o.ncu = 1 + (int32_t)rnd(300);
    if (iter % 3 == 1) o.no_split = 1;
    ta_plan* p = NULL;
    CHECK(plan_tree(&t, &o, &p) == TA_OK, "plan %d", iter);
    if (!p) continue;
    ++plans;
    int32_t nq = 0, ni = 0;
    int64_t ws = 0;
    CHECK(tree_attn_plan_info(p, &nq, &ws, &ni) == TA_OK && ws > 0, "info %d", iter);
    export_all(p);
    int32_t lens[64], next_page = t.ptr[t.n];
    memcpy(lens, t.len, sizeof lens);
    for (int step = 0; step < 4; ++step) CHECK(grow(p, &t, lens, &next_page) == TA_OK, "extend %d", iter);
    export_all(p);
    tree_attn_plan_destroy(p);
  }

  /* allocation failure at every host step of a host-only plan, then one
   * past them (succeeds); an extend whose host step fails leaves the plan
   * as it was and usable */
  random_tree(&t);
  for (int32_t k = 1; k <= 4; ++k) {
    ta_plan_opts o;
    memset(&o, 0, sizeof o);
    o.host_only = 1;
    o.fail_alloc_after = k;
    ta_plan* p = NULL;
    const ta_status s = plan_tree(&t, &o, &p);
    if (k <= 3) {
      CHECK(s == TA_ENOMEM && p == NULL, "fail_alloc_after %d", k);
      CHECK(strlen(tree_attn_last_error()) > 0, "message after ENOMEM");
    } else {
      CHECK(s == TA_OK && p != NULL, "fail_alloc_after %d (past the host steps)", k);
      int32_t lens[64], next_page = t.ptr[t.n];
      memcpy(lens, t.len, sizeof lens);
      CHECK(grow(p, &t, lens, &next_page) == TA_ENOMEM, "extend's host step fails");
      CHECK(grow(p, &t, lens, &next_page) == TA_OK, "next extend succeeds");
      export_all(p);
      tree_attn_plan_destroy(p);
    }
  }

  /* documented error codes */
  {
    const int32_t par[3] = {-1, 0, 0}, len[3] = {20, 5, 7}, ptr[4] = {0, 2, 3, 4}, ids[4] = {0, 1, 2, 3};
    ta_plan_opts o;
    memset(&o, 0, sizeof o);
    o.host_only = 1;
    ta_plan* p = NULL;
    const int32_t cyc[3] = {1, 2, 0}, two_roots[3] = {-1, -1, 0}, zero_len[3] = {20, 0, 7};
    const int32_t bad_ptr[4] = {0, 1, 3, 4};
    CHECK(tree_attn_plan(cyc, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "cycle");
    CHECK(tree_attn_plan(two_roots, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "two roots");
    CHECK(tree_attn_plan(par, 3, zero_len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "zero length");
    CHECK(tree_attn_plan(par, 3, len, bad_ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "page CSR");
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 6, 4, 4, 128, &o, &p) == TA_EINVAL, "leaf shorter than qpl");
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 1, 6, 4, 128, &o, &p) == TA_EINVAL, "heads");
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 1, 4, 4, 96, &o, &p) == TA_EUNSUPPORTED, "head_dim");
    CHECK(tree_attn_plan(NULL, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "null parent");
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, NULL) == TA_EINVAL, "null out");
    o.fail_alloc_after = -1;
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_EINVAL, "negative option");
    o.fail_alloc_after = 0;
    CHECK(tree_attn_plan(par, 3, len, ptr, ids, 16, 1, 4, 4, 128, &o, &p) == TA_OK, "valid plan");
    const int32_t add_bad[2] = {1, -1};
    CHECK(tree_attn_plan_extend(p, add_bad, NULL, 0, NULL, NULL) == TA_EINVAL, "negative growth");
    int64_t len_out = 0;
    CHECK(tree_attn_plan_export(p, 99, NULL, &len_out) == TA_EINVAL, "table id");
    CHECK(tree_attn_decode(NULL, TA_BF16, NULL, p, NULL, NULL) == TA_EINVAL, "decode host-only");
    tree_attn_plan_destroy(p);
    tree_attn_plan_destroy(NULL);
  }
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok %d\n", plans);
  return 0;
}
