// host_capi.cpp - C exports of the HIP-free host core for CPU-only tests.
// Built into libdflash_host.so (g++, no HIP); not part of libdflash.so.
#include <climits>
#include <string>
#include <vector>

#include "host_core.hpp"

using namespace dflash;

namespace {
thread_local std::string g_err;
}

extern "C" {

const char *dfh_last_error(void) { return g_err.c_str(); }

int dfh_validate(const dflash_config *c) {
  g_err.clear();
  return validate_config(*c, nullptr, &g_err);
}

void *dfh_pool_new(int32_t n) { return new BlockPool(n); }
void dfh_pool_delete(void *p) { delete (BlockPool *)p; }
int32_t dfh_pool_free_count(void *p) { return ((BlockPool *)p)->free_count(); }

void *dfh_seq_new(void *pool, int64_t budget, const int32_t *ids, int32_t n_ids, int32_t max_seq_len, int *status) {
  SeqRows *s = new SeqRows();
  g_err.clear();
  *status = seq_init(s, (BlockPool *)pool, budget, ids, n_ids, max_seq_len, &g_err);
  if (*status != DFLASH_OK) {
    delete s;
    return nullptr;
  }
  return s;
}

// reserve + commit n rows (what a precompute call does to the bookkeeping)
int dfh_seq_append(void *seq, void *pool, int32_t n) {
  SeqRows *s = (SeqRows *)seq;
  g_err.clear();
  int32_t first = 0;
  int rc = seq_reserve(s, (BlockPool *)pool, n, &first, &g_err);
  if (rc == DFLASH_OK) s->ctx_len += n;
  return rc;
}

int dfh_seq_trim(void *seq, int32_t a) {
  g_err.clear();
  return seq_trim((SeqRows *)seq, a, &g_err);
}

int32_t dfh_seq_ctx_len(void *seq) { return ((SeqRows *)seq)->ctx_len; }
int32_t dfh_seq_pending(void *seq) { return ((SeqRows *)seq)->ctx_len - ((SeqRows *)seq)->pending_base; }

int32_t dfh_seq_blocks(void *seq, int32_t *out, int32_t cap) {
  SeqRows *s = (SeqRows *)seq;
  int32_t n = (int32_t)s->blocks.size();
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = s->blocks[i];
  return n;
}

void dfh_seq_release(void *seq, void *pool) { seq_release((SeqRows *)seq, (BlockPool *)pool); }

// take: blocks into out (cap entries), returns the block count; *rows the rows moved
int32_t dfh_seq_take(void *seq, int32_t *out, int32_t cap, int32_t *rows) {
  std::vector<int32_t> b;
  seq_take((SeqRows *)seq, &b, rows);
  for (size_t i = 0; i < b.size() && (int32_t)i < cap; ++i) out[i] = b[i];
  return (int32_t)b.size();
}

int dfh_seq_install(void *seq, void *pool, const int32_t *blocks, int32_t n, int32_t rows, int32_t max_seq_len) {
  g_err.clear();
  return seq_install((SeqRows *)seq, (BlockPool *)pool, blocks, n, rows, max_seq_len, &g_err);
}

// the all-or-nothing reservation of a multi-state precompute
int dfh_reserve_rows(void **seqs, int32_t n, const int32_t *n_new, const int32_t *cap_blocks, void *pool) {
  g_err.clear();
  return reserve_rows((SeqRows *const *)seqs, n, n_new, cap_blocks, (BlockPool *)pool, &g_err);
}

int32_t dfh_attn_tiles(int32_t ctx_len, int32_t window) { return attn_tiles(ctx_len, window); }

// the propose's split plan: *tps and *n_split on success
int dfh_attn_plan(int32_t n, const int32_t *tiles, int32_t n_kv, int32_t max_tps, int64_t slot_cap, int32_t target_wgs,
                  int32_t *tps, int32_t *n_split, int32_t *nsplit_out, int32_t *split0_out) {
  g_err.clear();
  AttnPlan p;
  const int rc = attn_plan(n, tiles, n_kv, max_tps, slot_cap, target_wgs, &p, &g_err);
  if (rc == DFLASH_OK) {
    *tps = p.tps;
    *n_split = p.n_split;
    for (int32_t i = 0; i < n; ++i) {
      if (nsplit_out) nsplit_out[i] = p.nsplit[i];
      if (split0_out) split0_out[i] = p.split0[i];
    }
  }
  return rc;
}

// what dflash_build checks before it allocates: the config and the attention
// capacity of its widest batch of longest contexts (max_tps ctx tiles per split)
int dfh_build_check(const dflash_config *c, int32_t max_tps) {
  g_err.clear();
  Geo g;
  int rc = validate_config(*c, &g, &g_err);
  if (rc == DFLASH_OK) rc = check_attn_capacity(g, c->max_seq_len, max_tps, &g_err);
  return rc;
}

int dflash_yarn_inv_freq(int32_t head_dim, float rope_theta, float factor, float beta_fast, float beta_slow,
                         int32_t original_max_positions, float *out) {
  g_err.clear();
  return yarn_inv_freq(head_dim, rope_theta, factor, beta_fast, beta_slow, original_max_positions, out, &g_err);
}
void dfh_seq_delete(void *seq) { delete (SeqRows *)seq; }

}  // extern "C"
