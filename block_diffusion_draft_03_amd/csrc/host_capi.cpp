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

int dfh_seq_install(void *seq, void *pool, const int32_t *blocks, int32_t n, int32_t rows) {
  g_err.clear();
  return seq_install((SeqRows *)seq, (BlockPool *)pool, blocks, n, rows, &g_err);
}

int dflash_yarn_inv_freq(int32_t head_dim, float rope_theta, float factor, float beta_fast, float beta_slow,
                         int32_t original_max_positions, float *out) {
  g_err.clear();
  return yarn_inv_freq(head_dim, rope_theta, factor, beta_fast, beta_slow, original_max_positions, out, &g_err);
}
void dfh_seq_delete(void *seq) { delete (SeqRows *)seq; }

}  // extern "C"
