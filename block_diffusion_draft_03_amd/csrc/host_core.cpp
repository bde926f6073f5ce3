// host_core.cpp - see host_core.hpp.
#include "host_core.hpp"

#include <algorithm>
#include <climits>
#include <cmath>

namespace dflash {

static int fail(std::string *err, int code, const std::string &msg) {
  if (err) *err = msg;
  return code;
}

int validate_config(const dflash_config &c, Geo *g, std::string *err) {
  auto bad = [&](const std::string &m) { return fail(err, DFLASH_E_INVALID, "config: " + m); };
  if (c.num_layers < 1 || c.num_layers > 64) return bad("num_layers must be in [1, 64]");
  if (c.hidden < 64 || c.hidden % 64) return bad("hidden must be a positive multiple of 64");
  if (c.intermediate < 64 || c.intermediate % 64) return bad("intermediate must be a positive multiple of 64");
  if (!(c.head_dim == 16 || c.head_dim == 32 || c.head_dim == 64 || c.head_dim == 128))
    return bad("head_dim must be 16, 32, 64 or 128");
  if (c.num_q_heads < 1 || c.num_kv_heads < 1 || c.num_q_heads % c.num_kv_heads)
    return bad("num_kv_heads must divide num_q_heads");
  if ((c.num_q_heads * c.head_dim) % 64 || (c.num_kv_heads * c.head_dim) % 16)
    return bad("num_q_heads * head_dim must be a multiple of 64");
  if (c.gamma < 2 || c.gamma > 64) return bad("gamma must be in [2, 64]");
  if ((c.num_q_heads / c.num_kv_heads) * c.gamma > 128)
    return bad("(num_q_heads / num_kv_heads) * gamma must be at most 128");
  if (c.vocab < 2) return bad("vocab must be >= 2");
  if (c.mask_token_id >= (uint32_t)c.vocab) return bad("mask_token_id must be < vocab");
  if (c.num_target_layers < 1 || c.target_hidden < 1) return bad("num_target_layers and target_hidden must be >= 1");
  if (((int64_t)c.num_target_layers * c.target_hidden) % 8)
    return bad("num_target_layers * target_hidden must be a multiple of 8");
  if (c.ctx_window < 0) return bad("ctx_window must be >= 0");
  if (!(c.rope_theta > 1.0f) || !std::isfinite(c.rope_theta)) return bad("rope_theta must be finite and > 1");
  if (!(c.rms_eps >= 0.0f) || !std::isfinite(c.rms_eps)) return bad("rms_eps must be finite and >= 0");
  if (c.kv_block_size != DFLASH_KV_BLOCK) return bad("kv_block_size must be 16");
  if (c.kv_pool_blocks < 1) return bad("kv_pool_blocks must be >= 1");
  if (c.max_batch < 1 || c.max_batch > DFLASH_MAX_BATCH) return bad("max_batch must be in [1, 64]");
  if (c.max_seq_len < 1) return bad("max_seq_len must be >= 1");
  if (c.weight_dtype != DFLASH_F32 && c.weight_dtype != DFLASH_BF16) return bad("weight_dtype must be F32 or BF16");
  if (c.lm_head_dtype != DFLASH_BF16 && c.lm_head_dtype != DFLASH_FP8_E4M3)
    return bad("lm_head_dtype must be BF16 or FP8_E4M3");
  if (c.kv_dtype != DFLASH_BF16 && c.kv_dtype != DFLASH_FP8_E4M3) return bad("kv_dtype must be BF16 or FP8_E4M3");
  if (c.kv_dtype == DFLASH_FP8_E4M3 && c.head_dim < 64) return bad("an FP8_E4M3 KV cache needs head_dim >= 64");
  if (c.shifted_rows != 0 && c.shifted_rows != 1) return bad("shifted_rows must be 0 or 1");
  if (c.fp8_weights != 0 && c.fp8_weights != 1) return bad("fp8_weights must be 0 or 1");
  if (c.lm_act_fp8 != 0 && c.lm_act_fp8 != 1) return bad("lm_act_fp8 must be 0 or 1");
  if (c.lm_act_fp8 && c.lm_head_dtype != DFLASH_FP8_E4M3) return bad("lm_act_fp8 needs an FP8_E4M3 LM head");
  if (c.lm_act_fp8 && (c.vocab % 256 != 0 || c.hidden % 128 != 0))
    return bad("lm_act_fp8 needs vocab a multiple of 256 and hidden a multiple of 128");
  if (g) {
    g->L = c.num_layers;
    g->h = c.hidden;
    g->I = c.intermediate;
    g->n_q = c.num_q_heads;
    g->n_kv = c.num_kv_heads;
    g->d = c.head_dim;
    g->V = c.vocab;
    g->gamma = c.gamma;
    g->T = c.num_target_layers;
    g->Ht = c.target_hidden;
    g->W = c.ctx_window;
    g->q_dim = c.num_q_heads * c.head_dim;
    g->kv_dim = c.num_kv_heads * c.head_dim;
    g->qkv_dim = g->q_dim + 2 * g->kv_dim;
    g->fc_in = c.num_target_layers * c.target_hidden;
    g->fkv_dim = c.num_layers * 2 * g->kv_dim;
    g->words = (c.vocab + 31) / 32;
    g->rep = c.num_q_heads / c.num_kv_heads;
    g->max_batch = c.max_batch;
    g->m_max = c.max_batch * c.gamma;
    g->mask_id = c.mask_token_id;
    g->kv_fp8 = c.kv_dtype == DFLASH_FP8_E4M3;
    g->head_fp8 = c.lm_head_dtype == DFLASH_FP8_E4M3;
    g->w_f32 = c.weight_dtype == DFLASH_F32;
    g->shifted = c.shifted_rows != 0;
    g->fp8w = c.fp8_weights != 0;
    g->a8 = c.lm_act_fp8 != 0;
  }
  return DFLASH_OK;
}

BlockPool::BlockPool(int32_t n) : used_(n > 0 ? n : 0, 0), free_(n > 0 ? n : 0) {}

int32_t BlockPool::alloc() {
  for (int32_t i = hint_; i < size(); ++i) {
    if (!used_[i]) {
      used_[i] = 1;
      --free_;
      hint_ = i + 1;
      return i;
    }
  }
  hint_ = size();
  return -1;
}

bool BlockPool::take(int32_t id) {
  if (!is_free(id)) return false;
  used_[id] = 1;
  --free_;
  return true;
}

void BlockPool::release(int32_t id) {
  if (id < 0 || id >= size() || !used_[id]) return;
  used_[id] = 0;
  ++free_;
  if (id < hint_) hint_ = id;
}

int seq_init(SeqRows *s, BlockPool *pool, int64_t budget_tokens, const int32_t *block_ids, int32_t n_ids,
             int32_t max_seq_len, std::string *err) {
  *s = SeqRows();
  if (budget_tokens < 0) return fail(err, DFLASH_E_INVALID, "budget_tokens must be >= 0");
  if (block_ids || n_ids) {
    if (!block_ids || n_ids <= 0) return fail(err, DFLASH_E_INVALID, "block_ids and n_ids must be given together");
    for (int32_t i = 0; i < n_ids; ++i) {
      if (!pool->is_free(block_ids[i])) {
        for (int32_t j = 0; j < i; ++j) pool->release(block_ids[j]);
        return fail(err, DFLASH_E_NO_BLOCKS, "explicit block " + std::to_string(block_ids[i]) + " is not a free pool block");
      }
      pool->take(block_ids[i]);
    }
    s->blocks.assign(block_ids, block_ids + n_ids);
    s->cap_rows = std::min<int64_t>((int64_t)n_ids * DFLASH_KV_BLOCK, max_seq_len);
    if (budget_tokens != INT64_MAX && budget_tokens < s->cap_rows) s->cap_rows = budget_tokens;
    s->grow = false;
    return DFLASH_OK;
  }
  if (budget_tokens == INT64_MAX) {
    s->cap_rows = max_seq_len;
    s->grow = true;
    return DFLASH_OK;
  }
  const int64_t cap = std::min<int64_t>(budget_tokens, max_seq_len);
  int64_t nb = (cap + DFLASH_KV_BLOCK - 1) / DFLASH_KV_BLOCK;
  if (nb > pool->free_count()) return fail(err, DFLASH_E_NO_BLOCKS, "KV pool has too few free blocks for the budget");
  for (int64_t i = 0; i < nb; ++i) s->blocks.push_back(pool->alloc());
  s->cap_rows = cap;
  s->grow = false;
  return DFLASH_OK;
}

int seq_reserve(SeqRows *s, BlockPool *pool, int32_t n, int32_t *first_new_block, std::string *err) {
  if (first_new_block) *first_new_block = (int32_t)s->blocks.size();
  if (n < 0) return fail(err, DFLASH_E_INVALID, "row count must be >= 0");
  int64_t need_rows = (int64_t)s->ctx_len + n;
  if (need_rows > s->cap_rows) return fail(err, DFLASH_E_NO_BLOCKS, "the state's token budget is exhausted");
  int64_t need_blocks = (need_rows + DFLASH_KV_BLOCK - 1) / DFLASH_KV_BLOCK;
  int64_t have = (int64_t)s->blocks.size();
  if (need_blocks <= have) return DFLASH_OK;
  if (!s->grow) return fail(err, DFLASH_E_NO_BLOCKS, "the state's blocks are exhausted");
  if (need_blocks - have > pool->free_count()) return fail(err, DFLASH_E_NO_BLOCKS, "the KV pool is exhausted");
  for (int64_t i = have; i < need_blocks; ++i) s->blocks.push_back(pool->alloc());
  return DFLASH_OK;
}

void seq_unreserve(SeqRows *s, BlockPool *pool, int32_t first_new_block) {
  while ((int32_t)s->blocks.size() > first_new_block) {
    pool->release(s->blocks.back());
    s->blocks.pop_back();
  }
}

int reserve_rows(SeqRows *const *s, int32_t n, const int32_t *n_new, const int32_t *cap_blocks, BlockPool *pool,
                 std::string *err) {
  std::vector<int32_t> first(n > 0 ? n : 0, 0);
  for (int32_t i = 0; i < n; ++i) {
    int rc = seq_reserve(s[i], pool, n_new[i], &first[i], err);
    if (rc == DFLASH_OK && cap_blocks && (int32_t)s[i]->blocks.size() > cap_blocks[i]) {
      seq_unreserve(s[i], pool, first[i]);
      rc = fail(err, DFLASH_E_NO_BLOCKS, "block table capacity exceeded");
    }
    if (rc != DFLASH_OK) {
      for (int32_t j = i - 1; j >= 0; --j) seq_unreserve(s[j], pool, first[j]);
      if (err) *err = "state " + std::to_string(i) + ": " + *err;
      return rc;
    }
  }
  return DFLASH_OK;
}

int seq_trim(SeqRows *s, int32_t a, std::string *err) {
  int32_t pending = s->ctx_len - s->pending_base;
  if (a < 0 || a > pending)
    return fail(err, DFLASH_E_INVALID,
                "num_accepted " + std::to_string(a) + " outside [0, " + std::to_string(pending) + "]");
  s->ctx_len = s->pending_base + a;
  s->pending_base = s->ctx_len;
  return DFLASH_OK;
}

void seq_release(SeqRows *s, BlockPool *pool) {
  for (int32_t b : s->blocks) pool->release(b);
  s->blocks.clear();
  s->ctx_len = 0;
  s->pending_base = 0;
}

void seq_take(SeqRows *s, std::vector<int32_t> *blocks, int32_t *rows) {
  *blocks = std::move(s->blocks);
  *rows = s->ctx_len;
  s->blocks.clear();
  s->ctx_len = 0;
  s->pending_base = 0;
  s->grow = true;
}

int seq_install(SeqRows *s, BlockPool *pool, const int32_t *blocks, int32_t n, int32_t rows, int32_t max_seq_len,
                std::string *err) {
  if (s->ctx_len != 0) return fail(err, DFLASH_E_INVALID, "install needs a state that holds no rows");
  if (!blocks || n < 1) return fail(err, DFLASH_E_INVALID, "install needs at least one block");
  if (rows < 0 || (int64_t)rows > (int64_t)n * DFLASH_KV_BLOCK)
    return fail(err, DFLASH_E_INVALID, "installed rows must fit the installed blocks");
  if (rows > max_seq_len) return fail(err, DFLASH_E_INVALID, "installed rows exceed max_seq_len");
  std::vector<uint8_t> seen(pool->size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= pool->size() || pool->is_free(b))
      return fail(err, DFLASH_E_INVALID, "block " + std::to_string(b) + " is not an allocated pool block");
    if (seen[b]++) return fail(err, DFLASH_E_INVALID, "block " + std::to_string(b) + " is given twice");
  }
  for (int32_t b : s->blocks) pool->release(b);
  s->blocks.assign(blocks, blocks + n);
  s->ctx_len = rows;
  s->pending_base = rows;
  s->cap_rows = std::min<int64_t>(std::max<int64_t>(s->cap_rows, (int64_t)n * DFLASH_KV_BLOCK), max_seq_len);
  s->grow = true;
  return DFLASH_OK;
}

int32_t attn_tiles(int32_t c, int32_t window) {
  const int32_t lo = window > 0 ? std::max(0, c - window) : c;
  return lo < c ? (c - lo / DFLASH_KV_BLOCK * DFLASH_KV_BLOCK + 31) / 32 : 0;
}

int32_t attn_tiles_worst(int32_t window, int32_t max_seq_len) {
  // tiles grow with c up to the window; past it the aligned start adds up to
  // 15 rows, so the worst case is among c = min(W, max) .. min(W + 15, max)
  int32_t worst = 0;
  const int32_t c0 = std::min(window, max_seq_len);
  for (int32_t c = c0; c <= std::min(c0 + DFLASH_KV_BLOCK - 1, max_seq_len); ++c)
    worst = std::max(worst, attn_tiles(c, window));
  return worst;
}

int attn_plan(int32_t n, const int32_t *tiles, int32_t n_kv, int32_t max_tps, int64_t slot_cap, int32_t target_wgs,
              AttnPlan *plan, std::string *err) {
  if (n < 1 || n > DFLASH_MAX_BATCH || n_kv < 1 || max_tps < 1 || target_wgs < 1)
    return fail(err, DFLASH_E_INVALID, "attention plan: bad batch, head count or tile limit");
  int32_t max_T = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (tiles[i] < 0) return fail(err, DFLASH_E_INVALID, "attention plan: negative tile count");
    max_T = std::max(max_T, tiles[i]);
  }
  // a sequence with t ctx tiles takes (t + tps) / tps splits of at most tps
  // units (its block tile counted as one more), so its last split is no
  // longer than the others
  auto splits_of = [](int64_t t, int64_t tps) { return (t + tps) / tps; };
  auto flat = [&](int32_t tps) {
    int64_t f = 0;
    for (int32_t i = 0; i < n; ++i) f += splits_of(tiles[i], tps);
    return f;
  };
  const int64_t cap = std::min<int64_t>(ATTN_MAX_FLAT, slot_cap);
  // the preferred split count, as far as the tile limit allows, and never
  // more than ATTN_MAX_SPLITS splits
  int32_t tps = std::min(max_tps, std::max(1, (max_T + ATTN_PREF_SPLITS - 1) / ATTN_PREF_SPLITS));
  tps = std::max(tps, (max_T + ATTN_MAX_SPLITS) / ATTN_MAX_SPLITS);
  while (tps < max_tps && (flat(tps) * n_kv > target_wgs || flat(tps) > cap)) ++tps;
  if (tps > max_tps || flat(tps) > cap || splits_of(max_T, tps) > ATTN_MAX_SPLITS)
    return fail(err, DFLASH_E_INVALID,
                "context window too long for the attention splits (" + std::to_string(max_T) + " tiles of 32 keys, " +
                    std::to_string(n) + " sequences)");
  // Each sequence's splits are one run of split numbers; the runs go out
  // longest split first (the kernel divides a sequence's T + 2 units evenly
  // among its splits). Workgroups start in split order, so when a launch takes
  // more than one round of workgroups the last to start are the shortest
  // (longest processing time first); ties keep the sequence order.
  int32_t order[DFLASH_MAX_BATCH];
  for (int32_t i = 0; i < n; ++i) {
    order[i] = i;
    plan->nsplit[i] = (int32_t)splits_of(tiles[i], tps);
  }
  auto units = [&](int32_t i) { return (int64_t)tiles[i] + 2; };
  std::stable_sort(order, order + n, [&](int32_t x, int32_t y) {
    return units(x) * plan->nsplit[y] > units(y) * plan->nsplit[x];
  });
  int32_t f = 0;
  for (int32_t k = 0; k < n; ++k) {
    plan->split0[order[k]] = f;
    f += plan->nsplit[order[k]];
  }
  plan->tps = tps;
  plan->n_split = f;
  return DFLASH_OK;
}

int64_t attn_slots(const Geo &g, int32_t max_seq_len, int32_t max_tps) {
  const int64_t worst = attn_tiles_worst(g.W, max_seq_len);
  const int64_t per_seq = std::min<int64_t>(ATTN_MAX_SPLITS, (worst + max_tps) / max_tps);
  return std::max<int64_t>({(int64_t)ATTN_TARGET_WGS * 2, (int64_t)g.max_batch * g.n_kv * per_seq,
                            (int64_t)g.n_kv * ATTN_MAX_SPLITS});
}

int check_attn_capacity(const Geo &g, int32_t max_seq_len, int32_t max_tps, std::string *err) {
  std::vector<int32_t> tiles(g.max_batch, attn_tiles_worst(g.W, max_seq_len));
  AttnPlan plan;
  std::string e;
  if (attn_plan(g.max_batch, tiles.data(), g.n_kv, max_tps, attn_slots(g, max_seq_len, max_tps) / g.n_kv,
                ATTN_TARGET_WGS, &plan, &e) !=
      DFLASH_OK)
    return fail(err, DFLASH_E_INVALID,
                "config: max_batch sequences of min(ctx_window, max_seq_len) rows exceed the attention splits: " + e);
  return DFLASH_OK;
}

// Pair i rotates at w_i = theta^(-2i/d); the fractional pair index whose
// wavelength 2 pi / w fits `turns` times into the original context L is
// d ln(L / (2 pi turns)) / (2 ln theta). Pairs up to floor(index(beta_fast))
// keep w_i, pairs from ceil(index(beta_slow)) on take w_i / factor, and the
// weight of the kept frequency falls linearly in i in between (YaRN's
// "NTK-by-parts" interpolation over the pair index). Double precision,
// rounded once to float.
int yarn_inv_freq(int32_t head_dim, double theta, double factor, double beta_fast, double beta_slow,
                  int32_t original_max, float *out, std::string *err) {
  if (!out || head_dim < 2 || head_dim % 2 != 0 || !(theta > 1.0) || !(factor >= 1.0) || !(beta_slow > 0.0) ||
      !(beta_fast > beta_slow) || original_max < 1) {
    *err = "yarn_inv_freq: need an even head_dim >= 2, theta > 1, factor >= 1, beta_fast > beta_slow > 0, "
           "original_max >= 1 and an output";
    return DFLASH_E_INVALID;
  }
  const double d = head_dim;
  auto pair_index = [&](double turns) {
    return d * std::log((double)original_max / (turns * 2.0 * 3.14159265358979323846)) / (2.0 * std::log(theta));
  };
  const double lo = std::max(std::floor(pair_index(beta_fast)), 0.0);
  double hi = std::min(std::ceil(pair_index(beta_slow)), d - 1.0);
  if (hi == lo) hi += 0.001;
  for (int32_t i = 0; i < head_dim / 2; ++i) {
    const double w = std::pow(theta, -2.0 * i / d);
    const double ramp = std::min(std::max((i - lo) / (hi - lo), 0.0), 1.0);
    const double keep = 1.0 - ramp;
    out[i] = (float)((w / factor) * (1.0 - keep) + w * keep);
  }
  return DFLASH_OK;
}

}  // namespace dflash
