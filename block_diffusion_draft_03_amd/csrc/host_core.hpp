// host_core.hpp - HIP-free host logic of the DFlash draft head: geometry
// validation, the paged-KV block pool, and per-sequence row bookkeeping
// (append planning and after-verify trimming). Built into the HIP library and,
// on its own, into a CPU-only test library.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/dflash.h"

namespace dflash {

// Sizes derived from a validated dflash_config.
struct Geo {
  int L, h, I, n_q, n_kv, d, V, gamma, T, Ht, W;
  int q_dim, kv_dim, qkv_dim, fc_in, fkv_dim, words, rep, max_batch, m_max;
  uint32_t mask_id;
  bool kv_fp8, head_fp8, w_f32, shifted, fp8w, a8;
};

// Validate a config; on success fill *g. Returns a dflash_status.
int validate_config(const dflash_config &c, Geo *g, std::string *err);

// Physical KV blocks of one head. Allocation hands out the lowest free id.
class BlockPool {
 public:
  explicit BlockPool(int32_t n = 0);
  int32_t size() const { return (int32_t)used_.size(); }
  int32_t free_count() const { return free_; }
  bool is_free(int32_t id) const { return id >= 0 && id < size() && !used_[id]; }
  int32_t alloc();             // -1 when exhausted
  bool take(int32_t id);       // claim a specific free block
  void release(int32_t id);

 private:
  std::vector<uint8_t> used_;
  int32_t free_ = 0;
  int32_t hint_ = 0;  // every id below hint_ is in use
};

// Row bookkeeping of one sequence. Row i of the sequence sits at RoPE
// position i and in slot blocks[i / 16] * 16 + i % 16.
struct SeqRows {
  std::vector<int32_t> blocks;  // physical blocks in logical order
  int64_t cap_rows = 0;         // rows the sequence may ever hold
  bool grow = false;            // take blocks from the pool as rows arrive
  int32_t ctx_len = 0;          // rows held
  int32_t pending_base = 0;     // ctx_len at the last after_verify
};

// Create the row bookkeeping: explicit blocks, a known budget (all blocks
// taken now) or an unknown budget (grow up to max_seq_len).
int seq_init(SeqRows *s, BlockPool *pool, int64_t budget_tokens, const int32_t *block_ids, int32_t n_ids,
             int32_t max_seq_len, std::string *err);

// Make room for n more rows; new blocks (if any) are appended to s->blocks
// and *first_new_block is the logical index of the first one. Does not
// change ctx_len. Returns DFLASH_E_NO_BLOCKS without side effects on failure.
int seq_reserve(SeqRows *s, BlockPool *pool, int32_t n, int32_t *first_new_block, std::string *err);

// Keep the first a pending rows (0 <= a <= ctx_len - pending_base).
int seq_trim(SeqRows *s, int32_t a, std::string *err);

// Give every block back to the pool.
void seq_release(SeqRows *s, BlockPool *pool);

// Carry a sequence's KV to a later turn: move all its blocks and its row
// count (ctx_len) out; the blocks stay allocated in the pool. The state is
// left empty, taking blocks from the pool as rows arrive, with the same row
// capacity (as a fresh state of unknown budget).
void seq_take(SeqRows *s, std::vector<int32_t> *blocks, int32_t *rows);

// Install carried blocks (allocated in the pool, distinct) holding `rows`
// committed rows into a state that holds no rows; the state's own blocks go
// back to the pool first. Rows must fit the blocks and the state's row
// capacity (which grows to the installed blocks). Errors leave the state
// and the pool unchanged.
int seq_install(SeqRows *s, BlockPool *pool, const int32_t *blocks, int32_t n, int32_t rows, std::string *err);

// YaRN-corrected RoPE table (dflash_yarn_inv_freq): out[head_dim / 2].
int yarn_inv_freq(int32_t head_dim, double theta, double factor, double beta_fast, double beta_slow,
                  int32_t original_max, float *out, std::string *err);

}  // namespace dflash
