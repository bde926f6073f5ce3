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
// taken now) or an unknown budget (grow up to max_seq_len). A state never
// holds more than max_seq_len rows: a larger budget or block list is capped.
int seq_init(SeqRows *s, BlockPool *pool, int64_t budget_tokens, const int32_t *block_ids, int32_t n_ids,
             int32_t max_seq_len, std::string *err);

// Make room for n more rows; new blocks (if any) are appended to s->blocks
// and *first_new_block is the logical index of the first one. Does not
// change ctx_len. Returns DFLASH_E_NO_BLOCKS without side effects on failure.
int seq_reserve(SeqRows *s, BlockPool *pool, int32_t n, int32_t *first_new_block, std::string *err);

// Undo a seq_reserve: give back the blocks from logical index
// first_new_block on (those the reservation appended).
void seq_unreserve(SeqRows *s, BlockPool *pool, int32_t first_new_block);

// Reserve n_new[i] more rows for each of n states, all or nothing: when state
// i cannot take its rows (budget, pool, or more blocks than cap_blocks[i]
// when cap_blocks is given), the reservations of states 0..i-1 are undone and
// the pool is as before. A state may appear more than once (at most once with
// rows to append). Does not change ctx_len.
int reserve_rows(SeqRows *const *s, int32_t n, const int32_t *n_new, const int32_t *cap_blocks, BlockPool *pool,
                 std::string *err);

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
int seq_install(SeqRows *s, BlockPool *pool, const int32_t *blocks, int32_t n, int32_t rows, int32_t max_seq_len,
                std::string *err);

// ---- attention split plan of a propose launch ----
// The block's attention over a sequence's context runs in splits of up to
// tps ctx tiles of 32 keys (from the window start aligned down to a KV
// block); the sequence's last split also takes the block's own keys, which
// count as one more tile. A launch aims for at most ATTN_TARGET_WGS
// workgroups over all sequences and kv heads: two per compute unit, one
// round in which every workgroup is resident (measured on batches of 32 and
// 64 sequences of 256 or 512 to 4096 ctx rows with bf16 and E4M3 caches:
// targets of 384, 640 and 768 were slower or, with an E4M3 cache, 0.3%
// slower). It prefers at most
// ATTN_PREF_SPLITS splits per sequence, and cannot exceed ATTN_MAX_SPLITS
// splits per sequence (one wave merges a row's splits) or ATTN_MAX_FLAT
// splits in all (the split-to-sequence map travels in the launch arguments).
constexpr int ATTN_MAX_FLAT = 1024;
constexpr int ATTN_TARGET_WGS = 512;
constexpr int ATTN_MAX_SPLITS = 64;
constexpr int ATTN_PREF_SPLITS = 16;

// Ctx tiles of 32 keys a sequence of ctx_len rows attends to: rows
// [max(0, c - W), c), from that start aligned down to 16; W = 0 keeps none.
int32_t attn_tiles(int32_t ctx_len, int32_t window);

// The most tiles any state of a head can need (0 <= ctx_len <= max_seq_len).
int32_t attn_tiles_worst(int32_t window, int32_t max_seq_len);

struct AttnPlan {
  int32_t tps = 0, n_split = 0;
  int32_t split0[DFLASH_MAX_BATCH], nsplit[DFLASH_MAX_BATCH];
};

// Plan n sequences (tiles[i] ctx tiles each) over n_kv kv heads, with at most
// max_tps tiles per split, slot_cap partial slots per kv head and about
// target_wgs workgroups. Sequence i owns splits [split0[i], split0[i] +
// nsplit[i]); the runs cover [0, n_split), sequences with longer splits
// first. Fails with DFLASH_E_INVALID, touching nothing, when no split size
// fits.
int attn_plan(int32_t n, const int32_t *tiles, int32_t n_kv, int32_t max_tps, int64_t slot_cap, int32_t target_wgs,
              AttnPlan *plan, std::string *err);

// Partial slots (per kv head) a head keeps for its attention splits.
int64_t attn_slots(const Geo &g, int32_t max_seq_len, int32_t max_tps);

// Build-time check that the widest batch of the longest contexts has a split
// plan: then every propose the head accepts has one (the plan is monotone in
// every sequence's tiles and in the batch width).
int check_attn_capacity(const Geo &g, int32_t max_seq_len, int32_t max_tps, std::string *err);

// YaRN-corrected RoPE table (dflash_yarn_inv_freq): out[head_dim / 2].
int yarn_inv_freq(int32_t head_dim, double theta, double factor, double beta_fast, double beta_slow,
                  int32_t original_max, float *out, std::string *err);

}  // namespace dflash
