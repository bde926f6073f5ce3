/*
 * dflash.h - C ABI of the MI355X (gfx950) block-diffusion (DFlash) draft head.
 *
 * The library implements the draft head's propose pass: a block of gamma rows
 * (the last verified token, then mask tokens) runs through the drafter layers,
 * attending to a window of context K/V that earlier calls derived from the
 * target model's captured hidden states, and ends in the shared-vocabulary LM
 * head with a per-row argmax. Every step runs in HIP kernels on the device;
 * the host side only validates arguments and keeps per-sequence bookkeeping.
 *
 * Sources, cited by page title and section:
 *   [Head/atlas]    "Struct BlockDiffusionDraftHead" (spark_model::layers::dflash_head)
 *   [Head/metrale]  "Struct BlockDiffusionDraftHead" (metrale_model_arch::dflash_head)
 *   [DraftProposer] "Trait DraftProposer" (spark_model::speculative)
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory. Each argument says which.
 *   - `stream` is a hipStream_t cast to uint64_t (0 = the null stream). All
 *     device work of a call is enqueued on it. The calls that wait on the
 *     host: dflash_build (its stream), dflash_destroy, dflash_state_create,
 *     dflash_state_free, dflash_take_kv and dflash_install_kv (the device),
 *     dflash_timing_read and dflash_timing_enable(0) (the recorded events),
 *     and a dflash_precompute_ctx_kv of more than 64 rows when one of its two
 *     pinned staging buffers (row positions and block tables of a 1024-row
 *     pass) is still being copied by an earlier pass of it or of an earlier
 *     such call: it waits for that copy. dflash_propose and
 *     dflash_propose_batch never wait.
 *   - A negative return value is a dflash_status error; dflash_last_error()
 *     then describes it. Every argument check runs on the host before any
 *     kernel is enqueued, so a failed call leaves the device untouched and
 *     the head's bookkeeping as it was (a HIP failure while enqueueing,
 *     DFLASH_E_HIP, is the exception).
 *   - A head's scratch buffers are shared by all calls on that head: calls on
 *     one head must be ordered on the device (use one stream, or synchronise
 *     between streams). Host-side calls on one head are serialised by an
 *     internal mutex. States are owned by the head that created them.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 1
#define DFLASH_MAX_BATCH 64     /* widest dflash_propose_batch */
#define DFLASH_KV_BLOCK 16      /* rows per paged KV block */
#define DFLASH_NO_TOKEN 0xFFFFFFFFu /* id of a row whose every token is masked */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,   /* an argument value or state is invalid */
  DFLASH_E_SHAPE = -2,     /* geometry mismatch (e.g. fc width != num_target_layers * target_hidden) */
  DFLASH_E_NOMEM = -3,     /* a device or host allocation failed */
  DFLASH_E_NO_BLOCKS = -4, /* the KV pool or the state's token budget is exhausted */
  DFLASH_E_DECLINED = -5,  /* batch width outside 1..max_batch: fall back to per-sequence propose */
  DFLASH_E_HIP = -6        /* a HIP runtime call failed */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1, DFLASH_FP8_E4M3 = 2 } dflash_dtype;

typedef struct dflash_head dflash_head;   /* opaque */
typedef struct dflash_state dflash_state; /* opaque, one per sequence */

/* Geometry and build options ([Head/atlas] struct fields num_layers ...
 * rms_norm_eps, ctx_window; all validated by dflash_build). */
typedef struct {
  int32_t num_layers;        /* drafter layers L (>= 1) */
  int32_t hidden;            /* drafter hidden size h, multiple of 128 or 64 (tiny) */
  int32_t intermediate;      /* SwiGLU width I, multiple of 64 */
  int32_t num_q_heads;       /* query heads */
  int32_t num_kv_heads;      /* kv heads (divides num_q_heads) */
  int32_t head_dim;          /* 16, 32, 64 or 128; RoPE covers the whole head */
  int32_t vocab;             /* shared vocabulary V */
  int32_t gamma;             /* block rows per sequence (2..64) */
  uint32_t mask_token_id;    /* id of rows 1..gamma-1 of the block (< vocab) */
  int32_t num_target_layers; /* T: target layers in the captured hidden stack */
  int32_t target_hidden;     /* Ht: target hidden size; fc input width = T * Ht */
  int32_t ctx_window;        /* most ctx rows a block attends to; 0 disables ctx */
  float rope_theta;          /* inv_freq[i] = theta^(-2i/head_dim) unless a table is given */
  float rms_eps;             /* RMSNorm epsilon */
  int32_t kv_block_size;     /* must be DFLASH_KV_BLOCK */
  int32_t kv_pool_blocks;    /* physical blocks in the head's paged KV pool */
  int32_t max_batch;         /* widest batch (1..DFLASH_MAX_BATCH) */
  int32_t max_seq_len;       /* most ctx rows any state holds (larger budgets and block lists are capped) */
  dflash_dtype weight_dtype;  /* F32 or BF16: dtype of the drafter tensors given at build */
  dflash_dtype lm_head_dtype; /* BF16, or FP8_E4M3 (a mirror is built unless one is given) */
  dflash_dtype kv_dtype;      /* BF16, or FP8_E4M3 with per-(layer, K|V, kv head) scales */
  int32_t shifted_rows;       /* draft-row convention ([Head/atlas] field shifted_rows): 0, block row j is the
                                 draft for position + j; 1, block row j's output is the token at position
                                 + j + 1, so ids and row_prob come out rotated right by one (entry j + 1
                                 holds row j, entry 0 the last row) and index j is position + j's draft
                                 either way; the chain confidence is the min over entries 1..num_drafts */
  int32_t fp8_weights;        /* 0: the drafter's matrices (fc, layers, fused ctx K/V) are streamed in bf16;
                                 1: as E4M3 codes with one f32 scale per output row, built from their bf16
                                 values (scale = row amax / 448, code = enc(w / scale), as the LM-head
                                 mirror); weight-only, the products still run in bf16 ([Head/metrale] field
                                 lm_head_shared_fp8: the FP8 LM head of FP8 drafter weights) */
  int32_t lm_act_fp8;         /* 0: the final-normed rows enter the LM head in bf16; 1 (needs an FP8_E4M3
                                 head, vocab a multiple of 256, hidden a multiple of 128): W8A8 head, each
                                 row is quantised to E4M3 with one f32 scale (scale = row amax / 448, code
                                 = enc(z / scale), as the LM-head mirror) and the head's products run on
                                 the E4M3 matrix cores, logit = s_v * scale * sum_k q_vk c_k; every
                                 propose then takes the tiled path ([Head/atlas] field lm_head_shared_fp8
                                 gives the FP8 head; its activation format is this library's reading) */
} dflash_config;

/* One drafter layer's tensors: device pointers in weight_dtype, matrices in
 * PyTorch Linear layout [out, in], row-major. */
typedef struct {
  const void *in_norm;   /* [h] input RMSNorm gain */
  const void *q;         /* [n_q * d, h] */
  const void *k;         /* [n_kv * d, h] */
  const void *v;         /* [n_kv * d, h] */
  const void *o;         /* [h, n_q * d] */
  const void *post_norm; /* [h] post-attention RMSNorm gain */
  const void *gate;      /* [I, h] */
  const void *up;        /* [I, h] */
  const void *down;      /* [h, I] */
} dflash_layer_weights;

/* Weights given to dflash_build. The drafter checkpoint's tensors (fc, norms,
 * layers) and the LM head (bf16, or the FP8 codes and scales) are copied into
 * the head's tile-major streaming layout during the call and may be freed
 * afterwards. The target's embedding is borrowed when it is bf16 and must
 * outlive the head ([Head/atlas], struct description: the drafter uses the
 * target's embed_tokens and lm_head). */
typedef struct {
  const void *fc;             /* device [h, T*Ht], weight_dtype ([Head/atlas] field fc) */
  const void *hidden_norm;    /* device [h] ([Head/atlas] field hidden_norm) */
  const void *norm;           /* device [h] final norm ([Head/atlas] field norm) */
  const void *embed_tokens;   /* device [V, h], weight_dtype (bf16: borrowed) */
  const void *lm_head;        /* device [V, h], weight_dtype (bf16: borrowed) */
  const void *lm_head_fp8;    /* optional device [V, h] E4M3 codes (borrowed); NULL = build a mirror */
  const float *lm_head_scale; /* device [V] f32 row scales of lm_head_fp8 (borrowed) */
  const float *kv_scale;      /* host [L][2][n_kv] f32 (K then V) when kv_dtype is FP8, else NULL */
  const float *inv_freq;      /* optional host [head_dim/2] f32 RoPE table; NULL = plain theta table */
  const dflash_layer_weights *layers; /* host array [num_layers] */
} dflash_weights;

/* Build a head ([Head/atlas] impl, from_weights and validate_against_target).
 * Validates the geometry (a mismatched fc width is DFLASH_E_SHAPE), stitches
 * the fused ctx-K/V weight [L * 2 * n_kv * d, h] with rows [K0; V0; K1; V1;
 * ...] ([Head/atlas] field fused_kv_weight), converts and repacks the drafter
 * tensors to bf16, builds the FP8 LM-head mirror when asked ([Head/atlas]
 * field lm_head_shared_fp8: E4M3 codes, per-row scale amax / 448), and
 * allocates the paged KV pool and the scratch. Synchronises `stream`.
 * DFLASH_E_INVALID, before anything is allocated, when max_batch sequences of
 * min(ctx_window, max_seq_len) ctx rows would not fit the attention's splits
 * (at most 64 splits of 64 tiles of 32 keys per sequence and 1024 splits per
 * launch); a head that builds accepts every batch up to max_batch.
 * On success *out owns all of it until dflash_destroy. */
int dflash_build(const dflash_config *cfg, const dflash_weights *w, uint64_t stream, dflash_head **out);

/* Free the head and everything it owns. States of the head must have been
 * freed first (remaining ones are freed here). NULL is a no-op. */
void dflash_destroy(dflash_head *head);

/* Block size gamma ([DraftProposer] block_gamma); callers draft gamma - 1. */
int dflash_block_gamma(const dflash_head *head);

/* Widest batch one dflash_propose_batch call can carry ([DraftProposer]
 * propose_batch_max): the build's max_batch. */
int dflash_propose_batch_max(const dflash_head *head);

/* Per-sequence state ([DraftProposer] alloc_state / alloc_state_for).
 * budget_tokens: most ctx rows the sequence will hold; INT64_MAX = unknown
 * (the build's max_seq_len applies and blocks are taken from the pool as
 * rows arrive). With a known budget every block is taken now. No state
 * holds more than max_seq_len rows: a larger budget is capped to it.
 * block_ids (host, optional): explicit physical pool blocks for the
 * sequence, in logical order; n_ids of them bound its capacity (and
 * max_seq_len). They must be free. Returns DFLASH_E_NO_BLOCKS when the pool
 * cannot supply the blocks. */
int dflash_state_create(dflash_head *head, int64_t budget_tokens, const int32_t *block_ids, int32_t n_ids,
                        dflash_state **out);

/* Release a state's KV blocks and device memory ([DraftProposer] free_state).
 * Synchronises the device before releasing. */
int dflash_state_free(dflash_head *head, dflash_state *st);

/* Ctx rows the state holds (appended and not trimmed); negative on error. */
int dflash_state_ctx_len(const dflash_state *st);

/* Append ctx rows to n states ([Head/atlas] field fused_kv_weight: the
 * precompute module). For each state i, n_new[i] rows of the captured hidden
 * stack (rows sum(n_new[0..i)) .. of `stack`) are projected by fc, normed by
 * hidden_norm, and turned into every layer's K and V by one fused GEMM; K is
 * rotated at positions ctx_len .. ctx_len + n_new[i] - 1 and both are written
 * into the state's paged blocks. The rows become the state's pending rows.
 *   states: host array [n]; n_new: host array [n], each >= 0;
 *   stack: device bf16 [sum(n_new), T * Ht], row-major, shallow-to-deep
 *          concatenation of the target layers ([DraftProposer] propose,
 *          argument target_hidden_stack).
 * A call of up to 64 rows in all streams the weights once per 64 rows; a
 * larger call (prompt-scale prefill) runs in passes of up to 1024 rows through
 * MFMA-tiled GEMMs. A row's cached K/V is bit-identical for any call of the
 * same kind; the two kinds agree to rounding.
 * DFLASH_E_NO_BLOCKS if a state would exceed its budget or the pool; the
 * blocks are reserved for all states or for none (a failure gives back what
 * the states before the failing one took). */
int dflash_precompute_ctx_kv(dflash_head *head, dflash_state *const *states, int32_t n, const int32_t *n_new,
                             const void *stack, uint64_t stream);

/* One propose ([DraftProposer] propose; [Head/atlas] last_confidence).
 * The block [last_token, mask_token_id x (gamma - 1)] at RoPE positions
 * position .. position + gamma - 1 attends to the state's ctx rows
 * [max(0, ctx_len - ctx_window), ctx_len) and to itself; after the final norm
 * and LM head each row takes its argmax (ties to the lowest id).
 * Numerics: the dense products take bf16 operands with f32 accumulation;
 * attention runs in fp16 (Q, K, V and the softmax weights, f32 accumulation),
 * so the block rows' Q/K/V and the cached K/V must lie within fp16's range
 * (|x| < 65504; larger values become infinite and poison the row).
 *   last_token < vocab; 0 <= position < 2^31 - gamma; 1 <= num_drafts <= gamma - 1.
 *   bitmask: optional device int32 [ceil(V/32)]; bit v&31 of word v>>5 set
 *            means token v is allowed ([DraftProposer] propose, grammar_bitmask).
 * Outputs (device, caller-owned, valid after the stream completes):
 *   ids      uint32 [gamma]: argmax of every block row (drafts are rows
 *            1..num_drafts); DFLASH_NO_TOKEN when the mask allows nothing;
 *   conf     f32 [1]: min over rows 1..num_drafts of the top-1 softmax prob;
 *   row_prob f32 [gamma] or NULL: top-1 softmax prob of every row;
 *   logits   f32 [gamma, V] or NULL: unmasked logits (inspection only). */
int dflash_propose(dflash_head *head, dflash_state *st, uint32_t last_token, int64_t position, int32_t num_drafts,
                   const int32_t *bitmask, uint32_t *ids, float *conf, float *row_prob, float *logits,
                   uint64_t stream);

/* Batched propose: ONE forward over n * gamma rows ([Head/atlas] and
 * [DraftProposer] propose_batch). Sequence i uses states[i], last_tokens[i]
 * and positions[i] (host arrays [n]); the result for each sequence is that of
 * dflash_propose. 1 <= n <= max_batch, else DFLASH_E_DECLINED (the caller
 * falls back to per-sequence calls, never a different answer).
 *   bitmasks: optional device int32 [n, ceil(V/32)], one mask per sequence.
 *   ids [n, gamma], conf [n], row_prob [n, gamma] or NULL,
 *   logits [n, gamma, V] or NULL: device, caller-owned. */
int dflash_propose_batch(dflash_head *head, dflash_state *const *states, int32_t n, const uint32_t *last_tokens,
                         const int64_t *positions, int32_t num_drafts, const int32_t *bitmasks, uint32_t *ids,
                         float *conf, float *row_prob, float *logits, uint64_t stream);

/* dflash_propose without the head's scratch, for callers that cannot
 * allocate device memory or must not touch the head's buffers: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * arguments, checks and results are those of dflash_propose (bit for bit the
 * same outputs); the call's scratch (activations, split partials, counters,
 * the block's V^T copy) lives in a static device array of the library, 16 MiB
 * per device, held from library load until the process ends. The call clears
 * what must start at zero with a fill kernel on `stream` and allocates
 * nothing (no hipMalloc, no events). Every call on one device shares that
 * array and it keeps the last call's contents: calls that overlap on one
 * device (other streams, other heads, other threads) race and must be
 * ordered by the caller. DFLASH_E_INVALID, before anything is enqueued, when
 * the propose needs more scratch than the array holds (the full DFlash
 * geometry needs at most ~10 MiB: 16 block rows, 64 attention splits per kv
 * head), or when the head's device could not resolve the array at build. */
int dflash_propose_noalloc(dflash_head *head, dflash_state *st, uint32_t last_token, int64_t position,
                           int32_t num_drafts, const int32_t *bitmask, uint32_t *ids, float *conf, float *row_prob,
                           float *logits, uint64_t stream);

/* Trim after verification ([DraftProposer] after_verify): keep the first
 * num_accepted rows appended since the previous dflash_after_verify (or since
 * the state was created) and drop the rest; the kept rows become committed.
 * 0 <= num_accepted <= pending rows, else DFLASH_E_INVALID. Host-only: no
 * device work; the dropped rows' slots are overwritten by later appends. */
int dflash_after_verify(dflash_head *head, dflash_state *st, int32_t num_accepted);

/* Carry a sequence's drafter KV across turns ([DraftProposer]
 * take_drafter_kv, install_drafter_kv, free_drafter_kv). Host-side
 * bookkeeping: no kernel runs and the cached values are not touched (each
 * call first waits for the device, so no launch still reads a block table).
 *
 * dflash_take_kv moves all of the state's physical blocks into blocks_out
 * (caller-owned host array of `cap` entries) and its row count into *rows;
 * the blocks stay allocated in the head's pool and belong to the caller. The
 * state is left empty, as a fresh state of unknown budget with the same row
 * capacity. *n_blocks = 0 (and DFLASH_OK) when there is nothing to carry;
 * DFLASH_E_INVALID, with *n_blocks set to the count needed and nothing
 * moved, when cap is too small. *last_pair_key returns the key given at
 * install (-1 when none).
 *
 * dflash_install_kv gives carried blocks (n_blocks >= 1 distinct allocated
 * blocks that no live state holds, at most the state's block-table capacity)
 * holding `rows` committed rows (0 <= rows <= min(16 n_blocks, max_seq_len)) to a state that
 * holds no rows; the state's own blocks return to the pool. A later propose
 * sees exactly the carried rows. DFLASH_E_INVALID otherwise, nothing changed.
 *
 * dflash_free_kv returns carried blocks that no live state holds to the
 * pool (a carried entry being replaced or dropped). */
int dflash_take_kv(dflash_head *head, dflash_state *st, int32_t *blocks_out, int32_t cap, int32_t *n_blocks,
                   int32_t *rows, int64_t *last_pair_key);
int dflash_install_kv(dflash_head *head, dflash_state *st, const int32_t *blocks, int32_t n_blocks, int32_t rows,
                      int64_t last_pair_key);
int dflash_free_kv(dflash_head *head, const int32_t *blocks, int32_t n_blocks);

/* Copy cached ctx rows [row0, row0 + n_rows) of one layer out of the paged
 * cache, in the cache's storage dtype (bf16: 2 bytes, FP8: 1 byte per value),
 * as K [n_rows, n_kv, d] and V [n_rows, n_kv, d] into device buffers k_out and
 * v_out (either may be NULL). Inspection of what precompute wrote. */
int dflash_state_read_kv(dflash_head *head, const dflash_state *st, int32_t layer, int32_t row0, int32_t n_rows,
                         void *k_out, void *v_out, uint64_t stream);

/* The LM head the propose reads when lm_head_dtype is FP8: copies the E4M3
 * codes [V, h] and row scales [V] into device buffers (either may be NULL).
 * DFLASH_E_INVALID on a bf16 head. */
int dflash_read_lm_head_fp8(dflash_head *head, void *codes_out, float *scale_out, uint64_t stream);

/* YaRN-corrected RoPE table ([Head/atlas] field yarn_inv_freq: a
 * precomputed f32 [head_dim/2] table from the drafter's rope_scaling, e.g.
 * factor 64, beta_fast 32, beta_slow 1, original_max_position_embeddings
 * 4096; [Head/metrale] field yarn_inv_freq). Host-only: writes head_dim / 2
 * floats to caller-owned host memory `out`, to be passed as
 * dflash_weights.inv_freq. Pair i keeps theta^(-2i/head_dim) when its
 * wavelength fits more than beta_fast times into original_max_positions, is
 * divided by `factor` when it fits fewer than beta_slow times, and blends
 * linearly in i in between (YaRN's NTK-by-parts interpolation; no magnitude
 * scaling). DFLASH_E_INVALID unless head_dim is even and >= 2, theta > 1,
 * factor >= 1, beta_fast > beta_slow > 0, original_max_positions >= 1 and
 * out is set. */
int dflash_yarn_inv_freq(int32_t head_dim, float rope_theta, float factor, float beta_fast, float beta_slow,
                         int32_t original_max_positions, float *out);

/* Kernel timing for benchmarks. While enabled, each propose and precompute
 * call records HIP events on its own stream around: DFLASH_PHASE_LM_HEAD,
 * the LM-head stage-1 launches (the dominant weight stream);
 * DFLASH_PHASE_PROPOSE, all launches of a propose; DFLASH_PHASE_PRECOMPUTE,
 * all launches of a precompute. dflash_timing_read waits for the recorded
 * events, returns the summed elapsed milliseconds and the number of timed
 * intervals of one phase, and clears that phase. Disabling drops pending
 * records. Recording adds one event pair per interval to the stream. */
#define DFLASH_PHASE_LM_HEAD 0
#define DFLASH_PHASE_PROPOSE 1
#define DFLASH_PHASE_PRECOMPUTE 2
int dflash_timing_enable(dflash_head *head, int enable);
int dflash_timing_read(dflash_head *head, int32_t phase, double *total_ms, int64_t *intervals);

/* Message of the calling thread's last error ("" if none). */
const char *dflash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
