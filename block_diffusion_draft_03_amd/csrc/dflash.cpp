// dflash.cpp - the C ABI of include/dflash.h: argument validation, the head's
// device memory (repacked weights, paged KV pool, scratch), per-sequence
// state, and the ordered launches of the propose and precompute passes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/dflash.h"
#include "host_core.hpp"
#include "kernels.hpp"

using namespace dflash;

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string &m) {
  g_err = m;
  return code;
}

constexpr uint64_t HEAD_MAGIC = 0x44464c4153484844ull;   // "DFLASHHD"
constexpr uint64_t STATE_MAGIC = 0x44464c4153485354ull;  // "DFLASHST"
constexpr uint64_t DEAD_MAGIC = 0xdeadull;
// bf16 proposes of up to this many rows stream the weights through the
// few-row kernels; from one more row on the tiled kernels are faster
// (measured at 48 and 64 rows: 16% less time per propose; at 32 rows the
// few-row path is 16% faster)
constexpr int PROPOSE_FEW_ROWS = 32;
constexpr int PREFILL_ROWS = 1024;    // rows of one tiled precompute pass

#define HIP_TRY(expr)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return set_err(DFLASH_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

hipStream_t to_stream(uint64_t s) { return (hipStream_t)(uintptr_t)s; }

}  // namespace

struct dflash_state {
  uint64_t magic = STATE_MAGIC;
  dflash_head *owner = nullptr;
  SeqRows rows;
  int32_t *d_bt = nullptr;   // device block table
  int32_t *h_bt = nullptr;   // pinned host copy (entries written once, then uploaded)
  int32_t cap_blocks = 0;
  int32_t uploaded = 0;      // leading entries of d_bt already uploaded
  int64_t pair_key = -1;     // opaque key carried with installed blocks (-1: none)
};

// Device scratch of one propose: written and read within the call (the
// split counters and the block V^T copy's padding must be zero when the call
// starts; the kernels leave the counters at zero). The head owns one sized for
// max_batch sequences; dflash_propose_noalloc carves one out of a static array.
struct Scratch {
  float *hid = nullptr;                        // residual stream [M][h]
  uint16_t *act = nullptr;                     // next GEMM's bf16 operand [M][h]
  uint8_t *act8 = nullptr;                     // W8A8 head: E4M3 codes of the final-normed rows [M][h]
  float *act8_scale = nullptr;                 // and their row scales [M]
  uint16_t *qkv = nullptr, *attn = nullptr, *mlp = nullptr;
  float2 *cs = nullptr;                        // RoPE (cos, sin) per row [M][d / 2]
  uint16_t *o_part = nullptr;                  // attention split outputs (fp16) [n_kv][splits][R][d]
  float *ml_part = nullptr;                    // and their (max, sum)
  int attn_slots = 0;                          // splits over all kv heads o_part holds
  float *lm_mx = nullptr, *lm_se = nullptr;    // LM-head partials [P][M]
  uint32_t *lm_idx = nullptr;
  float *lm_p1 = nullptr;                      // [M]
  int *fin_counters = nullptr;                 // [sequences], zero between launches
  float *ss = nullptr;                         // per-unit row sums of squares [h / 16][M] (few-row path)
  int *tile_ctr = nullptr;                     // split counters of the residual GEMMs [h / 16], zero between launches
  uint16_t *vtb = nullptr;                     // V^T of the block rows [seqs][n_kv][d][gp], zero padded
  float *part = nullptr;                       // split-K partial sums [splits][rows][h]
};

// A repacked drafter matrix: tile-major bf16 (s null) or tile-major E4M3
// codes with one f32 scale per output row.
struct Wt {
  const void *w;
  const float *s;
};

struct dflash_head {
  uint64_t magic = HEAD_MAGIC;
  dflash_config cfg{};
  Geo g{};
  std::mutex mu;
  BlockPool pool;
  std::vector<dflash_state *> states;
  std::vector<void *> dev_allocs;

  // repacked drafter weights (bf16 unless noted), layer-major
  uint16_t *w_qkv = nullptr, *w_o = nullptr, *w_gu = nullptr, *w_down = nullptr, *w_fc = nullptr, *w_fkv = nullptr;
  size_t sz_qkv = 0, sz_o = 0, sz_gu = 0, sz_down = 0;  // tiled elements per layer
  // FP8 drafter weights: the same matrices as tiled E4M3 codes (one byte per
  // element, same element offsets) and f32 scales per output row, layer-major
  uint8_t *w8_qkv = nullptr, *w8_o = nullptr, *w8_gu = nullptr, *w8_down = nullptr, *w8_fc = nullptr,
          *w8_fkv = nullptr;
  float *s_qkv = nullptr, *s_o = nullptr, *s_gu = nullptr, *s_down = nullptr, *s_fc = nullptr, *s_fkv = nullptr;

  Wt pick(const uint16_t *b, const uint8_t *q, const float *s, size_t elem_off, size_t row_off) const {
    return g.fp8w ? Wt{q + elem_off, s + row_off} : Wt{b + elem_off, nullptr};
  }
  Wt wqkv(int l) const { return pick(w_qkv, w8_qkv, s_qkv, (size_t)l * sz_qkv, (size_t)l * g.qkv_dim); }
  Wt wo(int l) const { return pick(w_o, w8_o, s_o, (size_t)l * sz_o, (size_t)l * g.h); }
  Wt wgu(int l) const { return pick(w_gu, w8_gu, s_gu, (size_t)l * sz_gu, (size_t)l * 2 * g.I); }
  Wt wdown(int l) const { return pick(w_down, w8_down, s_down, (size_t)l * sz_down, (size_t)l * g.h); }
  Wt wfc() const { return pick(w_fc, w8_fc, s_fc, 0, 0); }
  Wt wfkv() const { return pick(w_fkv, w8_fkv, s_fkv, 0, 0); }
  float *g_in = nullptr, *g_post = nullptr, *g_hidden = nullptr, *g_final = nullptr;
  const uint16_t *embed = nullptr, *lm = nullptr;
  const uint8_t *lm8 = nullptr;
  const float *lm8_scale = nullptr;
  double *inv_freq = nullptr;
  float *kv_scale = nullptr;
  void *kv_pool = nullptr;
  size_t kv_elem = 2;

  // scratch of the propose (max_batch sequences) and of the precompute
  Scratch sc;
  int dev = 0;  // device the head lives on
  int lm_P = 0;
  int gp = 0;   // block rows padded to 32 (the vtb copy's row stride)
  float *pre_u = nullptr;
  uint16_t *pre_c = nullptr;
  // tiled precompute of many rows: row positions and block tables, double
  // buffered (pinned staging + device copy; ev[i] marks staging i free)
  bool tiled_prefill = false;
  int32_t *h_pos = nullptr, *d_pos = nullptr;
  const int32_t **h_bts = nullptr, **d_bts = nullptr;
  hipEvent_t pre_ev[2] = {nullptr, nullptr};
  bool pre_ev_used[2] = {false, false};

  // benchmark timing: recorded (start, stop) event pairs per phase
  bool timing = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> timed[3];
  std::vector<hipEvent_t> event_pool;

  hipEvent_t take_event() {
    if (!event_pool.empty()) {
      hipEvent_t e = event_pool.back();
      event_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }

  // Open an interval of `phase` on stream s; returns the stop event to
  // record at the end, or nullptr when timing is off.
  hipEvent_t interval_begin(int phase, hipStream_t s) {
    if (!timing) return nullptr;
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) return nullptr;
    if (hipEventRecord(a, s) != hipSuccess) return nullptr;
    timed[phase].push_back({a, b});
    return b;
  }

  template <class T>
  int alloc(T **p, size_t count) {
    void *q = nullptr;
    const size_t bytes = std::max<size_t>(count * sizeof(T), 256);
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess) return set_err(DFLASH_E_NOMEM, std::string("hipMalloc of ") + std::to_string(bytes) + " bytes: " + hipGetErrorString(e));
    dev_allocs.push_back(q);
    *p = (T *)q;
    return DFLASH_OK;
  }
};

namespace {

bool head_ok(const dflash_head *h) { return h && h->magic == HEAD_MAGIC; }
bool state_ok(const dflash_head *h, const dflash_state *s) { return s && s->magic == STATE_MAGIC && s->owner == h; }

void free_head_memory(dflash_head *h) {
  for (void *p : h->dev_allocs) (void)hipFree(p);
  h->dev_allocs.clear();
  if (h->h_pos) (void)hipHostFree(h->h_pos);
  if (h->h_bts) (void)hipHostFree((void *)h->h_bts);
  h->h_pos = nullptr;
  h->h_bts = nullptr;
  for (hipEvent_t &e : h->pre_ev)
    if (e) {
      (void)hipEventDestroy(e);
      e = nullptr;
    }
}

void free_state_memory(dflash_state *s) {
  if (s->d_bt) (void)hipFree(s->d_bt);
  if (s->h_bt) (void)hipHostFree(s->h_bt);
  s->d_bt = nullptr;
  s->h_bt = nullptr;
}

#define TRY(expr)                  \
  do {                             \
    int r_ = (expr);               \
    if (r_ != DFLASH_OK) return r_; \
  } while (0)

// Repack the drafter tensors and allocate everything; called under no lock
// on a fresh head.
// FP8 drafter weights: every drafter matrix in the row order of its bf16
// tiles, quantised per output row (scale = row amax / 448 of the bf16 values,
// code = enc(w / scale), the LM-head mirror's recipe) and tiled as E4M3. The
// fused ctx K/V rows get the same codes and scales as the layers' K/V rows.
int build_fp8_weights(dflash_head *H, const dflash_weights *w, hipStream_t st) {
  const Geo &g = H->g;
  const bool f32 = g.w_f32;
  const int h = g.h, d = g.d;
  TRY(H->alloc(&H->w8_qkv, (size_t)g.L * H->sz_qkv));
  TRY(H->alloc(&H->w8_o, (size_t)g.L * H->sz_o));
  TRY(H->alloc(&H->w8_gu, (size_t)g.L * H->sz_gu));
  TRY(H->alloc(&H->w8_down, (size_t)g.L * H->sz_down));
  TRY(H->alloc(&H->w8_fc, tiled_elems(h, g.fc_in)));
  TRY(H->alloc(&H->w8_fkv, tiled_elems(g.fkv_dim, h)));
  TRY(H->alloc(&H->s_qkv, (size_t)g.L * g.qkv_dim));
  TRY(H->alloc(&H->s_o, (size_t)g.L * h));
  TRY(H->alloc(&H->s_gu, (size_t)g.L * 2 * g.I));
  TRY(H->alloc(&H->s_down, (size_t)g.L * h));
  TRY(H->alloc(&H->s_fc, (size_t)h));
  TRY(H->alloc(&H->s_fkv, (size_t)g.fkv_dim));
  // row-major bf16 staging of one matrix and its row-major codes (freed below)
  const size_t most = std::max({(size_t)g.qkv_dim * h, (size_t)h * g.q_dim, (size_t)2 * g.I * h, (size_t)h * g.I,
                                (size_t)h * g.fc_in, (size_t)g.fkv_dim * h});
  uint16_t *tmp = nullptr;
  uint8_t *codes = nullptr;
  HIP_TRY(hipMalloc(&tmp, most * sizeof(uint16_t)));
  hipError_t e = hipMalloc(&codes, most);
  if (e != hipSuccess) {
    (void)hipFree(tmp);
    HIP_TRY(e);
  }
  int rc = DFLASH_OK;
  auto run = [&](hipError_t x) {
    if (rc == DFLASH_OK && x != hipSuccess) rc = set_err(DFLASH_E_HIP, std::string("FP8 weight build: ") + hipGetErrorString(x));
  };
  auto pack = [&](uint8_t *dst, float *scale, int rows, int cols) {
    run(launch_fp8_mirror(tmp, rows, cols, codes, scale, st));
    run(launch_tile_fp8(dst, codes, rows, cols, st));
  };
  for (int l = 0; l < g.L && rc == DFLASH_OK; ++l) {
    const dflash_layer_weights &lw = w->layers[l];
    run(launch_convert_rows(tmp, lw.q, nullptr, g.q_dim, h, f32, ROWS_ROPE_PAIRS, d, st));
    run(launch_convert_rows(tmp + (size_t)g.q_dim * h, lw.k, nullptr, g.kv_dim, h, f32, ROWS_ROPE_PAIRS, d, st));
    run(launch_convert_rows(tmp + (size_t)(g.q_dim + g.kv_dim) * h, lw.v, nullptr, g.kv_dim, h, f32, ROWS_SAME, d, st));
    pack(H->w8_qkv + (size_t)l * H->sz_qkv, H->s_qkv + (size_t)l * g.qkv_dim, g.qkv_dim, h);
    run(launch_convert_rows(tmp, lw.o, nullptr, h, g.q_dim, f32, ROWS_SAME, d, st));
    pack(H->w8_o + (size_t)l * H->sz_o, H->s_o + (size_t)l * h, h, g.q_dim);
    run(launch_convert_rows(tmp, lw.gate, lw.up, 2 * g.I, h, f32, ROWS_GATE_UP, d, st));
    pack(H->w8_gu + (size_t)l * H->sz_gu, H->s_gu + (size_t)l * 2 * g.I, 2 * g.I, h);
    run(launch_convert_rows(tmp, lw.down, nullptr, h, g.I, f32, ROWS_SAME, d, st));
    pack(H->w8_down + (size_t)l * H->sz_down, H->s_down + (size_t)l * h, h, g.I);
  }
  for (int l = 0; l < g.L && rc == DFLASH_OK; ++l) {
    const dflash_layer_weights &lw = w->layers[l];
    run(launch_convert_rows(tmp + (size_t)2 * l * g.kv_dim * h, lw.k, nullptr, g.kv_dim, h, f32, ROWS_ROPE_PAIRS, d, st));
    run(launch_convert_rows(tmp + (size_t)(2 * l + 1) * g.kv_dim * h, lw.v, nullptr, g.kv_dim, h, f32, ROWS_SAME, d, st));
  }
  if (rc == DFLASH_OK) pack(H->w8_fkv, H->s_fkv, g.fkv_dim, h);
  if (rc == DFLASH_OK) run(launch_convert_rows(tmp, w->fc, nullptr, h, g.fc_in, f32, ROWS_SAME, d, st));
  if (rc == DFLASH_OK) pack(H->w8_fc, H->s_fc, h, g.fc_in);
  const hipError_t se = hipStreamSynchronize(st);
  (void)hipFree(tmp);
  (void)hipFree(codes);
  if (rc != DFLASH_OK) return rc;
  HIP_TRY(se);
  return DFLASH_OK;
}

int build_impl(dflash_head *H, const dflash_weights *w, hipStream_t st) {
  const Geo &g = H->g;
  const bool f32 = g.w_f32;
  const size_t h = g.h;
  if (!w->fc || !w->hidden_norm || !w->norm || !w->embed_tokens || !w->layers)
    return set_err(DFLASH_E_INVALID, "weights: fc, hidden_norm, norm, embed_tokens and layers are required");
  if (!w->lm_head && !(g.head_fp8 && w->lm_head_fp8))
    return set_err(DFLASH_E_INVALID, "weights: lm_head is required (or lm_head_fp8 for an FP8 head)");
  if (w->lm_head_fp8 && (!g.head_fp8 || !w->lm_head_scale))
    return set_err(DFLASH_E_INVALID, "weights: lm_head_fp8 needs lm_head_dtype FP8_E4M3 and lm_head_scale");
  if (g.kv_fp8 && !w->kv_scale) return set_err(DFLASH_E_INVALID, "weights: kv_scale is required for an FP8 KV cache");
  for (int l = 0; l < g.L; ++l) {
    const dflash_layer_weights &lw = w->layers[l];
    if (!lw.in_norm || !lw.q || !lw.k || !lw.v || !lw.o || !lw.post_norm || !lw.gate || !lw.up || !lw.down)
      return set_err(DFLASH_E_INVALID, "weights: layer " + std::to_string(l) + " has a NULL tensor");
  }
  if (g.kv_fp8) {
    for (int i = 0; i < g.L * 2 * g.n_kv; ++i)
      if (!(w->kv_scale[i] > 0.0f) || !std::isfinite(w->kv_scale[i]))
        return set_err(DFLASH_E_INVALID, "weights: kv_scale entries must be finite and > 0");
  }

  // drafter tensors -> bf16, repacked into the tile-major GEMM layout
  H->sz_qkv = tiled_elems(g.qkv_dim, g.h);
  H->sz_o = tiled_elems(g.h, g.q_dim);
  H->sz_gu = tiled_elems(2 * g.I, g.h);
  H->sz_down = tiled_elems(g.h, g.I);
  TRY(H->alloc(&H->g_in, (size_t)g.L * h));
  TRY(H->alloc(&H->g_post, (size_t)g.L * h));
  TRY(H->alloc(&H->g_hidden, h));
  TRY(H->alloc(&H->g_final, h));
  const int d = g.d;
  for (int l = 0; l < g.L; ++l) {
    const dflash_layer_weights &lw = w->layers[l];
    HIP_TRY(launch_to_f32(H->g_in + (size_t)l * h, lw.in_norm, g.h, f32, st));
    HIP_TRY(launch_to_f32(H->g_post + (size_t)l * h, lw.post_norm, g.h, f32, st));
  }
  HIP_TRY(launch_to_f32(H->g_hidden, w->hidden_norm, g.h, f32, st));
  HIP_TRY(launch_to_f32(H->g_final, w->norm, g.h, f32, st));
  if (g.fp8w) {
    TRY(build_fp8_weights(H, w, st));
  } else {
  TRY(H->alloc(&H->w_qkv, (size_t)g.L * H->sz_qkv));
  TRY(H->alloc(&H->w_o, (size_t)g.L * H->sz_o));
  TRY(H->alloc(&H->w_gu, (size_t)g.L * H->sz_gu));
  TRY(H->alloc(&H->w_down, (size_t)g.L * H->sz_down));
  TRY(H->alloc(&H->w_fc, tiled_elems(g.h, g.fc_in)));
  TRY(H->alloc(&H->w_fkv, tiled_elems(g.fkv_dim, g.h)));
  for (int l = 0; l < g.L; ++l) {
    const dflash_layer_weights &lw = w->layers[l];
    // [Q; K; V] with Q and K rows in RoPE pair order
    uint16_t *qkv = H->w_qkv + (size_t)l * H->sz_qkv;
    HIP_TRY(launch_tile_rows(qkv, 0, lw.q, nullptr, g.q_dim, g.h, f32, ROWS_ROPE_PAIRS, d, st));
    HIP_TRY(launch_tile_rows(qkv, g.q_dim, lw.k, nullptr, g.kv_dim, g.h, f32, ROWS_ROPE_PAIRS, d, st));
    HIP_TRY(launch_tile_rows(qkv, g.q_dim + g.kv_dim, lw.v, nullptr, g.kv_dim, g.h, f32, ROWS_SAME, d, st));
    HIP_TRY(launch_tile_rows(H->w_o + (size_t)l * H->sz_o, 0, lw.o, nullptr, g.h, g.q_dim, f32, ROWS_SAME, d, st));
    HIP_TRY(launch_tile_rows(H->w_gu + (size_t)l * H->sz_gu, 0, lw.gate, lw.up, 2 * g.I, g.h, f32, ROWS_GATE_UP, d, st));
    HIP_TRY(launch_tile_rows(H->w_down + (size_t)l * H->sz_down, 0, lw.down, nullptr, g.h, g.I, f32, ROWS_SAME, d, st));
    // fused ctx K/V weight: rows [K0; V0; K1; V1; ...] (K rows in RoPE pair order)
    HIP_TRY(launch_tile_rows(H->w_fkv, 2 * l * g.kv_dim, lw.k, nullptr, g.kv_dim, g.h, f32, ROWS_ROPE_PAIRS, d, st));
    HIP_TRY(launch_tile_rows(H->w_fkv, (2 * l + 1) * g.kv_dim, lw.v, nullptr, g.kv_dim, g.h, f32, ROWS_SAME, d, st));
  }
  HIP_TRY(launch_tile_rows(H->w_fc, 0, w->fc, nullptr, g.h, g.fc_in, f32, ROWS_SAME, d, st));
  }

  // target's shared tensors: the embedding is borrowed when bf16 (rows are
  // gathered); the LM head is streamed from a tiled copy the head owns
  if (f32) {
    uint16_t *e = nullptr;
    TRY(H->alloc(&e, (size_t)g.V * h));
    HIP_TRY(launch_convert_rows(e, w->embed_tokens, nullptr, g.V, g.h, true, ROWS_SAME, d, st));
    H->embed = e;
  } else {
    H->embed = (const uint16_t *)w->embed_tokens;
  }
  if (!g.head_fp8) {
    uint16_t *m = nullptr;
    TRY(H->alloc(&m, tiled_elems(g.V, g.h)));
    HIP_TRY(launch_tile_rows(m, 0, w->lm_head, nullptr, g.V, g.h, f32, ROWS_SAME, d, st));
    H->lm = m;
  } else {
    // E4M3 codes + per-row scales: the given native head, or a mirror of the
    // bf16 head (amax / 448 per row); tiled into a copy the head owns
    uint8_t *tiled = nullptr;
    TRY(H->alloc(&tiled, tiled_elems(g.V, g.h)));
    if (w->lm_head_fp8) {
      float *s = nullptr;
      TRY(H->alloc(&s, (size_t)g.V));
      HIP_TRY(hipMemcpyAsync(s, w->lm_head_scale, (size_t)g.V * sizeof(float), hipMemcpyDeviceToDevice, st));
      HIP_TRY(launch_tile_fp8(tiled, (const uint8_t *)w->lm_head_fp8, g.V, g.h, st));
      H->lm8_scale = s;
    } else {
      const uint16_t *src = (const uint16_t *)w->lm_head;
      uint16_t *conv = nullptr;
      if (f32) {  // bf16 view of an f32 head, for the mirror only
        HIP_TRY(hipMalloc(&conv, (size_t)g.V * h * 2));
        HIP_TRY(launch_convert_rows(conv, w->lm_head, nullptr, g.V, g.h, true, ROWS_SAME, d, st));
        src = conv;
      }
      uint8_t *rowmajor = nullptr;
      float *s = nullptr;
      TRY(H->alloc(&s, (size_t)g.V));
      HIP_TRY(hipMalloc(&rowmajor, (size_t)g.V * h));
      HIP_TRY(launch_fp8_mirror(src, g.V, g.h, rowmajor, s, st));
      HIP_TRY(launch_tile_fp8(tiled, rowmajor, g.V, g.h, st));
      HIP_TRY(hipStreamSynchronize(st));
      (void)hipFree(rowmajor);
      if (conv) (void)hipFree(conv);
      H->lm8_scale = s;
    }
    H->lm8 = tiled;
  }

  // RoPE inverse frequencies in double
  std::vector<double> inv(g.d / 2);
  for (int i = 0; i < g.d / 2; ++i)
    inv[i] = w->inv_freq ? (double)w->inv_freq[i] : std::pow((double)H->cfg.rope_theta, -2.0 * i / g.d);
  TRY(H->alloc(&H->inv_freq, inv.size()));
  HIP_TRY(hipMemcpyAsync(H->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice, st));
  TRY(H->alloc(&H->kv_scale, (size_t)g.L * 2 * g.n_kv));
  if (g.kv_fp8)
    HIP_TRY(hipMemcpyAsync(H->kv_scale, w->kv_scale, (size_t)g.L * 2 * g.n_kv * sizeof(float), hipMemcpyHostToDevice, st));

  // paged KV pool [block][L][K|V][n_kv][16][d]
  H->kv_elem = g.kv_fp8 ? 1 : 2;
  const size_t pool_bytes = (size_t)H->cfg.kv_pool_blocks * g.L * 2 * g.n_kv * DFLASH_KV_BLOCK * g.d * H->kv_elem;
  {
    uint8_t *p = nullptr;
    TRY(H->alloc(&p, pool_bytes));
    HIP_TRY(hipMemsetAsync(p, 0, pool_bytes, st));
    H->kv_pool = p;
  }
  H->pool = BlockPool(H->cfg.kv_pool_blocks);

  // scratch sized for max_batch * gamma rows
  const size_t M = g.m_max;
  TRY(H->alloc(&H->sc.hid, M * h));
  TRY(H->alloc(&H->sc.act, M * h));
  if (g.a8) {
    TRY(H->alloc(&H->sc.act8, M * h));
    TRY(H->alloc(&H->sc.act8_scale, M));
  }
  TRY(H->alloc(&H->sc.qkv, M * g.qkv_dim));
  TRY(H->alloc(&H->sc.attn, M * g.q_dim));
  TRY(H->alloc(&H->sc.mlp, M * g.I));
  TRY(H->alloc(&H->sc.cs, M * (g.d / 2)));
  // split-K partials of the GEMMs that feed the residual stream (N = h)
  int max_splits = 1;
  for (int K : {g.q_dim, g.I, g.fc_in}) {
    max_splits = std::max(max_splits, gemm_plan(g.h, K, true).splits);
    if (bgemm_ok(EPI_PARTIAL, g.h, K)) max_splits = std::max(max_splits, bgemm_splits(g.h, K, (int)M));
  }
  // precompute passes of PREFILL_ROWS rows run through the tiled kernels
  H->tiled_prefill = !g.fp8w && bgemm_ok(EPI_PARTIAL, g.h, g.fc_in) && bgemm_ok(EPI_KV_SCATTER, g.fkv_dim, g.h);
  const size_t pre_rows = H->tiled_prefill ? PREFILL_ROWS : GEMM_MAX_ROWS;
  if (H->tiled_prefill) max_splits = std::max(max_splits, bgemm_splits(g.h, g.fc_in, PREFILL_ROWS));
  TRY(H->alloc(&H->sc.part, (size_t)max_splits * std::max({M, (size_t)GEMM_MAX_ROWS, pre_rows}) * h));
  const size_t R = (size_t)g.rep * g.gamma;
  // partial slots: every plan the propose takes fits (checked at build)
  H->sc.attn_slots = (int)attn_slots(g, H->cfg.max_seq_len, attn_max_tiles_per_split());
  TRY(H->alloc(&H->sc.ss, (size_t)((g.h + 15) / 16) * GEMM_MAX_ROWS));
  TRY(H->alloc(&H->sc.tile_ctr, (size_t)((g.h + 15) / 16)));
  HIP_TRY(hipMemsetAsync(H->sc.tile_ctr, 0, (size_t)((g.h + 15) / 16) * sizeof(int), st));
  H->gp = (g.gamma + 31) / 32 * 32;
  TRY(H->alloc(&H->sc.vtb, (size_t)g.max_batch * g.n_kv * g.d * H->gp));
  HIP_TRY(hipMemsetAsync(H->sc.vtb, 0, (size_t)g.max_batch * g.n_kv * g.d * H->gp * sizeof(uint16_t), st));
  TRY(H->alloc(&H->sc.o_part, (size_t)H->sc.attn_slots * R * g.d));
  TRY(H->alloc(&H->sc.ml_part, (size_t)H->sc.attn_slots * R * 2));
  H->lm_P = lm_parts(g.V);
  const size_t lm_slots = (size_t)std::max(H->lm_P, blm_parts(g.V)) * M;
  TRY(H->alloc(&H->sc.lm_mx, lm_slots));
  TRY(H->alloc(&H->sc.lm_se, lm_slots));
  TRY(H->alloc(&H->sc.lm_idx, lm_slots));
  TRY(H->alloc(&H->sc.lm_p1, M));
  TRY(H->alloc(&H->sc.fin_counters, (size_t)g.max_batch));
  HIP_TRY(hipMemsetAsync(H->sc.fin_counters, 0, (size_t)g.max_batch * sizeof(int), st));
  TRY(H->alloc(&H->pre_u, pre_rows * h));
  TRY(H->alloc(&H->pre_c, pre_rows * h));
  if (H->tiled_prefill) {
    TRY(H->alloc(&H->d_pos, 2 * (size_t)PREFILL_ROWS));
    TRY(H->alloc(&H->d_bts, 2 * (size_t)PREFILL_ROWS));
    HIP_TRY(hipHostMalloc((void **)&H->h_pos, 2 * PREFILL_ROWS * sizeof(int32_t), hipHostMallocDefault));
    HIP_TRY(hipHostMalloc((void **)&H->h_bts, 2 * PREFILL_ROWS * sizeof(const int32_t *), hipHostMallocDefault));
    for (hipEvent_t &e : H->pre_ev) HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  HIP_TRY(hipStreamSynchronize(st));
  return DFLASH_OK;
}

// One GEMM over M rows in chunks of GEMM_MAX_ROWS. The epilogue output
// pointers and the RoPE table are advanced with the rows. EPI_PARTIAL
// outputs are laid out [splits][M][N] over all M rows of the call.
// tiled: take the tiled kernel for any row count (else only above GEMM_MAX_ROWS).
int gemm_rows(dflash_head *H, int epi, const uint16_t *A, int lda, int M, Wt W, int N, int K,
              EpiArgs e, hipStream_t st, int *splits_out = nullptr, RowScale rs = RowScale{}, bool tiled = false) {
  GemmArgs ga{};
  ga.lda = lda;
  ga.W = W.w;
  ga.wscale = W.s;
  ga.N = N;
  ga.K = K;
  const GemmPlan p = gemm_plan(N, K, epi == EPI_PARTIAL);
  ga.tn = p.tn;
  ga.nw = p.nw;
  ga.st = p.st;
  ga.splits = p.splits;
  ga.kslice = p.kslice;
  if (splits_out) *splits_out = p.splits;
  e.ld_split = M;
  if ((M > GEMM_MAX_ROWS || tiled) && bgemm_ok(epi, N, K) && !rs.ss && !e.tile_ctr && !W.s) {
    // all rows in one tiled launch
    ga.A = A;
    ga.M = M;
    e.row0 = 0;
    if (epi == EPI_PARTIAL) {
      ga.splits = bgemm_splits(N, K, M);
      ga.kslice = K / ga.splits;
      if (splits_out) *splits_out = ga.splits;
    }
    HIP_TRY(launch_bgemm(epi, ga, e, st));
    return DFLASH_OK;
  }
  const int half = H->g.d / 2;
  for (int r0 = 0; r0 < M; r0 += GEMM_MAX_ROWS) {
    ga.A = A + (size_t)r0 * lda;
    ga.M = std::min(GEMM_MAX_ROWS, M - r0);
    EpiArgs ec = e;
    ec.row0 = r0;
    if (e.out_f32) ec.out_f32 = e.out_f32 + (size_t)r0 * e.ldo;
    if (e.out_bf16) ec.out_bf16 = e.out_bf16 + (size_t)r0 * e.ldo;
    if (e.cs) ec.cs = e.cs + (size_t)r0 * half;
    if (e.res_h) ec.res_h = e.res_h + (size_t)r0 * N;
    if (e.res_act) ec.res_act = e.res_act + (size_t)r0 * N;
    if (e.ss_out) ec.ss_out = e.ss_out + r0;
    ga.rs = rs;
    if (rs.ss) ga.rs.ss = rs.ss + r0;
    HIP_TRY(launch_gemm(epi, ga, ec, st));
  }
  return DFLASH_OK;
}

// h += W A^T for a GEMM into the residual stream (split over K, then the
// splits are added in order), followed by out = bf16(RMSNorm(h) * gain).
int resid_gemm(dflash_head *H, const Scratch &sc, const uint16_t *A, int lda, int M, Wt W, int K, float *h,
               const float *gain, uint16_t *out, bool init_zero, hipStream_t st, bool tiled = false) {
  EpiArgs e{};
  e.out_f32 = sc.part;
  e.ldo = H->g.h;
  int splits = 1;
  TRY(gemm_rows(H, EPI_PARTIAL, A, lda, M, W, H->g.h, K, e, st, &splits, RowScale{}, tiled));
  ResidNormArgs r{};
  r.h = h;
  r.part = sc.part;
  r.splits = splits;
  r.ld_split = M;
  r.n = H->g.h;
  r.init_zero = init_zero ? 1 : 0;
  r.gain = gain;
  r.eps = H->cfg.rms_eps;
  r.out = out;
  HIP_TRY(launch_resid_norm(r, M, st));
  return DFLASH_OK;
}

// h += W A^T into the residual stream for few rows: the split GEMM's last
// split of every 16-row unit adds the splits in order, writes bf16(h * gain)
// and the unit's per-row sums of squares (Scratch::ss); the consumer applies the
// RMSNorm row scale. Returns the units the consumer sums.
int resid_gemm_fused(dflash_head *H, const Scratch &sc, const uint16_t *A, int lda, int M, Wt W, int K,
                     const float *gain, hipStream_t st, int *units) {
  EpiArgs e{};
  e.out_f32 = sc.part;
  e.ldo = H->g.h;
  e.res_h = sc.hid;
  e.res_gain = gain;
  e.res_act = sc.act;
  e.ss_out = sc.ss;
  e.ss_ld = M;
  e.tile_ctr = sc.tile_ctr;
  TRY(gemm_rows(H, EPI_PARTIAL, A, lda, M, W, H->g.h, K, e, st));
  const GemmPlan p = gemm_plan(H->g.h, K, true);
  *units = (H->g.h + 16 * p.tn - 1) / (16 * p.tn);
  return DFLASH_OK;
}

// few rows: the residual GEMMs finish their own splits and every consumer
// applies the RMSNorm row scale from per-unit sums of squares (Scratch::ss);
// the W8A8 head needs the final-normed rows in act (no deferred row scale)
bool propose_fused(const Geo &g, int M) { return !g.a8 && M <= (g.fp8w ? GEMM_MAX_ROWS : PROPOSE_FEW_ROWS); }

bool propose_tiled_lm(const Geo &g, int M) {
  return !propose_fused(g, M) && (M > GEMM_MAX_ROWS || !g.fp8w || g.a8) && blm_ok(g.V, g.h);
}

// Argument checks of a propose and its attention plan: nothing is enqueued.
int propose_check(dflash_head *H, dflash_state *const *states, int n, const uint32_t *tokens, const int64_t *positions,
                  int num_drafts, uint32_t *ids, float *conf, int attn_slots, AttnPlan *plan) {
  const Geo &g = H->g;
  if (n < 1 || n > g.max_batch)
    return set_err(DFLASH_E_DECLINED, "batch of " + std::to_string(n) + " outside [1, " + std::to_string(g.max_batch) + "]");
  if (!states || !tokens || !positions) return set_err(DFLASH_E_INVALID, "states, last_tokens and positions are required");
  if (num_drafts < 1 || num_drafts > g.gamma - 1)
    return set_err(DFLASH_E_INVALID, "num_drafts must be in [1, gamma - 1]");
  if (!ids || !conf) return set_err(DFLASH_E_INVALID, "ids and conf outputs are required");
  for (int i = 0; i < n; ++i) {
    if (!state_ok(H, states[i])) return set_err(DFLASH_E_INVALID, "state " + std::to_string(i) + " is not a live state of this head");
    if (tokens[i] >= (uint32_t)g.V) return set_err(DFLASH_E_INVALID, "last_token " + std::to_string(tokens[i]) + " >= vocab");
    if (positions[i] < 0 || positions[i] > (int64_t)INT_MAX - g.gamma)
      return set_err(DFLASH_E_INVALID, "position out of range");
  }
  const int M = n * g.gamma;
  if (g.a8 && !propose_tiled_lm(g, M)) return set_err(DFLASH_E_INVALID, "the W8A8 LM head needs the tiled head");
  // attention splits, planned before anything is enqueued
  int32_t tiles[DFLASH_MAX_BATCH];
  for (int i = 0; i < n; ++i) tiles[i] = attn_tiles(states[i]->rows.ctx_len, g.W);
  std::string err;
  const int rc = attn_plan(n, tiles, g.n_kv, attn_max_tiles_per_split(), attn_slots / g.n_kv,
                           ATTN_TARGET_WGS, plan, &err);
  if (rc != DFLASH_OK) return set_err(rc, err);
  return DFLASH_OK;
}

// The launches of a checked propose, with its scratch.
int propose_launch(dflash_head *H, const Scratch &sc, const AttnPlan &plan, dflash_state *const *states, int n,
                   const uint32_t *tokens, const int64_t *positions, int num_drafts, const int32_t *bitmasks,
                   uint32_t *ids, float *conf, float *row_prob, float *logits, hipStream_t st, bool timed) {
  const Geo &g = H->g;
  const int M = n * g.gamma;
  const int h = g.h;
  const bool fused = propose_fused(g, M);
  const bool tiled_lm = propose_tiled_lm(g, M);
  hipEvent_t t_all = timed ? H->interval_begin(DFLASH_PHASE_PROPOSE, st) : nullptr;

  SetupArgs sa{};
  sa.embed = H->embed;
  sa.gain = H->g_in;
  sa.eps = H->cfg.rms_eps;
  sa.h = h;
  sa.gamma = g.gamma;
  sa.half_dim = g.d / 2;
  sa.mask_id = g.mask_id;
  sa.inv_freq = H->inv_freq;
  sa.hid = sc.hid;
  sa.a = sc.act;
  sa.ss_out = fused ? sc.ss : nullptr;
  sa.cs = sc.cs;
  for (int i = 0; i < n; ++i) {
    sa.token[i] = tokens[i];
    sa.position[i] = (int32_t)positions[i];
  }
  HIP_TRY(launch_setup(sa, M, st));

  AttnArgs aa{};
  aa.qkv = sc.qkv;
  aa.vtb = sc.vtb;
  aa.ld = g.qkv_dim;
  aa.gamma = g.gamma;
  aa.rep = g.rep;
  aa.n_kv = g.n_kv;
  aa.head_dim = g.d;
  aa.k_off = g.q_dim;
  aa.v_off = g.q_dim + g.kv_dim;
  aa.pool = H->kv_pool;
  aa.L = g.L;
  aa.kv_fp8 = g.kv_fp8;
  aa.kv_scale = H->kv_scale;
  aa.o_part = sc.o_part;
  aa.ml_part = sc.ml_part;
  aa.out = sc.attn;
  aa.out_ld = g.q_dim;
  // ctx tiles of 32 positions from the block-aligned window start, in the
  // splits of the plan (attn_plan: the last split of a sequence also takes
  // the block tile)
  for (int i = 0; i < n; ++i) {
    const int c = states[i]->rows.ctx_len;
    aa.seq[i].ctx_len = c;
    aa.seq[i].win_start = g.W > 0 ? std::max(0, c - g.W) : c;
    aa.seq[i].bt = states[i]->d_bt;
    aa.seq[i].split0 = plan.split0[i];
    aa.seq[i].nsplit = plan.nsplit[i];
    for (int c2 = 0; c2 < plan.nsplit[i]; ++c2) aa.split_seq[plan.split0[i] + c2] = (uint8_t)i;
  }
  aa.tps = plan.tps;
  aa.n_split = plan.n_split;

  // act holds RMSNorm(h) with the next consumer's gain: layer 0's input norm
  // comes from the setup kernel, every later one from the residual finish.
  EpiArgs e{};
  RowScale rs{};
  if (fused) rs = RowScale{sc.ss, 1, M, H->cfg.rms_eps};
  for (int l = 0; l < g.L; ++l) {
    e = EpiArgs{};
    e.out_bf16 = sc.qkv;
    e.ldo = g.qkv_dim;
    e.cs = sc.cs;
    e.head_dim = g.d;
    e.q_dim = g.q_dim;
    e.kv_dim = g.kv_dim;
    e.vtb = sc.vtb;
    e.gamma = g.gamma;
    e.gp = H->gp;
    TRY(gemm_rows(H, EPI_QKV_ROPE, sc.act, h, M, H->wqkv(l), g.qkv_dim, h, e, st, nullptr, rs, !fused));
    aa.layer = l;
    HIP_TRY(launch_attention(aa, n, st));
    const float *post_gain = H->g_post + (size_t)l * h;
    if (fused) {
      TRY(resid_gemm_fused(H, sc, sc.attn, g.q_dim, M, H->wo(l), g.q_dim, post_gain, st, &rs.units));
    } else {
      TRY(resid_gemm(H, sc, sc.attn, g.q_dim, M, H->wo(l), g.q_dim, sc.hid, post_gain, sc.act, false, st, true));
    }
    e = EpiArgs{};
    e.out_bf16 = sc.mlp;
    e.ldo = g.I;
    TRY(gemm_rows(H, EPI_SWIGLU, sc.act, h, M, H->wgu(l), 2 * g.I, h, e, st, nullptr, rs, !fused));
    const float *next_gain = l + 1 < g.L ? H->g_in + (size_t)(l + 1) * h : H->g_final;
    if (fused) {
      TRY(resid_gemm_fused(H, sc, sc.mlp, g.I, M, H->wdown(l), g.I, next_gain, st, &rs.units));
    } else {
      TRY(resid_gemm(H, sc, sc.mlp, g.I, M, H->wdown(l), g.I, sc.hid, next_gain, sc.act, false, st, true));
    }
  }

  LmArgs la{};
  la.K = h;
  la.W = g.head_fp8 ? (const void *)H->lm8 : (const void *)H->lm;
  la.scale = H->lm8_scale;
  la.V = g.V;
  la.bitmask = bitmasks;
  la.words = g.words;
  la.gamma = g.gamma;
  la.ld_part = M;
  la.part_mx = sc.lm_mx;
  la.part_se = sc.lm_se;
  la.part_idx = sc.lm_idx;
  la.rs = rs;
  if (tiled_lm) {
    la.z = sc.act;
    la.M = M;
    la.row0 = 0;
    la.logits = logits;
    if (g.a8) {
      HIP_TRY(launch_quant_rows_a8(sc.act, M, h, sc.act8, sc.act8_scale, st));
      la.z8 = sc.act8;
      la.ascale = sc.act8_scale;
    }
    hipEvent_t t_lm = timed ? H->interval_begin(DFLASH_PHASE_LM_HEAD, st) : nullptr;
    HIP_TRY(launch_blm_head(g.head_fp8, g.a8, la, st));
    if (t_lm) HIP_TRY(hipEventRecord(t_lm, st));
  }
  for (int r0 = 0; !tiled_lm && r0 < M; r0 += GEMM_MAX_ROWS) {
    la.z = sc.act + (size_t)r0 * h;
    la.M = std::min(GEMM_MAX_ROWS, M - r0);
    la.row0 = r0;
    la.logits = logits ? logits + (size_t)r0 * g.V : nullptr;
    hipEvent_t t_lm = timed ? H->interval_begin(DFLASH_PHASE_LM_HEAD, st) : nullptr;
    HIP_TRY(launch_lm_head(g.head_fp8, la, st));
    if (t_lm) HIP_TRY(hipEventRecord(t_lm, st));
  }
  LmFinishArgs fa{};
  fa.part_mx = sc.lm_mx;
  fa.part_se = sc.lm_se;
  fa.part_idx = sc.lm_idx;
  fa.P = tiled_lm ? blm_parts(g.V) : H->lm_P;
  fa.M = M;
  fa.gamma = g.gamma;
  fa.num_drafts = num_drafts;
  fa.shifted = g.shifted ? 1 : 0;
  fa.ids = ids;
  fa.conf = conf;
  fa.row_prob = row_prob;
  fa.p1 = sc.lm_p1;
  fa.counters = sc.fin_counters;
  HIP_TRY(launch_lm_finish(fa, n, st));
  if (t_all) HIP_TRY(hipEventRecord(t_all, st));
  return DFLASH_OK;
}

// Upload block-table entries that are not yet on the device.
int sync_block_table(dflash_state *s, hipStream_t st) {
  const int32_t nb = (int32_t)s->rows.blocks.size();
  if (nb <= s->uploaded) return DFLASH_OK;
  if (nb > s->cap_blocks) return set_err(DFLASH_E_NO_BLOCKS, "block table capacity exceeded");
  for (int32_t i = s->uploaded; i < nb; ++i) s->h_bt[i] = s->rows.blocks[i];
  HIP_TRY(hipMemcpyAsync(s->d_bt + s->uploaded, s->h_bt + s->uploaded, (size_t)(nb - s->uploaded) * sizeof(int32_t),
                         hipMemcpyHostToDevice, st));
  s->uploaded = nb;
  return DFLASH_OK;
}

}  // namespace

// ---- allocation-free propose ------------------------------------------------
// Scratch of dflash_propose_noalloc, for callers that cannot allocate device
// memory. Every device the library runs on holds its own copy of this array
// (at its own address) until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns on that device, never
// through the array's name. All calls on one device share it.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on device dev: resolved once per device, with
// dev current (dflash_build calls this for its device; a later call on
// another current device cannot resolve it).
int scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= MAX_DEVICES) return set_err(DFLASH_E_INVALID, "device id out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    HIP_TRY(hipGetDevice(&cur));
    if (cur != dev) return set_err(DFLASH_E_INVALID, "the static scratch is resolved with the head's device current");
    void *p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return set_err(DFLASH_E_HIP, "hipGetSymbolAddress gave no address for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH_OK;
}

// Lay out the scratch of a one-sequence propose with attention plan `plan`
// from `base` (256-byte aligned pieces); with base null only the size is
// computed. The split counters and the block V^T copy (which must be zero
// when a call starts) are placed side by side, from sc->fin_counters on, and
// *zero_bytes is their extent.
size_t carve_scratch(const dflash_head *H, const AttnPlan &plan, uint8_t *base, Scratch *sc, size_t *zero_bytes) {
  const Geo &g = H->g;
  const size_t M = g.gamma, h = g.h, R = (size_t)g.rep * g.gamma;
  size_t off = 0;
  auto take = [&](auto **p, size_t count) {
    off = (off + 255) & ~(size_t)255;
    *p = base ? (std::remove_reference_t<decltype(*p)>)(base + off) : nullptr;
    off += count * sizeof(**p);
  };
  take(&sc->hid, M * h);
  take(&sc->act, M * h);
  if (g.a8) {
    take(&sc->act8, M * h);
    take(&sc->act8_scale, M);
  }
  take(&sc->qkv, M * g.qkv_dim);
  take(&sc->attn, M * g.q_dim);
  take(&sc->mlp, M * g.I);
  take(&sc->cs, M * (g.d / 2));
  sc->attn_slots = plan.n_split * g.n_kv;
  take(&sc->o_part, (size_t)sc->attn_slots * R * g.d);
  take(&sc->ml_part, (size_t)sc->attn_slots * R * 2);
  const size_t P = (size_t)std::max(lm_parts(g.V), blm_parts(g.V));
  take(&sc->lm_mx, P * M);
  take(&sc->lm_se, P * M);
  take(&sc->lm_idx, P * M);
  take(&sc->lm_p1, M);
  take(&sc->ss, (h + 15) / 16 * M);
  int splits = 1;
  for (int K : {g.q_dim, g.I}) {
    splits = std::max(splits, gemm_plan(g.h, K, true).splits);
    if (bgemm_ok(EPI_PARTIAL, g.h, K)) splits = std::max(splits, bgemm_splits(g.h, K, (int)M));
  }
  take(&sc->part, (size_t)splits * M * h);
  off = (off + 255) & ~(size_t)255;
  const size_t zero0 = off;  // sc->fin_counters starts here
  take(&sc->fin_counters, 1);
  take(&sc->tile_ctr, (h + 15) / 16);
  take(&sc->vtb, (size_t)g.n_kv * g.d * H->gp);
  off = (off + 255) & ~(size_t)255;
  *zero_bytes = off - zero0;
  return off;
}

}  // namespace

extern "C" {

const char *dflash_last_error(void) { return g_err.c_str(); }

int dflash_build(const dflash_config *cfg, const dflash_weights *w, uint64_t stream, dflash_head **out) {
  if (!cfg || !w || !out) return set_err(DFLASH_E_INVALID, "cfg, weights and out are required");
  *out = nullptr;
  Geo g;
  std::string err;
  int rc = validate_config(*cfg, &g, &err);
  if (rc == DFLASH_OK) rc = check_attn_capacity(g, cfg->max_seq_len, attn_max_tiles_per_split(), &err);
  if (rc != DFLASH_OK) return set_err(rc, err);
  int dev_count = 0;
  if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count < 1) return set_err(DFLASH_E_HIP, "no HIP device");
  dflash_head *H = new dflash_head();
  H->cfg = *cfg;
  H->g = g;
  if (hipGetDevice(&H->dev) != hipSuccess) H->dev = 0;
  rc = build_impl(H, w, to_stream(stream));
  if (rc != DFLASH_OK) {
    (void)hipStreamSynchronize(to_stream(stream));
    free_head_memory(H);
    H->magic = DEAD_MAGIC;
    delete H;
    return rc;
  }
  // the static scratch of dflash_propose_noalloc, resolved on the head's
  // device while it is current (a failure is reported by that call)
  void *unused = nullptr;
  (void)scratch_address(H->dev, &unused);
  *out = H;
  g_err.clear();
  return DFLASH_OK;
}

void dflash_destroy(dflash_head *head) {
  if (!head_ok(head)) return;
  (void)hipDeviceSynchronize();
  for (dflash_state *s : head->states) {
    free_state_memory(s);
    s->magic = DEAD_MAGIC;
    delete s;
  }
  head->states.clear();
  for (auto &q : head->timed)
    for (auto &p : q) {
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    }
  for (hipEvent_t e : head->event_pool) (void)hipEventDestroy(e);
  free_head_memory(head);
  head->magic = DEAD_MAGIC;
  delete head;
}

int dflash_block_gamma(const dflash_head *head) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  return head->g.gamma;
}

int dflash_propose_batch_max(const dflash_head *head) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  return head->g.max_batch;
}

int dflash_state_create(dflash_head *head, int64_t budget_tokens, const int32_t *block_ids, int32_t n_ids,
                        dflash_state **out) {
  if (!head_ok(head) || !out) return set_err(DFLASH_E_INVALID, "invalid head or out");
  *out = nullptr;
  std::lock_guard<std::mutex> lk(head->mu);
  dflash_state *s = new dflash_state();
  s->owner = head;
  std::string err;
  int rc = seq_init(&s->rows, &head->pool, budget_tokens, block_ids, n_ids, head->cfg.max_seq_len, &err);
  if (rc != DFLASH_OK) {
    delete s;
    return set_err(rc, err);
  }
  s->cap_blocks = (int32_t)((s->rows.cap_rows + DFLASH_KV_BLOCK - 1) / DFLASH_KV_BLOCK);
  s->cap_blocks = std::max<int32_t>(s->cap_blocks, (int32_t)s->rows.blocks.size());
  s->cap_blocks = std::max<int32_t>(s->cap_blocks, 1);
  hipError_t e = hipMalloc(&s->d_bt, (size_t)s->cap_blocks * sizeof(int32_t));
  if (e == hipSuccess) e = hipHostMalloc(&s->h_bt, (size_t)s->cap_blocks * sizeof(int32_t), hipHostMallocDefault);
  if (e == hipSuccess) e = hipMemset(s->d_bt, 0, (size_t)s->cap_blocks * sizeof(int32_t));
  if (e == hipSuccess && !s->rows.blocks.empty()) {
    for (size_t i = 0; i < s->rows.blocks.size(); ++i) s->h_bt[i] = s->rows.blocks[i];
    e = hipMemcpy(s->d_bt, s->h_bt, s->rows.blocks.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    s->uploaded = (int32_t)s->rows.blocks.size();
  }
  if (e != hipSuccess) {
    seq_release(&s->rows, &head->pool);
    free_state_memory(s);
    delete s;
    return set_err(DFLASH_E_NOMEM, std::string("state allocation: ") + hipGetErrorString(e));
  }
  head->states.push_back(s);
  *out = s;
  return DFLASH_OK;
}

int dflash_state_free(dflash_head *head, dflash_state *st) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (!state_ok(head, st)) return set_err(DFLASH_E_INVALID, "not a live state of this head");
  HIP_TRY(hipDeviceSynchronize());
  seq_release(&st->rows, &head->pool);
  free_state_memory(st);
  head->states.erase(std::remove(head->states.begin(), head->states.end(), st), head->states.end());
  st->magic = DEAD_MAGIC;
  delete st;
  return DFLASH_OK;
}

int dflash_state_ctx_len(const dflash_state *st) {
  if (!st || st->magic != STATE_MAGIC) return set_err(DFLASH_E_INVALID, "invalid state");
  return st->rows.ctx_len;
}

int dflash_precompute_ctx_kv(dflash_head *head, dflash_state *const *states, int32_t n, const int32_t *n_new,
                             const void *stack, uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  dflash_head *H = head;
  const Geo &g = H->g;
  if (n < 1 || !states || !n_new) return set_err(DFLASH_E_INVALID, "n >= 1, states and n_new are required");
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (!state_ok(H, states[i])) return set_err(DFLASH_E_INVALID, "state " + std::to_string(i) + " is not a live state of this head");
    if (n_new[i] < 0) return set_err(DFLASH_E_INVALID, "n_new must be >= 0");
    for (int j = 0; j < i; ++j)
      if (states[j] == states[i] && n_new[i] > 0 && n_new[j] > 0)
        return set_err(DFLASH_E_INVALID, "a state appears twice with rows to append");
    total += n_new[i];
  }
  if (total > INT_MAX / 2) return set_err(DFLASH_E_INVALID, "too many rows");
  if (total > 0 && !stack) return set_err(DFLASH_E_INVALID, "stack is required when rows are appended");
  // reserve blocks for every state first, all or nothing (no device work yet)
  {
    std::vector<SeqRows *> rows(n);
    std::vector<int32_t> caps(n);
    for (int i = 0; i < n; ++i) {
      rows[i] = &states[i]->rows;
      caps[i] = states[i]->cap_blocks;
    }
    std::string err;
    const int rc = reserve_rows(rows.data(), n, n_new, caps.data(), &H->pool, &err);
    if (rc != DFLASH_OK) return set_err(rc, err);
  }
  hipStream_t st = to_stream(stream);
  for (int i = 0; i < n; ++i) TRY(sync_block_table(states[i], st));
  if (total == 0) return DFLASH_OK;

  // row -> (position, block table)
  std::vector<int> pos;
  std::vector<const int32_t *> bts;
  pos.reserve(total);
  bts.reserve(total);
  for (int i = 0; i < n; ++i)
    for (int k = 0; k < n_new[i]; ++k) {
      pos.push_back(states[i]->rows.ctx_len + k);
      bts.push_back(states[i]->d_bt);
    }
  const int h = g.h;
  hipEvent_t t_all = H->interval_begin(DFLASH_PHASE_PRECOMPUTE, st);
  if (H->tiled_prefill && total > GEMM_MAX_ROWS) {
    // passes of up to PREFILL_ROWS rows through the tiled kernels; the rows'
    // positions and block tables go to the device through pinned staging
    for (int r0 = 0, pass = 0; r0 < (int)total; r0 += PREFILL_ROWS, ++pass) {
      const int m = std::min<int>(PREFILL_ROWS, (int)total - r0);
      const int b = pass & 1;
      if (H->pre_ev_used[b]) HIP_TRY(hipEventSynchronize(H->pre_ev[b]));  // the copy that read staging b is done
      int32_t *hp = H->h_pos + (size_t)b * PREFILL_ROWS;
      const int32_t **hb = H->h_bts + (size_t)b * PREFILL_ROWS;
      for (int r = 0; r < m; ++r) {
        hp[r] = pos[r0 + r];
        hb[r] = bts[r0 + r];
      }
      int32_t *dp = H->d_pos + (size_t)b * PREFILL_ROWS;
      const int32_t **db = H->d_bts + (size_t)b * PREFILL_ROWS;
      HIP_TRY(hipMemcpyAsync(dp, hp, m * sizeof(int32_t), hipMemcpyHostToDevice, st));
      HIP_TRY(hipMemcpyAsync((void *)db, (const void *)hb, m * sizeof(const int32_t *), hipMemcpyHostToDevice, st));
      HIP_TRY(hipEventRecord(H->pre_ev[b], st));
      H->pre_ev_used[b] = true;
      TRY(resid_gemm(H, H->sc, (const uint16_t *)stack + (size_t)r0 * g.fc_in, g.fc_in, m, H->wfc(), g.fc_in, H->pre_u,
                     H->g_hidden, H->pre_c, true, st));
      EpiArgs e{};
      e.head_dim = g.d;
      e.pool = H->kv_pool;
      e.L = g.L;
      e.n_kv = g.n_kv;
      e.kv_fp8 = g.kv_fp8;
      e.kv_scale = H->kv_scale;
      e.inv_freq = H->inv_freq;
      e.d_row_pos = dp;
      e.d_row_bt = db;
      TRY(gemm_rows(H, EPI_KV_SCATTER, H->pre_c, h, m, H->wfkv(), g.fkv_dim, h, e, st));
    }
    if (t_all) HIP_TRY(hipEventRecord(t_all, st));
    for (int i = 0; i < n; ++i) states[i]->rows.ctx_len += n_new[i];
    return DFLASH_OK;
  }
  for (int r0 = 0; r0 < (int)total; r0 += GEMM_MAX_ROWS) {
    const int m = std::min<int>(GEMM_MAX_ROWS, (int)total - r0);
    // u = S fc^T (split over K, summed in split order), c = RMSNorm(u) bf16
    TRY(resid_gemm(H, H->sc, (const uint16_t *)stack + (size_t)r0 * g.fc_in, g.fc_in, m, H->wfc(), g.fc_in, H->pre_u,
                   H->g_hidden, H->pre_c, true, st));
    EpiArgs e{};
    e.head_dim = g.d;
    e.pool = H->kv_pool;
    e.L = g.L;
    e.n_kv = g.n_kv;
    e.kv_fp8 = g.kv_fp8;
    e.kv_scale = H->kv_scale;
    e.inv_freq = H->inv_freq;
    for (int r = 0; r < m; ++r) {
      e.row_pos[r] = pos[r0 + r];
      e.row_bt[r] = bts[r0 + r];
    }
    TRY(gemm_rows(H, EPI_KV_SCATTER, H->pre_c, h, m, H->wfkv(), g.fkv_dim, h, e, st));
  }
  if (t_all) HIP_TRY(hipEventRecord(t_all, st));
  for (int i = 0; i < n; ++i) states[i]->rows.ctx_len += n_new[i];
  return DFLASH_OK;
}

int dflash_propose(dflash_head *head, dflash_state *st, uint32_t last_token, int64_t position, int32_t num_drafts,
                   const int32_t *bitmask, uint32_t *ids, float *conf, float *row_prob, float *logits,
                   uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  dflash_state *states[1] = {st};
  AttnPlan plan;
  int rc = propose_check(head, states, 1, &last_token, &position, num_drafts, ids, conf, head->sc.attn_slots, &plan);
  if (rc == DFLASH_E_DECLINED) return set_err(DFLASH_E_INVALID, g_err);
  if (rc != DFLASH_OK) return rc;
  return propose_launch(head, head->sc, plan, states, 1, &last_token, &position, num_drafts, bitmask, ids, conf,
                        row_prob, logits, to_stream(stream), true);
}

int dflash_propose_batch(dflash_head *head, dflash_state *const *states, int32_t n, const uint32_t *last_tokens,
                         const int64_t *positions, int32_t num_drafts, const int32_t *bitmasks, uint32_t *ids,
                         float *conf, float *row_prob, float *logits, uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  AttnPlan plan;
  const int rc = propose_check(head, states, n, last_tokens, positions, num_drafts, ids, conf, head->sc.attn_slots, &plan);
  if (rc != DFLASH_OK) return rc;
  return propose_launch(head, head->sc, plan, states, n, last_tokens, positions, num_drafts, bitmasks, ids, conf,
                        row_prob, logits, to_stream(stream), true);
}

int dflash_propose_noalloc(dflash_head *head, dflash_state *st, uint32_t last_token, int64_t position,
                           int32_t num_drafts, const int32_t *bitmask, uint32_t *ids, float *conf, float *row_prob,
                           float *logits, uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  dflash_state *states[1] = {st};
  // the plan of dflash_propose, so the two give the same result bit for bit
  AttnPlan plan;
  int rc = propose_check(head, states, 1, &last_token, &position, num_drafts, ids, conf, head->sc.attn_slots, &plan);
  if (rc == DFLASH_E_DECLINED) return set_err(DFLASH_E_INVALID, g_err);
  if (rc != DFLASH_OK) return rc;
  Scratch sc;
  size_t zero_bytes = 0;
  const size_t need = carve_scratch(head, plan, nullptr, &sc, &zero_bytes);
  if (need > NOALLOC_SCRATCH_BYTES)
    return set_err(DFLASH_E_INVALID, "this propose needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                         std::to_string(NOALLOC_SCRATCH_BYTES) + " of the static array");
  void *base = nullptr;
  TRY(scratch_address(head->dev, &base));
  carve_scratch(head, plan, (uint8_t *)base, &sc, &zero_bytes);
  const hipStream_t s = to_stream(stream);
  // the previous call on this device left its own counters and V^T rows here
  HIP_TRY(launch_zero(sc.fin_counters, zero_bytes, s));
  return propose_launch(head, sc, plan, states, 1, &last_token, &position, num_drafts, bitmask, ids, conf, row_prob,
                        logits, s, false);
}

int dflash_after_verify(dflash_head *head, dflash_state *st, int32_t num_accepted) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (!state_ok(head, st)) return set_err(DFLASH_E_INVALID, "not a live state of this head");
  std::string err;
  int rc = seq_trim(&st->rows, num_accepted, &err);
  return rc == DFLASH_OK ? rc : set_err(rc, err);
}

// Whether a live state of the head holds block b.
static bool block_owned(const dflash_head *head, int32_t b) {
  for (const dflash_state *s : head->states)
    for (int32_t x : s->rows.blocks)
      if (x == b) return true;
  return false;
}

int dflash_take_kv(dflash_head *head, dflash_state *st, int32_t *blocks_out, int32_t cap, int32_t *n_blocks,
                   int32_t *rows, int64_t *last_pair_key) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (!state_ok(head, st)) return set_err(DFLASH_E_INVALID, "not a live state of this head");
  if (!n_blocks || !rows || !last_pair_key) return set_err(DFLASH_E_INVALID, "n_blocks, rows and last_pair_key are required");
  const int32_t nb = (int32_t)st->rows.blocks.size();
  *n_blocks = nb;
  *rows = 0;
  *last_pair_key = -1;
  if (nb == 0) return DFLASH_OK;  // nothing to carry
  if (!blocks_out || cap < nb) return set_err(DFLASH_E_INVALID, "blocks_out holds fewer than the state's blocks");
  HIP_TRY(hipDeviceSynchronize());  // no launch still reads the state's block table
  std::vector<int32_t> taken;
  seq_take(&st->rows, &taken, rows);
  std::copy(taken.begin(), taken.end(), blocks_out);
  *last_pair_key = st->pair_key;
  st->pair_key = -1;
  st->uploaded = 0;
  return DFLASH_OK;
}

int dflash_install_kv(dflash_head *head, dflash_state *st, const int32_t *blocks, int32_t n_blocks, int32_t rows,
                      int64_t last_pair_key) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (!state_ok(head, st)) return set_err(DFLASH_E_INVALID, "not a live state of this head");
  if (!blocks || n_blocks < 1) return set_err(DFLASH_E_INVALID, "install needs at least one block");
  if (n_blocks > st->cap_blocks) return set_err(DFLASH_E_INVALID, "more blocks than the state's block table holds");
  for (int32_t i = 0; i < n_blocks; ++i)
    if (block_owned(head, blocks[i]))
      return set_err(DFLASH_E_INVALID, "block " + std::to_string(blocks[i]) + " is held by a live state");
  HIP_TRY(hipDeviceSynchronize());  // no launch still reads the state's block table
  std::string err;
  const int rc = seq_install(&st->rows, &head->pool, blocks, n_blocks, rows, head->cfg.max_seq_len, &err);
  if (rc != DFLASH_OK) return set_err(rc, err);
  for (int32_t i = 0; i < n_blocks; ++i) st->h_bt[i] = blocks[i];
  HIP_TRY(hipMemcpy(st->d_bt, st->h_bt, (size_t)n_blocks * sizeof(int32_t), hipMemcpyHostToDevice));
  st->uploaded = n_blocks;
  st->pair_key = last_pair_key;
  return DFLASH_OK;
}

int dflash_free_kv(dflash_head *head, const int32_t *blocks, int32_t n_blocks) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (n_blocks < 0 || (n_blocks > 0 && !blocks)) return set_err(DFLASH_E_INVALID, "bad block list");
  std::vector<uint8_t> seen(head->pool.size(), 0);
  for (int32_t i = 0; i < n_blocks; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= head->pool.size() || head->pool.is_free(b) || seen[b]++)
      return set_err(DFLASH_E_INVALID, "block " + std::to_string(b) + " is not an allocated pool block (or given twice)");
    if (block_owned(head, b)) return set_err(DFLASH_E_INVALID, "block " + std::to_string(b) + " is held by a live state");
  }
  for (int32_t i = 0; i < n_blocks; ++i) head->pool.release(blocks[i]);
  return DFLASH_OK;
}

int dflash_state_read_kv(dflash_head *head, const dflash_state *st, int32_t layer, int32_t row0, int32_t n_rows,
                         void *k_out, void *v_out, uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (!state_ok(head, st)) return set_err(DFLASH_E_INVALID, "not a live state of this head");
  const Geo &g = head->g;
  if (layer < 0 || layer >= g.L) return set_err(DFLASH_E_INVALID, "layer out of range");
  if (row0 < 0 || n_rows < 0 || (int64_t)row0 + n_rows > st->rows.ctx_len)
    return set_err(DFLASH_E_INVALID, "rows outside [0, ctx_len)");
  if (n_rows == 0) return DFLASH_OK;
  HIP_TRY(launch_read_kv(head->kv_pool, st->d_bt, g.L, layer, g.n_kv, g.d, (int)head->kv_elem, row0, n_rows, k_out,
                         v_out, to_stream(stream)));
  return DFLASH_OK;
}

int dflash_yarn_inv_freq(int32_t head_dim, float rope_theta, float factor, float beta_fast, float beta_slow,
                         int32_t original_max_positions, float *out) {
  std::string err;
  const int rc = yarn_inv_freq(head_dim, rope_theta, factor, beta_fast, beta_slow, original_max_positions, out, &err);
  if (rc != DFLASH_OK) return set_err(rc, err);
  return DFLASH_OK;
}

int dflash_timing_enable(dflash_head *head, int enable) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  head->timing = enable != 0;
  if (!head->timing) {
    for (auto &q : head->timed) {
      for (auto &p : q) {
        (void)hipEventSynchronize(p.second);
        head->event_pool.push_back(p.first);
        head->event_pool.push_back(p.second);
      }
      q.clear();
    }
  }
  return DFLASH_OK;
}

int dflash_timing_read(dflash_head *head, int32_t phase, double *total_ms, int64_t *intervals) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  if (phase < 0 || phase > 2 || !total_ms || !intervals) return set_err(DFLASH_E_INVALID, "bad phase or outputs");
  double sum = 0.0;
  int64_t n = 0;
  for (auto &p : head->timed[phase]) {
    HIP_TRY(hipEventSynchronize(p.second));
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, p.first, p.second));
    sum += ms;
    ++n;
    head->event_pool.push_back(p.first);
    head->event_pool.push_back(p.second);
  }
  head->timed[phase].clear();
  *total_ms = sum;
  *intervals = n;
  return DFLASH_OK;
}

int dflash_read_lm_head_fp8(dflash_head *head, void *codes_out, float *scale_out, uint64_t stream) {
  if (!head_ok(head)) return set_err(DFLASH_E_INVALID, "invalid head");
  std::lock_guard<std::mutex> lk(head->mu);
  const Geo &g = head->g;
  if (!g.head_fp8) return set_err(DFLASH_E_INVALID, "the head's LM head is bf16");
  hipStream_t st = to_stream(stream);
  if (codes_out) HIP_TRY(launch_untile_fp8((uint8_t *)codes_out, head->lm8, g.V, g.h, st));
  if (scale_out) HIP_TRY(hipMemcpyAsync(scale_out, head->lm8_scale, (size_t)g.V * sizeof(float), hipMemcpyDeviceToDevice, st));
  return DFLASH_OK;
}

}  // extern "C"
