// kernels.hpp - argument structs and host launchers of the gfx950 kernels.
// Every launcher enqueues on `stream` and returns hipSuccess or the launch
// error; shapes are validated by the caller (dflash.cpp) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"
#include "host_core.hpp"

namespace dflash {

// ---------------------------------------------------------------- GEMMs ----
// out[m, n] = sum_k A[m, k] * W[n, k]: bf16 activations A [M, lda] against a
// tile-major weight matrix W [N, K]. launch_gemm is the weight-streaming
// kernel for M <= 64 rows (one workgroup per 16 * tn weight rows and K slice,
// nw waves splitting the slice); launch_bgemm is the LDS-tiled kernel for
// many rows. Both follow the K order of gemm_plan, so they give identical
// results for a row. With splits > 1 the epilogue must be EPI_PARTIAL and
// k_resid_norm finishes the sum.

enum Epi : int {
  EPI_F32 = 0,        // out_f32[m, n] = acc
  EPI_SWIGLU = 2,     // W rows alternate gate / up; out_bf16[m, i] = silu(gate_i) * up_i
  EPI_QKV_ROPE = 3,   // columns [Q | K | V] (Q, K in pair order); RoPE on Q and K from the cos/sin table
  EPI_KV_SCATTER = 4, // columns [K0 | V0 | K1 | V1 ...]; RoPE on K at the row position, store into the paged pool
  EPI_PARTIAL = 5     // out_f32[(split * ld_split + m) * ldo + n] = this split's partial sum
};

constexpr int GEMM_MAX_ROWS = 64;

// Launch shape of one GEMM; a function of (N, K) only, so a row's result does
// not depend on how many rows share the launch. Each K slice of kslice
// columns is summed as four consecutive parts (the nw = 4 waves of the
// weight-streaming kernel), added in order.
struct GemmPlan {
  int tn, nw, st, splits, kslice;
};
GemmPlan gemm_plan(int N, int K, bool allow_split);

// Row scale of an activation that is not yet normalised: A holds
// bf16(h * gain) and r[m] = 1 / sqrt(sum_u ss[u * ld + m] / K + eps) from the
// producer's per-unit sums of squares of h; the GEMM multiplies row m of its
// result by r[m] (null ss: A is already normalised).
struct RowScale {
  const float *ss;
  int units, ld;
  float eps;
};

struct GemmArgs {
  const uint16_t *A;  // bf16 activations [M, lda]
  int lda, M;
  const void *W;      // [N, K] bf16, tile-major
  int N, K;
  int tn, nw, st, splits, kslice;
  RowScale rs;        // weight-streaming kernel only
  const float *wscale;  // E4M3 weights: W is tiled E4M3 and output n is scaled by wscale[n] (weight-streaming kernel only)
};

struct EpiArgs {
  float *out_f32;
  uint16_t *out_bf16;  // bf16 bit patterns (SwiGLU), fp16 (QKV)
  int ldo, ld_split;
  // QKV RoPE
  const float2 *cs;   // [M][head_dim / 2] (cos, sin) of each row's position
  int head_dim, q_dim, kv_dim;
  uint16_t *vtb;      // QKV: V^T of the block rows (fp16), [seq][n_kv][gp / 16][head_dim][16] (gp = gamma rounded up to 32)
  int gamma, gp, row0;  // row0: row of the call that this launch's row 0 is
  // KV scatter
  void *pool;
  int L, n_kv, kv_fp8;
  const float *kv_scale;   // device [L][2][n_kv]
  const double *inv_freq;  // device [head_dim / 2]
  int row_pos[GEMM_MAX_ROWS];
  const int32_t *row_bt[GEMM_MAX_ROWS];
  // KV scatter over more rows (tiled kernel): device [M] positions and block
  // tables of the launch's rows, used instead of row_pos / row_bt when set
  const int32_t *d_row_pos;
  const int32_t *const *d_row_bt;
  // EPI_PARTIAL, weight-streaming kernel: when tile_ctr is set, the last
  // split of every unit adds the splits in order to the fp32 residual res_h
  // [M][N], writes res_act = bf16(res_h * res_gain) and the unit's per-row
  // sum of squares to ss_out[unit * ss_ld + m] (counters start and end at 0)
  float *res_h;
  const float *res_gain;
  uint16_t *res_act;
  float *ss_out;
  int ss_ld;
  int *tile_ctr;
};

hipError_t launch_gemm(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s);

// The tiled kernel takes any M (one launch for all rows) when N and K are
// multiples of 128 (EPI_KV_SCATTER then reads d_row_pos / d_row_bt).
bool bgemm_ok(int epi, int N, int K);
// K splits of a tiled EPI_PARTIAL GEMM over M rows (at most 4; K a multiple of 128 * splits).
int bgemm_splits(int N, int K, int M);
hipError_t launch_bgemm(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s);

// Finish of a split GEMM into the residual stream, one workgroup per row:
// h[m] = (init_zero ? 0 : h[m]) + sum over splits of part[s][m]; then, if out
// is set, out[m] = bf16(RMSNorm(h[m]) * gain).
struct ResidNormArgs {
  float *h;
  const float *part;   // [splits][ld_split][n]
  int splits, ld_split, n, init_zero;
  const float *gain;
  float eps;
  uint16_t *out;
};
hipError_t launch_resid_norm(const ResidNormArgs &a, int M, hipStream_t s);

// --------------------------------------------------------------- LM head ---
struct LmArgs {
  const uint16_t *z;     // [M, K] bf16 final-normed rows (rows row0 .. row0 + M - 1 of the call)
  int M, K;
  int row0, ld_part;     // global row of z[0]; partial row stride (all rows of the call)
  const void *W;         // [V, K] bf16 or E4M3
  const float *scale;    // [V] for E4M3
  int V;
  const int32_t *bitmask;  // [n_seq, words] or null
  int words, gamma;
  float *logits;         // [M, V] or null, already offset to row0
  float *part_mx, *part_se;
  uint32_t *part_idx;    // [P, ld_part]
  RowScale rs;           // weight-streaming kernel only (rows row0 + m)
  const uint8_t *z8;     // tiled W8A8 head only: [M, K] E4M3 codes of z
  const float *ascale;   // and their [M] row scales
};
int lm_parts(int V);     // P of launch_lm_head, a function of V only
hipError_t launch_lm_head(bool w_fp8, const LmArgs &a, hipStream_t s);
// Tiled LM head for any M (one launch for all rows; row0 = 0, ld_part = M)
// when blm_ok(V, K), blm_parts(V) partials per row. Logits are bit-identical
// to launch_lm_head's (both sum K in one pass). a_fp8 (needs w_fp8): W8A8,
// the rows come as E4M3 codes z8 with row scales ascale (z unused).
bool blm_ok(int V, int K);
int blm_parts(int V);
hipError_t launch_blm_head(bool w_fp8, bool a_fp8, const LmArgs &a, hipStream_t s);

struct LmFinishArgs {
  const float *part_mx, *part_se;
  const uint32_t *part_idx;
  int P, M, gamma, num_drafts;
  int shifted;     // row j goes to entry (j + 1) % gamma of ids, row_prob and p1
  uint32_t *ids;
  float *conf, *row_prob;
  float *p1;       // [M] scratch: top-1 probability of every row
  int *counters;   // [n_seq] zero between launches
};
hipError_t launch_lm_finish(const LmFinishArgs &a, int n_seq, hipStream_t s);

// ------------------------------------------------------------- attention ---
struct AttnSeq {
  int ctx_len, win_start;
  const int32_t *bt;
  int split0, nsplit;  // this sequence's first split (over all sequences of the launch) and split count (1..64)
};

// ATTN_MAX_FLAT (splits over all sequences of one launch): host_core.hpp

struct AttnArgs {
  const uint16_t *qkv;   // [n_seq * gamma, ld] fp16 rows [Q | K | V], RoPE applied
  const uint16_t *vtb;   // fp16 V^T of the block rows, [n_seq][n_kv][roundup(gamma, 32) / 16][head_dim][16], zero padded
  int ld, gamma, rep, n_kv, head_dim, k_off, v_off;
  const void *pool;      // [block][L][K|V][n_kv] tiles: K [16][head_dim], V^T [head_dim][16]
  int L, layer, kv_fp8;
  const float *kv_scale;
  int tps, n_split;      // ctx tiles (32 positions) per split; splits over all sequences (per kv head)
  uint16_t *o_part;      // fp16 normalised output of each split [slot][R][head_dim]
  float *ml_part;        // (max, sum) of each split's rows
  uint16_t *out;         // [n_seq * gamma, n_q * head_dim] bf16
  int out_ld;
  AttnSeq seq[DFLASH_MAX_BATCH];
  uint8_t split_seq[ATTN_MAX_FLAT];  // sequence of each split
};
hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s);
int attn_max_tiles_per_split();

// ------------------------------------------------------------------ misc ---
struct SetupArgs {
  const uint16_t *embed;    // [V, h] bf16
  const float *gain;        // [h] first layer input norm
  float eps;
  int h, gamma, half_dim;
  uint32_t mask_id;
  const double *inv_freq;   // [half_dim]
  float *hid;               // [M, h] fp32
  uint16_t *a;              // [M, h] bf16: RMSNorm(h) * gain, or h * gain when ss_out is set
  float *ss_out;            // [M] sum of squares of each row (the row scale is left to the consumer), or null
  float2 *cs;               // [M, half_dim]
  uint32_t token[DFLASH_MAX_BATCH];
  int32_t position[DFLASH_MAX_BATCH];
};
hipError_t launch_setup(const SetupArgs &a, int M, hipStream_t s);

// Row orders of the repacked weights.
enum RowOrder : int {
  ROWS_SAME = 0,      // dst row r = src row r
  ROWS_GATE_UP = 1,   // dst row 2i = src (gate) row i, dst row 2i+1 = src2 (up) row i
  ROWS_ROPE_PAIRS = 2 // within each head of head_dim rows: dst row j = src row j/2 + (j%2) * head_dim/2
};

// dst rows [0, rows) of [rows, cols] bf16 from src rows (bf16 or f32) in the
// given row order.
hipError_t launch_convert_rows(uint16_t *dst, const void *src, const void *src2, int rows, int cols, bool src_f32,
                               int order, int head_dim, hipStream_t s);

// Tile-major weight layout read by the GEMM kernels. A [rows, cols] matrix
// becomes ceil(rows/16) tiles of 16 rows; each tile holds ceil(cols/128)
// steps of 128 columns; a bf16 step is 4 k-groups x 64 lanes x 8 values, lane
// l of k-group c holding row l % 16, columns 32c + 8(l / 16) .. +7. Rows and
// columns past the matrix are zero. An E4M3 step is 2 pairs x 64 lanes x 16
// bytes: pair j of lane l holds the 8 codes of k-group 2j then of 2j + 1.
size_t tiled_elems(int rows, int cols);
// bf16 tiled copy of src rows (bf16 or f32) in the given row order, written
// at tile row offset dst_row0 (a multiple of 16) of a matrix with `cols`.
hipError_t launch_tile_rows(uint16_t *dst, int dst_row0, const void *src, const void *src2, int rows, int cols,
                            bool src_f32, int order, int head_dim, hipStream_t s);
// E4M3 tiled copy of row-major codes [rows, cols].
hipError_t launch_tile_fp8(uint8_t *dst, const uint8_t *src, int rows, int cols, hipStream_t s);
// Row-major copy of a tiled E4M3 matrix.
hipError_t launch_untile_fp8(uint8_t *dst, const uint8_t *src, int rows, int cols, hipStream_t s);
hipError_t launch_to_f32(float *dst, const void *src, int n, bool src_f32, hipStream_t s);

// FP8 mirror of a bf16 [V, h] head: per-row scale amax / 448, E4M3 codes.
hipError_t launch_fp8_mirror(const uint16_t *src, int V, int h, uint8_t *codes, float *scale, hipStream_t s);
// E4M3 rows for the W8A8 LM head: launch_fp8_mirror's codes and scales, each
// 128-column step's codes permuted into the head's K order (h % 128 == 0)
hipError_t launch_quant_rows_a8(const uint16_t *src, int M, int h, uint8_t *codes, float *scale, hipStream_t s);
// Zero `bytes` (a multiple of 4, 4-byte aligned) at device address p.
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

// Gather ctx rows of one layer out of the paged pool (storage dtype bytes).
hipError_t launch_read_kv(const void *pool, const int32_t *bt, int L, int layer, int n_kv, int d, int elem_bytes,
                          int row0, int n_rows, void *k_out, void *v_out, hipStream_t s);

}  // namespace dflash
