// kernels.hpp - argument structs and host launchers of the gfx950 kernels.
// Every launcher enqueues on `stream` and returns hipSuccess or the launch
// error; shapes are validated by the caller (dflash.hip) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// ---------------------------------------------------------------- GEMMs ----
// Skinny weight-streaming GEMM: out[m, n] = sum_k A[m, k] * W[n, k] for
// M <= 64 activation rows (bf16, row stride lda) against a weight matrix W
// [N, K] (bf16, or E4M3 codes with per-row f32 scales). Work: one workgroup
// per 128 output columns and K slice; split-K partials are reduced in fixed
// split order by the last workgroup of each column group.

enum Epi : int {
  EPI_F32 = 0,        // out_f32[m, n] = acc
  EPI_RESID = 1,      // out_f32[m, n] += acc (the fp32 residual stream)
  EPI_SWIGLU = 2,     // W rows are 64-row gate / up blocks; out_bf16[m, i] = silu(gate) * up
  EPI_QKV_ROPE = 3,   // columns [Q | K | V]; RoPE on Q and K from the per-row cos/sin table
  EPI_KV_SCATTER = 4  // columns [K0 | V0 | K1 | V1 ...]; RoPE on K at the row position, store into the paged pool
};

constexpr int GEMM_MAX_ROWS = 64;

struct GemmArgs {
  const uint16_t *A;
  int lda, M;
  const void *W;      // [N, K] bf16 or E4M3
  int N, K;
  int kslice, splits; // K slice per workgroup (multiple of 128), number of slices
  float *ws;          // split-K partials
  int *counters;      // per column group, zero between launches
};

struct EpiArgs {
  float *out_f32;
  uint16_t *out_bf16;
  int ldo;
  // QKV RoPE
  const float2 *cs;   // [M][head_dim / 2] (cos, sin) of each row's position
  int head_dim, q_dim, kv_dim;
  // KV scatter
  void *pool;
  int L, n_kv, kv_fp8;
  const float *kv_scale;   // device [L][2][n_kv]
  const double *inv_freq;  // device [head_dim / 2]
  int row_pos[GEMM_MAX_ROWS];
  const int32_t *row_bt[GEMM_MAX_ROWS];
};

// Split choice depends only on (N, K) so a row's result does not depend on
// how many rows share the launch.
void gemm_plan(int N, int K, int *kslice, int *splits);
size_t gemm_ws_floats(int N, int K);   // workspace for M up to 64
int gemm_groups(int N);

hipError_t launch_gemm(int epi, bool w_fp8, const GemmArgs &g, const EpiArgs &e, hipStream_t s);

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
};
int lm_parts(int V);     // P, a function of V only
hipError_t launch_lm_head(bool w_fp8, const LmArgs &a, hipStream_t s);

struct LmFinishArgs {
  const float *part_mx, *part_se;
  const uint32_t *part_idx;
  int P, M, gamma, num_drafts;
  uint32_t *ids;
  float *conf, *row_prob;
};
hipError_t launch_lm_finish(const LmFinishArgs &a, int n_seq, hipStream_t s);

// ------------------------------------------------------------- attention ---
struct AttnSeq {
  int ctx_len, win_start;
  const int32_t *bt;
};

struct AttnArgs {
  const uint16_t *qkv;   // [n_seq * gamma, ld] rows [Q | K | V], RoPE applied
  int ld, gamma, rep, n_kv, head_dim, k_off, v_off;
  const void *pool;
  int L, layer, kv_fp8;
  const float *kv_scale;
  int chunk, max_splits;
  float *o_part, *ml_part;
  uint16_t *out;         // [n_seq * gamma, n_q * head_dim] bf16
  int out_ld;
  AttnSeq seq[DFLASH_MAX_BATCH];
};
hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s);

// ------------------------------------------------------------------ misc ---
struct SetupArgs {
  const uint16_t *embed;    // [V, h] bf16
  const float *gain;        // [h] first layer input norm
  float eps;
  int h, gamma, half_dim;
  uint32_t mask_id;
  const double *inv_freq;   // [half_dim]
  float *hid;               // [M, h] fp32
  uint16_t *a;              // [M, h] bf16
  float2 *cs;               // [M, half_dim]
  uint32_t token[DFLASH_MAX_BATCH];
  int32_t position[DFLASH_MAX_BATCH];
};
hipError_t launch_setup(const SetupArgs &a, int M, hipStream_t s);

// out[m] = bf16(RMSNorm(x[m]) * gain), x fp32 [M, n] row stride ldx.
hipError_t launch_rmsnorm(const float *x, int ldx, const float *gain, float eps, int n, uint16_t *out, int ldo,
                          int M, hipStream_t s);

// dst rows [0, rows) of [rows, cols] bf16 from src rows (bf16 or f32);
// interleave != 0: dst is the 64-row gate / up interleave of src (gate) and
// src2 (up), each [rows / 2, cols].
hipError_t launch_convert_rows(uint16_t *dst, const void *src, const void *src2, int rows, int cols, bool src_f32,
                               bool interleave, hipStream_t s);
hipError_t launch_to_f32(float *dst, const void *src, int n, bool src_f32, hipStream_t s);

// FP8 mirror of a bf16 [V, h] head: per-row scale amax / 448, E4M3 codes.
hipError_t launch_fp8_mirror(const uint16_t *src, int V, int h, uint8_t *codes, float *scale, hipStream_t s);

// Gather ctx rows of one layer out of the paged pool (storage dtype bytes).
hipError_t launch_read_kv(const void *pool, const int32_t *bt, int L, int layer, int n_kv, int d, int elem_bytes,
                          int row0, int n_rows, void *k_out, void *v_out, hipStream_t s);

}  // namespace dflash
