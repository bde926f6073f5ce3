// gemm_epi.hpp - lane-local epilogues shared by the weight-streaming GEMM
// kernels (few activation rows) and the tiled GEMM kernels (many rows).
//
// Both compute D^T = W A^T with v_mfma_f32_16x16x32_bf16, so a lane ends with
// four consecutive output columns n .. n+3 (weight rows 4g .. 4g+3 of a
// 16-row tile) for one activation row m. The build repacks weight rows in
// pairs: Q and K rows of a head are ordered (dim i, dim i + d/2), and the MLP
// weight alternates gate and up rows, so (n, n+1) and (n+2, n+3) are a RoPE
// pair or a gate/up pair and every epilogue stays inside the lane.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

// (cos, sin) of the two RoPE pairs in columns n .. n+3 of row m (unused for
// V columns): 16 contiguous bytes of the row's table, so a kernel can load
// them before its weight stream.
__device__ __forceinline__ float4 qkv_cs(int m, int n, const EpiArgs &ea) {
  if (n >= ea.q_dim + ea.kv_dim) return float4{1.0f, 0.0f, 1.0f, 0.0f};
  const int p = (n % ea.head_dim) >> 1;  // pair index of rows n, n+1 (even)
  return *(const float4 *)(ea.cs + (size_t)m * (ea.head_dim >> 1) + p);
}

// EPI_QKV_ROPE with the row's (cos, sin) pairs cs = (c0, s0, c1, s1).
__device__ __forceinline__ void epilogue4_qkv(const f32x4 v, int m, int n, const float4 cs, const EpiArgs &ea) {
  float y[4] = {v[0], v[1], v[2], v[3]};
  if (n < ea.q_dim + ea.kv_dim) {
    y[0] = v[0] * cs.x - v[1] * cs.y;
    y[1] = v[1] * cs.x + v[0] * cs.y;
    y[2] = v[2] * cs.z - v[3] * cs.w;
    y[3] = v[3] * cs.z + v[2] * cs.w;
  }
  // fp16: Q, K and V are only read by the attention kernel, which multiplies
  // in fp16 (8 more significand bits than bf16 on the same matrix cores)
  uint2 o;
  o.x = pack_f16x2(y[0], y[1]);
  o.y = pack_f16x2(y[2], y[3]);
  *(uint2 *)(ea.out_bf16 + (size_t)m * ea.ldo + n) = o;
  if (n >= ea.q_dim + ea.kv_dim && ea.vtb) {
    // V of the block rows, transposed per kv head for the attention kernel
    const int vn = n - ea.q_dim - ea.kv_dim, hd = vn / ea.head_dim, dim = vn % ea.head_dim;
    const int seq = (ea.row0 + m) / ea.gamma, j = (ea.row0 + m) % ea.gamma;
    const int n_kv = ea.kv_dim / ea.head_dim, nb16 = ea.gp / 16;
    uint16_t *vt = ea.vtb + (((size_t)(seq * n_kv + hd) * nb16 + j / 16) * ea.head_dim + dim) * 16 + (j & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) vt[(size_t)r * 16] = (uint16_t)(pack_f16x2(y[r], 0.0f) & 0xFFFFu);
  }
}

// EPI_F32:      out_f32[m, n..n+3] = v
// EPI_PARTIAL:  out_f32[split][m][n..n+3] = v   (row stride ldo, split stride ld_split rows)
// EPI_SWIGLU:   out_bf16[m, n/2], [m, n/2 + 1] = silu(gate) * up
// EPI_QKV_ROPE: out_bf16[m, n..n+3] = v as fp16, rotated by row m's (cos, sin) when n is a Q or K column
// EPI_KV_SCATTER: columns [K0 | V0 | K1 | V1 ...]; K rotated at the row's position; stored
//               (bf16 or E4M3 with the per-head scale) into the row's pool slot
template <int EPI>
__device__ __forceinline__ void epilogue4(const f32x4 v, int m, int n, int split, const EpiArgs &ea) {
  if constexpr (EPI == EPI_F32 || EPI == EPI_PARTIAL) {
    float *o = EPI == EPI_F32 ? ea.out_f32 + (size_t)m * ea.ldo + n
                              : ea.out_f32 + ((size_t)split * ea.ld_split + m) * ea.ldo + n;
    *(f32x4 *)o = v;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // rows (gate_i, up_i, gate_i+1, up_i+1) with i = n / 2
    *(uint32_t *)(ea.out_bf16 + (size_t)m * ea.ldo + n / 2) = pack_bf16x2(silu(v[0]) * v[1], silu(v[2]) * v[3]);
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    epilogue4_qkv(v, m, n, qkv_cs(m, n, ea), ea);
  } else if constexpr (EPI == EPI_KV_SCATTER) {
    const int d = ea.head_dim;
    const int kv_dim = ea.n_kv * d;
    const int l = n / (2 * kv_dim), rem = n % (2 * kv_dim);
    const int kv = rem / kv_dim, hd = (rem % kv_dim) / d, j = n % d;
    const int pos = ea.d_row_pos ? ea.d_row_pos[m] : ea.row_pos[m];
    float y[4] = {v[0], v[1], v[2], v[3]};
    if (kv == 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        double sn, cs;
        sincos((double)pos * ea.inv_freq[(j >> 1) + q], &sn, &cs);
        const float c = (float)cs, s = (float)sn;
        const float x0 = v[2 * q], x1 = v[2 * q + 1];
        y[2 * q] = x0 * c - x1 * s;
        y[2 * q + 1] = x1 * c + x0 * s;
      }
    }
    // K tile [16 slots][d]; V tile transposed, [d][16 slots]
    const int32_t blk = (ea.d_row_pos ? ea.d_row_bt[m] : ea.row_bt[m])[pos >> 4];
    const size_t tile = ((((size_t)blk * ea.L + l) * 2 + kv) * ea.n_kv + hd) * (size_t)(DFLASH_KV_BLOCK * d);
    const int slot = pos & 15;
    if (ea.kv_fp8) {
      const float sc = ea.kv_scale[(l * 2 + kv) * ea.n_kv + hd];
      uint8_t *p = (uint8_t *)ea.pool + tile;
      if (kv == 0) {
        uint32_t w = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) w |= (uint32_t)f32_to_e4m3(y[r] / sc) << (8 * r);
        *(uint32_t *)(p + (size_t)slot * d + j) = w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[(size_t)(j + r) * DFLASH_KV_BLOCK + slot] = f32_to_e4m3(y[r] / sc);
      }
    } else {
      uint16_t *p = (uint16_t *)ea.pool + tile;
      if (kv == 0) {
        *(uint2 *)(p + (size_t)slot * d + j) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[(size_t)(j + r) * DFLASH_KV_BLOCK + slot] = f32_to_bf16(y[r]);
      }
    }
  }
}

}  // namespace dflash
