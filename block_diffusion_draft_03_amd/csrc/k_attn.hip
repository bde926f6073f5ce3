// k_attn.hip - GQA attention of the block rows over the paged ctx window and
// the block itself, for gfx950.
//
// One workgroup per (sequence, kv head, key chunk). The rep = n_q / n_kv
// query heads of a kv head times the gamma block rows form up to 128 query
// rows, 32 per wave. Keys are the ctx rows [win_start, ctx_len) read through
// the block table from the paged pool, followed by the gamma block rows (K/V
// straight from the QKV output). Every 32-key tile is staged in LDS (K
// row-major, V transposed), with FP8 codes widened to bf16 on the way.
//
// The products are computed transposed so every per-query quantity stays in
// one lane: S^T = K Q^T (MFMA A = 16 keys x 32 dims, B = Q^T), giving lane l
// the scores of query l % 16 for keys 4g + r (g = l / 16); the PV product is
// O^T = V^T P^T, whose B operand is exactly the lane's own probabilities for
// keys {4g..4g+3, 16+4g..16+4g+3} and whose A operand reads V^T for the same
// key set. Online softmax in base 2; the running max is shared across the
// four lane groups with two shuffles, the running sum stays per lane until
// the end. Each workgroup writes an unnormalised partial (O, max, sum) and a
// combine kernel merges the chunks of a (sequence, kv head).
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int KT = 32;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int KS = D >= 32 ? D / 32 : 1;  // 32-dim MFMA k-steps
  constexpr int DT = D / 16;                // 16-dim output tiles
  constexpr int KP = D + 8;                 // padded LDS row of K
  constexpr int VP = KT + 8;                // padded LDS row of V^T
  __shared__ uint16_t Ks[KT][KP];
  __shared__ uint16_t Vt[D][VP];

  const int s = blockIdx.z, g = blockIdx.y, c = blockIdx.x;
  const AttnSeq sq = a.seq[s];
  const int S_ctx = sq.ctx_len - sq.win_start;
  const int S = S_ctx + a.gamma;
  const int nsplit = (S + a.chunk - 1) / a.chunk;
  if (c >= nsplit) return;
  const int key_lo = c * a.chunk, key_hi = min(S, key_lo + a.chunk);
  const int R = a.rep * a.gamma;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lg = lane >> 4, r16 = lane & 15;
  const uint4 z4 = {0u, 0u, 0u, 0u};

  // Q fragments (B operand of S^T = K Q^T): query column r16 of each tile.
  bf16x8 qf[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = min((wave * 2 + qt) * 16 + r16, R - 1);
    const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
    const uint16_t *qrow = a.qkv + (size_t)(s * a.gamma + j) * a.ld + hq * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dd = ks * 32 + 8 * lg;
      qf[qt][ks] = as_bf16x8(dd < D ? *(const uint4 *)(qrow + dd) : z4);
    }
  }

  float kscale = 1.0f, vscale = 1.0f;
  if (a.kv_fp8) {
    kscale = a.kv_scale[(a.layer * 2 + 0) * a.n_kv + g];
    vscale = a.kv_scale[(a.layer * 2 + 1) * a.n_kv + g];
  }
  const float sc_ctx = LOG2E / sqrtf((float)D) * kscale;  // scores in base-2 units
  const float sc_blk = LOG2E / sqrtf((float)D);

  f32x4 o[2][DT];
  float m_run[2], l_run[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    m_run[qt] = -__builtin_huge_valf();
    l_run[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t head_stride = (size_t)DFLASH_KV_BLOCK * D;  // one (block, layer, K|V, head) tile
  for (int t0 = key_lo; t0 < key_hi; t0 += KT) {
    __syncthreads();
    // Stage K and V^T for keys t0 .. t0 + 31 (8 dims per item).
    for (int e = threadIdx.x; e < KT * (D / 8); e += blockDim.x) {
      const int key = e / (D / 8), dc = (e % (D / 8)) * 8;
      const int kidx = t0 + key;
      uint4 kv8 = z4, vv8 = z4;
      if (kidx < key_hi) {
        if (kidx < S_ctx) {
          const int pos = sq.win_start + kidx;
          const int32_t blk = sq.bt[pos >> 4];
          const size_t base = (((size_t)blk * a.L + a.layer) * 2 * a.n_kv + g) * head_stride + (size_t)(pos & 15) * D + dc;
          const size_t vofs = (size_t)a.n_kv * head_stride;
          if (a.kv_fp8) {
            const uint8_t *p = (const uint8_t *)a.pool;
            const uint2 kc = *(const uint2 *)(p + base), vc = *(const uint2 *)(p + base + vofs);
            uint2 lo = e4m3x4_to_bf16x4(kc.x), hi = e4m3x4_to_bf16x4(kc.y);
            kv8 = uint4{lo.x, lo.y, hi.x, hi.y};
            lo = e4m3x4_to_bf16x4(vc.x);
            hi = e4m3x4_to_bf16x4(vc.y);
            vv8 = uint4{lo.x, lo.y, hi.x, hi.y};
          } else {
            const uint16_t *p = (const uint16_t *)a.pool;
            kv8 = *(const uint4 *)(p + base);
            vv8 = *(const uint4 *)(p + base + vofs);
          }
        } else {
          const uint16_t *brow = a.qkv + (size_t)(s * a.gamma + (kidx - S_ctx)) * a.ld;
          kv8 = *(const uint4 *)(brow + a.k_off + g * D + dc);
          vv8 = *(const uint4 *)(brow + a.v_off + g * D + dc);
        }
      }
      *(uint4 *)&Ks[key][dc] = kv8;
      const uint16_t *vh = (const uint16_t *)&vv8;
#pragma unroll
      for (int i = 0; i < 8; ++i) Vt[dc + i][key] = vh[i];
    }
    __syncthreads();

#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if ((wave * 2 + qt) * 16 >= R) continue;  // wave-uniform
      f32x4 sacc[2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        sacc[ks2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int dd = ks * 32 + 8 * lg;
          const bf16x8 kf = as_bf16x8(dd < D ? *(const uint4 *)&Ks[ks2 * 16 + r16][dd] : z4);
          sacc[ks2] = mfma16x16x32(kf, qf[qt][ks], sacc[ks2]);
        }
      }
      float x[2][4];
      float tmax = -__builtin_huge_valf();
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kidx = t0 + ks2 * 16 + 4 * lg + r;
          const float sc = kidx < S_ctx ? sc_ctx : sc_blk;
          x[ks2][r] = kidx < key_hi ? sacc[ks2][r] * sc : -__builtin_huge_valf();
          tmax = fmaxf(tmax, x[ks2][r]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
      const float m_new = fmaxf(m_run[qt], tmax);
      const float alpha = fast_exp2(m_run[qt] - m_new);
      // P feeds the PV product; ctx keys of an FP8 cache carry the V scale
      // in P (their V codes are staged unscaled), block keys do not.
      float p[2][4], psum = 0.0f;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(x[ks2][r] - m_new);
          psum += e;
          p[ks2][r] = t0 + ks2 * 16 + 4 * lg + r < S_ctx ? e * vscale : e;
        }
      l_run[qt] = l_run[qt] * alpha + psum;
      m_run[qt] = m_new;
      uint4 pk;
      pk.x = pack_bf16x2(p[0][0], p[0][1]);
      pk.y = pack_bf16x2(p[0][2], p[0][3]);
      pk.z = pack_bf16x2(p[1][0], p[1][1]);
      pk.w = pack_bf16x2(p[1][2], p[1][3]);
      const bf16x8 pf = as_bf16x8(pk);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[qt][dt] *= alpha;
        const uint16_t *vr = &Vt[dt * 16 + r16][0];
        const uint2 v0 = *(const uint2 *)(vr + 4 * lg), v1 = *(const uint2 *)(vr + 16 + 4 * lg);
        const bf16x8 vf = as_bf16x8(uint4{v0.x, v0.y, v1.x, v1.y});
        o[qt][dt] = mfma16x16x32(vf, pf, o[qt][dt]);
      }
    }
  }

  // Unnormalised partial of this chunk: O, running max (base 2), sum.
  const size_t part = ((size_t)(s * a.n_kv + g) * a.max_splits + c) * R;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = (wave * 2 + qt) * 16 + r16;
    float l_tot = l_run[qt];
    l_tot += __shfl_xor(l_tot, 16, WAVE);
    l_tot += __shfl_xor(l_tot, 32, WAVE);
    if ((wave * 2 + qt) * 16 >= R || q >= R) continue;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *(f32x4 *)(a.o_part + (part + q) * D + dt * 16 + 4 * lg) = o[qt][dt];
    }
    if (lg == 0) {
      a.ml_part[(part + q) * 2 + 0] = m_run[qt];
      a.ml_part[(part + q) * 2 + 1] = l_tot;
    }
  }
}

// Merge the key chunks of every (sequence, kv head, query row, dim).
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int n_seq) {
  const int R = a.rep * a.gamma, D = a.head_dim;
  const size_t total = (size_t)n_seq * a.n_kv * R * D;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int dd = (int)(e % D);
    const int q = (int)((e / D) % R);
    const int g = (int)((e / ((size_t)D * R)) % a.n_kv);
    const int s = (int)(e / ((size_t)D * R * a.n_kv));
    const AttnSeq sq = a.seq[s];
    const int S = sq.ctx_len - sq.win_start + a.gamma;
    const int nsplit = (S + a.chunk - 1) / a.chunk;
    const size_t base = (size_t)(s * a.n_kv + g) * a.max_splits;
    float M = -__builtin_huge_valf();
    for (int c = 0; c < nsplit; ++c) M = fmaxf(M, a.ml_part[((base + c) * R + q) * 2]);
    float num = 0.0f, den = 0.0f;
    for (int c = 0; c < nsplit; ++c) {
      const size_t pr = (base + c) * R + q;
      const float w = fast_exp2(a.ml_part[pr * 2] - M);
      den += w * a.ml_part[pr * 2 + 1];
      num += w * a.o_part[pr * D + dd];
    }
    const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
    a.out[(size_t)(s * a.gamma + j) * a.out_ld + hq * D + dd] = f32_to_bf16(num / den);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s) {
  dim3 grid(a.max_splits, a.n_kv, n_seq), block(256);
  switch (a.head_dim) {
    case 16: hipLaunchKernelGGL(k_attn<16>, grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL(k_attn<32>, grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL(k_attn<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn<128>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)n_seq * a.n_kv * a.rep * a.gamma * a.head_dim;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(k_attn_combine, dim3(blocks), dim3(256), 0, s, a, n_seq);
  return hipGetLastError();
}

}  // namespace dflash
