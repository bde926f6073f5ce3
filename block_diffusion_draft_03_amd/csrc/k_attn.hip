// k_attn.hip - GQA attention of the block rows over the paged ctx window and
// the block itself, for gfx950.
//
// One workgroup per (sequence, kv head, key chunk). The rep = n_q / n_kv
// query heads of a kv head times the gamma block rows form up to 128 query
// rows, 32 per wave. Keys are the ctx rows [win_start, ctx_len) read through
// the block table from the paged pool, followed by the gamma block rows (K/V
// straight from the QKV output). Every 32-key tile is staged in LDS (K
// row-major, V transposed), FP8 codes widened to bf16 on the way; the global
// loads of tile t + 1 are issued before tile t is computed.
//
// The products are computed transposed so every per-query quantity stays in
// one lane: S^T = K Q^T (MFMA A = 16 keys x 32 dims, B = Q^T), giving lane l
// the scores of query l % 16 for keys 4g + r (g = l / 16); the PV product is
// O^T = V^T P^T, whose B operand is exactly the lane's own probabilities for
// keys {4g..4g+3, 16+4g..16+4g+3} and whose A operand reads V^T for the same
// key set. Online softmax in base 2; the running max is shared across the
// four lane groups with two shuffles, the running sum stays per lane until
// the end. Each workgroup writes an unnormalised partial (O, max, sum); the
// combine kernel merges the chunks of every query row with one wave.
//
// Q and K carry their head dimensions in RoPE pair order (the QKV epilogue and
// the cache use the same order), which leaves every score unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int KT = 32;          // keys per tile
constexpr int GT = 2;           // tiles whose loads are issued together
constexpr int MAX_BT = 64;      // block ids staged per workgroup (chunk <= 1008 keys)

struct Staged {
  uint4 k[2], v[2];
};

template <int D>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int KS = D >= 32 ? D / 32 : 1;  // 32-dim MFMA k-steps
  constexpr int DT = D / 16;                // 16-dim output tiles
  constexpr int KP = D + 8;                 // padded LDS row of K
  constexpr int VP = KT + 8;                // padded LDS row of V^T
  constexpr int ITEMS = KT * (D / 8);       // 8-dim chunks per tile
  constexpr int PER = (ITEMS + 255) / 256;  // chunks per thread (<= 2)
  __shared__ uint16_t Ks[KT][KP];
  __shared__ uint16_t Vt[D][VP];
  __shared__ int32_t s_bt[MAX_BT];

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

  // block ids covering this chunk's ctx rows
  const int pos_lo = sq.win_start + key_lo;
  const int blk_lo = pos_lo >> 4;
  if (key_lo < S_ctx) {
    const int blk_hi = (sq.win_start + min(key_hi, S_ctx) - 1) >> 4;
    for (int i = threadIdx.x; i <= blk_hi - blk_lo; i += blockDim.x) s_bt[i] = sq.bt[blk_lo + i];
  }

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
  __syncthreads();  // s_bt

  const size_t head_stride = (size_t)DFLASH_KV_BLOCK * D;  // one (block, layer, K|V, head) tile
  auto load_tile = [&](int t0, Staged &st) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * 256;
      st.k[i] = z4;
      st.v[i] = z4;
      if (e >= ITEMS) continue;
      const int key = e / (D / 8), dc = (e % (D / 8)) * 8;
      const int kidx = t0 + key;
      if (kidx >= key_hi) continue;
      if (kidx < S_ctx) {
        const int pos = sq.win_start + kidx;
        const int32_t blk = s_bt[(pos >> 4) - blk_lo];
        const size_t base = (((size_t)blk * a.L + a.layer) * 2 * a.n_kv + g) * head_stride + (size_t)(pos & 15) * D + dc;
        const size_t vofs = (size_t)a.n_kv * head_stride;
        if (a.kv_fp8) {
          const uint8_t *p = (const uint8_t *)a.pool;
          const uint2 kc = *(const uint2 *)(p + base), vc = *(const uint2 *)(p + base + vofs);
          st.k[i] = uint4{kc.x, kc.y, 0u, 1u};  // raw codes, widened when staged
          st.v[i] = uint4{vc.x, vc.y, 0u, 1u};
        } else {
          const uint16_t *p = (const uint16_t *)a.pool;
          st.k[i] = *(const uint4 *)(p + base);
          st.v[i] = *(const uint4 *)(p + base + vofs);
        }
      } else {
        const uint16_t *brow = a.qkv + (size_t)(s * a.gamma + (kidx - S_ctx)) * a.ld;
        st.k[i] = *(const uint4 *)(brow + a.k_off + g * D + dc);
        st.v[i] = *(const uint4 *)(brow + a.v_off + g * D + dc);
      }
    }
  };
  auto store_tile = [&](int t0, const Staged &st) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * 256;
      if (e >= ITEMS) continue;
      const int key = e / (D / 8), dc = (e % (D / 8)) * 8;
      const int kidx = t0 + key;
      uint4 kv8 = st.k[i], vv8 = st.v[i];
      if (a.kv_fp8 && kidx < S_ctx && kidx < key_hi) {
        uint2 lo = e4m3x4_to_bf16x4(kv8.x), hi = e4m3x4_to_bf16x4(kv8.y);
        kv8 = uint4{lo.x, lo.y, hi.x, hi.y};
        lo = e4m3x4_to_bf16x4(vv8.x);
        hi = e4m3x4_to_bf16x4(vv8.y);
        vv8 = uint4{lo.x, lo.y, hi.x, hi.y};
      }
      *(uint4 *)&Ks[key][dc] = kv8;
      const uint16_t *vh = (const uint16_t *)&vv8;
#pragma unroll
      for (int q = 0; q < 8; ++q) Vt[dc + q][key] = vh[q];
    }
  };

  // Groups of GT tiles: all global loads of a group are issued together,
  // then its tiles are staged and computed one by one.
  for (int g0 = key_lo; g0 < key_hi; g0 += GT * KT) {
    Staged grp[GT];
#pragma unroll
    for (int t = 0; t < GT; ++t) load_tile(g0 + t * KT, grp[t]);
#pragma unroll
    for (int t = 0; t < GT; ++t) {
    const int t0 = g0 + t * KT;
    if (t0 >= key_hi) break;
    __syncthreads();  // previous tile's readers are done
    store_tile(t0, grp[t]);
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
    for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(a.o_part + (part + q) * D + dt * 16 + 4 * lg) = o[qt][dt];
    if (lg == 0) {
      a.ml_part[(part + q) * 2 + 0] = m_run[qt];
      a.ml_part[(part + q) * 2 + 1] = l_tot;
    }
  }
}

// Merge the key chunks of one query row per wave: lane s < nsplit reads
// chunk s's (max, sum); the weights exp2(m_s - M) are shared by shuffles and
// every lane accumulates its dimensions over the chunks in order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int n_seq) {
  constexpr int DPL = D >= 64 ? D / 64 : 1;  // dims per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int R = a.rep * a.gamma;
  const int row = blockIdx.x * 4 + wave;  // (s, g, q)
  if (row >= n_seq * a.n_kv * R) return;
  const int q = row % R, g = (row / R) % a.n_kv, s = row / (R * a.n_kv);
  const AttnSeq sq = a.seq[s];
  const int S = sq.ctx_len - sq.win_start + a.gamma;
  const int nsplit = (S + a.chunk - 1) / a.chunk;  // <= 64
  const size_t base = (size_t)(s * a.n_kv + g) * a.max_splits;
  float m = -__builtin_huge_valf(), l = 0.0f;
  if (lane < nsplit) {
    m = a.ml_part[((base + lane) * R + q) * 2];
    l = a.ml_part[((base + lane) * R + q) * 2 + 1];
  }
  float M = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, WAVE));
  const float w = lane < nsplit ? fast_exp2(m - M) : 0.0f;
  const float den = wave_sum(w * l);
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  const bool active = D >= 64 || lane < D;
#pragma unroll 8
  for (int c = 0; c < nsplit; ++c) {
    const float wc = __shfl(w, c, WAVE);
    const float *op = a.o_part + ((base + c) * R + q) * D;
#pragma unroll
    for (int i = 0; i < DPL; ++i)
      if (active) acc[i] += wc * op[lane + 64 * i];
  }
  const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
  uint16_t *out = a.out + (size_t)(s * a.gamma + j) * a.out_ld + hq * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i)
    if (active) out[lane + 64 * i] = f32_to_bf16(acc[i] / den);
}

}  // namespace

int attn_max_chunk_blocks() { return MAX_BT; }

hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s) {
  if (a.chunk % KT || (a.chunk / DFLASH_KV_BLOCK) + 2 > MAX_BT || a.max_splits > 64) return hipErrorInvalidValue;
  dim3 grid(a.max_splits, a.n_kv, n_seq), block(256);
  const int rows = n_seq * a.n_kv * a.rep * a.gamma;
  dim3 cgrid((rows + 3) / 4);
  switch (a.head_dim) {
    case 16:
      hipLaunchKernelGGL(k_attn<16>, grid, block, 0, s, a);
      hipLaunchKernelGGL(k_attn_combine<16>, cgrid, block, 0, s, a, n_seq);
      break;
    case 32:
      hipLaunchKernelGGL(k_attn<32>, grid, block, 0, s, a);
      hipLaunchKernelGGL(k_attn_combine<32>, cgrid, block, 0, s, a, n_seq);
      break;
    case 64:
      hipLaunchKernelGGL(k_attn<64>, grid, block, 0, s, a);
      hipLaunchKernelGGL(k_attn_combine<64>, cgrid, block, 0, s, a, n_seq);
      break;
    case 128:
      hipLaunchKernelGGL(k_attn<128>, grid, block, 0, s, a);
      hipLaunchKernelGGL(k_attn_combine<128>, cgrid, block, 0, s, a, n_seq);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dflash
