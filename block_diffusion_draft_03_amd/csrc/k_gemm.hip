// k_gemm.hip - weight-streaming MFMA GEMMs of the DFlash head for gfx950.
//
// All contractions of the propose path have few activation rows (gamma per
// sequence) against large bf16 (or E4M3) weight matrices, so they are bound
// by streaming the weights from HBM once. The kernels compute the transposed
// product D^T = W A^T with v_mfma_f32_16x16x32_bf16: the MFMA's A operand is
// 16 weight rows, its B operand 16 activation rows. For k-step c of a
// 128-wide K step, lane l (row l % 16, group g = l / 16) loads the 8 values
// at k0 + 32c + 8g, so one load instruction covers 16 weight rows x 64
// contiguous bytes. A lane then holds outputs (rows) 4g .. 4g+3 of a tile
// for activation row l % 16.
//
// Work unit: 16 * TN consecutive weight rows. The NW waves of a workgroup
// split the unit's K range into NW contiguous parts and reduce through LDS in
// wave order. A GEMM may also be split over K across workgroups; then every
// split writes its partial sums and a separate kernel (k_resid_norm) adds
// them in split order. Every reduction order is fixed, so results are
// deterministic and a row's result does not depend on the other rows.
//
// Epilogues are lane-local because the build repacks weight rows in pairs:
// Q and K rows of a head are ordered (dim i, dim i + d/2) for i = 0 .. d/2-1,
// and the MLP weight alternates gate and up rows. Lane rows 4g, 4g+1 and
// 4g+2, 4g+3 are therefore a RoPE pair (or a gate/up pair). Q and K stay in
// that pair order everywhere inside the library (attention is invariant to a
// common permutation of the Q and K dimensions).
//
// With ANORM the A operand is the RMSNorm of the fp32 residual stream,
// formed while loading: bf16(h * r * gain) with r = 1 / sqrt(mean(h^2) + eps)
// from per-unit sums of squares that the producing GEMM wrote.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

template <int MT, int TN>
struct Frag {
  uint4 w[TN][4];
  uint4 a[MT][4];
};

// 8 bf16 of normalised activations: h[k .. k+8) * r * gain[k .. k+8)
__device__ __forceinline__ uint4 norm_bf16x8(const float *h, const float *gain, float r) {
  const float4 x0 = *(const float4 *)h, x1 = *(const float4 *)(h + 4);
  const float4 g0 = *(const float4 *)gain, g1 = *(const float4 *)(gain + 4);
  uint4 o;
  o.x = pack_bf16x2(x0.x * r * g0.x, x0.y * r * g0.y);
  o.y = pack_bf16x2(x0.z * r * g0.z, x0.w * r * g0.w);
  o.z = pack_bf16x2(x1.x * r * g1.x, x1.y * r * g1.y);
  o.w = pack_bf16x2(x1.z * r * g1.z, x1.w * r * g1.w);
  return o;
}

struct AOperand {
  const uint16_t *a;   // bf16 activations (plain)
  const float *h;      // fp32 residual (ANORM)
  const float *gain;   // ANORM
  const float *rinv;   // ANORM: per activation row (LDS)
  int lda;
};

template <int MT, int TN, bool WFP8, bool ANORM, bool TILED = false>
__device__ __forceinline__ void load_step(Frag<MT, TN> &f, const void *__restrict__ Wv, int K, const int (&wrow)[TN],
                                          const AOperand &A, const int (&arow)[MT], int k0, int ke, int g) {
  const uint4 z = {0u, 0u, 0u, 0u};
  if constexpr (TILED && !WFP8) {
    // tile-major weights: 16-row tile, 128-wide step, k-group c, lane -> 8 values
    const uint16_t *W = (const uint16_t *)Wv;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint16_t *p = W + (((size_t)(wrow[t] >> 4) * ((K + 127) >> 7) + (k0 >> 7)) * 4 * 64 + lane) * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) f.w[t][c] = (k0 + 32 * c + 8 * g < ke) ? *(const uint4 *)(p + c * 64 * 8) : z;
    }
  } else if constexpr (TILED && WFP8) {
    // tile-major E4M3: pair j of lane l = codes of k-groups 2j and 2j + 1
    const uint8_t *W = (const uint8_t *)Wv;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint8_t *p = W + (((size_t)(wrow[t] >> 4) * ((K + 127) >> 7) + (k0 >> 7)) * 2 * 64 + lane) * 16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 q = z;
        if (k0 + 64 * j + 8 * g < ke) q = *(const uint4 *)(p + j * 64 * 16);
        uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
        f.w[t][2 * j] = uint4{lo.x, lo.y, hi.x, hi.y};
        lo = e4m3x4_to_bf16x4(q.z);
        hi = e4m3x4_to_bf16x4(q.w);
        f.w[t][2 * j + 1] = (k0 + 64 * j + 32 + 8 * g < ke) ? uint4{lo.x, lo.y, hi.x, hi.y} : z;
      }
    }
  } else if constexpr (!WFP8) {
    const uint16_t *W = (const uint16_t *)Wv;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint16_t *p = W + (size_t)wrow[t] * K + k0 + 8 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) f.w[t][c] = (k0 + 32 * c + 8 * g < ke) ? *(const uint4 *)(p + 32 * c) : z;
    }
  } else {
    const uint8_t *W = (const uint8_t *)Wv;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint8_t *p = W + (size_t)wrow[t] * K + k0 + 8 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint2 q = {0u, 0u};
        if (k0 + 32 * c + 8 * g < ke) q = *(const uint2 *)(p + 32 * c);
        const uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
        f.w[t][c] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = k0 + 32 * c + 8 * g;
      if (k >= ke) {
        f.a[mt][c] = z;
      } else if constexpr (ANORM) {
        f.a[mt][c] = norm_bf16x8(A.h + (size_t)arow[mt] * A.lda + k, A.gain + k, A.rinv[mt * 16 + (threadIdx.x & 15)]);
      } else {
        f.a[mt][c] = *(const uint4 *)(A.a + (size_t)arow[mt] * A.lda + k);
      }
    }
  }
}

template <int MT, int TN>
__device__ __forceinline__ void mma_step(const Frag<MT, TN> &f, f32x4 (&acc)[TN][MT]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[t][mt] = mfma16x16x32(as_bf16x8(f.w[t][c]), as_bf16x8(f.a[mt][c]), acc[t][mt]);
}

template <int MT, int TN>
__device__ __forceinline__ void zero(f32x4 (&acc)[TN][MT]) {
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc[t][mt][r] += sum over k in [kb, ke) of W[row0 + 16t + 4g + r, k] * A[mt*16 + l%16, k]
// The range is walked in batches of ST 128-wide steps: all loads of a batch
// are issued before its MFMAs (steps past ke load nothing and add zeros), so
// a wave keeps ST steps of weight rows in flight.
template <int MT, int TN, int ST, bool WFP8, bool ANORM, bool TILED = false>
__device__ __forceinline__ void stream_rows(const void *__restrict__ W, int N, int K, const AOperand &A, int M,
                                            int row0, int kb, int ke, f32x4 (&acc)[TN][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  int wrow[TN], arow[MT];
#pragma unroll
  for (int t = 0; t < TN; ++t) wrow[t] = min(row0 + 16 * t + r16, N - 1);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + r16, M - 1);
  for (int k0 = kb; k0 < ke; k0 += 128 * ST) {
    Frag<MT, TN> f[ST];
#pragma unroll
    for (int s = 0; s < ST; ++s) load_step<MT, TN, WFP8, ANORM, TILED>(f[s], W, K, wrow, A, arow, k0 + 128 * s, ke, g);
#pragma unroll
    for (int s = 0; s < ST; ++s) mma_step<MT, TN>(f[s], acc);
  }
}

// Sum the NW waves' partials in wave order; the result ends in wave 0.
template <int MT, int TN, int NW>
__device__ __forceinline__ void wave_reduce(f32x4 (&acc)[TN][MT], float *red) {
  if constexpr (NW == 1) return;
  constexpr int V = TN * MT * 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave - 1) * V + (t * MT + mt) * 4 + r) * 64 + lane] = acc[t][mt][r];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][mt][r] += red[((w - 1) * V + (t * MT + mt) * 4 + r) * 64 + lane];
  }
}

// Per-row inverse RMS from the producer's per-unit sums of squares, into LDS.
template <int MT>
__device__ __forceinline__ void load_rinv(const GemmArgs &ga, float *rinv, float *tmp) {
  // thread t: row t % (16 MT), units t / (16 MT), + stride
  constexpr int R = 16 * MT;
  const int nthr = blockDim.x;
  const int row = threadIdx.x % R, lane_u = threadIdx.x / R, nu = nthr / R;
  float s = 0.0f;
  if (row < ga.M)
    for (int u = lane_u; u < ga.ss_units; u += nu) s += ga.ss_in[(size_t)u * ga.ss_ld + ga.ss_row0 + row];
  tmp[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < R) {
    float t = 0.0f;
    for (int i = 0; i < nu; ++i) t += tmp[i * R + threadIdx.x];
    rinv[threadIdx.x] = 1.0f / sqrtf(t / (float)ga.K + ga.eps);
  }
  __syncthreads();
}

template <int MT, int TN, int NW, int ST, int EPI, bool ANORM, bool TILED = false>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmArgs ga, EpiArgs ea) {
  __shared__ float red[(NW > 1 ? NW - 1 : 1) * TN * MT * 4 * 64];
  __shared__ float rinv[16 * MT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int row0 = blockIdx.x * 16 * TN;
  const int kb = blockIdx.y * ga.kslice, ke = min(ga.K, kb + ga.kslice);
  const int steps = (ke - kb + 127) / 128;
  const int s0 = (steps * wave) / NW, s1 = (steps * (wave + 1)) / NW;
  AOperand A{ga.A, ga.H, ga.gain, rinv, ga.lda};
  if constexpr (ANORM) load_rinv<MT>(ga, rinv, red);
  f32x4 acc[TN][MT];
  zero<MT, TN>(acc);
  stream_rows<MT, TN, ST, false, ANORM, TILED>(ga.W, ga.N, ga.K, A, ga.M, row0, kb + 128 * s0, min(ke, kb + 128 * s1),
                                               acc);
  wave_reduce<MT, TN, NW>(acc, red);
  if (wave != 0) return;

  float ss_acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) ss_acc[mt] = 0.0f;
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      const int n = row0 + 16 * t + 4 * g;  // first of this lane's 4 rows
      const bool ok = m < ga.M && n < ga.N;
      const f32x4 v = acc[t][mt];
      if constexpr (EPI == EPI_F32 || EPI == EPI_PARTIAL) {
        if (ok) {
          float *o = EPI == EPI_F32 ? ea.out_f32 + (size_t)m * ea.ldo + n
                                    : ea.out_f32 + ((size_t)blockIdx.y * ea.ld_split + m) * ea.ldo + n;
          *(f32x4 *)o = v;
        }
      } else if constexpr (EPI == EPI_RESID) {
        // h += acc, and this unit's sum of squares of the new h per row
        float ss = 0.0f;
        if (ok) {
          float *o = ea.out_f32 + (size_t)m * ea.ldo + n;
          const f32x4 x = v + *(const f32x4 *)o;
          *(f32x4 *)o = x;
          ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
        ss += __shfl_xor(ss, 16, WAVE);
        ss += __shfl_xor(ss, 32, WAVE);
        ss_acc[mt] += ss;
      } else if constexpr (EPI == EPI_SWIGLU) {
        // rows (gate_i, up_i, gate_i+1, up_i+1) with i = n / 2
        if (ok)
          *(uint32_t *)(ea.out_bf16 + (size_t)m * ea.ldo + n / 2) = pack_bf16x2(silu(v[0]) * v[1], silu(v[2]) * v[3]);
      } else if constexpr (EPI == EPI_QKV_ROPE) {
        if (!ok) continue;
        const int half = ea.head_dim >> 1;
        float y[4] = {v[0], v[1], v[2], v[3]};
        if (n < ea.q_dim + ea.kv_dim) {
          const int p = (n % ea.head_dim) >> 1;  // pair index of rows n, n+1
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float2 c = ea.cs[(size_t)m * half + p + q];
            const float x0 = v[2 * q], x1 = v[2 * q + 1];
            y[2 * q] = x0 * c.x - x1 * c.y;
            y[2 * q + 1] = x1 * c.x + x0 * c.y;
          }
        }
        uint2 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        *(uint2 *)(ea.out_bf16 + (size_t)m * ea.ldo + n) = o;
      } else {  // EPI_KV_SCATTER: columns [K0 | V0 | K1 | V1 ...], K in pair order
        if (!ok) continue;
        const int d = ea.head_dim;
        const int kv_dim = ea.n_kv * d;
        const int l = n / (2 * kv_dim), rem = n % (2 * kv_dim);
        const int kv = rem / kv_dim, hd = (rem % kv_dim) / d, j = n % d;
        const int pos = ea.row_pos[m];
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
        const int32_t blk = ea.row_bt[m][pos >> 4];
        const size_t off = ((((size_t)blk * ea.L + l) * 2 + kv) * ea.n_kv + hd) * (size_t)(DFLASH_KV_BLOCK * d) +
                           (size_t)(pos & 15) * d + j;
        if (ea.kv_fp8) {
          const float sc = ea.kv_scale[(l * 2 + kv) * ea.n_kv + hd];
          uint32_t w = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) w |= (uint32_t)f32_to_e4m3(y[r] / sc) << (8 * r);
          *(uint32_t *)((uint8_t *)ea.pool + off) = w;
        } else {
          uint2 o;
          o.x = pack_bf16x2(y[0], y[1]);
          o.y = pack_bf16x2(y[2], y[3]);
          *(uint2 *)((uint16_t *)ea.pool + off) = o;
        }
      }
    }
  if constexpr (EPI == EPI_RESID) {
    if (ea.ss_out && g == 0)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16;
        if (m < ga.M) ea.ss_out[(size_t)blockIdx.x * ea.ss_ld + ea.ss_row0 + m] = ss_acc[mt];
      }
  }
}

// Split-K finish for the residual GEMMs: one workgroup per activation row
// adds the splits' partial sums (in split order) to the fp32 residual row,
// then writes the RMSNorm of the new row (with `gain`) as bf16 and, when
// asked, the row's sum of squares.
__global__ __launch_bounds__(256) void k_resid_norm(ResidNormArgs a) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  float *hr = a.h + (size_t)m * a.n;
  float ss = 0.0f;
  for (int i = threadIdx.x * 4; i < a.n; i += blockDim.x * 4) {
    f32x4 x = a.init_zero ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4 *)(hr + i);
    for (int s = 0; s < a.splits; ++s) x += *(const f32x4 *)(a.part + ((size_t)s * a.ld_split + m) * a.n + i);
    *(f32x4 *)(hr + i) = x;
    ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
  ss = block_sum(ss, red);
  if (!a.out) return;
  const float r = 1.0f / sqrtf(ss / (float)a.n + a.eps);
  uint16_t *o = a.out + (size_t)m * a.n;
  for (int i = threadIdx.x * 4; i < a.n; i += blockDim.x * 4) {
    const f32x4 x = *(const f32x4 *)(hr + i);
    const float4 gg = *(const float4 *)(a.gain + i);
    uint2 w;
    w.x = pack_bf16x2(x[0] * r * gg.x, x[1] * r * gg.y);
    w.y = pack_bf16x2(x[2] * r * gg.z, x[3] * r * gg.w);
    *(uint2 *)(o + i) = w;
  }
}

// ------------------------------------------------------------- LM head ----
// Stage 1: every wave streams (16 * TN)-row vocab units u = wave_id,
// wave_id + total_waves, ... over the full K and keeps, per lane, a running
// (max, argmax, sum exp) of its activation row over the vocab entries it sees
// (masked entries skipped). Lanes, then the workgroup's waves, are merged in
// a fixed order; one partial per workgroup and row is written.
template <int MT, int TN, int ST, bool WFP8, bool TILED = false>
__global__ __launch_bounds__(256) void k_lm_head(LmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  constexpr int UNIT = 16 * TN;
  const int units = (a.V + UNIT - 1) / UNIT;
  ArgState st[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arg_init(st[mt]);
  const int32_t *mask_row[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r16, a.M - 1);
    mask_row[mt] = a.bitmask ? a.bitmask + (size_t)((a.row0 + m) / a.gamma) * a.words : nullptr;
  }
  AOperand A{a.z, nullptr, nullptr, nullptr, a.K};
  const int nw = gridDim.x * 4;
  for (int u = blockIdx.x * 4 + wave; u < units; u += nw) {
    const int row0 = u * UNIT;
    f32x4 acc[TN][MT];
    zero<MT, TN>(acc);
    stream_rows<MT, TN, ST, WFP8, false, TILED>(a.W, a.V, a.K, A, a.M, row0, 0, a.K, acc);
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = row0 + 16 * t + 4 * g + r;
        if (v >= a.V) continue;
        const float sc = WFP8 ? a.scale[v] : 1.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float x = acc[t][mt][r] * sc;
          const int m = mt * 16 + r16;
          if (a.logits && m < a.M) a.logits[(size_t)m * a.V + v] = x;
          if (mask_row[mt] && !((((uint32_t)mask_row[mt][v >> 5]) >> (v & 31)) & 1u)) continue;
          arg_push(st[mt], x, (uint32_t)v);
        }
      }
  }
  __shared__ float s_mx[4][MT * 16], s_se[4][MT * 16];
  __shared__ uint32_t s_idx[4][MT * 16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st[mt] = arg_merge(st[mt], arg_shfl_xor(st[mt], 16));
    st[mt] = arg_merge(st[mt], arg_shfl_xor(st[mt], 32));
    if (g == 0) {
      s_mx[wave][mt * 16 + r16] = st[mt].mx;
      s_se[wave][mt * 16 + r16] = st[mt].se;
      s_idx[wave][mt * 16 + r16] = st[mt].idx;
    }
  }
  __syncthreads();
  if (threadIdx.x < MT * 16) {
    const int m = threadIdx.x;
    ArgState r;
    r.mx = s_mx[0][m];
    r.se = s_se[0][m];
    r.idx = s_idx[0][m];
    for (int w = 1; w < 4; ++w) {
      ArgState o;
      o.mx = s_mx[w][m];
      o.se = s_se[w][m];
      o.idx = s_idx[w][m];
      r = arg_merge(r, o);
    }
    if (m < a.M) {
      const size_t o = (size_t)blockIdx.x * a.ld_part + a.row0 + m;
      a.part_mx[o] = r.mx;
      a.part_se[o] = r.se;
      a.part_idx[o] = r.idx;
    }
  }
}

// Stage 2: one workgroup per block row merges the row's P partials (fixed
// tree order) and writes its id and top-1 probability; the last row of a
// sequence to finish (atomic ticket) writes the chain confidence
// min(p1) over rows 1..num_drafts.
__global__ __launch_bounds__(256) void k_lm_finish(LmFinishArgs a) {
  __shared__ float s_mx[256], s_se[256];
  __shared__ uint32_t s_idx[256];
  const int m = blockIdx.x, seq = m / a.gamma;
  ArgState st;
  arg_init(st);
  constexpr int PER = 4;
  ArgState q[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = threadIdx.x + i * blockDim.x;
    arg_init(q[i]);
    if (p < a.P) {
      const size_t o = (size_t)p * a.M + m;
      q[i].mx = a.part_mx[o];
      q[i].se = a.part_se[o];
      q[i].idx = a.part_idx[o];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) st = arg_merge(st, q[i]);
  for (int p = threadIdx.x + PER * blockDim.x; p < a.P; p += blockDim.x) {
    const size_t o = (size_t)p * a.M + m;
    ArgState x;
    x.mx = a.part_mx[o];
    x.se = a.part_se[o];
    x.idx = a.part_idx[o];
    st = arg_merge(st, x);
  }
  s_mx[threadIdx.x] = st.mx;
  s_se[threadIdx.x] = st.se;
  s_idx[threadIdx.x] = st.idx;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      ArgState x, y;
      x.mx = s_mx[threadIdx.x];
      x.se = s_se[threadIdx.x];
      x.idx = s_idx[threadIdx.x];
      y.mx = s_mx[threadIdx.x + w];
      y.se = s_se[threadIdx.x + w];
      y.idx = s_idx[threadIdx.x + w];
      x = arg_merge(x, y);
      s_mx[threadIdx.x] = x.mx;
      s_se[threadIdx.x] = x.se;
      s_idx[threadIdx.x] = x.idx;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const bool none = s_mx[0] == -__builtin_huge_valf();
    const float p1 = none ? 0.0f : 1.0f / s_se[0];
    a.ids[m] = none ? DFLASH_NO_TOKEN : s_idx[0];
    if (a.row_prob) a.row_prob[m] = p1;
    a.p1[m] = p1;
    __threadfence();
    const int prev = atomicAdd(&a.counters[seq], 1);
    if (prev == a.gamma - 1) {
      __threadfence();
      float c = a.p1[seq * a.gamma + 1];
      for (int j = 2; j <= a.num_drafts; ++j) c = fminf(c, a.p1[seq * a.gamma + j]);
      a.conf[seq] = c;
      a.counters[seq] = 0;
    }
  }
}

template <int MT, int TN, int NW, int ST, bool ANORM>
hipError_t launch_cfg(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  dim3 grid((g.N + 16 * TN - 1) / (16 * TN), g.splits), block(NW * 64);
#define DFL_CASE(E)                                                                         \
  case E:                                                                                   \
    hipLaunchKernelGGL((k_gemm<MT, TN, NW, ST, E, ANORM, true>), grid, block, 0, s, g, e);      \
    break;
  switch (epi) {
    DFL_CASE(EPI_F32)
    DFL_CASE(EPI_RESID)
    DFL_CASE(EPI_SWIGLU)
    DFL_CASE(EPI_QKV_ROPE)
    DFL_CASE(EPI_KV_SCATTER)
    DFL_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef DFL_CASE
  return hipGetLastError();
}

template <int MT, bool ANORM>
hipError_t launch_mt(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  // configurations chosen by gemm_plan
  if (g.tn == 1 && g.nw == 4 && g.st == 4) return launch_cfg<MT, 1, 4, 4, ANORM>(epi, g, e, s);
  if (g.tn == 2 && g.nw == 4 && g.st == 4) return launch_cfg<MT, 2, 4, 4, ANORM>(epi, g, e, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Measured on MI355X over the propose shapes with tiled weights: 4 waves per
// workgroup with 4 steps in flight each; 32-row units for wide matrices;
// 16-row units split over K (up to 4 ways) for the N = hidden GEMMs.
GemmPlan gemm_plan(int N, int K, bool allow_split) {
  GemmPlan p;
  const int steps = (K + 127) / 128;
  p.tn = N > 4096 ? 2 : 1;
  p.nw = 4;
  p.st = 4;
  p.splits = 1;
  const int units = (N + 16 * p.tn - 1) / (16 * p.tn);
  if (allow_split && units < 256) {
    int want = (256 + units - 1) / units;
    if (want > 4) want = 4;
    if (want > steps) want = steps;
    p.splits = want < 1 ? 1 : want;
  }
  const int per = (steps + p.splits - 1) / p.splits;
  p.kslice = per * 128;
  p.splits = (K + p.kslice - 1) / p.kslice;
  return p;
}

hipError_t launch_gemm(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  if (g.M < 1 || g.M > GEMM_MAX_ROWS || g.splits < 1) return hipErrorInvalidValue;
  if (g.splits > 1 && epi != EPI_PARTIAL) return hipErrorInvalidValue;
  const int mt = g.M <= 16 ? 1 : (g.M <= 32 ? 2 : 4);
  if (g.H) return hipErrorInvalidValue;  // the norm-fused A operand is not used by the library
  return mt == 1 ? launch_mt<1, false>(epi, g, e, s) : mt == 2 ? launch_mt<2, false>(epi, g, e, s)
                                                               : launch_mt<4, false>(epi, g, e, s);
}

hipError_t launch_resid_norm(const ResidNormArgs &a, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_resid_norm, dim3(M), dim3(256), 0, s, a);
  return hipGetLastError();
}

int lm_parts(int V) {
  // one workgroup per CU measured best for the 248k x 2048 head
  const int units = (V + 31) / 32;
  const int wgs = (units + 3) / 4;
  return wgs < 256 ? wgs : 256;
}

hipError_t launch_lm_head(bool w_fp8, const LmArgs &a, hipStream_t s) {
  if (a.M < 1 || a.M > GEMM_MAX_ROWS) return hipErrorInvalidValue;
  const int mt = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  dim3 grid(lm_parts(a.V)), block(256);
  if (w_fp8) {
    if (mt == 1) hipLaunchKernelGGL((k_lm_head<1, 2, 2, true, true>), grid, block, 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL((k_lm_head<2, 2, 2, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_lm_head<4, 2, 2, true, true>), grid, block, 0, s, a);
  } else {
    if (mt == 1) hipLaunchKernelGGL((k_lm_head<1, 2, 2, false, true>), grid, block, 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL((k_lm_head<2, 2, 2, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_lm_head<4, 2, 2, false, true>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_lm_finish(const LmFinishArgs &a, int n_seq, hipStream_t s) {
  hipLaunchKernelGGL(k_lm_finish, dim3(n_seq * a.gamma), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
