// k_gemm.hip - weight-streaming MFMA GEMMs of the DFlash head for gfx950.
//
// A propose forward has few activation rows (gamma per sequence) against
// large bf16 (or E4M3) weight matrices, so these kernels are bound by
// streaming the weights from HBM once. They compute the transposed product
// D^T = W A^T with v_mfma_f32_16x16x32_bf16: the MFMA's A operand is 16
// weight rows, its B operand 16 activation rows. For k-step c of a 128-wide
// K step, lane l (row l % 16, group g = l / 16) loads the 8 values at
// k0 + 32c + 8g, so one load instruction covers 16 weight rows x 64
// contiguous bytes. A lane then holds outputs (rows) 4g .. 4g+3 of a tile
// for activation row l % 16.
//
// Work unit: 16 * TN consecutive weight rows. The NW waves of a workgroup
// split the unit's K range into NW contiguous parts and reduce through LDS in
// wave order. A GEMM may also be split over K across workgroups; then every
// split writes its partial sums and a separate kernel (k_resid_norm) adds
// them in split order. Every reduction order is fixed, so results are
// deterministic and a row's result does not depend on the other rows. The
// tiled kernels for many rows (k_bgemm.hip) sum each K slice in one pass, so
// their layer GEMMs agree with these to rounding; their LM head, which sums
// K in one pass like the one here, is bit-identical.
#include "common.hpp"
#include "gemm_epi.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int NUM_CUS = 256;  // compute units of the MI355X

template <int MT, int TN>
struct Frag {
  uint4 w[TN][4];
  uint4 a[MT][4];
  uint4 q8[TN][2];  // tile-major E4M3: raw codes, widened into w just before the products
};

template <int MT, int TN, bool WFP8, bool TILED = false>
__device__ __forceinline__ void load_step(Frag<MT, TN> &f, const void *__restrict__ Wv, int K, const int (&wrow)[TN],
                                          const uint16_t *__restrict__ A, int lda, const int (&arow)[MT], int k0,
                                          int ke, int g) {
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
    // tile-major E4M3: pair j of lane l = codes of k-groups 2j and 2j + 1,
    // kept raw (widen_e4m3 converts them after the whole batch is issued, so
    // the loads stay in flight together); columns past K are zero codes in
    // the tiled copy
    const uint8_t *W = (const uint8_t *)Wv;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint8_t *p = W + (((size_t)(wrow[t] >> 4) * ((K + 127) >> 7) + (k0 >> 7)) * 2 * 64 + lane) * 16;
#pragma unroll
      for (int j = 0; j < 2; ++j) f.q8[t][j] = (k0 + 64 * j + 8 * g < ke) ? *(const uint4 *)(p + j * 64 * 16) : z;
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
      f.a[mt][c] = k < ke ? *(const uint4 *)(A + (size_t)arow[mt] * lda + k) : z;
    }
  }
}

template <int MT, int TN>
__device__ __forceinline__ void widen_e4m3(Frag<MT, TN> &f) {
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 q = f.q8[t][j];
      uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
      f.w[t][2 * j] = uint4{lo.x, lo.y, hi.x, hi.y};
      lo = e4m3x4_to_bf16x4(q.z);
      hi = e4m3x4_to_bf16x4(q.w);
      f.w[t][2 * j + 1] = uint4{lo.x, lo.y, hi.x, hi.y};
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
template <int MT, int TN, int ST, bool WFP8, bool TILED = false>
__device__ __forceinline__ void stream_rows(const void *__restrict__ W, int N, int K, const uint16_t *__restrict__ A,
                                            int lda, int M, int row0, int kb, int ke, f32x4 (&acc)[TN][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  int wrow[TN], arow[MT];
#pragma unroll
  for (int t = 0; t < TN; ++t) wrow[t] = min(row0 + 16 * t + r16, N - 1);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + r16, M - 1);
  for (int k0 = kb; k0 < ke; k0 += 128 * ST) {
    Frag<MT, TN> f[ST];
#pragma unroll
    for (int s = 0; s < ST; ++s) load_step<MT, TN, WFP8, TILED>(f[s], W, K, wrow, A, lda, arow, k0 + 128 * s, ke, g);
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      if constexpr (TILED && WFP8) widen_e4m3<MT, TN>(f[s]);
      mma_step<MT, TN>(f[s], acc);
    }
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

// r[m] = 1 / sqrt(sum_u ss[u * ld + m] / n + eps) for the R = 16 MT rows of
// the launch, into LDS: every thread sums a strided subset of the units of
// one row, the subsets are added in a fixed order. The first RS_PRE loads of
// every thread are issued by row_scale_issue (before the weight stream) and
// consumed by row_scale_finish (after it).
constexpr int RS_PRE = 8;

template <int MT>
__device__ __forceinline__ void row_scale_issue(const RowScale &rs, int M, float (&v)[RS_PRE]) {
  constexpr int R = 16 * MT;
  const int row = threadIdx.x % R, grp = threadIdx.x / R, ngrp = blockDim.x / R;
#pragma unroll
  for (int i = 0; i < RS_PRE; ++i) {
    const int u = grp + i * ngrp;
    v[i] = (row < M && u < rs.units) ? rs.ss[(size_t)u * rs.ld + row] : 0.0f;
  }
}

template <int MT>
__device__ __forceinline__ void row_scale_finish(const RowScale &rs, int M, int n, const float (&v)[RS_PRE],
                                                 float *rinv, float *tmp) {
  constexpr int R = 16 * MT;
  const int row = threadIdx.x % R, grp = threadIdx.x / R, ngrp = blockDim.x / R;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < RS_PRE; ++i) s += v[i];
  if (row < M)
    for (int u = grp + RS_PRE * ngrp; u < rs.units; u += ngrp) s += rs.ss[(size_t)u * rs.ld + row];
  __syncthreads();
  tmp[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < R) {
    float t = 0.0f;
    for (int i = 0; i < ngrp; ++i) t += tmp[i * R + threadIdx.x];
    rinv[threadIdx.x] = 1.0f / sqrtf(t / (float)n + rs.eps);
  }
  __syncthreads();
}

template <int MT>
__device__ __forceinline__ void load_row_scale(const RowScale &rs, int M, int n, float *rinv, float *tmp) {
  float v[RS_PRE];
  row_scale_issue<MT>(rs, M, v);
  row_scale_finish<MT>(rs, M, n, v, rinv, tmp);
}

// Split finish of a residual GEMM (EPI_PARTIAL with ea.tile_ctr), wave 0 of
// each workgroup: publish this split's partial with write-through stores,
// count the unit's splits, and in the last one add the splits in split order
// onto the residual, write the gain-scaled bf16 row part and the unit's per-row
// sums of squares.
template <int MT, int TN>
__device__ __forceinline__ void finish_residual(const GemmArgs &ga, const EpiArgs &ea, const f32x4 (&acc)[TN][MT],
                                                int row0) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int split = blockIdx.y, splits = gridDim.y;
  // the residual part and the gain are final before this launch: every split
  // loads them ahead of the split count, off the critical path of the last one
  f32x4 hx[TN][MT];
  float4 gg[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = min(row0 + 16 * t + 4 * g, ga.N - 4);
    gg[t] = *(const float4 *)(ea.res_gain + n);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) hx[t][mt] = *(const f32x4 *)(ea.res_h + (size_t)min(mt * 16 + r16, ga.M - 1) * ga.N + n);
  }
  if (splits > 1) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16, n = row0 + 16 * t + 4 * g;
        if (m >= ga.M || n >= ga.N) continue;
        float *o = ea.out_f32 + ((size_t)split * ea.ld_split + m) * ea.ldo + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) __hip_atomic_store(o + r, acc[t][mt][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    __builtin_amdgcn_s_waitcnt(0x0F70 & ~0xF);  // vmcnt(0): the partial is written through
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(&ea.tile_ctr[blockIdx.x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, WAVE);
    if (prev != splits - 1) return;
    if (lane == 0) __hip_atomic_store(&ea.tile_ctr[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float ss[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) ss[mt] = 0.0f;
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16, n = row0 + 16 * t + 4 * g;
      if (m >= ga.M || n >= ga.N) continue;
      f32x4 x = hx[t][mt];
      for (int sp = 0; sp < splits; ++sp) {
        if (sp == split) {
          x += acc[t][mt];
        } else {
          const float *o = ea.out_f32 + ((size_t)sp * ea.ld_split + m) * ea.ldo + n;
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] += __hip_atomic_load(o + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      *(f32x4 *)(ea.res_h + (size_t)m * ga.N + n) = x;
      *(uint2 *)(ea.res_act + (size_t)m * ga.N + n) =
          uint2{pack_bf16x2(x[0] * gg[t].x, x[1] * gg[t].y), pack_bf16x2(x[2] * gg[t].z, x[3] * gg[t].w)};
      ss[mt] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float v = ss[mt];
    v += __shfl_xor(v, 16, WAVE);
    v += __shfl_xor(v, 32, WAVE);
    const int m = mt * 16 + r16;
    if (g == 0 && m < ga.M) ea.ss_out[(size_t)blockIdx.x * ea.ss_ld + m] = v;
  }
}

// WFP8: W is a tiled E4M3 matrix, widened to bf16 in registers; output
// row n of the product is scaled by ga.wscale[n] before any epilogue.
template <int MT, int TN, int NW, int ST, int EPI, bool TILED = false, bool WFP8 = false>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmArgs ga, EpiArgs ea) {
  __shared__ float red[(NW > 1 ? NW - 1 : 1) * TN * MT * 4 * 64 > 256 ? (NW > 1 ? NW - 1 : 1) * TN * MT * 4 * 64 : 256];
  __shared__ float rinv[16 * MT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int row0 = blockIdx.x * 16 * TN;
  const int kb = blockIdx.y * ga.kslice, ke = min(ga.K, kb + ga.kslice);
  const int steps = (ke - kb + 127) / 128;
  const int s0 = (steps * wave) / NW, s1 = (steps * (wave + 1)) / NW;
  float rs_v[RS_PRE];
  if (ga.rs.ss) row_scale_issue<MT>(ga.rs, ga.M, rs_v);
  // wave 0 writes the epilogue: its RoPE (cos, sin) pairs are loaded now
  float4 cs4[TN][MT];
  if constexpr (EPI == EPI_QKV_ROPE) {
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          cs4[t][mt] = qkv_cs(min(mt * 16 + r16, ga.M - 1), min(row0 + 16 * t + 4 * g, ga.N - 4), ea);
    }
  }
  f32x4 acc[TN][MT];
  zero<MT, TN>(acc);
  stream_rows<MT, TN, ST, WFP8, TILED>(ga.W, ga.N, ga.K, ga.A, ga.lda, ga.M, row0, kb + 128 * s0,
                                       min(ke, kb + 128 * s1), acc);
  wave_reduce<MT, TN, NW>(acc, red);
  if (ga.rs.ss) row_scale_finish<MT>(ga.rs, ga.M, ga.K, rs_v, rinv, red);
  if (wave != 0) return;
  if constexpr (WFP8) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = ga.wscale[min(row0 + 16 * t + 4 * g + r, ga.N - 1)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][mt][r] *= sc[r];
    }
  }
  if constexpr (EPI == EPI_PARTIAL) {
    if (ea.tile_ctr) {
      finish_residual<MT, TN>(ga, ea, acc, row0);
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      const int n = row0 + 16 * t + 4 * g;  // first of this lane's 4 rows
      const f32x4 v = ga.rs.ss ? acc[t][mt] * rinv[min(m, 16 * MT - 1)] : acc[t][mt];
      if (m < ga.M && n < ga.N) {
        if constexpr (EPI == EPI_QKV_ROPE) epilogue4_qkv(v, m, n, cs4[t][mt], ea);
        else epilogue4<EPI>(v, m, n, blockIdx.y, ea);
      }
    }
}

// Split-K finish for the residual GEMMs: one workgroup per activation row
// adds the splits' partial sums (in split order) to the fp32 residual row,
// then writes the RMSNorm of the new row (with `gain`) as bf16 and, when
// asked, the row's sum of squares.
__global__ __launch_bounds__(256) void k_resid_norm(ResidNormArgs a) {
  constexpr int MAXC = 4;  // row chunks (of 4 values per thread) kept in registers
  constexpr int MAXS = 4;  // splits whose loads are all issued before the sum
  __shared__ float red[4];
  const int m = blockIdx.x;
  float *hr = a.h + (size_t)m * a.n;
  const int step = blockDim.x * 4;
  const bool fast = a.n <= MAXC * step && a.splits <= MAXS;
  float ss = 0.0f;
  f32x4 xs[MAXC];
  if (fast) {
    // every load of the row is in flight at once; the sum keeps split order
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int i = c * step + threadIdx.x * 4;
      if (i < a.n) {
        f32x4 p[MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
          if (s < a.splits) p[s] = *(const f32x4 *)(a.part + ((size_t)s * a.ld_split + m) * a.n + i);
        f32x4 x = a.init_zero ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4 *)(hr + i);
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
          if (s < a.splits) x += p[s];
        *(f32x4 *)(hr + i) = x;
        ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        xs[c] = x;
      }
    }
  } else {
    for (int i = threadIdx.x * 4; i < a.n; i += step) {
      f32x4 x = a.init_zero ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4 *)(hr + i);
      for (int s = 0; s < a.splits; ++s) x += *(const f32x4 *)(a.part + ((size_t)s * a.ld_split + m) * a.n + i);
      *(f32x4 *)(hr + i) = x;
      ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
  }
  ss = block_sum(ss, red);
  if (!a.out) return;
  const float r = 1.0f / sqrtf(ss / (float)a.n + a.eps);
  uint16_t *o = a.out + (size_t)m * a.n;
  auto put = [&](int i, const f32x4 x) {
    const float4 gg = *(const float4 *)(a.gain + i);
    uint2 w;
    w.x = pack_bf16x2(x[0] * r * gg.x, x[1] * r * gg.y);
    w.y = pack_bf16x2(x[2] * r * gg.z, x[3] * r * gg.w);
    *(uint2 *)(o + i) = w;
  };
  if (fast) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int i = c * step + threadIdx.x * 4;
      if (i < a.n) put(i, xs[c]);
    }
  } else {
    for (int i = threadIdx.x * 4; i < a.n; i += step) put(i, *(const f32x4 *)(hr + i));
  }
}

// ------------------------------------------------------------- LM head ----
// Stage 1: every wave streams (16 * TN)-row vocab units u = wave_id,
// wave_id + total_waves, ... over the full K and keeps, per lane, a running
// (max, argmax, sum exp) of its activation row over the vocab entries it sees
// (masked entries skipped). Lanes, then the workgroup's waves, are merged in
// a fixed order; one partial per workgroup and row is written. Wave ids run
// over the workgroups first (wave w of workgroup b is w * workgroups + b), so
// the units that do not divide evenly are dealt one per CU: every CU streams
// within one unit of the same bytes, and a CU's rate bounds the kernel.
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
  __shared__ float rinv[16 * MT], tmp[256];
  if (a.rs.ss) {
    RowScale rs = a.rs;
    rs.ss = a.rs.ss + a.row0;
    load_row_scale<MT>(rs, a.M, a.K, rinv, tmp);
  }
  float rsc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) rsc[mt] = a.rs.ss ? rinv[min(mt * 16 + r16, 16 * MT - 1)] : 1.0f;
  const int nw = gridDim.x * 4;
  for (int u = wave * gridDim.x + blockIdx.x; u < units; u += nw) {
    const int row0 = u * UNIT;
    f32x4 acc[TN][MT];
    zero<MT, TN>(acc);
    stream_rows<MT, TN, ST, WFP8, TILED>(a.W, a.V, a.K, a.z, a.K, a.M, row0, 0, a.K, acc);
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = row0 + 16 * t + 4 * g + r;
        if (v >= a.V) continue;
        const float sc = WFP8 ? a.scale[v] : 1.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float x = a.rs.ss ? acc[t][mt][r] * rsc[mt] * sc : acc[t][mt][r] * sc;
          const int m = mt * 16 + r16;
          if (a.logits && m < a.M) a.logits[(size_t)m * a.V + v] = x;
          const bool ok = !mask_row[mt] || ((((uint32_t)mask_row[mt][v >> 5]) >> (v & 31)) & 1u);
          arg_push(st[mt], x, (uint32_t)v, ok);
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
// tree order) and writes its id and top-1 probability at the row's entry
// (row j at entry j, or at (j + 1) % gamma with the shifted-row convention);
// the last row of a sequence to finish (atomic ticket) writes the chain
// confidence min(p1) over entries 1..num_drafts.
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
    const int j = m - seq * a.gamma;
    const int e = seq * a.gamma + (a.shifted ? (j + 1) % a.gamma : j);  // entry of row j
    a.ids[e] = none ? DFLASH_NO_TOKEN : s_idx[0];
    if (a.row_prob) a.row_prob[e] = p1;
    a.p1[e] = p1;
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

template <int MT, int TN, int NW, int ST>
hipError_t launch_cfg(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  dim3 grid((g.N + 16 * TN - 1) / (16 * TN), g.splits), block(NW * 64);
#define DFL_CASE(E)                                                                           \
  case E:                                                                                     \
    if (g.wscale) hipLaunchKernelGGL((k_gemm<MT, TN, NW, ST, E, true, true>), grid, block, 0, s, g, e); \
    else hipLaunchKernelGGL((k_gemm<MT, TN, NW, ST, E, true, false>), grid, block, 0, s, g, e);         \
    break;
  switch (epi) {
    DFL_CASE(EPI_F32)
    DFL_CASE(EPI_SWIGLU)
    DFL_CASE(EPI_QKV_ROPE)
    DFL_CASE(EPI_KV_SCATTER)
    DFL_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef DFL_CASE
  return hipGetLastError();
}

template <int MT, int TN, int ST>
hipError_t launch_partial(const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  dim3 grid((g.N + 16 * TN - 1) / (16 * TN), g.splits), block(4 * 64);
  if (g.wscale) hipLaunchKernelGGL((k_gemm<MT, TN, 4, ST, EPI_PARTIAL, true, true>), grid, block, 0, s, g, e);
  else hipLaunchKernelGGL((k_gemm<MT, TN, 4, ST, EPI_PARTIAL, true, false>), grid, block, 0, s, g, e);
  return hipGetLastError();
}

// Busiest CU's 16-row tiles when N rows go out in units of 16 * tn rows, one
// unit per workgroup and NUM_CUS workgroups per round.
int tiles_per_cu(int N, int tn) {
  const int units = (N + 16 * tn - 1) / (16 * tn);
  return (units + NUM_CUS - 1) / NUM_CUS * tn;
}

// The plan fixes the K order (nw, splits, kslice); the launch shape below
// does not change it. For one 16-row group of activations (the registers
// allow it): a split of a residual GEMM loads a wave's 5 or 6 steps in one
// batch, and a wide matrix goes out in 48-row units when that lowers the
// busiest CU's share (12288 rows: 256 units of 48 instead of 384 of 32, which
// leave half the CUs with two).
template <int MT>
hipError_t launch_mt(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  if (g.nw != 4 || g.st != 4 || (g.tn != 1 && g.tn != 2)) return hipErrorInvalidValue;
  if constexpr (MT == 1) {
    if (epi == EPI_PARTIAL && g.tn == 1) {
      const int per_wave = ((g.kslice + 127) / 128 + 3) / 4;
      if (per_wave == 6) return launch_partial<1, 1, 6>(g, e, s);
      if (per_wave == 5) return launch_partial<1, 1, 5>(g, e, s);
    }
    if (epi != EPI_PARTIAL && g.tn == 2 && tiles_per_cu(g.N, 3) < tiles_per_cu(g.N, 2))
      return launch_cfg<MT, 3, 4, 4>(epi, g, e, s);
  }
  if (g.tn == 1) return launch_cfg<MT, 1, 4, 4>(epi, g, e, s);
  return launch_cfg<MT, 2, 4, 4>(epi, g, e, s);
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
  return mt == 1 ? launch_mt<1>(epi, g, e, s) : mt == 2 ? launch_mt<2>(epi, g, e, s) : launch_mt<4>(epi, g, e, s);
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
