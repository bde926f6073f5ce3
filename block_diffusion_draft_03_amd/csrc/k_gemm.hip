// k_gemm.hip - weight-streaming MFMA GEMMs of the DFlash head for gfx950.
//
// All contractions of the propose path have few activation rows (gamma per
// sequence) against large bf16 (or E4M3) weight matrices, so they are bound
// by streaming the weights from HBM once. The kernel computes the transposed
// product D^T = W A^T with v_mfma_f32_16x16x32_bf16: the A operand of the
// MFMA is 16 weight rows, the B operand 16 activation rows. Lane l loads 64
// contiguous bytes (32 bf16) of weight row n0 + l % 16 per 128-wide K step,
// so a wave reads 16 rows x 256 contiguous bytes per step; the 32 values are
// split into the four 8-value MFMA k-groups, and the activations are loaded
// with the same k permutation, which leaves the dot products unchanged.
//
// Each wave owns two 16-row weight tiles 64 rows apart (tiles w and w + 4 of
// a 128-row column group), so a RoPE pair (i, i + 64) of a 128-wide head, or
// a gate / up pair of the interleaved MLP weight, lands in one lane.
//
// Split-K: the workgroups of one column group write partial tiles to a
// workspace; the last to arrive (atomic ticket) sums them in split order
// 0, 1, 2, ... and runs the epilogue, so results are deterministic and do not
// depend on which rows share the launch.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

template <int MT>
struct Frag {
  uint4 w0[4], w1[4];
  uint4 a[MT][4];
};

// Load one 128-wide K step for this lane into registers.
template <int MT, bool WFP8>
__device__ __forceinline__ void load_step(Frag<MT> &f, const void *__restrict__ Wv, int K, int n0, int n1,
                                          const uint16_t *__restrict__ A, int lda, const int (&arow)[MT], int kk,
                                          int ke) {
  const uint4 z = {0u, 0u, 0u, 0u};
  if constexpr (!WFP8) {
    const uint16_t *W = (const uint16_t *)Wv;
    const uint16_t *p0 = W + (size_t)n0 * K + kk;
    const uint16_t *p1 = W + (size_t)n1 * K + kk;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool ok = kk + 8 * c < ke;
      f.w0[c] = ok ? *(const uint4 *)(p0 + 8 * c) : z;
      f.w1[c] = ok ? *(const uint4 *)(p1 + 8 * c) : z;
    }
  } else {
    const uint8_t *W = (const uint8_t *)Wv;
    const bool ok = kk < ke;  // K % 32 == 0: a lane's 32 codes are all in or all out
    uint4 q0a = z, q0b = z, q1a = z, q1b = z;
    if (ok) {
      const uint8_t *p0 = W + (size_t)n0 * K + kk;
      const uint8_t *p1 = W + (size_t)n1 * K + kk;
      q0a = *(const uint4 *)p0;
      q0b = *(const uint4 *)(p0 + 16);
      q1a = *(const uint4 *)p1;
      q1b = *(const uint4 *)(p1 + 16);
    }
    const uint32_t d0[8] = {q0a.x, q0a.y, q0a.z, q0a.w, q0b.x, q0b.y, q0b.z, q0b.w};
    const uint32_t d1[8] = {q1a.x, q1a.y, q1a.z, q1a.w, q1b.x, q1b.y, q1b.z, q1b.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint2 lo = e4m3x4_to_bf16x4(d0[2 * c]), hi = e4m3x4_to_bf16x4(d0[2 * c + 1]);
      f.w0[c] = uint4{lo.x, lo.y, hi.x, hi.y};
      lo = e4m3x4_to_bf16x4(d1[2 * c]);
      hi = e4m3x4_to_bf16x4(d1[2 * c + 1]);
      f.w1[c] = uint4{lo.x, lo.y, hi.x, hi.y};
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint16_t *pa = A + (size_t)arow[mt] * lda + kk;
#pragma unroll
    for (int c = 0; c < 4; ++c) f.a[mt][c] = (kk + 8 * c < ke) ? *(const uint4 *)(pa + 8 * c) : z;
  }
}

template <int MT>
__device__ __forceinline__ void mma_step(const Frag<MT> &f, f32x4 (&acc)[2][MT]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[0][mt] = mfma16x16x32(as_bf16x8(f.w0[c]), as_bf16x8(f.a[mt][c]), acc[0][mt]);
      acc[1][mt] = mfma16x16x32(as_bf16x8(f.w1[c]), as_bf16x8(f.a[mt][c]), acc[1][mt]);
    }
  }
}

// acc[t][mt][r] = sum_k W[n_t + 4g + r, k] * A[mt*16 + l%16, k] over [kb, ke).
template <int MT, bool WFP8>
__device__ __forceinline__ void mainloop(const void *__restrict__ W, int N, int K, const uint16_t *__restrict__ A,
                                         int lda, int M, int n_t0, int n_t1, int kb, int ke, f32x4 (&acc)[2][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int n0 = min(n_t0 + r16, N - 1), n1 = min(n_t1 + r16, N - 1);
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + r16, M - 1);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb >= ke) return;
  Frag<MT> cur, nxt;
  load_step<MT, WFP8>(cur, W, K, n0, n1, A, lda, arow, kb + 32 * g, ke);
  for (int k0 = kb; k0 < ke; k0 += 128) {
    const bool more = k0 + 128 < ke;
    if (more) load_step<MT, WFP8>(nxt, W, K, n0, n1, A, lda, arow, k0 + 128 + 32 * g, ke);
    mma_step<MT>(cur, acc);
    if (more) cur = nxt;
  }
}

// Deterministic split-K reduction. Returns false in every workgroup except
// the last one of the column group, which ends holding the full sums.
template <int MT>
__device__ __forceinline__ bool splitk_reduce(const GemmArgs &ga, f32x4 (&acc)[2][MT]) {
  if (ga.splits <= 1) return true;
  __shared__ int s_last;
  const int cg = blockIdx.x, split = blockIdx.y;
  f32x4 *my = (f32x4 *)ga.ws + ((size_t)(split * gridDim.x + cg) * blockDim.x + threadIdx.x) * (2 * MT);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) my[t * MT + mt] = acc[t][mt];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&ga.counters[cg], 1);
    s_last = (prev == ga.splits - 1);
  }
  __syncthreads();
  if (!s_last) return false;
  __threadfence();
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ga.splits; ++s) {
    const f32x4 *p = (const f32x4 *)ga.ws + ((size_t)(s * gridDim.x + cg) * blockDim.x + threadIdx.x) * (2 * MT);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[t][mt] += p[t * MT + mt];
      }
  }
  if (threadIdx.x == 0) ga.counters[cg] = 0;
  return true;
}

template <int MT, bool WFP8, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs ga, EpiArgs ea) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int cg = blockIdx.x;
  const int n_t0 = cg * 128 + wave * 16, n_t1 = n_t0 + 64;
  const int kb = blockIdx.y * ga.kslice, ke = min(ga.K, kb + ga.kslice);
  f32x4 acc[2][MT];
  mainloop<MT, WFP8>(ga.W, ga.N, ga.K, ga.A, ga.lda, ga.M, n_t0, n_t1, kb, ke, acc);
  if (!splitk_reduce<MT>(ga, acc)) return;

  if constexpr (EPI == EPI_F32 || EPI == EPI_RESID) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16;
        if (m >= ga.M) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = (t ? n_t1 : n_t0) + 4 * g + r;
          if (n >= ga.N) continue;
          float *o = ea.out_f32 + (size_t)m * ea.ldo + n;
          if constexpr (EPI == EPI_F32)
            *o = acc[t][mt][r];
          else
            *o += acc[t][mt][r];
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m >= ga.M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = cg * 64 + wave * 16 + 4 * g + r;  // intermediate index
        if (cg * 128 + wave * 16 + 4 * g + r >= ga.N) continue;
        ea.out_bf16[(size_t)m * ea.ldo + i] = f32_to_bf16(silu(acc[0][mt][r]) * acc[1][mt][r]);
      }
    }
  } else {
    // RoPE epilogues: stage the 128-column tile in LDS, then rotate pairs.
    __shared__ float tile[MT * 16][129];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile[mt * 16 + r16][t * 64 + wave * 16 + 4 * g + r] = acc[t][mt][r];
    __syncthreads();
    const int d = ea.head_dim, half = d >> 1;
    for (int e = threadIdx.x; e < MT * 16 * 128; e += blockDim.x) {
      const int m = e >> 7, col = e & 127;
      const int n = cg * 128 + col;
      if (m >= ga.M || n >= ga.N) continue;
      const int i = n % d;  // dim within the head (heads align to d inside a group)
      const float x = tile[m][col];
      if constexpr (EPI == EPI_QKV_ROPE) {
        float y = x;
        if (n < ea.q_dim + ea.kv_dim) {
          const int ip = i < half ? i : i - half;
          const float xp = tile[m][i < half ? col + half : col - half];
          const float2 c = ea.cs[(size_t)m * half + ip];
          y = i < half ? x * c.x - xp * c.y : x * c.x + xp * c.y;
        }
        ea.out_bf16[(size_t)m * ea.ldo + n] = f32_to_bf16(y);
      } else {  // EPI_KV_SCATTER
        const int kv_dim = ea.n_kv * d;
        const int l = n / (2 * kv_dim), rem = n % (2 * kv_dim);
        const int kv = rem / kv_dim, hd = (rem % kv_dim) / d;
        const int pos = ea.row_pos[m];
        float y = x;
        if (kv == 0) {
          const int ip = i < half ? i : i - half;
          const float xp = tile[m][i < half ? col + half : col - half];
          double sn, cs;
          sincos((double)pos * ea.inv_freq[ip], &sn, &cs);
          const float c = (float)cs, s = (float)sn;
          y = i < half ? x * c - xp * s : x * c + xp * s;
        }
        const int32_t blk = ea.row_bt[m][pos >> 4];
        const size_t off = ((((size_t)blk * ea.L + l) * 2 + kv) * ea.n_kv + hd) * (size_t)(DFLASH_KV_BLOCK * d) +
                           (size_t)(pos & 15) * d + i;
        if (ea.kv_fp8) {
          const float sc = ea.kv_scale[(l * 2 + kv) * ea.n_kv + hd];
          ((uint8_t *)ea.pool)[off] = f32_to_e4m3(y / sc);
        } else {
          ((uint16_t *)ea.pool)[off] = f32_to_bf16(y);
        }
      }
    }
  }
}

template <int MT, bool WFP8>
hipError_t launch_t(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  dim3 grid(gemm_groups(g.N), g.splits), block(256);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((k_gemm<MT, WFP8, EPI_F32>), grid, block, 0, s, g, e); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<MT, WFP8, EPI_RESID>), grid, block, 0, s, g, e); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm<MT, WFP8, EPI_SWIGLU>), grid, block, 0, s, g, e); break;
    case EPI_QKV_ROPE: hipLaunchKernelGGL((k_gemm<MT, WFP8, EPI_QKV_ROPE>), grid, block, 0, s, g, e); break;
    case EPI_KV_SCATTER: hipLaunchKernelGGL((k_gemm<MT, WFP8, EPI_KV_SCATTER>), grid, block, 0, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- LM head ----
// Stage 1: every workgroup streams 128-row vocab groups cg = blockIdx.x,
// blockIdx.x + P, ... and keeps, per lane, a running (max, argmax, sum exp)
// of its activation row over the vocab entries it sees (masked entries are
// skipped). Lanes, then waves, are merged in a fixed order and one partial
// per workgroup and row is written.
template <int MT, bool WFP8>
__global__ __launch_bounds__(256) void k_lm_head(LmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int groups = (a.V + 127) / 128;
  ArgState st[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arg_init(st[mt]);
  const int32_t *mask_row[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r16, a.M - 1);
    mask_row[mt] = a.bitmask ? a.bitmask + (size_t)((a.row0 + m) / a.gamma) * a.words : nullptr;
  }
  for (int cg = blockIdx.x; cg < groups; cg += gridDim.x) {
    const int n_t0 = cg * 128 + wave * 16, n_t1 = n_t0 + 64;
    f32x4 acc[2][MT];
    mainloop<MT, WFP8>(a.W, a.V, a.K, a.z, a.K, a.M, n_t0, n_t1, 0, a.K, acc);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = (t ? n_t1 : n_t0) + 4 * g + r;
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

// Stage 2: one workgroup per sequence merges the P partials of each of its
// gamma rows (fixed tree order), writes the ids and top-1 probabilities, and
// the chain confidence min(p1) over rows 1..num_drafts.
__global__ __launch_bounds__(256) void k_lm_finish(LmFinishArgs a) {
  __shared__ float s_mx[256], s_se[256];
  __shared__ uint32_t s_idx[256];
  __shared__ float s_p1[64];
  const int seq = blockIdx.x;
  for (int j = 0; j < a.gamma; ++j) {
    const int m = seq * a.gamma + j;
    ArgState st;
    arg_init(st);
    for (int p = threadIdx.x; p < a.P; p += blockDim.x) {
      const size_t o = (size_t)p * a.M + m;
      ArgState q;
      q.mx = a.part_mx[o];
      q.se = a.part_se[o];
      q.idx = a.part_idx[o];
      st = arg_merge(st, q);
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
      s_p1[j] = p1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float c = s_p1[1];
    for (int j = 2; j <= a.num_drafts; ++j) c = fminf(c, s_p1[j]);
    a.conf[seq] = c;
  }
}

}  // namespace

int gemm_groups(int N) { return (N + 127) / 128; }

void gemm_plan(int N, int K, int *kslice, int *splits) {
  const int groups = gemm_groups(N);
  const int steps = (K + 127) / 128;
  int want = 512 / groups;
  if (want < 1) want = 1;
  if (want > steps) want = steps;
  const int per = (steps + want - 1) / want;
  *kslice = per * 128;
  *splits = (K + *kslice - 1) / *kslice;
}

size_t gemm_ws_floats(int N, int K) {
  int ks, sp;
  gemm_plan(N, K, &ks, &sp);
  if (sp <= 1) return 0;
  return (size_t)sp * gemm_groups(N) * 256 * (2 * 4 * 4);
}

hipError_t launch_gemm(int epi, bool w_fp8, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  if (g.M < 1 || g.M > GEMM_MAX_ROWS) return hipErrorInvalidValue;
  const int mt = g.M <= 16 ? 1 : (g.M <= 32 ? 2 : 4);
  if (w_fp8) return hipErrorInvalidValue;  // only the LM head streams E4M3 weights
  return mt == 1 ? launch_t<1, false>(epi, g, e, s) : mt == 2 ? launch_t<2, false>(epi, g, e, s)
                                                              : launch_t<4, false>(epi, g, e, s);
}

int lm_parts(int V) {
  const int groups = (V + 127) / 128;
  return groups < 1024 ? groups : 1024;
}

hipError_t launch_lm_head(bool w_fp8, const LmArgs &a, hipStream_t s) {
  if (a.M < 1 || a.M > GEMM_MAX_ROWS) return hipErrorInvalidValue;
  const int mt = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  dim3 grid(lm_parts(a.V)), block(256);
  if (w_fp8) {
    if (mt == 1) hipLaunchKernelGGL((k_lm_head<1, true>), grid, block, 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL((k_lm_head<2, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_lm_head<4, true>), grid, block, 0, s, a);
  } else {
    if (mt == 1) hipLaunchKernelGGL((k_lm_head<1, false>), grid, block, 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL((k_lm_head<2, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_lm_head<4, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_lm_finish(const LmFinishArgs &a, int n_seq, hipStream_t s) {
  hipLaunchKernelGGL(k_lm_finish, dim3(n_seq), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
