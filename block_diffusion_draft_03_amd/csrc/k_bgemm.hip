// k_bgemm.hip - LDS-tiled MFMA GEMMs for many activation rows (batched
// propose) on gfx950.
//
// A workgroup of 4 waves computes a 128 x 128 block of D^T = W A^T: 8 weight
// tiles of 16 rows against 8 activation tiles of 16 rows, each wave a 64 x 64
// quarter with v_mfma_f32_16x16x32_bf16. K advances in stages of 64 columns
// (half of one 128-wide step of the tile-major weight layout). A stage's
// operands are staged in LDS already in MFMA fragment order (the weights come
// from HBM in that order; activation rows are scattered into it), so every
// fragment read is one contiguous 1 KB ds_read_b128 per wave. The next
// stage's global loads are in flight while the current stage is multiplied;
// two LDS buffers, one barrier per stage.
//
// K order: each K slice of the GemmPlan is summed sequentially in 32-wide
// MFMA steps, whatever the number of rows, so results are deterministic and
// row-independent; they agree with the weight-streaming kernel (which sums
// each slice as four parts) to rounding. The LM head's logits are
// bit-identical to the weight-streaming kernel's (both sum K in one pass).
//
// Block placement is XCD-aware: workgroup b runs on XCD b % 8, and the
// activation blocks that share one weight block are consecutive workgroups of
// one XCD, so the weight block is read from HBM once and then from that
// XCD's L2.
#include "common.hpp"
#include "gemm_epi.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int BN = 128;                // weight rows per workgroup
constexpr int BM = 128;                // activation rows per workgroup
constexpr int NT = BN / 16;            // weight tiles
constexpr int MTL = BM / 16;           // activation tiles
constexpr int WN = NT / 2, WM = MTL / 2;  // tiles per wave (2 x 2 waves)
constexpr int SW = NT * 2 * 64;        // uint4 of weights per stage
constexpr int SA = MTL * 2 * 64;       // uint4 of activations per stage
constexpr int NTHR = 256;
constexpr int LM_TILES = 8;            // vocab tiles of 128 per LM-head workgroup

// Global loads of the stage that starts at absolute column k (a multiple of 64).
template <bool WFP8>
__device__ __forceinline__ void gload(uint4 (&rw)[SW / NTHR], uint4 (&ra)[SA / NTHR], const void *__restrict__ W,
                                      int steps_w, int tile0,
                                      const uint16_t *__restrict__ A, int lda, int M, int m0, int k) {
  const int step = k >> 7, half = (k >> 6) & 1;
  if constexpr (!WFP8) {
    const uint4 *Wq = (const uint4 *)W;
#pragma unroll
    for (int i = 0; i < SW / NTHR; ++i) {
      const int j = threadIdx.x + NTHR * i;
      const int t = j >> 7, c = (j >> 6) & 1, lane = j & 63;
      rw[i] = Wq[(((size_t)(tile0 + t) * steps_w + step) * 4 + half * 2 + c) * 64 + lane];
    }
  } else {
    // one E4M3 pair (k-groups 2 half, 2 half + 1) per (tile, lane)
    const uint4 *Wq = (const uint4 *)W;
#pragma unroll
    for (int i = 0; i < SW / NTHR / 2; ++i) {
      const int j = threadIdx.x + NTHR * i;
      const int t = j >> 6, lane = j & 63;
      const uint4 q = Wq[(((size_t)(tile0 + t) * steps_w + step) * 2 + half) * 64 + lane];
      uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
      rw[2 * i] = uint4{lo.x, lo.y, hi.x, hi.y};
      lo = e4m3x4_to_bf16x4(q.z);
      hi = e4m3x4_to_bf16x4(q.w);
      rw[2 * i + 1] = uint4{lo.x, lo.y, hi.x, hi.y};
    }
  }
#pragma unroll
  for (int i = 0; i < SA / NTHR; ++i) {
    const int j = threadIdx.x + NTHR * i;
    const int lane = j & 63, rest = j >> 6, c = rest & 1, mt = rest >> 1;
    const int m = min(m0 + mt * 16 + (lane & 15), M - 1);
    ra[i] = *(const uint4 *)(A + (size_t)m * lda + k + 32 * c + 8 * (lane >> 4));
  }
}

// LDS image of a stage: [tile][c][lane] weight fragments, then
// [act tile][c][lane] activation fragments.
template <bool WFP8>
__device__ __forceinline__ void lstore(const uint4 (&rw)[SW / NTHR], const uint4 (&ra)[SA / NTHR], uint4 *buf) {
  if constexpr (!WFP8) {
#pragma unroll
    for (int i = 0; i < SW / NTHR; ++i) buf[threadIdx.x + NTHR * i] = rw[i];
  } else {
#pragma unroll
    for (int i = 0; i < SW / NTHR / 2; ++i) {
      const int j = threadIdx.x + NTHR * i;
      const int t = j >> 6, lane = j & 63;
      buf[(t * 2 + 0) * 64 + lane] = rw[2 * i];
      buf[(t * 2 + 1) * 64 + lane] = rw[2 * i + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < SA / NTHR; ++i) buf[SW + threadIdx.x + NTHR * i] = ra[i];
}

__device__ __forceinline__ void mma_stage(const uint4 *buf, int wn, int wm, int lane, f32x4 (&acc)[WN][WM]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint4 wf[WN], af[WM];
#pragma unroll
    for (int i = 0; i < WN; ++i) wf[i] = buf[((wn * WN + i) * 2 + c) * 64 + lane];
#pragma unroll
    for (int j = 0; j < WM; ++j) af[j] = buf[SW + ((wm * WM + j) * 2 + c) * 64 + lane];
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WM; ++j) acc[i][j] = mfma16x16x32(as_bf16x8(wf[i]), as_bf16x8(af[j]), acc[i][j]);
  }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[WN][WM]) {
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Block (weight block nb, activation block mb) of workgroup b; false for the
// padding workgroups of the last XCD round.
__device__ __forceinline__ bool place(int b, int n_nb, int n_mb, int &nb, int &mb) {
  const int x = b & 7, k = b >> 3;
  nb = (k / n_mb) * 8 + x;
  mb = k % n_mb;
  return nb < n_nb;
}

// acc += W[tile0 .. tile0 + 8 tiles) x A[m0 .. m0 + 128) over columns
// [kb, kb + 128 * S), summed sequentially.
template <bool WFP8>
__device__ __forceinline__ void block_product(const void *W, int steps_w, int tile0, const uint16_t *A, int lda, int M,
                                              int m0, int kb, int S, uint4 (*lds)[SW + SA], f32x4 (&acc)[WN][WM]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave & 1, wm = wave >> 1;
  const int NS = 2 * S;
  uint4 rw[SW / NTHR], ra[SA / NTHR];
  gload<WFP8>(rw, ra, W, steps_w, tile0, A, lda, M, m0, kb);
  lstore<WFP8>(rw, ra, lds[0]);
  __syncthreads();
  for (int st = 0; st + 1 < NS; ++st) {
    gload<WFP8>(rw, ra, W, steps_w, tile0, A, lda, M, m0, kb + 64 * (st + 1));
    mma_stage(lds[st & 1], wn, wm, lane, acc);
    lstore<WFP8>(rw, ra, lds[(st + 1) & 1]);
    __syncthreads();
  }
  mma_stage(lds[(NS - 1) & 1], wn, wm, lane, acc);
  __syncthreads();
}

template <int EPI>
__global__ __launch_bounds__(NTHR, 2) void k_bgemm(GemmArgs ga, EpiArgs ea, int n_nb, int n_mb) {
  __shared__ uint4 lds[2][SW + SA];
  int nb, mb;
  if (!place(blockIdx.x, n_nb, n_mb, nb, mb)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int wn = wave & 1, wm = wave >> 1;
  const int split = blockIdx.y;
  const int kb = split * ga.kslice, ke = min(ga.K, kb + ga.kslice);
  f32x4 acc[WN][WM];
  zero_acc(acc);
  block_product<false>(ga.W, ga.K >> 7, nb * NT, ga.A, ga.lda, ga.M, mb * BM, kb, (ke - kb) >> 7, lds, acc);
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int n = nb * BN + (wn * WN + i) * 16 + 4 * g;
      const int m = mb * BM + (wm * WM + j) * 16 + r16;
      if (m < ga.M) epilogue4<EPI>(acc[i][j], m, n, split, ea);
    }
}

// LM head: workgroup (vocab range p, activation block mb) multiplies its
// LM_TILES vocab blocks of 128 rows and keeps, per lane and activation row, a
// running (max, argmax, sum exp) over the unmasked entries; lanes, then the
// two waves sharing a row, are merged in a fixed order and one partial per
// (p, row) is written.
template <bool WFP8>
__global__ __launch_bounds__(NTHR, 2) void k_blm_head(LmArgs a, int n_p, int n_mb) {
  __shared__ uint4 lds[2][SW + SA];
  __shared__ float s_mx[2][BM], s_se[2][BM];
  __shared__ uint32_t s_idx[2][BM];
  int p, mb;
  if (!place(blockIdx.x, n_p, n_mb, p, mb)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int wn = wave & 1, wm = wave >> 1;
  const int n_vb = a.V / BN;
  const int steps_w = a.K >> 7;
  ArgState st[WM];
  const int32_t *mask_row[WM];
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    arg_init(st[j]);
    const int m = min(mb * BM + (wm * WM + j) * 16 + r16, a.M - 1);
    mask_row[j] = a.bitmask ? a.bitmask + (size_t)(m / a.gamma) * a.words : nullptr;
  }
  for (int vb = p * LM_TILES; vb < min(n_vb, (p + 1) * LM_TILES); ++vb) {
    f32x4 acc[WN][WM];
    zero_acc(acc);
    block_product<WFP8>(a.W, steps_w, vb * NT, a.z, a.K, a.M, mb * BM, 0, steps_w, lds, acc);
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = vb * BN + (wn * WN + i) * 16 + 4 * g + r;
        const float sc = WFP8 ? a.scale[v] : 1.0f;
#pragma unroll
        for (int j = 0; j < WM; ++j) {
          const float x = acc[i][j][r] * sc;
          const int m = mb * BM + (wm * WM + j) * 16 + r16;
          if (a.logits && m < a.M) a.logits[(size_t)m * a.V + v] = x;
          const bool ok = !mask_row[j] || ((((uint32_t)mask_row[j][v >> 5]) >> (v & 31)) & 1u);
          arg_push(st[j], x, (uint32_t)v, ok);
        }
      }
  }
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    st[j] = arg_merge(st[j], arg_shfl_xor(st[j], 16));
    st[j] = arg_merge(st[j], arg_shfl_xor(st[j], 32));
    if (g == 0) {
      const int row = (wm * WM + j) * 16 + r16;
      s_mx[wn][row] = st[j].mx;
      s_se[wn][row] = st[j].se;
      s_idx[wn][row] = st[j].idx;
    }
  }
  __syncthreads();
  if (threadIdx.x < BM) {
    const int row = threadIdx.x, m = mb * BM + row;
    ArgState x, y;
    x.mx = s_mx[0][row];
    x.se = s_se[0][row];
    x.idx = s_idx[0][row];
    y.mx = s_mx[1][row];
    y.se = s_se[1][row];
    y.idx = s_idx[1][row];
    x = arg_merge(x, y);
    if (m < a.M) {
      const size_t o = (size_t)p * a.ld_part + m;
      a.part_mx[o] = x.mx;
      a.part_se[o] = x.se;
      a.part_idx[o] = x.idx;
    }
  }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  const int n_nb = g.N / BN, n_mb = (g.M + BM - 1) / BM;
  dim3 grid(((n_nb + 7) / 8) * 8 * n_mb, g.splits);
  hipLaunchKernelGGL((k_bgemm<EPI>), grid, dim3(NTHR), 0, s, g, e, n_nb, n_mb);
  return hipGetLastError();
}

}  // namespace

bool bgemm_ok(int epi, int N, int K) {
  return epi != EPI_KV_SCATTER && N % BN == 0 && K % 128 == 0 && N > 0 && K > 0;
}

hipError_t launch_bgemm(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  if (g.M < 1 || !bgemm_ok(epi, g.N, g.K) || g.splits < 1 || g.kslice % 128 != 0) return hipErrorInvalidValue;
  if (g.splits > 1 && epi != EPI_PARTIAL) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_F32: return launch_epi<EPI_F32>(g, e, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(g, e, s);
    case EPI_QKV_ROPE: return launch_epi<EPI_QKV_ROPE>(g, e, s);
    case EPI_PARTIAL: return launch_epi<EPI_PARTIAL>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

int blm_parts(int V) { return (V / BN + LM_TILES - 1) / LM_TILES; }

hipError_t launch_blm_head(bool w_fp8, const LmArgs &a, hipStream_t s) {
  if (a.M < 1 || a.V % BN != 0 || a.K % 128 != 0 || a.row0 != 0) return hipErrorInvalidValue;
  const int n_p = blm_parts(a.V), n_mb = (a.M + BM - 1) / BM;
  dim3 grid(((n_p + 7) / 8) * 8 * n_mb);
  if (w_fp8) hipLaunchKernelGGL((k_blm_head<true>), grid, dim3(NTHR), 0, s, a, n_p, n_mb);
  else hipLaunchKernelGGL((k_blm_head<false>), grid, dim3(NTHR), 0, s, a, n_p, n_mb);
  return hipGetLastError();
}

}  // namespace dflash
