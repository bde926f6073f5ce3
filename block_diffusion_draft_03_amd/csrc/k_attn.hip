// k_attn.hip - GQA attention of the block rows over the paged ctx window and
// the block itself, for gfx950.
//
// One workgroup (4 waves) per (sequence, kv head, split). The rep = n_q / n_kv
// query heads of the kv head times the gamma block rows form up to 128 query
// rows, 32 per wave. Keys come in tiles of 32: ctx tiles are aligned to two
// 16-row KV blocks (positions outside [win_start, ctx_len) are masked), and
// the gamma block rows form the block tile(s), whose K rows come straight
// from the QKV output and whose V^T from the copy the QKV epilogue writes.
// A split owns a run of ctx tiles; the last split also owns the block tiles.
//
// The pool stores K row-major and V transposed ([dim][16 slots]) per block,
// so every MFMA fragment of a tile is one contiguous 16-byte piece per lane
// in global memory and is copied straight into LDS in fragment order with
// direct-to-LDS loads (one 1 KB fragment per wave instruction, no register
// staging). Ctx tiles stream through a ring of NSTAGE LDS slots with
// NSTAGE - 1 tiles in flight.
//
// Products are transposed so every per-query quantity stays in one lane:
// S^T = K Q^T (MFMA A = 16 keys x 32 dims, B = Q^T). The 16 MFMA rows of key
// sub-tile u hold keys (r / 4) * 8 + 4u + r % 4, so lane group g ends with
// the scores of keys 8g .. 8g+7 for its query; those are exactly the B
// operand of O^T = V^T P^T, whose A operand (16 dims x keys 8g .. 8g+7) is a
// 16-byte piece of V^T. Online softmax in base 2; the FP8 V scale of ctx keys
// is folded into P. With head_dim >= 64 the K fragments of k-steps 2j and
// 2j+1 take dims 64j + 16g .. +15 of lane group g (one 16-byte piece of an
// E4M3 row), and Q uses the same dim order. Q and K also carry their head
// dims in RoPE pair order; every score is unchanged by these permutations.
//
// Each split writes an unnormalised partial (O, max, sum) that the combine
// kernel merges (one wave per query row); with a single split the output is
// written directly.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int KT = 32;          // keys per tile
constexpr int MAX_TPS = 32;     // ctx tiles per split (2 KV blocks each)

typedef __attribute__((address_space(3))) uint4 lds_uint4;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_uint4 *)p);
}

// One wave-wide direct-to-LDS load: lane l's 16 bytes at g land at LDS byte
// address lds + 16 l. Issued as assembly so that the only waits on it are
// the explicit vmcnt waits below; m0 is restored afterwards.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds)
               : "memory");
}

// s_waitcnt vmcnt(n), expcnt / lgkmcnt untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool FP8>
struct Geom {
  static constexpr int KS = D >= 32 ? D / 32 : 1;  // 32-dim MFMA k-steps
  static constexpr int DT = D / 16;                // 16-dim output tiles
  static constexpr bool PAIRED = KS >= 2;          // k-steps 2j, 2j+1 share a 16-dim piece per lane group
  static_assert(!FP8 || (PAIRED && DT % 2 == 0), "an E4M3 cache needs head_dim >= 64");
  // fragments (1 KB) per tile: K [u][ks] then V^T [dt]; E4M3: K [u][ks / 2], V^T [dt / 2]
  static constexpr int CF = FP8 ? KS + DT / 2 : 2 * KS + DT;  // ctx tile
  static constexpr int BF = 2 * KS + DT;                      // block tile (bf16)
  static constexpr int PW = (CF + 3) / 4;                     // ctx-tile loads per wave
  static constexpr int PB = (BF + 3) / 4;                     // block-tile loads per wave
  static constexpr int NSTAGE = FP8 ? 4 : 3;
};

// First dim of the 8 that lane group gq holds in k-step ks.
template <int D>
__device__ __forceinline__ int kdim(int ks, int gq) {
  if constexpr (D >= 64) return (ks & ~1) * 32 + 16 * gq + 8 * (ks & 1);
  else return 8 * gq;
}

// Key within the tile held by MFMA row r of sub-tile u.
__device__ __forceinline__ int key_of(int u, int r) { return (r >> 2) * 8 + 4 * u + (r & 3); }

struct TileSrc {
  const uint8_t *pool;
  size_t head_bytes;   // bytes of one (block, layer, K|V, kv head) tile
  int L, layer, n_kv, g;
  int32_t bA, bB;      // the tile's two KV blocks
};

// Issue this wave's direct-to-LDS loads of one ctx tile into `slot`.
template <int D, bool FP8>
__device__ __forceinline__ void issue_ctx(const TileSrc &t, uint32_t slot, int wave, int lane) {
  using G = Geom<D, FP8>;
  const int r = lane & 15, gq = lane >> 4;
  constexpr int EB = FP8 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < G::PW; ++j) {
    const int i = (wave + 4 * j) % G::CF;  // wave-uniform; duplicates reload an item with the same bytes
    const uint8_t *src;
    bool active = true;
    if (i < (FP8 ? G::KS : 2 * G::KS)) {
      int u, dim;
      if constexpr (FP8) {
        u = i / (G::KS / 2);
        dim = kdim<D>(2 * (i % (G::KS / 2)), gq);
      } else {
        u = i / G::KS;
        dim = kdim<D>(i % G::KS, gq);
        active = dim < D;
      }
      const int kt = key_of(u, r);
      const int32_t blk = kt < 16 ? t.bA : t.bB;
      src = t.pool + ((((size_t)blk * t.L + t.layer) * 2 + 0) * t.n_kv + t.g) * t.head_bytes +
            ((size_t)(kt & 15) * D + dim) * EB;
    } else {
      int dim, slot0;
      int32_t blk;
      if constexpr (FP8) {
        const int dt = 2 * (i - G::KS) + (lane >> 5);
        dim = dt * 16 + r;
        blk = ((lane >> 4) & 1) ? t.bB : t.bA;
        slot0 = 0;
      } else {
        dim = (i - 2 * G::KS) * 16 + r;
        blk = gq < 2 ? t.bA : t.bB;
        slot0 = 8 * (gq & 1);
      }
      src = t.pool + ((((size_t)blk * t.L + t.layer) * 2 + 1) * t.n_kv + t.g) * t.head_bytes +
            ((size_t)dim * 16 + slot0) * EB;
    }
    if (active) dma16(src, slot + i * 1024);
  }
}

// Issue this wave's loads of block tile bt (keys 32 bt .. of the gamma rows).
template <int D>
__device__ __forceinline__ void issue_block(const AttnArgs &a, int s, int g, int bt, uint32_t slot, int wave,
                                            int lane) {
  using G = Geom<D, false>;
  const int r = lane & 15, gq = lane >> 4;
  const int GP = (a.gamma + 31) & ~31;
#pragma unroll
  for (int j = 0; j < G::PB; ++j) {
    const int i = (wave + 4 * j) % G::BF;
    const uint16_t *src;
    bool active = true;
    if (i < 2 * G::KS) {
      const int u = i / G::KS, dim = kdim<D>(i % G::KS, gq);
      active = dim < D;
      const int tok = min(32 * bt + key_of(u, r), a.gamma - 1);
      src = a.qkv + (size_t)(s * a.gamma + tok) * a.ld + a.k_off + g * D + dim;
    } else {
      const int dim = (i - 2 * G::KS) * 16 + r;
      src = a.vtb + ((size_t)(s * a.n_kv + g) * D + dim) * GP + 32 * bt + 8 * gq;
    }
    if (active) dma16(src, slot + i * 1024);
  }
}

__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 q) {
  const uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
  return uint4{lo.x, lo.y, hi.x, hi.y};
}

template <int D>
struct WaveState {
  f32x4 o[2][Geom<D, false>::DT];
  float m[2], l[2];
};

// One tile for this wave's two query tiles. `valid` says whether key kt of
// the tile takes part; sc scales the raw scores into base-2 units; vs is
// folded into P (E4M3 V of ctx keys).
template <int D, bool FP8CTX, class Valid>
__device__ __forceinline__ void tile_step(const uint4 *slot, const bf16x8 (&qf)[2][Geom<D, false>::KS], int nqt,
                                          Valid valid, float sc, float vs, WaveState<D> &w, int lane) {
  using G = Geom<D, FP8CTX>;
  const int gq = lane >> 4;
  bf16x8 kf[2][G::KS];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      if constexpr (FP8CTX) {
        const uint8_t *p = (const uint8_t *)(slot + (u * (G::KS / 2) + ks / 2) * 64 + lane) + 8 * (ks & 1);
        kf[u][ks] = as_bf16x8(e4m3x8_to_bf16x8(*(const uint2 *)p));
      } else {
        kf[u][ks] = as_bf16x8(slot[(u * G::KS + ks) * 64 + lane]);
      }
    }
  uint4 pk[2];
  float alpha[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if (qt >= nqt) continue;
    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) sacc[u] = mfma16x16x32(kf[u][ks], qf[qt][ks], sacc[u]);
    }
    float x[2][4];
    float tmax = -__builtin_huge_valf();
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[u][r] = valid(8 * gq + 4 * u + r) ? sacc[u][r] * sc : -__builtin_huge_valf();
        tmax = fmaxf(tmax, x[u][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
    const float m_new = fmaxf(w.m[qt], tmax);
    alpha[qt] = fast_exp2(w.m[qt] - m_new);
    float p[2][4], psum = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(x[u][r] - m_new);
        psum += e;
        p[u][r] = e * vs;
      }
    w.l[qt] = w.l[qt] * alpha[qt] + psum;
    w.m[qt] = m_new;
    pk[qt].x = pack_bf16x2(p[0][0], p[0][1]);
    pk[qt].y = pack_bf16x2(p[0][2], p[0][3]);
    pk[qt].z = pack_bf16x2(p[1][0], p[1][1]);
    pk[qt].w = pack_bf16x2(p[1][2], p[1][3]);
  }
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    bf16x8 vf;
    if constexpr (FP8CTX) {
      const uint8_t *base = (const uint8_t *)(slot + (G::KS + dt / 2) * 64);
      const uint8_t *p = base + (((dt & 1) * 32 + (gq >> 1) * 16 + (lane & 15)) * 16) + 8 * (gq & 1);
      vf = as_bf16x8(e4m3x8_to_bf16x8(*(const uint2 *)p));
    } else {
      vf = as_bf16x8(slot[(2 * G::KS + dt) * 64 + lane]);
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (qt >= nqt) continue;
      w.o[qt][dt] = mfma16x16x32(vf, as_bf16x8(pk[qt]), w.o[qt][dt] * alpha[qt]);
    }
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  using G = Geom<D, FP8>;
  using GB = Geom<D, false>;
  constexpr int NS = G::NSTAGE;
  __shared__ uint4 ring[NS][G::CF * 64];
  __shared__ uint4 blkt[GB::BF * 64];
  __shared__ int32_t s_bt[2 * MAX_TPS];

  const int s = blockIdx.z, g = blockIdx.y, c = blockIdx.x;
  const AttnSeq sq = a.seq[s];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int gq = lane >> 4, r16 = lane & 15;
  const int R = a.rep * a.gamma;
  const bool has_ctx = sq.win_start < sq.ctx_len;
  const int p0 = has_ctx ? (sq.win_start >> 4) << 4 : 0;
  const int T = has_ctx ? (sq.ctx_len - p0 + KT - 1) / KT : 0;
  const int t0 = c * a.tps, nt = max(0, min(T, t0 + a.tps) - t0);
  const bool last = c == a.max_splits - 1;
  const int NBT = (a.gamma + KT - 1) / KT;

  if constexpr (D < 32) {
    // lanes whose dims are past head_dim load nothing: their LDS stays zero
    uint4 *z = &ring[0][0];
    for (int i = threadIdx.x; i < NS * G::CF * 64; i += 256) z[i] = uint4{0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < GB::BF * 64; i += 256) blkt[i] = uint4{0u, 0u, 0u, 0u};
  }
  {
    // block ids of this split's tiles; blocks past the sequence reuse its
    // last block (their keys are masked)
    const int nbv = (sq.ctx_len + 15) >> 4;
    for (int i = threadIdx.x; i < 2 * nt; i += 256) s_bt[i] = sq.bt[min((p0 >> 4) + 2 * t0 + i, nbv - 1)];
  }

  // Q fragments (B operand of S^T): query column r16 of this wave's tiles
  const int nqt = min(2, max(0, (R - wave * 32 + 15) / 16));
  bf16x8 qf[2][GB::KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = min((wave * 2 + qt) * 16 + r16, R - 1);
    const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
    const uint16_t *qrow = a.qkv + (size_t)(s * a.gamma + j) * a.ld + hq * D;
#pragma unroll
    for (int ks = 0; ks < GB::KS; ++ks) {
      const int dd = kdim<D>(ks, gq);
      qf[qt][ks] = as_bf16x8(dd < D ? *(const uint4 *)(qrow + dd) : uint4{0u, 0u, 0u, 0u});
    }
  }

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (FP8) {
    kscale = a.kv_scale[(a.layer * 2 + 0) * a.n_kv + g];
    vscale = a.kv_scale[(a.layer * 2 + 1) * a.n_kv + g];
  }
  const float sc_blk = LOG2E / sqrtf((float)D);
  const float sc_ctx = sc_blk * kscale;

  WaveState<D> w;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    w.m[qt] = -__builtin_huge_valf();
    w.l[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < GB::DT; ++dt) w.o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // s_bt, zeroed LDS

  TileSrc src;
  src.pool = (const uint8_t *)a.pool;
  src.head_bytes = (size_t)DFLASH_KV_BLOCK * D * (FP8 ? 1 : 2);
  src.L = a.L;
  src.layer = a.layer;
  src.n_kv = a.n_kv;
  src.g = g;
  const uint32_t ring0 = lds_addr(&ring[0][0]), blk0 = lds_addr(blkt);
  constexpr uint32_t SLOT_BYTES = G::CF * 1024;
  auto issue_tile = [&](int t, int slot_idx) {
    src.bA = s_bt[2 * t];
    src.bB = s_bt[2 * t + 1];
    issue_ctx<D, FP8>(src, ring0 + slot_idx * SLOT_BYTES, wave, lane);
  };

  if (last) issue_block<D>(a, s, g, 0, blk0, wave, lane);
  if (nt > 0)
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue_tile(min(j, nt - 1), j);

  if (last) {
    for (int bt = 0; bt < NBT; ++bt) {
      if (bt == 0) {
        if (nt > 0) wait_vm<(NS - 1) * G::PW>();
        else wait_vm<0>();
      } else {
        lds_barrier();  // everyone is done with the previous block tile
        issue_block<D>(a, s, g, bt, blk0, wave, lane);
        wait_vm<0>();
      }
      lds_barrier();
      const int nvalid = min(KT, a.gamma - 32 * bt);
      tile_step<D, false>(blkt, qf, nqt, [&](int kt) { return kt < nvalid; }, sc_blk, 1.0f, w, lane);
    }
  }

  const int pos_base = p0 + t0 * KT;
#pragma unroll 1
  for (int t = 0; t < nt; ++t) {
    wait_vm<(NS - 2) * G::PW>();
    lds_barrier();
    issue_tile(min(t + NS - 1, nt - 1), (t + NS - 1) % NS);
    const int pos0 = pos_base + t * KT;
    const int lo = sq.win_start - pos0, hi = sq.ctx_len - pos0;
    tile_step<D, FP8>(&ring[t % NS][0], qf, nqt, [&](int kt) { return kt >= lo && kt < hi; }, sc_ctx,
                      FP8 ? vscale : 1.0f, w, lane);
  }
  wait_vm<0>();

  // partial (O, max, sum) of this split, or the output with one split
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l_tot = w.l[qt];
    l_tot += __shfl_xor(l_tot, 16, WAVE);
    l_tot += __shfl_xor(l_tot, 32, WAVE);
    const int q = (wave * 2 + qt) * 16 + r16;
    if (qt >= nqt || q >= R) continue;
    if (a.max_splits == 1) {
      const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
      uint16_t *out = a.out + (size_t)(s * a.gamma + j) * a.out_ld + hq * D;
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int dt = 0; dt < GB::DT; ++dt) {
        const f32x4 v = w.o[qt][dt];
        *(uint2 *)(out + dt * 16 + 4 * gq) = uint2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
      }
    } else {
      const size_t part = ((size_t)(s * a.n_kv + g) * a.max_splits + c) * R + q;
#pragma unroll
      for (int dt = 0; dt < GB::DT; ++dt) *(f32x4 *)(a.o_part + part * D + dt * 16 + 4 * gq) = w.o[qt][dt];
      if (gq == 0) {
        a.ml_part[part * 2 + 0] = w.m[qt];
        a.ml_part[part * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge the splits of one query row per wave: lane s reads split s's (max,
// sum); the weights exp2(m_s - M) are shared by shuffles and every lane
// accumulates its dimensions over the splits in order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int n_seq) {
  constexpr int DPL = D >= 64 ? D / 64 : 1;  // dims per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int R = a.rep * a.gamma;
  const int row = blockIdx.x * 4 + wave;  // (s, g, q)
  if (row >= n_seq * a.n_kv * R) return;
  const int q = row % R, g = (row / R) % a.n_kv, s = row / (R * a.n_kv);
  const int nsplit = a.max_splits;  // <= 64
  const size_t base = (size_t)(s * a.n_kv + g) * nsplit;
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

template <int D, bool FP8>
hipError_t launch_d(const AttnArgs &a, int n_seq, hipStream_t s) {
  dim3 grid(a.max_splits, a.n_kv, n_seq), block(256);
  hipLaunchKernelGGL((k_attn<D, FP8>), grid, block, 0, s, a);
  if (a.max_splits > 1) {
    const int rows = n_seq * a.n_kv * a.rep * a.gamma;
    hipLaunchKernelGGL(k_attn_combine<D>, dim3((rows + 3) / 4), block, 0, s, a, n_seq);
  }
  return hipGetLastError();
}

}  // namespace

int attn_max_tiles_per_split() { return MAX_TPS; }

hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s) {
  if (a.tps < 1 || a.tps > MAX_TPS || a.max_splits < 1 || a.max_splits > 64 || a.gamma > 64 ||
      a.rep * a.gamma > 128)
    return hipErrorInvalidValue;
  if (a.kv_fp8) {
    switch (a.head_dim) {
      case 64: return launch_d<64, true>(a, n_seq, s);
      case 128: return launch_d<128, true>(a, n_seq, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 16: return launch_d<16, false>(a, n_seq, s);
    case 32: return launch_d<32, false>(a, n_seq, s);
    case 64: return launch_d<64, false>(a, n_seq, s);
    case 128: return launch_d<128, false>(a, n_seq, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dflash
