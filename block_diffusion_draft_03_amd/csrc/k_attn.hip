// k_attn.hip - GQA attention of the block rows over the paged ctx window and
// the block itself, for gfx950.
//
// One workgroup (NWAVE waves) per (split, kv head); a sequence has as many splits
// as its own context needs, so short sequences take no idle workgroups.
// Workgroups start split by split in the planner's numbering, which puts the
// sequences with the longest splits first. The rep = n_q / n_kv
// query heads of the kv head times the gamma block rows form up to 128 query
// rows, 16 QT per wave. Keys come in tiles of 32: ctx tiles are aligned to two
// 16-row KV blocks (positions outside [win_start, ctx_len) are masked), and
// the gamma block rows form the block tile(s), whose K rows come straight
// from the QKV output and whose V^T from the copy the QKV epilogue writes.
// A sequence's ctx tiles and its block tile(s), counted as two more tiles,
// are divided evenly among its splits; the last split owns the block tile(s).
//
// The pool stores K row-major and V transposed ([dim][16 slots]) per block,
// so every 16-byte piece of an MFMA fragment is contiguous in global memory.
// Direct-to-LDS loads copy one 1 KB fragment per wave instruction (no
// register staging); the four lanes of each quad load 64 contiguous bytes (one
// K row segment, or two V^T rows), and the piece order keeps the 128-bit
// fragment reads from LDS free of bank conflicts (an XOR swizzle for K). Ctx tiles stream
// through a ring of NSTAGE LDS slots with NSTAGE - 1 tiles in flight.
//
// Products are transposed so every per-query quantity stays in one lane:
// S^T = K Q^T (MFMA A = 16 keys x 32 dims, B = Q^T). The 16 MFMA rows of key
// sub-tile u hold keys (r / 4) * 8 + 4u + r % 4, so lane group g ends with
// the scores of keys 8g .. 8g+7 for its query; those are exactly the B
// operand of O^T = V^T P^T, whose A operand (16 dims x keys 8g .. 8g+7) is a
// 16-byte piece of V^T. Online softmax in base 2. Both products run on the
// fp16 matrix cores (f32 accumulation): the block rows' Q, K and V come from
// the QKV epilogue as fp16, a bf16 ctx tile is widened to fp16 in LDS by the
// waves that loaded it, an E4M3 ctx tile is decoded once per workgroup (each
// wave its own fragments) into an fp16 LDS tile of the block-tile layout,
// and P is rounded to fp16 (three more significand bits than bf16 at every
// step). With an E4M3 cache O accumulates ctx V in code units (the block
// tile's P is divided by the V scale) and is multiplied by the scale at the
// end, and the softmax base of the ctx tiles moves only when a score exceeds
// it by more than 2^8 (the loop is bound by VALU work: the decode and the
// rescale of O were most of it). With an E4M3 cache the K fragments of k-steps 2j and 2j+1
// take dims 64j + 16g .. +15 of lane group g (one 16-byte piece of an E4M3
// row), and Q (and the block tile's K) use the same dim order. Q and K also
// carry their head dims in RoPE pair order; every score is unchanged by these
// permutations.
//
// Each split writes its own normalised output (fp16, bounded by max |V|) with
// its max and sum (f32); the combine kernel merges them (one wave per query
// row) with weights exp2(m_s - M) l_s. With a single split the output is
// written directly.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

constexpr int KT = 32;          // keys per tile
constexpr int QT = 1;           // 16-row query tiles per wave
constexpr int NWAVE = 8 / QT;   // waves per workgroup (128 query rows)
constexpr int NTHR = 64 * NWAVE;
constexpr int MAX_TPS = 64;     // ctx tiles per split (2 KV blocks each)

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
  static constexpr int PW = (CF + NWAVE - 1) / NWAVE;         // ctx-tile loads per wave
  static constexpr int PB = (BF + NWAVE - 1) / NWAVE;         // block-tile loads per wave
  static constexpr int NSTAGE = FP8 ? 4 : 3;
  // a bf16 ctx tile is widened to fp16 in LDS by the waves that loaded it
  // (each fragment has exactly one loader when CF is a multiple of NWAVE)
  static constexpr bool CONV = !FP8 && CF % NWAVE == 0;
  // an E4M3 ctx tile is decoded once per workgroup, by the waves that loaded
  // it, into a double-buffered fp16 tile of the block-tile layout
  static constexpr bool WIDEN = FP8;
};

// First dim of the 8 that lane group gq holds in k-step ks.
template <bool PAIRED>
__device__ __forceinline__ int kdim(int ks, int gq) {
  if constexpr (PAIRED) return (ks & ~1) * 32 + 16 * gq + 8 * (ks & 1);
  else return 32 * ks + 8 * gq;
}

// LDS piece (16 bytes) of fragment row r (0..15), lane group gq, in a K
// fragment: the quad of row r holds its four pieces, XOR-swizzled by r / 2 so
// that 128-bit reads of the fragment are free of bank conflicts on gfx950
// (measured: 489 B/ns per CU against 292 with the swizzle by r / 4, 455-500
// for contiguous reads).
__device__ __forceinline__ int k_piece(int r, int gq) { return 4 * r + (gq ^ ((r >> 1) & 3)); }
// The K row / lane group loaded by DMA lane L (inverse of k_piece).
__device__ __forceinline__ int k_row_of(int L) { return L >> 2; }
__device__ __forceinline__ int k_gq_of(int L) { return (L & 3) ^ ((L >> 3) & 3); }

// LDS piece of a bf16 V^T fragment for dim d (0..15) and lane group gq (keys
// 8gq .. 8gq+7: block gq / 2, half gq % 2): the quad of dims (2k, 2k+1)
// holds both halves of both rows, unswizzled (128-bit reads conflict-free:
// 494 B/ns per CU, against 292 with the halves swapped by d / 8).
__device__ __forceinline__ int v_piece(int d, int gq) { return (gq >> 1) * 32 + 2 * d + (gq & 1); }
__device__ __forceinline__ void v_of(int L, int &blk, int &d, int &half) {
  blk = L >> 5;
  d = (L & 31) >> 1;
  half = L & 1;
}

// Key within the tile held by MFMA row r of sub-tile u.
__device__ __forceinline__ int key_of(int u, int r) { return (r >> 2) * 8 + 4 * u + (r & 3); }

// This wave's share of the loads of a ctx tile, fixed for the whole kernel:
// item j is fragment dst[j] of the slot, read from the K (kv = 0) or V^T
// (kv = 1) tile of block A or B (per lane) at lane byte offset off[j].
template <int D, bool FP8>
struct IssuePlan {
  static constexpr int PW = Geom<D, FP8>::PW;
  uint32_t off[PW], dst[PW];
  int kv[PW];
  bool selB[PW], act[PW];
};

template <int D, bool FP8>
__device__ __forceinline__ IssuePlan<D, FP8> make_issue_plan(int wave, int lane) {
  using G = Geom<D, FP8>;
  IssuePlan<D, FP8> p;
  constexpr int EB = FP8 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < G::PW; ++j) {
    const int i = (wave + NWAVE * j) % G::CF;  // duplicates reload an item with the same bytes
    p.dst[j] = i * 1024;
    p.act[j] = true;
    if (i < (FP8 ? G::KS : 2 * G::KS)) {
      // K: this lane loads row k_row_of(lane), lane group k_gq_of(lane)
      const int r = k_row_of(lane), gq = k_gq_of(lane);
      int u, dim;
      if constexpr (FP8) {
        u = i / (G::KS / 2);
        dim = kdim<true>(2 * (i % (G::KS / 2)), gq);
      } else {
        u = i / G::KS;
        dim = kdim<false>(i % G::KS, gq);
        p.act[j] = dim < D;
      }
      const int kt = key_of(u, r);
      p.kv[j] = 0;
      p.selB[j] = kt >= 16;
      p.off[j] = ((kt & 15) * D + (dim < D ? dim : 0)) * EB;
    } else {
      int dim, slot0;
      if constexpr (FP8) {
        dim = (2 * (i - G::KS) + (lane >> 5)) * 16 + (lane & 15);
        p.selB[j] = (lane >> 4) & 1;
        slot0 = 0;
      } else {
        int blk, d, half;
        v_of(lane, blk, d, half);
        dim = (i - 2 * G::KS) * 16 + d;
        p.selB[j] = blk;
        slot0 = 8 * half;
      }
      p.kv[j] = 1;
      p.off[j] = (dim * 16 + slot0) * EB;
    }
  }
  return p;
}

struct TileSrc {
  const uint8_t *pool;
  size_t head_bytes;   // bytes of one (block, layer, K|V, kv head) tile
  int L, layer, n_kv, g;
};

// Issue this wave's direct-to-LDS loads of the ctx tile on blocks (bA, bB).
template <int D, bool FP8>
__device__ __forceinline__ void issue_ctx(const TileSrc &t, const IssuePlan<D, FP8> &p, int32_t bA, int32_t bB,
                                          uint32_t slot) {
  const size_t stride = (size_t)t.n_kv * t.head_bytes;  // K -> V of one (block, layer)
  const uint8_t *kA = t.pool + (((size_t)bA * t.L + t.layer) * 2 * t.n_kv + t.g) * t.head_bytes;
  const uint8_t *kB = t.pool + (((size_t)bB * t.L + t.layer) * 2 * t.n_kv + t.g) * t.head_bytes;
#pragma unroll
  for (int j = 0; j < IssuePlan<D, FP8>::PW; ++j) {
    const uint8_t *base = (p.selB[j] ? kB : kA) + (p.kv[j] ? stride : 0);
    if (p.act[j]) dma16(base + p.off[j], slot + p.dst[j]);
  }
}

// Issue this wave's loads of block tile bt (keys 32 bt .. of the gamma rows):
// K from the QKV rows (dims in the kernel's K order), V^T from the block
// copy [seq][kv][16-key block][dim][16].
template <int D, bool PAIRED>
__device__ __forceinline__ void issue_block(const AttnArgs &a, int s, int g, int bt, uint32_t slot, int wave,
                                            int lane) {
  using G = Geom<D, false>;
  const int nb16 = ((a.gamma + 31) & ~31) / 16;
#pragma unroll
  for (int j = 0; j < G::PB; ++j) {
    const int i = (wave + NWAVE * j) % G::BF;
    const uint16_t *src;
    bool active = true;
    if (i < 2 * G::KS) {
      const int r = k_row_of(lane), gq = k_gq_of(lane);
      const int u = i / G::KS, dim = kdim<PAIRED>(i % G::KS, gq);
      active = dim < D;
      const int tok = min(32 * bt + key_of(u, r), a.gamma - 1);
      src = a.qkv + (size_t)(s * a.gamma + tok) * a.ld + a.k_off + g * D + (active ? dim : 0);
    } else {
      int blk, d, half;
      v_of(lane, blk, d, half);
      const int dim = (i - 2 * G::KS) * 16 + d;
      src = a.vtb + ((((size_t)(s * a.n_kv + g) * nb16 + 2 * bt + blk) * D + dim) * 16 + 8 * half);
    }
    if (active) dma16(src, slot + i * 1024);
  }
}

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column's four lane
// groups), by the gfx950 row swaps instead of LDS permutes.
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint2 q) {
  const uint2 lo = e4m3x4_to_f16x4(q.x), hi = e4m3x4_to_f16x4(q.y);
  return as_f16x8(uint4{lo.x, lo.y, hi.x, hi.y});
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u) {
  return uint4{bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y), bf16x2_to_f16x2(u.z), bf16x2_to_f16x2(u.w)};
}

// What a tile slot holds: fp16 (the block tile, or a bf16 ctx tile already
// widened in place), bf16 (widened to fp16 as its fragments are read) or
// E4M3 codes (decoded to fp16 as they are read).
enum TileFmt { T_F16 = 0, T_BF16 = 1, T_E4M3 = 2 };

template <int D>
struct WaveState {
  f32x4 o[QT][Geom<D, false>::DT];
  float m[QT], l[QT];
};

// One tile for this wave's query tiles. `valid` says whether key kt of the
// tile takes part; sc scales the raw scores into base-2 units; P is
// multiplied by ps before it meets V (1 / V scale on the block tile of an
// E4M3 cache, whose ctx V stays in code units until the end). Both products
// run on the fp16 matrix cores with f32 accumulation.
template <int D, int FMT, bool LAZY = false, class Valid>
__device__ __forceinline__ void tile_step(const uint4 *slot, const f16x8 (&qf)[QT][Geom<D, false>::KS], bool full,
                                          Valid valid, float sc, float ps, WaveState<D> &w, int lane) {
  using G = Geom<D, FMT == T_E4M3>;
  const int gq = lane >> 4;
  f16x8 kf[2][G::KS];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const int piece = k_piece(lane & 15, gq);
      if constexpr (FMT == T_E4M3) {
        const uint8_t *p = (const uint8_t *)(slot + (u * (G::KS / 2) + ks / 2) * 64 + piece) + 8 * (ks & 1);
        kf[u][ks] = e4m3x8_to_f16x8(*(const uint2 *)p);
      } else if constexpr (FMT == T_BF16) {
        kf[u][ks] = as_f16x8(bf16x8_to_f16x8(slot[(u * G::KS + ks) * 64 + piece]));
      } else {
        kf[u][ks] = as_f16x8(slot[(u * G::KS + ks) * 64 + piece]);
      }
    }
  uint4 pk[QT];
  float alpha[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) sacc[u] = mfma16x16x32_f16(kf[u][ks], qf[qt][ks], sacc[u]);
    }
    // raw scores; sc > 0, so the max commutes with the scaling
    float x[2][4];
    if (!full) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[u][r] = valid(8 * gq + 4 * u + r) ? sacc[u][r] : -__builtin_huge_valf();
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[u][r] = sacc[u][r];
    }
    float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    tmax = max_lane_groups(tmax);
    float m_new = fmaxf(w.m[qt], tmax * sc);
    // LAZY: the base moves only when the max exceeds it by more than 2^8 (p
    // stays below 256: fp16 P loses nothing, f32 O and l take the scale)
    if constexpr (LAZY) m_new = m_new - w.m[qt] > 8.0f ? m_new : w.m[qt];
    alpha[qt] = fast_exp2(w.m[qt] - m_new);
    float p[2][4], psum = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(fmaf(x[u][r], sc, -m_new));
        psum += e;
        p[u][r] = e * ps;
      }
    w.l[qt] = w.l[qt] * alpha[qt] + psum;
    w.m[qt] = m_new;
    pk[qt].x = pack_f16x2(p[0][0], p[0][1]);
    pk[qt].y = pack_f16x2(p[0][2], p[0][3]);
    pk[qt].z = pack_f16x2(p[1][0], p[1][1]);
    pk[qt].w = pack_f16x2(p[1][2], p[1][3]);
  }
  // rescale O only when some lane's running max moved (alpha == 1 is exact)
  bool moved = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) moved = moved || alpha[qt] != 1.0f;
  if (__any(moved)) {
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) w.o[qt][dt] *= alpha[qt];
  }
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    f16x8 vf;
    if constexpr (FMT == T_E4M3) {
      const uint8_t *base = (const uint8_t *)(slot + (G::KS + dt / 2) * 64);
      const uint8_t *p = base + (((dt & 1) * 32 + (gq >> 1) * 16 + (lane & 15)) * 16) + 8 * (gq & 1);
      vf = e4m3x8_to_f16x8(*(const uint2 *)p);
    } else if constexpr (FMT == T_BF16) {
      vf = as_f16x8(bf16x8_to_f16x8(slot[(2 * G::KS + dt) * 64 + v_piece(lane & 15, gq)]));
    } else {
      vf = as_f16x8(slot[(2 * G::KS + dt) * 64 + v_piece(lane & 15, gq)]);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) w.o[qt][dt] = mfma16x16x32_f16(vf, as_f16x8(pk[qt]), w.o[qt][dt]);
  }
}

// Decode the E4M3 ctx-tile fragments this wave loaded (items wave,
// wave + NWAVE, ... below CF: one owner each) into the fp16 tile `dst`, laid
// out as a block tile: K fragment (u, k-step pair j) piece L becomes fp16 K
// fragments (u, 2j) and (u, 2j + 1) at piece L; V fragment pair p, whose
// piece L holds 8 + 8 codes of dim 16 (2p + L / 32) + L % 16 for keys
// 16 ((L / 16) % 2) + 0..7 and + 8..15, becomes fp16 V^T fragment 2p + L / 32
// at the block tile's pieces of those key groups.
template <int D>
__device__ __forceinline__ void widen_e4m3(const uint4 *ring_slot, uint4 *dst, int wave, int lane) {
  using G = Geom<D, true>;
#pragma unroll
  for (int j = 0; j < G::PW; ++j) {
    const int i = wave + NWAVE * j;
    if (i >= G::CF) continue;
    const uint4 q = ring_slot[i * 64 + lane];
    const uint2 a0 = e4m3x4_to_f16x4(q.x), a1 = e4m3x4_to_f16x4(q.y);
    const uint2 b0 = e4m3x4_to_f16x4(q.z), b1 = e4m3x4_to_f16x4(q.w);
    const uint4 lo = uint4{a0.x, a0.y, a1.x, a1.y}, hi = uint4{b0.x, b0.y, b1.x, b1.y};
    if (i < G::KS) {
      const int u = i / (G::KS / 2), jp = i % (G::KS / 2);
      dst[(u * G::KS + 2 * jp) * 64 + lane] = lo;
      dst[(u * G::KS + 2 * jp + 1) * 64 + lane] = hi;
    } else {
      const int dt = 2 * (i - G::KS) + (lane >> 5), d = lane & 15, gh = (lane >> 4) & 1;
      uint4 *v = dst + (2 * G::KS + dt) * 64;
      v[v_piece(d, 2 * gh)] = lo;
      v[v_piece(d, 2 * gh + 1)] = hi;
    }
  }
}

template <int D, bool FP8, int NS = Geom<D, FP8>::NSTAGE>
__global__ __launch_bounds__(NTHR, 2) void k_attn(AttnArgs a) {
  using G = Geom<D, FP8>;
  using GB = Geom<D, false>;
  __shared__ uint4 ring[NS][G::CF * 64];
  // fp16 tiles: the block tile, and with an E4M3 cache the two decoded ctx
  // tiles (the block tile shares the second, which tile 1 first overwrites
  // after every wave has passed tile 0's barrier)
  constexpr int NFB = G::WIDEN ? 2 : 1;
  __shared__ uint4 fb[NFB][GB::BF * 64];
  uint4 *const blkt = fb[NFB - 1];
  __shared__ int32_t s_bt[2 * (MAX_TPS + 1)];

  const int flat = blockIdx.y, g = blockIdx.x;
  const int s = a.split_seq[flat];
  const AttnSeq sq = a.seq[s];
  const int c = flat - sq.split0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int gq = lane >> 4, r16 = lane & 15;
  const int R = a.rep * a.gamma;
  const bool has_ctx = sq.win_start < sq.ctx_len;
  const int p0 = has_ctx ? (sq.win_start >> 4) << 4 : 0;
  const int T = has_ctx ? (sq.ctx_len - p0 + KT - 1) / KT : 0;
  // the sequence's T ctx tiles and its block tile, which costs about two
  // (its own load, ahead of the ctx loop), are divided evenly among its
  // splits: T + 2 units, the last split owning the block tile. The planner
  // sized the splits for T + 1 units of at most tps, so a split holds at most
  // tps + 1 ctx tiles.
  const int U = T + 2;
  const int t0 = (int)((int64_t)c * U / sq.nsplit), t1 = min(T, (int)((int64_t)(c + 1) * U / sq.nsplit));
  const int nt = max(0, t1 - t0);
  const bool last = c == sq.nsplit - 1;
  const int NBT = (a.gamma + KT - 1) / KT;

  if constexpr (D < 32) {
    // lanes whose dims are past head_dim load nothing: their LDS stays zero
    uint4 *z = &ring[0][0];
    for (int i = threadIdx.x; i < NS * G::CF * 64; i += NTHR) z[i] = uint4{0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < NFB * GB::BF * 64; i += NTHR) (&fb[0][0])[i] = uint4{0u, 0u, 0u, 0u};
  }
  // Q fragments (B operand of S^T): query column r16 of this wave's tiles
  // (rows past R repeat row R - 1 and are not written), loaded first so that
  // their latency overlaps the block table's
  f16x8 qf[QT][GB::KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = min((wave * QT + qt) * 16 + r16, R - 1);
    const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
    const uint16_t *qrow = a.qkv + (size_t)(s * a.gamma + j) * a.ld + hq * D;
#pragma unroll
    for (int ks = 0; ks < GB::KS; ++ks) {
      const int dd = kdim<FP8>(ks, gq);
      qf[qt][ks] = as_f16x8(dd < D ? *(const uint4 *)(qrow + dd) : uint4{0u, 0u, 0u, 0u});
    }
  }

  {
    // block ids of this split's tiles; blocks past the sequence reuse its
    // last block (their keys are masked)
    const int nbv = (sq.ctx_len + 15) >> 4;
    for (int i = threadIdx.x; i < 2 * nt; i += NTHR) s_bt[i] = sq.bt[min((p0 >> 4) + 2 * t0 + i, nbv - 1)];
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
  for (int qt = 0; qt < QT; ++qt) {
    w.m[qt] = -__builtin_huge_valf();
    w.l[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < GB::DT; ++dt) w.o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // s_bt, zeroed LDS
  // The Q loads complete here, before any direct-to-LDS load is issued. The
  // tile loads are assembly, which the compiler does not see but the hardware
  // counts: a Q load still pending in the compiler's view would make it wait
  // for vmcnt(0) inside the tile loop, i.e. for every tile in flight.
  wait_vm<0>();

  TileSrc src;
  src.pool = (const uint8_t *)a.pool;
  src.head_bytes = (size_t)DFLASH_KV_BLOCK * D * (FP8 ? 1 : 2);
  src.L = a.L;
  src.layer = a.layer;
  src.n_kv = a.n_kv;
  src.g = g;
  const uint32_t ring0 = lds_addr(&ring[0][0]), blk0 = lds_addr(blkt);
  constexpr uint32_t SLOT_BYTES = G::CF * 1024;
  const IssuePlan<D, FP8> plan = make_issue_plan<D, FP8>(wave, lane);
  auto issue_tile = [&](int t, int slot_idx) {
    const int32_t bA = __builtin_amdgcn_readfirstlane(s_bt[2 * t]);
    const int32_t bB = __builtin_amdgcn_readfirstlane(s_bt[2 * t + 1]);
    issue_ctx<D, FP8>(src, plan, bA, bB, ring0 + slot_idx * SLOT_BYTES);
  };

  if (last) issue_block<D, FP8>(a, s, g, 0, blk0, wave, lane);
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
        issue_block<D, FP8>(a, s, g, bt, blk0, wave, lane);
        wait_vm<0>();
      }
      lds_barrier();
      const int nvalid = min(KT, a.gamma - 32 * bt);
      // with an E4M3 cache O is kept in V-code units (times vscale at the end)
      tile_step<D, T_F16>(blkt, qf, nvalid >= KT, [&](int kt) { return kt < nvalid; }, sc_blk,
                          FP8 ? 1.0f / vscale : 1.0f, w, lane);
    }
  }

  const int pos_base = p0 + t0 * KT;
#pragma unroll 1
  for (int t = 0; t < nt; ++t) {
    wait_vm<(NS - 2) * G::PW>();
    if constexpr (G::CONV) {
      // this wave's own fragments of tile t, bf16 -> fp16 in place, then
      // published by the barrier
      asm volatile("" ::: "memory");
      uint4 *sl = &ring[t % NS][0];
#pragma unroll
      for (int j = 0; j < G::PW; ++j) {
        uint4 *q = sl + (plan.dst[j] >> 4) + lane;
        *q = bf16x8_to_f16x8(*q);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    if constexpr (G::WIDEN) {
      // this wave's own fragments of tile t, E4M3 -> fp16 into fp16 tile
      // t % 2 (whose last readers, at tile t - 2, have all passed tile t - 1's
      // barrier), then published by the barrier
      asm volatile("" ::: "memory");
      widen_e4m3<D>(&ring[t % NS][0], fb[t & 1], wave, lane);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    lds_barrier();
    issue_tile(min(t + NS - 1, nt - 1), (t + NS - 1) % NS);
    const int pos0 = pos_base + t * KT;
    const int lo = sq.win_start - pos0, hi = sq.ctx_len - pos0;
    constexpr int FMT = G::WIDEN || G::CONV ? T_F16 : FP8 ? T_E4M3 : T_BF16;
    tile_step<D, FMT, G::WIDEN>(G::WIDEN ? fb[t & 1] : &ring[t % NS][0], qf, lo <= 0 && hi >= KT,
                      [&](int kt) { return kt >= lo && kt < hi; }, sc_ctx, 1.0f, w, lane);
  }
  wait_vm<0>();

  // partial (O, max, sum) of this split, or the output with one split
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l_tot = w.l[qt];
    l_tot += __shfl_xor(l_tot, 16, WAVE);
    l_tot += __shfl_xor(l_tot, 32, WAVE);
    const int q = (wave * QT + qt) * 16 + r16;
    if (q >= R) continue;
    if (sq.nsplit == 1) {
      const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
      uint16_t *out = a.out + (size_t)(s * a.gamma + j) * a.out_ld + hq * D;
      const float inv = vscale / l_tot;  // vscale 1 without an E4M3 cache
#pragma unroll
      for (int dt = 0; dt < GB::DT; ++dt) {
        const f32x4 v = w.o[qt][dt];
        *(uint2 *)(out + dt * 16 + 4 * gq) = uint2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
      }
    } else {
      const size_t part = ((size_t)g * a.n_split + flat) * R + q;
#pragma unroll
      for (int dt = 0; dt < GB::DT; ++dt) {
        const f32x4 v = w.o[qt][dt];
        const float nrm = vscale / l_tot;  // the split's own softmax output, |O| <= max |V|
        *(uint2 *)(a.o_part + part * D + dt * 16 + 4 * gq) = uint2{pack_f16x2(v[0] * nrm, v[1] * nrm), pack_f16x2(v[2] * nrm, v[3] * nrm)};
      }
      if (gq == 0) {
        a.ml_part[part * 2 + 0] = w.m[qt];
        a.ml_part[part * 2 + 1] = l_tot;
      }
    }
  }
}

// Reduction over the 16 lanes of each DPP row (lanes 16k .. 16k + 15): quad
// permutes, then row rotates. Every lane of the row ends with the result; the
// order is fixed.
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));   // quad_perm [1, 0, 3, 2]
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));   // quad_perm [2, 3, 0, 1]
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror 4
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror 8
  return x;
}

// Merge the splits of four query rows per wave, one 16-lane row group per
// row. Lane l of a group reads the (max, sum) of splits l, l + 16, ... and
// holds dims DPL l .. DPL l + DPL - 1 (DPL = head_dim / 16) of every split's
// output; the row's maximum M and the sum of the weights exp2(m_s - M) l_s
// come from reductions inside the group, each split's weight from the lane
// that holds it. The outputs of the first PRE splits are loaded together
// with the (max, sum) pairs, before the weights are known; splits are added
// in order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int n_seq) {
  constexpr int DPL = D / 16;                  // dims per lane
  constexpr int NW = DPL >= 2 ? DPL / 2 : 1;   // 32-bit words of fp16 per lane and split
  constexpr int PRE = 16;
  constexpr int SL = ATTN_MAX_SPLITS / 16;     // (max, sum) slots per lane
  static_assert(SL == 4, "the weight sum pairs four 16-split slots");
  static_assert(D % 16 == 0, "head_dim a multiple of 16");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sl = lane & 15;
  const int R = a.rep * a.gamma;
  const int rows = n_seq * a.n_kv * R;
  const int row = (blockIdx.x * 4 + wave) * 4 + (lane >> 4);  // (s, g, q)
  const int rowc = min(row, rows - 1);
  const int q = rowc % R, g = (rowc / R) % a.n_kv, s = rowc / (R * a.n_kv);
  const int nsplit = a.seq[s].nsplit;  // <= 64
  // a row with one split was written by the attention kernel
  const int ns = (row < rows && nsplit > 1) ? nsplit : 0;
  const size_t base = (size_t)g * a.n_split + a.seq[s].split0;
  auto o_bits = [&](int c, uint32_t (&b)[NW]) {
    const uint16_t *op = a.o_part + ((base + c) * R + q) * D + DPL * sl;
    if constexpr (DPL == 8) {
      const uint4 v = *(const uint4 *)op;
      b[0] = v.x, b[1] = v.y, b[2] = v.z, b[3] = v.w;
    } else if constexpr (DPL == 4) {
      const uint2 v = *(const uint2 *)op;
      b[0] = v.x, b[1] = v.y;
    } else if constexpr (DPL == 2) {
      b[0] = *(const uint32_t *)op;
    } else {
      b[0] = *op;
    }
  };
  auto widen = [&](const uint32_t (&b)[NW], float (&v)[DPL]) {
    if constexpr (DPL == 1) {
      v[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)b[0]);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const f16x2_t x = __builtin_bit_cast(f16x2_t, b[i]);
        v[2 * i] = (float)x[0];
        v[2 * i + 1] = (float)x[1];
      }
    }
  };
  uint32_t pre[PRE][NW];
#pragma unroll
  for (int c = 0; c < PRE; ++c) {
#pragma unroll
    for (int i = 0; i < NW; ++i) pre[c][i] = 0u;
    if (c < ns) o_bits(c, pre[c]);
  }
  float mm[SL], ll[SL];
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    const int c = sl + 16 * k;
    mm[k] = -__builtin_huge_valf();
    ll[k] = 0.0f;
    if (c < ns) {
      mm[k] = a.ml_part[((base + c) * R + q) * 2];
      ll[k] = a.ml_part[((base + c) * R + q) * 2 + 1];
    }
  }
  float mx = mm[0];
#pragma unroll
  for (int k = 1; k < SL; ++k) mx = fmaxf(mx, mm[k]);
  const float M = row16_reduce<true>(mx);
  float w[SL], t[SL];
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    w[k] = sl + 16 * k < ns ? fast_exp2(mm[k] - M) * ll[k] : 0.0f;  // weight of split sl + 16 k
    t[k] = row16_reduce<false>(w[k]);
  }
  // splits 0..15, 16..31, 32..47, 48..63 each by the same 16-lane tree, then
  // the four sums pairwise
  const float den = (t[0] + t[1]) + (t[2] + t[3]);
  // the wave's largest split count (row groups may differ)
  int ns_max = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) ns_max = max(ns_max, __builtin_amdgcn_readlane(ns, 16 * r));
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  static_assert(PRE == 16, "the preloaded splits are the first weight slot");
#pragma unroll
  for (int c = 0; c < PRE; ++c) {
    const float wc = __shfl(w[0], (lane & 48) | c, WAVE);
    float v[DPL];
    widen(pre[c], v);
    if (c < ns)
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] += wc * v[i];
  }
  for (int c = PRE; c < ns_max; ++c) {
    const int k = c >> 4;  // wave-uniform
    const float wk = k == 1 ? w[1] : k == 2 ? w[2] : w[3];
    const float wc = __shfl(wk, (lane & 48) | (c & 15), WAVE);
    uint32_t b[NW];
    if (c < ns) {
      o_bits(c, b);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) b[i] = 0u;
    }
    float v[DPL];
    widen(b, v);
    if (c < ns)
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] += wc * v[i];
  }
  if (ns > 0) {
    const int hq = g * a.rep + q / a.gamma, j = q % a.gamma;
    uint16_t *out = a.out + (size_t)(s * a.gamma + j) * a.out_ld + hq * D + DPL * sl;
    if constexpr (DPL == 1) {
      out[0] = f32_to_bf16(acc[0] / den);
    } else {
      uint32_t o[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) o[i] = pack_bf16x2(acc[2 * i] / den, acc[2 * i + 1] / den);
      if constexpr (DPL == 8) *(uint4 *)out = uint4{o[0], o[1], o[2], o[3]};
      else if constexpr (DPL == 4) *(uint2 *)out = uint2{o[0], o[1]};
      else *(uint32_t *)out = o[0];
    }
  }
}

template <int D, bool FP8>
hipError_t launch_d(const AttnArgs &a, int n_seq, bool merge, hipStream_t s) {
  // kv heads fastest: workgroups start split by split, in the plan's order
  dim3 grid(a.n_kv, a.n_split);
  hipLaunchKernelGGL((k_attn<D, FP8>), grid, dim3(NTHR), 0, s, a);
  if (merge) {
    const int rows = n_seq * a.n_kv * a.rep * a.gamma;
    hipLaunchKernelGGL(k_attn_combine<D>, dim3((rows + 15) / 16), dim3(256), 0, s, a, n_seq);
  }
  return hipGetLastError();
}

}  // namespace

int attn_max_tiles_per_split() { return MAX_TPS; }

hipError_t launch_attention(const AttnArgs &a, int n_seq, hipStream_t s) {
  if (a.tps < 1 || a.tps > MAX_TPS || a.n_split < n_seq || a.n_split > ATTN_MAX_FLAT || a.gamma > 64 ||
      a.rep * a.gamma > 128 || n_seq < 1 || n_seq > DFLASH_MAX_BATCH)
    return hipErrorInvalidValue;
  // each sequence's splits are one run [split0, split0 + nsplit) mapped back
  // to it by split_seq; runs of distinct sequences cannot overlap, so runs
  // whose sizes add up to n_split cover [0, n_split) exactly
  bool merge = false;
  int total = 0;
  for (int i = 0; i < n_seq; ++i) {
    const AttnSeq &q = a.seq[i];
    if (q.nsplit < 1 || q.nsplit > 64 || q.split0 < 0 || q.split0 + q.nsplit > a.n_split) return hipErrorInvalidValue;
    for (int c = 0; c < q.nsplit; ++c)
      if (a.split_seq[q.split0 + c] != i) return hipErrorInvalidValue;
    total += q.nsplit;
    merge = merge || q.nsplit > 1;
  }
  if (total != a.n_split) return hipErrorInvalidValue;
  if (a.kv_fp8) {
    switch (a.head_dim) {
      case 64: return launch_d<64, true>(a, n_seq, merge, s);
      case 128: return launch_d<128, true>(a, n_seq, merge, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 16: return launch_d<16, false>(a, n_seq, merge, s);
    case 32: return launch_d<32, false>(a, n_seq, merge, s);
    case 64: return launch_d<64, false>(a, n_seq, merge, s);
    case 128: return launch_d<128, false>(a, n_seq, merge, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dflash
