// k_bgemm.hip - LDS-tiled MFMA GEMMs for many activation rows (batched
// propose) on gfx950.
//
// A workgroup computes a block of D^T = W A^T with v_mfma_f32_16x16x32_bf16:
// 128 x 128 (weight rows x activation rows) on 4 waves of 64 x 64 for the
// layer GEMMs, 256 x 256 on 8 waves of 128 x 64 for the LM head (larger wave
// tiles read fewer LDS bytes per MFMA). K advances in stages of 64 columns
// (half of one 128-wide step of the tile-major weight layout). A stage's
// weights are staged in LDS already in MFMA fragment order (they come from HBM
// in that order), so every weight fragment read is one contiguous 1 KB
// ds_read_b128 per wave. Activation rows are staged row-major, 128 bytes (64
// columns) per row, each load instruction bringing whole 128-byte row segments
// of 8 rows (rows scattered in 64-byte halves load at well under half the
// rate); the 16-byte chunks of a row are XOR-swizzled so that the fragment
// reads of 16 rows fall on distinct LDS banks. The next
// stage's global loads are in flight while the current stage is multiplied,
// each wave's loads issued between its matrix instructions; two LDS buffers,
// one barrier per stage.
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

// Workgroup tile: BN weight rows x BM activation rows on WAVES_N x WAVES_M
// waves, each wave multiplying WN weight tiles by WM activation tiles.
template <int BN_, int BM_, int WAVES_N_, int WAVES_M_>
struct Tiling {
  static constexpr int BN = BN_, BM = BM_;
  static constexpr int NT = BN / 16, MTL = BM / 16;   // 16-row tiles
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NWAVES = WAVES_N * WAVES_M, NTHR = 64 * NWAVES;
  static constexpr int WN = NT / WAVES_N, WM = MTL / WAVES_M;  // tiles per wave
  static_assert(NT % WAVES_N == 0 && MTL % WAVES_M == 0 && NWAVES % 2 == 0, "tiles divide among the waves");
};
// Layer GEMMs: 8 waves (two per SIMD, so one wave's multiplies cover the
// other's waits) on 128 x 128 or 256 x 128 blocks, whichever needs fewer
// rounds of workgroups over the chip; LM head: 8 waves of 128 x 64.
using TileG = Tiling<128, 128, 4, 2>;   // waves of 32 x 64
using TileW = Tiling<256, 128, 4, 2>;   // waves of 64 x 64
using TileL = Tiling<256, 256, 2, 4>;
using TileLW = Tiling<256, 256, 2, 4>;  // the E4M3-weight LM head (weights widened in registers)
using TileH = Tiling<192, 256, 2, 4>;   // waves of 96 x 64: layer GEMMs over many rows (fewer L2 bytes per product)
using TileQ = Tiling<160, 128, 2, 2>;   // 4 waves of 80 x 64: N = 32 x 160 (the QKV product) in one round

constexpr int NSTAGE_G = 4;            // LDS ring depth (stages in flight + the one multiplied): 128 KB
constexpr int NSTAGE_W = 3;            // 144 KB
constexpr int NSTAGE_LM = 2;
constexpr int NSTAGE_H = 2;             // 112 KB
constexpr int NSTAGE_Q = 4;             // 144 KB
constexpr int NUM_CUS = 256;           // compute units of the MI355X
constexpr int LM_TILES = 4;            // vocab blocks per LM-head workgroup

typedef __attribute__((address_space(3))) uint4 lds_uint4;
typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer resource of a global array of `bytes` bytes (offsets past the end
// read as zero).
__device__ __forceinline__ int4v make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  int4v r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

// One wave-wide direct-to-LDS load: lane l's 16 bytes at buffer offset
// voff + soff land at LDS byte address lds + 16 l (lds wave-uniform). Issued
// as assembly so that the only waits on it are the pipeline's explicit vmcnt
// waits (the compiler would drain every such load before any LDS read); m0
// is restored afterwards.
__device__ __forceinline__ void dma16(int4v r, uint32_t voff, uint32_t soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(soff), "s"(lds)
      : "memory");
}

// As dma16 with 4 bytes per lane (lane l's dword lands at lds + 4 l).
__device__ __forceinline__ void dma4(int4v r, uint32_t voff, uint32_t soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(soff), "s"(lds)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_uint4 *)(const uint4 *)p);
}

// A stage is a list of 1 KB pieces (64 lanes x 16 bytes): the weight
// fragments [tile][c] (bf16) or [tile] (E4M3: the 16 codes of k-groups c = 0
// and 1 of each lane), then the activation rows, 8 rows of 128 bytes per
// piece. Pieces are dealt to the waves round-robin (piece i * NWAVES + w to
// wave w), so every wave issues WP weight and AP activation loads per stage.
template <bool WFP8, class TL>
struct StageShape {
  static constexpr int WF = WFP8 ? TL::NT : TL::NT * 2;
  static constexpr int AF = TL::BM / 8;
  static constexpr int F = WF + AF;
  static constexpr int WP = WF / TL::NWAVES, AP = AF / TL::NWAVES;
  static constexpr int PER = WP + AP;  // loads per wave and stage
  static_assert(WF % TL::NWAVES == 0 && AF % TL::NWAVES == 0, "pieces divide among the waves");
};

// Per-lane offsets of a wave's loads, fixed for the whole K loop.
template <bool WFP8, class TL>
struct LoadPlan {
  int4v rw, ra;             // weight and activation buffers
  uint32_t w_base;          // byte offset of the block's first weight tile (step 0)
  uint32_t w_tile;          // bytes of one 16-row weight tile over all of K
  uint32_t w_step;          // bytes per 128-wide step of one tile
  uint32_t wv;              // lane offset inside a weight piece
  uint32_t va[StageShape<WFP8, TL>::AP];  // activation pieces: lane offset at column 0
};

template <bool WFP8, class TL>
__device__ __forceinline__ LoadPlan<WFP8, TL> make_plan(const void *W, size_t w_bytes, int steps_w, int tile0,
                                                        const uint16_t *A, int lda, int M, int m0, int wave,
                                                        int lane) {
  using S = StageShape<WFP8, TL>;
  LoadPlan<WFP8, TL> p;
  p.rw = make_rsrc(W, (uint32_t)w_bytes);
  p.ra = make_rsrc(A, (uint32_t)((size_t)M * lda * 2));
  p.w_step = WFP8 ? 2048u : 4096u;
  p.w_tile = (uint32_t)steps_w * p.w_step;
  p.w_base = (uint32_t)tile0 * p.w_tile;
  // bf16 piece i * NWAVES + w is k-group (w & 1) of its tile
  p.wv = (uint32_t)lane * 16 + (WFP8 ? 0u : (uint32_t)(wave & 1) * 1024);
#pragma unroll
  for (int i = 0; i < S::AP; ++i) {
    // lane l lands at LDS chunk l & 7 of local row `row`; it fetches the chunk that swizzles there
    const int row = 8 * (i * TL::NWAVES + wave) + (lane >> 3);
    const int m = min(m0 + row, M - 1);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    p.va[i] = (uint32_t)(((size_t)m * lda + 8 * chunk) * 2);
  }
  return p;
}

// Direct-to-LDS loads of the stage at absolute column k (a multiple of 64)
// into the slot at LDS byte address `slot`.
template <bool WFP8, class TL>
__device__ __forceinline__ void issue_stage(uint32_t slot, const LoadPlan<WFP8, TL> &p, int wave, int k) {
  using S = StageShape<WFP8, TL>;
  const uint32_t step_off = (uint32_t)(k >> 7) * p.w_step + (uint32_t)((k >> 6) & 1) * (p.w_step / 2);
#pragma unroll
  for (int i = 0; i < S::WP; ++i) {
    const int piece = i * TL::NWAVES + wave;
    const int tile = WFP8 ? piece : piece >> 1;
    dma16(p.rw, p.wv, p.w_base + (uint32_t)tile * p.w_tile + step_off, slot + piece * 1024);
  }
#pragma unroll
  for (int i = 0; i < S::AP; ++i)
    dma16(p.ra, p.va[i], (uint32_t)k * 2, slot + (S::WF + i * TL::NWAVES + wave) * 1024);
}

// The q-th of this wave's loads of the stage at column k (weights first,
// then activation rows), as issue_stage issues them.
template <bool WFP8, class TL>
__device__ __forceinline__ void issue_one(uint32_t slot, const LoadPlan<WFP8, TL> &p, int wave, int k, int q) {
  using S = StageShape<WFP8, TL>;
  if (q < S::WP) {
    const uint32_t step_off = (uint32_t)(k >> 7) * p.w_step + (uint32_t)((k >> 6) & 1) * (p.w_step / 2);
    const int piece = q * TL::NWAVES + wave;
    const int tile = WFP8 ? piece : piece >> 1;
    dma16(p.rw, p.wv, p.w_base + (uint32_t)tile * p.w_tile + step_off, slot + piece * 1024);
  } else {
    const int i = q - S::WP;
    dma16(p.ra, p.va[i], (uint32_t)k * 2, slot + (S::WF + i * TL::NWAVES + wave) * 1024);
  }
}

// A wave issues its loads of the next stage one at a time, one before every
// DMA_GAP of its matrix instructions, instead of all at once after the
// barrier: a direct-to-LDS load that cannot yet enter the memory pipeline
// holds up the wave's in-order issue, and issued in a burst by every wave
// together they kept the matrix cores idle (gate/up product at 1024 rows 6%
// faster, QKV 7%, with spacings 1, 2 and 4 measured).
constexpr int DMA_GAP = 2;

// Issue load q = n / DMA_GAP before product n of a stage (n counts the
// wave's products of the stage), fenced so the scheduler keeps the order.
template <int PER, class Issue>
__device__ __forceinline__ void issue_at(int n, Issue &issue) {
  if (n % DMA_GAP == 0 && n / DMA_GAP < PER) {
    __builtin_amdgcn_sched_barrier(0);
    issue(n / DMA_GAP);
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <int PER, int TOT, class Issue>
__device__ __forceinline__ void issue_rest(Issue &issue) {
#pragma unroll
  for (int q = (TOT + DMA_GAP - 1) / DMA_GAP; q < PER; ++q) issue(q);
}

// Wait until at most `later` stages of this wave's loads are outstanding.
template <bool WFP8, class TL>
__device__ __forceinline__ void wait_stages(int later) {
  constexpr int P = StageShape<WFP8, TL>::PER;
  // s_waitcnt vmcnt(n) with expcnt / lgkmcnt left at their maximum
#define DFL_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0xF70)
  if (later >= 3) DFL_VMCNT(3 * P);
  else if (later == 2) DFL_VMCNT(2 * P);
  else if (later == 1) DFL_VMCNT(P);
  else DFL_VMCNT(0);
#undef DFL_VMCNT
}

template <bool WFP8, class TL, class Issue>
__device__ __forceinline__ void mma_stage(const uint4 *slot, int wn, int wm, int lane,
                                          f32x4 (&acc)[TL::WN][TL::WM], Issue &issue) {
  constexpr int PER = StageShape<WFP8, TL>::PER;
  using S = StageShape<WFP8, TL>;
  constexpr int WN = TL::WN, WM = TL::WM;
  const int r16 = lane & 15, g = lane >> 4, swz = (r16 >> 1) & 7;
  const uint4 *arow = slot + S::WF * 64 + (wm * WM * 16 + r16) * 8;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint4 wf[WN], af[WM];
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      if constexpr (WFP8) {
        // k-group c of the lane's E4M3 pair, widened to bf16
        const uint2 q = *(const uint2 *)((const uint8_t *)(slot + (wn * WN + i) * 64 + lane) + 8 * c);
        const uint2 lo = e4m3x4_to_bf16x4(q.x), hi = e4m3x4_to_bf16x4(q.y);
        wf[i] = uint4{lo.x, lo.y, hi.x, hi.y};
      } else {
        wf[i] = slot[((wn * WN + i) * 2 + c) * 64 + lane];
      }
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) af[j] = arow[j * 16 * 8 + ((4 * c + g) ^ swz)];
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        issue_at<PER>((c * WN + i) * WM + j, issue);
        acc[i][j] = mfma16x16x32(as_bf16x8(wf[i]), as_bf16x8(af[j]), acc[i][j]);
      }
  }
  issue_rest<PER, 2 * WN * WM>(issue);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// acc += A B^T over 128 columns of E4M3 codes (format 0 for both operands,
// unit E8M0 block scales).
__device__ __forceinline__ f32x4 mfma16x16x128_e4m3(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// W8A8 stage: 128 columns of E4M3 weights and E4M3 activation codes, staged
// with the bf16 stage shape (a weight tile's two 1 KB pieces are the two
// 64-column halves of its 128-column step; an activation row is 128 code
// bytes). Lane group g of a weight tile holds, in its two pieces, the codes
// of columns 32c + 8g + e (c = 0..3, e = 0..7) in that order; the product
// only needs both operands in one K order, and the activation rows come
// with each step's codes stored in exactly that order per lane group
// (launch_quant_rows_a8), so a lane's operand is 16-byte chunks g and g + 4
// of its row. Weight fragments are read one tile ahead.
template <class TL>
__device__ __forceinline__ void mma_stage_a8(const uint4 *slot, int wn, int wm, int lane,
                                             f32x4 (&acc)[TL::WN][TL::WM]) {
  using S = StageShape<false, TL>;
  constexpr int WN = TL::WN, WM = TL::WM;
  const int r16 = lane & 15, g = lane >> 4, swz = (r16 >> 1) & 7;
  const uint4 *arow = slot + S::WF * 64 + (wm * WM * 16 + r16) * 8;
  auto wfrag = [&](int i) {
    const uint4 lo = slot[((wn * WN + i) * 2) * 64 + lane], hi = slot[((wn * WN + i) * 2 + 1) * 64 + lane];
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  i32x8 af[WM];
  i32x8 wcur = wfrag(0);
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const uint4 *row = arow + j * 16 * 8;
    const uint4 x0 = row[g ^ swz], x1 = row[(g + 4) ^ swz];
    af[j] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    i32x8 wnext = wcur;
    if (i + 1 < WN) wnext = wfrag(i + 1);
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = mfma16x16x128_e4m3(wcur, af[j], acc[i][j]);
    wcur = wnext;
  }
}

// Fragments of one stage held in registers (bf16 weights): [k-group][tile].
template <class TL>
struct StageFrags {
  uint4 w[2][TL::WN], a[2][TL::WM];
};

template <class TL>
__device__ __forceinline__ void read_frags(const uint4 *slot, int wn, int wm, int lane, StageFrags<TL> &f) {
  using S = StageShape<false, TL>;
  const int r16 = lane & 15, g = lane >> 4, swz = (r16 >> 1) & 7;
  const uint4 *arow = slot + S::WF * 64 + (wm * TL::WM * 16 + r16) * 8;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int i = 0; i < TL::WN; ++i) f.w[c][i] = slot[((wn * TL::WN + i) * 2 + c) * 64 + lane];
#pragma unroll
    for (int j = 0; j < TL::WM; ++j) f.a[c][j] = arow[j * 16 * 8 + ((4 * c + g) ^ swz)];
  }
}

template <class TL, class Issue>
__device__ __forceinline__ void mma_frags(const StageFrags<TL> &f, f32x4 (&acc)[TL::WN][TL::WM], Issue &issue) {
  constexpr int PER = StageShape<false, TL>::PER;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < TL::WN; ++i)
#pragma unroll
      for (int j = 0; j < TL::WM; ++j) {
        issue_at<PER>((c * TL::WN + i) * TL::WM + j, issue);
        acc[i][j] = mfma16x16x32(as_bf16x8(f.w[c][i]), as_bf16x8(f.a[c][j]), acc[i][j]);
      }
  issue_rest<PER, 2 * TL::WN * TL::WM>(issue);
}

template <int WN, int WM>
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

// Barrier between the waves of the workgroup with no memory fence: the
// direct-to-LDS loads of later stages stay in flight across it (each wave has
// already waited for its own loads of the stage about to be read). The empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// acc += W[block tiles] x A[block rows] over NS stages from column kb,
// summed sequentially. NSTAGE - 1 stages are in flight ahead of the one
// being multiplied (ring of NSTAGE slots in `lds`); one barrier per stage.
// Every iteration issues one stage (the last ones reload the final stage
// into a slot nobody reads), so the wait count is constant. A8: W8A8 stages
// (bf16 stage shape holding E4M3 codes, mma_stage_a8).
template <bool WFP8, int NSTAGE, class TL, bool A8 = false>
__device__ __forceinline__ void block_product(const LoadPlan<WFP8, TL> &p, int kb, int NS, uint4 *lds,
                                              f32x4 (&acc)[TL::WN][TL::WM]) {
  static_assert(!(A8 && WFP8), "W8A8 stages use the bf16 stage shape");
  constexpr int SLOT = StageShape<WFP8, TL>::F * 64;
  constexpr uint32_t SLOT_BYTES = SLOT * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave % TL::WAVES_N, wm = wave / TL::WAVES_N;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    issue_stage<WFP8, TL>(base + s * SLOT_BYTES, p, wave, kb + 64 * min(s, NS - 1));
#pragma unroll 1
  for (int s = 0; s < NS; ++s) {
    wait_stages<WFP8, TL>(NSTAGE - 2);
    stage_barrier();
    const int sn = s + NSTAGE - 1;
    const uint32_t nslot = base + (sn % NSTAGE) * SLOT_BYTES;
    const int nk = kb + 64 * min(sn, NS - 1);
    if constexpr (A8) {
      issue_stage<WFP8, TL>(nslot, p, wave, nk);
      mma_stage_a8<TL>(lds + (s % NSTAGE) * SLOT, wn, wm, lane, acc);
    } else {
      auto issue = [&](int q) { issue_one<WFP8, TL>(nslot, p, wave, nk, q); };
      mma_stage<WFP8, TL>(lds + (s % NSTAGE) * SLOT, wn, wm, lane, acc, issue);
    }
  }
  wait_stages<WFP8, TL>(0);
  __syncthreads();
}

// Same product as block_product for bf16 weights, with the fragment reads
// of stage s + 1 issued while stage s is multiplied (two register sets), so
// the LDS reads overlap the matrix cores. Iteration s waits for stage s + 1,
// then (after every wave has finished reading stage s, whose fragments were
// read in iteration s - 1) refills stage s's slot with stage s + NSTAGE.
template <int NSTAGE, class TL>
__device__ __forceinline__ void block_product_pipelined(const LoadPlan<false, TL> &p, int kb, int S, uint4 *lds,
                                                        f32x4 (&acc)[TL::WN][TL::WM]) {
  constexpr int SLOT = StageShape<false, TL>::F * 64;
  constexpr uint32_t SLOT_BYTES = SLOT * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave % TL::WAVES_N, wm = wave / TL::WAVES_N;
  const int NS = 2 * S;  // even
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) issue_stage<false, TL>(base + s * SLOT_BYTES, p, wave, kb + 64 * min(s, NS - 1));
  StageFrags<TL> f0, f1;
  wait_stages<false, TL>(NSTAGE - 1);
  stage_barrier();
  read_frags<TL>(lds, wn, wm, lane, f0);
  // sched_barrier(0) keeps the scheduler from pulling the multiplies of a
  // stage up to its fragment reads (they have no memory dependence on the
  // barrier), which would serialise the reads and the matrix cores again.
  auto step = [&](int s, StageFrags<TL> &cur, StageFrags<TL> &next) {
    __builtin_amdgcn_sched_barrier(0);
    wait_stages<false, TL>(NSTAGE - 2);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage s are done
    stage_barrier();
    const uint32_t nslot = base + (s % NSTAGE) * SLOT_BYTES;
    const int nk = kb + 64 * min(s + NSTAGE, NS - 1);
    auto issue = [&](int q) { issue_one<false, TL>(nslot, p, wave, nk, q); };
    read_frags<TL>(lds + ((s + 1) % NSTAGE) * SLOT, wn, wm, lane, next);
    __builtin_amdgcn_sched_barrier(0);
    mma_frags<TL>(cur, acc, issue);
  };
#pragma unroll 1
  for (int s = 0; s < NS; s += 2) {
    step(s, f0, f1);
    step(s + 1, f1, f0);
  }
  wait_stages<false, TL>(0);
  __syncthreads();
}

template <int EPI, int NSTAGE, class TL>
__global__ __launch_bounds__(TL::NTHR) void k_bgemm(GemmArgs ga, EpiArgs ea, int n_nb, int n_mb) {
  constexpr int WN = TL::WN, WM = TL::WM, BN = TL::BN, BM = TL::BM;
  __shared__ uint4 lds[NSTAGE * StageShape<false, TL>::F * 64];
  int nb, mb;
  if (!place(blockIdx.x, n_nb, n_mb, nb, mb)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int wn = wave % TL::WAVES_N, wm = wave / TL::WAVES_N;
  const int split = blockIdx.y;
  const int kb = split * ga.kslice, ke = min(ga.K, kb + ga.kslice);
  f32x4 acc[WN][WM];
  zero_acc(acc);
  const LoadPlan<false, TL> p = make_plan<false, TL>(ga.W, (size_t)ga.N * ga.K * 2, ga.K >> 7, nb * TL::NT, ga.A, ga.lda, ga.M,
                                      mb * BM, __builtin_amdgcn_readfirstlane(wave), lane);
  // the 256-row blocks hold too many accumulators for a second register set
  // of fragments: their reads are not overlapped with the matrix cores
  if constexpr (TL::BM == 256) block_product<false, NSTAGE, TL>(p, kb, (ke - kb) >> 6, lds, acc);
  else block_product_pipelined<NSTAGE, TL>(p, kb, (ke - kb) >> 7, lds, acc);
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
// LM_TILES vocab blocks of BN rows and keeps, per lane and activation row, a
// running (max, argmax, sum exp) over the unmasked entries; lanes, then the
// two waves sharing a row, are merged in a fixed order and one partial per
// (p, row) is written. The vocab block's row scales (E4M3) and the bitmask
// words of the block's sequences are brought into LDS by direct loads issued
// ahead of the block's product (they complete before its first stage), so the
// epilogue reads no global memory.
//
// MODE: LM_BF16 (bf16 weights and rows), LM_W8 (E4M3 weights widened to
// bf16, bf16 rows), LM_W8A8 (E4M3 weights and E4M3 row codes z8 with row
// scales ascale, 128-column stages on the E4M3 matrix cores; logit =
// acc * s_v * a_m).
enum { LM_BF16 = 0, LM_W8 = 1, LM_W8A8 = 2 };

template <int MODE, int NSTAGE, class TL>
__global__ __launch_bounds__(TL::NTHR) void k_blm_head(LmArgs a, int n_p, int n_mb, int stride_p) {
  constexpr bool WFP8 = MODE != LM_BF16;          // E4M3 weights with row scales
  constexpr bool A8 = MODE == LM_W8A8;
  constexpr bool SW8 = MODE == LM_W8;             // E4M3 stage shape
  constexpr int WN = TL::WN, WM = TL::WM, BN = TL::BN, BM = TL::BM, NT = TL::NT;
  constexpr int MW = BN / 32;        // mask words of a vocab block
  constexpr int MSEQ = BM / 2 + 1;   // sequences one block of rows can touch (gamma >= 2)
  constexpr int WNS = TL::WAVES_N;  // waves that share each activation row
  __shared__ uint4 lds[NSTAGE * StageShape<SW8, TL>::F * 64];
  __shared__ float s_mx[WNS][BM], s_se[WNS][BM];
  __shared__ uint32_t s_idx[WNS][BM];
  __shared__ __align__(16) float s_scale[BN];
  __shared__ uint32_t s_mask[((MSEQ + 7) / 8) * 8 * MW];  // [local sequence][word], whole loads of 8 sequences
  // Persistent placement: workgroup b sits on XCD x = b % 8 with activation
  // block mb and group q of its XCD, and loops over the vocab ranges
  // q * 8 + x, + stride_p, ...: the n_mb workgroups that share a range run
  // side by side on one XCD for the whole launch and stay in step, so more of
  // a range's weight lines are still in that XCD's L2 when the partners read
  // them than when each range's workgroups are dispatched as others finish.
  const int xcd = blockIdx.x & 7, slot_k = blockIdx.x >> 3;
  const int mb = slot_k % n_mb;
  for (int p = (slot_k / n_mb) * 8 + xcd; p < n_p; p += stride_p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4,
              r16 = lane & 15;
    const int wn = wave % TL::WAVES_N, wm = wave / TL::WAVES_N;
    const int n_vb = a.V / BN;
    const int steps_w = a.K >> 7;
    const int seq0 = (mb * BM) / a.gamma;
    const int n_s = (min(mb * BM + BM, a.M) - 1) / a.gamma - seq0 + 1;  // <= MSEQ
    const int4v r_scale = make_rsrc(a.scale, WFP8 ? (uint32_t)a.V * 4u : 0u);
    const int4v r_mask = make_rsrc(a.bitmask, a.bitmask ? (uint32_t)((a.M + a.gamma - 1) / a.gamma) * a.words * 4u : 0u);
    const bool masked = a.bitmask != nullptr;
    ArgState st[WM];
    int sl[WM];     // local sequence of each row this lane holds
    float am[WM];   // W8A8: the rows' activation scales
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      arg_init(st[j]);
      const int m = min(mb * BM + (wm * WM + j) * 16 + r16, a.M - 1);
      sl[j] = m / a.gamma - seq0;
      am[j] = A8 ? a.ascale[m] : 1.0f;
    }
    for (int vb = p * LM_TILES; vb < min(n_vb, (p + 1) * LM_TILES); ++vb) {
      if (WFP8 || masked) __syncthreads();  // the previous block's epilogue is done with s_scale / s_mask
      if (WFP8 && wave == 0) dma16(r_scale, lane * 16, (uint32_t)vb * BN * 4, lds_addr(s_scale));
      if (masked)
        for (int q = wave; q * 8 < n_s; q += TL::NWAVES) {
          const int ls = min(q * 8 + (lane >> 3), n_s - 1);
          dma4(r_mask, (uint32_t)(((seq0 + ls) * a.words + vb * MW + (lane & 7)) * 4), 0, lds_addr(s_mask + q * 64));
        }
      f32x4 acc[WN][WM];
      zero_acc(acc);
      if constexpr (A8) {
        // codes staged as if bf16 of half the width: a 64-"column" stage is 128
        // code columns, one 2 KB step of a weight tile
        LoadPlan<false, TL> pl = make_plan<false, TL>(a.W, (size_t)a.V * a.K, steps_w, vb * NT,
                                                      (const uint16_t *)a.z8, a.K / 2, a.M, mb * BM, wave, lane);
        pl.w_tile = (uint32_t)steps_w * 2048u;
        pl.w_base = (uint32_t)(vb * NT) * pl.w_tile;
        block_product<false, NSTAGE, TL, true>(pl, 0, steps_w, lds, acc);
      } else {
        const LoadPlan<SW8, TL> pl = make_plan<SW8, TL>(a.W, (size_t)a.V * a.K * (WFP8 ? 1 : 2), steps_w, vb * NT, a.z,
                                                        a.K, a.M, mb * BM, wave, lane);
        block_product<SW8, NSTAGE, TL>(pl, 0, 2 * steps_w, lds, acc);
      }
      // This lane's entries: vocab vl = (wn * WN + i) * 16 + 4 g + r of the
      // block, rows (wm * WM + j) * 16 + r16. Their row scales (four
      // consecutive entries per read) and the rows' mask words (two vocab
      // tiles per 32-bit word) are read from LDS once per block.
      static_assert(BN % 32 == 0 && (WN * 16) % 32 == 0, "a wave's vocab range covers whole mask words");
      f32x4 scv[WN];
#pragma unroll
      for (int i = 0; i < WN; ++i)
        scv[i] = WFP8 ? *(const f32x4 *)(s_scale + (wn * WN + i) * 16 + 4 * g) : f32x4{1.f, 1.f, 1.f, 1.f};
      uint32_t mw[WM][WN / 2];
#pragma unroll
      for (int j = 0; j < WM; ++j)
#pragma unroll
        for (int w = 0; w < WN / 2; ++w) mw[j][w] = masked ? s_mask[sl[j] * MW + (wn * WN) / 2 + w] : ~0u;
      if (a.logits) {
        // the optional logits output (before the mask)
#pragma unroll
        for (int i = 0; i < WN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < WM; ++j) {
              const int m = mb * BM + (wm * WM + j) * 16 + r16, v = vb * BN + (wn * WN + i) * 16 + 4 * g + r;
              if (m < a.M) a.logits[(size_t)m * a.V + v] = A8 ? acc[i][j][r] * scv[i][r] * am[j] : acc[i][j][r] * scv[i][r];
            }
      }
      // Two passes per row: the block's logits (masked ones as -inf, kept in
      // acc) with this lane's largest and its first index, then one
      // exponential per logit against the row's merged maximum.
      float bm[WM];
      uint32_t bi[WM];
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        bm[j] = -__builtin_huge_valf();
        bi[j] = 0xFFFFFFFFu;
      }
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vl = (wn * WN + i) * 16 + 4 * g + r, v = vb * BN + vl;
          const int bit = (i & 1) * 16 + 4 * g + r;  // vl & 31
#pragma unroll
          for (int j = 0; j < WM; ++j) {
            const float x = A8 ? acc[i][j][r] * scv[i][r] * am[j] : acc[i][j][r] * scv[i][r];
            const bool ok = (mw[j][i >> 1] >> bit) & 1u;
            const float xo = ok ? x : -__builtin_huge_valf();
            acc[i][j][r] = xo;
            // values come in increasing v, so a strict > keeps the lowest id of a tie
            bi[j] = xo > bm[j] ? (uint32_t)v : bi[j];
            bm[j] = fmaxf(bm[j], xo);
          }
        }
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const float mn = fmaxf(st[j].mx, bm[j]);
        const float off = -mn * LOG2E;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < WN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) s += fast_exp2(fmaf(acc[i][j][r], LOG2E, off));
        const bool any = mn > -__builtin_huge_valf();  // else every value so far is masked
        const float se = st[j].se * fast_exp2(fmaf(st[j].mx, LOG2E, off)) + s;
        st[j].se = any ? se : st[j].se;
        st[j].idx = bm[j] > st[j].mx ? bi[j] : st[j].idx;
        st[j].mx = any ? mn : st[j].mx;
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
      ArgState x;
      x.mx = s_mx[0][row];
      x.se = s_se[0][row];
      x.idx = s_idx[0][row];
      // the row's waves in wave order
#pragma unroll
      for (int w = 1; w < WNS; ++w) {
        ArgState y;
        y.mx = s_mx[w][row];
        y.se = s_se[w][row];
        y.idx = s_idx[w][row];
        x = arg_merge(x, y);
      }
      if (m < a.M) {
        const size_t o = (size_t)p * a.ld_part + m;
        a.part_mx[o] = x.mx;
        a.part_se[o] = x.se;
        a.part_idx[o] = x.idx;
      }
    }
    __syncthreads();  // s_mx / s_se / s_idx are read before the next range writes them
  }
}

template <int EPI, class TL, int NSTAGE>
hipError_t launch_epi(const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  const int n_nb = g.N / TL::BN, n_mb = (g.M + TL::BM - 1) / TL::BM;
  dim3 grid(((n_nb + 7) / 8) * 8 * n_mb, g.splits);
  hipLaunchKernelGGL((k_bgemm<EPI, NSTAGE, TL>), grid, dim3(TL::NTHR), 0, s, g, e, n_nb, n_mb);
  return hipGetLastError();
}

// Workgroup rounds over the chip of a tiling.
int rounds(int N, int M, int BN, int BM, int splits) {
  const long wgs = (long)(N / BN) * ((M + BM - 1) / BM) * splits;
  return (int)((wgs + NUM_CUS - 1) / NUM_CUS);
}

// The 256-row blocks do twice the work of the 128-row ones in about 1.55
// times the time (fewer LDS bytes per product): use them when that wins.
bool wide_tiles(int epi, int N, int M) {
  if (epi == EPI_PARTIAL || N % TileW::BN != 0) return false;
  return 31 * rounds(N, M, TileW::BN, TileW::BM, 1) < 20 * rounds(N, M, TileG::BN, TileG::BM, 1);
}

// The tiled GEMMs are bound by L2 -> LDS traffic: a round of workgroups over
// the chip takes about (BN + BM) x K bytes per compute unit, so a launch
// costs about rounds x (BN + BM). Each launch takes the eligible tiling of
// least cost (ties to the earlier one): 128 x 128 and 256 x 128 for any
// epilogue, 192 x 256 and 160 x 128 for the others when N is a multiple of
// their BN (the gate/up product of 1024 rows: one round of 256 blocks of
// 192 x 256 instead of three of 768; the QKV product, N = 5120: one round of
// 256 blocks of 160 x 128 instead of 160 blocks of 256 x 128). The 256 x 128
// tiling is taken over 128 x 128 only at less than 20 / 31 of its cost
// (measured: the wider blocks do twice the work in about 1.55 times the time).
enum TileId { T_G = 0, T_W = 1, T_H = 2, T_Q = 3 };

int pick_tiles(int epi, int N, int M) {
  auto cost = [&](int bn, int bm) { return (long)rounds(N, M, bn, bm, 1) * (bn + bm); };
  int best = T_G;
  long c_best = cost(TileG::BN, TileG::BM);
  if (wide_tiles(epi, N, M)) {
    best = T_W;
    c_best = cost(TileW::BN, TileW::BM);
  }
  if (epi == EPI_PARTIAL) return best;
  if (N % TileH::BN == 0 && cost(TileH::BN, TileH::BM) < c_best) {
    best = T_H;
    c_best = cost(TileH::BN, TileH::BM);
  }
  if (N % TileQ::BN == 0 && cost(TileQ::BN, TileQ::BM) < c_best) best = T_Q;
  return best;
}

template <int EPI>
hipError_t launch_pick(const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  switch (pick_tiles(EPI, g.N, g.M)) {
    case T_H: return launch_epi<EPI, TileH, NSTAGE_H>(g, e, s);
    case T_Q: return launch_epi<EPI, TileQ, NSTAGE_Q>(g, e, s);
    case T_W: return launch_epi<EPI, TileW, NSTAGE_W>(g, e, s);
    default: return launch_epi<EPI, TileG, NSTAGE_G>(g, e, s);
  }
}

}  // namespace

bool bgemm_ok(int epi, int N, int K) {
  return (epi == EPI_F32 || epi == EPI_SWIGLU || epi == EPI_QKV_ROPE || epi == EPI_PARTIAL || epi == EPI_KV_SCATTER) &&
         N % TileG::BN == 0 && K % 128 == 0 && N > 0 && K > 0;
}

int bgemm_splits(int N, int K, int M) {
  // about one workgroup per compute unit; every split a multiple of 128 columns
  const int blocks = (N / TileG::BN) * ((M + TileG::BM - 1) / TileG::BM);
  int splits = std::max(1, std::min(4, (NUM_CUS + blocks / 2) / std::max(blocks, 1)));
  while (splits > 1 && K % (splits * 128) != 0) --splits;
  return splits;
}

hipError_t launch_bgemm(int epi, const GemmArgs &g, const EpiArgs &e, hipStream_t s) {
  if (g.M < 1 || !bgemm_ok(epi, g.N, g.K) || g.splits < 1 || g.kslice % 128 != 0) return hipErrorInvalidValue;
  if (g.splits > 1 && epi != EPI_PARTIAL) return hipErrorInvalidValue;
  if (epi == EPI_KV_SCATTER && (!e.d_row_pos || !e.d_row_bt)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_F32: return launch_pick<EPI_F32>(g, e, s);
    case EPI_KV_SCATTER: return launch_pick<EPI_KV_SCATTER>(g, e, s);
    case EPI_SWIGLU: return launch_pick<EPI_SWIGLU>(g, e, s);
    case EPI_QKV_ROPE: return launch_pick<EPI_QKV_ROPE>(g, e, s);
    case EPI_PARTIAL: return launch_pick<EPI_PARTIAL>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

int blm_parts(int V) { return (V / TileL::BN + LM_TILES - 1) / LM_TILES; }

bool blm_ok(int V, int K) { return V > 0 && K > 0 && V % TileL::BN == 0 && K % 128 == 0; }

hipError_t launch_blm_head(bool w_fp8, bool a_fp8, const LmArgs &a, hipStream_t s) {
  if (a.M < 1 || a.V % TileL::BN != 0 || a.K % 128 != 0 || a.row0 != 0) return hipErrorInvalidValue;
  if (a_fp8 && (!w_fp8 || !a.z8 || !a.ascale)) return hipErrorInvalidValue;
  const int n_p = blm_parts(a.V), n_mb = (a.M + TileL::BM - 1) / TileL::BM;
  // one workgroup per CU (the ring fills the LDS): groups of n_mb per XCD,
  // at most as many groups as there are vocab ranges per XCD
  const int groups = std::max(1, std::min(NUM_CUS / 8 / n_mb, (n_p + 7) / 8));
  const int stride_p = groups * 8;
  dim3 grid(stride_p * n_mb);
  if (a_fp8) hipLaunchKernelGGL((k_blm_head<LM_W8A8, NSTAGE_LM, TileL>), grid, dim3(TileL::NTHR), 0, s, a, n_p, n_mb, stride_p);
  else if (w_fp8) hipLaunchKernelGGL((k_blm_head<LM_W8, NSTAGE_LM, TileLW>), grid, dim3(TileLW::NTHR), 0, s, a, n_p, n_mb, stride_p);
  else hipLaunchKernelGGL((k_blm_head<LM_BF16, NSTAGE_LM, TileL>), grid, dim3(TileL::NTHR), 0, s, a, n_p, n_mb, stride_p);
  return hipGetLastError();
}

}  // namespace dflash
