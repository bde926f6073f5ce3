// common.hpp - device helpers shared by the gfx950 kernels of the DFlash head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float E4M3_MAX = 448.0f;

// bf16 is stored as uint16_t bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3FN codes (one dword) -> four bf16 (two dwords), bytes 0, 1 into
// the first dword and 2, 3 into the second. E4M3 values are exactly
// representable in bf16; the conversion's scale of 1.0 leaves them unchanged.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  return v[0];
}

// float -> E4M3FN code: round to nearest even, saturate to +-448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  x = fminf(fmaxf(x, -E4M3_MAX), E4M3_MAX);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false);
  return (uint8_t)(r & 0xFF);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

// ---- fp16 (the attention operands: Q, K, V and P) ----
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// float -> fp16 pair, round to nearest even (fp16 is stored as uint16_t bit patterns).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Two bf16 (one dword) -> two fp16: exact for magnitudes in fp16's normal
// range [2^-14, 65504] (a bf16 significand has 8 bits, fp16's 11).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}

// Four E4M3FN codes (one dword) -> four fp16 (two dwords), bytes 0, 1 into
// the first dword and 2, 3 into the second; exact (every E4M3 value is an
// fp16 value).
__device__ __forceinline__ uint2 e4m3x4_to_f16x4(uint32_t w) {
  const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
  const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ f16x8 as_f16x8(const uint4 &u) { return __builtin_bit_cast(f16x8, u); }

__device__ __forceinline__ f32x4 mfma16x16x32_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float silu(float x) { return x / (1.0f + fast_exp2(-x * LOG2E)); }

// Sum over a wave with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Block-wide sum of one float per thread (blockDim.x a multiple of 64,
// at most 1024); `red` is LDS scratch of blockDim.x / 64 floats. Fixed order.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Running (max, argmax, sum of exp(x - max)) of a softmax row. Ties keep the
// lower index; `se` is relative to `mx` (natural exponent).
struct ArgState {
  float mx;
  float se;
  uint32_t idx;
};

__device__ __forceinline__ void arg_init(ArgState &s) {
  s.mx = -__builtin_huge_valf();
  s.se = 0.0f;
  s.idx = 0xFFFFFFFFu;
}

// Add one value with an index larger than every index already in s (when
// `take` is set). Branch-free: one exponential either way.
__device__ __forceinline__ void arg_push(ArgState &s, float x, uint32_t v, bool take = true) {
  const bool up = x > s.mx;
  const float e = fast_exp2((up ? s.mx - x : x - s.mx) * LOG2E);
  const float se = up ? s.se * e + 1.0f : s.se + e;
  s.se = take ? se : s.se;
  s.idx = take && up ? v : s.idx;
  s.mx = take && up ? x : s.mx;
}

// Merge two states (any index order); ties go to the lower index.
__device__ __forceinline__ ArgState arg_merge(const ArgState a, const ArgState b) {
  const float ninf = -__builtin_huge_valf();
  const bool pick_a = a.mx > b.mx || (a.mx == b.mx && a.idx < b.idx);
  ArgState r;
  r.mx = pick_a ? a.mx : b.mx;
  r.idx = pick_a ? a.idx : b.idx;
  r.se = a.se * fast_exp2((a.mx - r.mx) * LOG2E) + b.se * fast_exp2((b.mx - r.mx) * LOG2E);
  // an empty side (nothing pushed) leaves the other unchanged
  const bool a_empty = a.mx == ninf, b_empty = b.mx == ninf;
  r.mx = b_empty ? a.mx : a_empty ? b.mx : r.mx;
  r.idx = b_empty ? a.idx : a_empty ? b.idx : r.idx;
  r.se = b_empty ? a.se : a_empty ? b.se : r.se;
  return r;
}

__device__ __forceinline__ ArgState arg_shfl_xor(const ArgState &s, int o) {
  ArgState t;
  t.mx = __shfl_xor(s.mx, o, WAVE);
  t.se = __shfl_xor(s.se, o, WAVE);
  t.idx = (uint32_t)__shfl_xor((int)s.idx, o, WAVE);
  return t;
}

}  // namespace dflash
