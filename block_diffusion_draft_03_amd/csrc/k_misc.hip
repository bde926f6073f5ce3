// k_misc.hip - row-wise kernels of the DFlash head for gfx950: block setup
// (embedding gather, first RMSNorm, RoPE table), RMSNorm, build-time weight
// conversion and repacking, the FP8 LM-head mirror, and KV inspection.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

namespace {

// One workgroup per block row m of the call: sequence s = m / gamma, row
// j = m % gamma. Token = last verified token for j == 0, else the mask
// token; position = position[s] + j. Writes the fp32 residual row (embedding
// row widened), its RMSNorm with the first layer's input gain as bf16 (or,
// with ss_out, the row times the gain and the row's sum of squares), and the
// row's (cos, sin) RoPE table computed in double precision.
__global__ __launch_bounds__(256) void k_setup(SetupArgs a) {
  constexpr int VPT = 8;  // embedding values per thread and chunk (one 16-byte load)
  constexpr int MAXC = 2; // chunks kept in registers (hidden <= 4096)
  __shared__ float red[4];
  const int m = blockIdx.x, s = m / a.gamma, j = m % a.gamma;
  const uint32_t tok = j == 0 ? a.token[s] : a.mask_id;
  const int pos = a.position[s] + j;
  const uint16_t *e = a.embed + (size_t)tok * a.h;
  float *hr = a.hid + (size_t)m * a.h;
  uint16_t *ar = a.a + (size_t)m * a.h;
  const int step = blockDim.x * VPT;
  const bool fast = a.h % VPT == 0 && a.h <= MAXC * step;
  // the row's loads go out first; the RoPE table is computed while they are in flight
  uint4 q[MAXC];
  if (fast) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int i = c * step + threadIdx.x * VPT;
      if (i < a.h) q[c] = *(const uint4 *)(e + i);
    }
  }
  for (int i = threadIdx.x; i < a.half_dim; i += blockDim.x) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[i], &sn, &cs);
    a.cs[(size_t)m * a.half_dim + i] = make_float2((float)cs, (float)sn);
  }
  float ss = 0.0f;
  if (fast) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int i = c * step + threadIdx.x * VPT;
      if (i < a.h) {
        const uint32_t w[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
        float x[VPT];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(w[k] << 16);
          x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) ss += x[k] * x[k];
        *(float4 *)(hr + i) = make_float4(x[0], x[1], x[2], x[3]);
        *(float4 *)(hr + i + 4) = make_float4(x[4], x[5], x[6], x[7]);
      }
    }
  } else {
    for (int i = threadIdx.x; i < a.h; i += blockDim.x) {
      const float x = bf16_to_f32(e[i]);
      hr[i] = x;
      ss += x * x;
    }
  }
  ss = block_sum(ss, red);
  const float r = a.ss_out ? 1.0f : 1.0f / sqrtf(ss / (float)a.h + a.eps);
  if (a.ss_out && threadIdx.x == 0) a.ss_out[m] = ss;
  if (fast) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int i = c * step + threadIdx.x * VPT;
      if (i < a.h) {
        const uint32_t w[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = pack_bf16x2(__uint_as_float(w[k] << 16) * r * a.gain[i + 2 * k],
                             __uint_as_float(w[k] & 0xFFFF0000u) * r * a.gain[i + 2 * k + 1]);
        *(uint4 *)(ar + i) = uint4{o[0], o[1], o[2], o[3]};
      }
    }
  } else {
    for (int i = threadIdx.x; i < a.h; i += blockDim.x) ar[i] = f32_to_bf16(bf16_to_f32(e[i]) * r * a.gain[i]);
  }
}

__device__ __forceinline__ uint16_t load_as_bf16(const void *src, size_t i, bool src_f32) {
  return src_f32 ? f32_to_bf16(((const float *)src)[i]) : ((const uint16_t *)src)[i];
}

__global__ void k_convert_rows(uint16_t *dst, const void *src, const void *src2, int rows, int cols, int src_f32,
                               int order, int head_dim) {
  const size_t total = (size_t)rows * cols;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int rr = (int)(e / cols), cc = (int)(e % cols);
    const void *s = src;
    int sr = rr;
    if (order == ROWS_GATE_UP) {
      s = (rr & 1) ? src2 : src;
      sr = rr >> 1;
    } else if (order == ROWS_ROPE_PAIRS) {
      const int head = rr / head_dim, j = rr % head_dim;
      sr = head * head_dim + (j >> 1) + (j & 1) * (head_dim >> 1);
    }
    dst[e] = load_as_bf16(s, (size_t)sr * cols + cc, src_f32 != 0);
  }
}

// Source row of destination row rr under a row order; *second selects src2.
__device__ __forceinline__ int src_row(int rr, int order, int head_dim, bool *second) {
  *second = false;
  if (order == ROWS_GATE_UP) {
    *second = (rr & 1) != 0;
    return rr >> 1;
  }
  if (order == ROWS_ROPE_PAIRS) {
    const int head = rr / head_dim, j = rr % head_dim;
    return head * head_dim + (j >> 1) + (j & 1) * (head_dim >> 1);
  }
  return rr;
}

// One thread per 16-byte lane chunk of the tiled layout (8 bf16).
__global__ void k_tile_rows(uint16_t *dst, int dst_tile0, const void *src, const void *src2, int rows, int cols,
                            int src_f32, int order, int head_dim) {
  const int steps = (cols + 127) / 128, tiles = (rows + 15) / 16;
  const size_t chunks = (size_t)tiles * steps * 256;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q & 63), c = (int)((q >> 6) & 3);
    const size_t ts = q >> 8;
    const int step = (int)(ts % steps), tile = (int)(ts / steps);
    const int r = tile * 16 + (lane & 15);
    const int k0 = step * 128 + 32 * c + 8 * (lane >> 4);
    uint16_t v[8];
    bool second = false;
    const int sr = r < rows ? src_row(r, order, head_dim, &second) : 0;
    const void *s = second ? src2 : src;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (r < rows && k0 + e < cols) ? load_as_bf16(s, (size_t)sr * cols + k0 + e, src_f32 != 0) : (uint16_t)0;
    const size_t o = (((size_t)(dst_tile0 + tile) * steps + step) * 4 + c) * 64 + lane;
    *(uint4 *)(dst + o * 8) = *(const uint4 *)v;
  }
}

// E4M3: one thread per 16-byte chunk (k-groups 2j and 2j+1 of one lane).
__global__ void k_tile_fp8(uint8_t *dst, const uint8_t *src, int rows, int cols, int untile) {
  const int steps = (cols + 127) / 128, tiles = (rows + 15) / 16;
  const size_t chunks = (size_t)tiles * steps * 128;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q & 63), j = (int)((q >> 6) & 1);
    const size_t ts = q >> 7;
    const int step = (int)(ts % steps), tile = (int)(ts / steps);
    const int r = tile * 16 + (lane & 15);
    uint8_t *t = dst + q * 16;
    const uint8_t *tt = src + q * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = step * 128 + 32 * (2 * j + h) + 8 * (lane >> 4) + e;
        if (r >= rows || k >= cols) {
          if (!untile) t[8 * h + e] = 0;
          continue;
        }
        if (untile)
          dst[(size_t)r * cols + k] = tt[8 * h + e];
        else
          t[8 * h + e] = src[(size_t)r * cols + k];
      }
  }
}

__global__ void k_to_f32(float *dst, const void *src, int n, int src_f32) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    dst[i] = src_f32 ? ((const float *)src)[i] : bf16_to_f32(((const uint16_t *)src)[i]);
}

// One workgroup per vocab row: s = amax / 448 (1 for an all-zero row),
// code = E4M3(w / s) with IEEE float32 division, round to nearest even.
__global__ __launch_bounds__(256) void k_fp8_mirror(const uint16_t *src, int h, uint8_t *codes, float *scale) {
  __shared__ float red[4];
  const int v = blockIdx.x;
  const uint16_t *row = src + (size_t)v * h;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < h; i += blockDim.x) amax = fmaxf(amax, fabsf(bf16_to_f32(row[i])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / E4M3_MAX : 1.0f;
  if (threadIdx.x == 0) scale[v] = s;
  uint8_t *out = codes + (size_t)v * h;
  for (int i = threadIdx.x; i < h; i += blockDim.x) out[i] = f32_to_e4m3(bf16_to_f32(row[i]) / s);
}

// E4M3 activation rows of the W8A8 LM head, one workgroup per row: the
// mirror's recipe (s = amax / 448, 1 for an all-zero row; code = E4M3(x / s)
// with IEEE float32 division), stored in the head's K order: inside each
// 128-column step, the 8 codes of columns 32c + 8g .. + 7 sit in half c & 1
// of 16-byte chunk g + 4 (c >> 1), so lane group g of a 16x16x128 operand
// takes chunks g and g + 4 (the bf16 head's read pattern).
__global__ __launch_bounds__(256) void k_quant_rows_a8(const uint16_t *src, int h, uint8_t *codes, float *scale) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const uint16_t *row = src + (size_t)m * h;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < h; i += blockDim.x) amax = fmaxf(amax, fabsf(bf16_to_f32(row[i])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / E4M3_MAX : 1.0f;
  if (threadIdx.x == 0) scale[m] = s;
  uint8_t *out = codes + (size_t)m * h;
  for (int p = threadIdx.x; p < h / 8; p += blockDim.x) {
    // output piece p: step p / 16, piece q of the step = half q & 1 of chunk
    // q / 2 = g + 4 (c >> 1), from columns 32c + 8g
    const int step = p >> 4, q = p & 15, g = (q >> 1) & 3, c = 2 * (q >> 3) + (q & 1);
    const uint4 x = *(const uint4 *)(row + step * 128 + 32 * c + 8 * g);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t v = w[e];
      const uint32_t c0 = (uint32_t)f32_to_e4m3(bf16_to_f32((uint16_t)(v & 0xFFFFu)) / s);
      const uint32_t c1 = (uint32_t)f32_to_e4m3(bf16_to_f32((uint16_t)(v >> 16)) / s);
      if (e < 2) lo |= (c0 | (c1 << 8)) << (16 * e);
      else hi |= (c0 | (c1 << 8)) << (16 * (e - 2));
    }
    *(uint2 *)(out + (size_t)p * 8) = uint2{lo, hi};
  }
}

// Cached K is stored with its head dimensions in RoPE pair order (dim i at
// position 2i for i < d/2, at 2(i - d/2) + 1 otherwise); the copy restores
// the natural order.
__global__ void k_read_kv(const uint8_t *pool, const int32_t *bt, int L, int layer, int n_kv, int d, int eb, int row0,
                          int n_rows, uint8_t *k_out, uint8_t *v_out) {
  const size_t row_bytes = (size_t)n_kv * d * eb;
  const size_t total = (size_t)n_rows * row_bytes;
  const int half = d >> 1;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(e / row_bytes);
    const size_t within = e % row_bytes;
    const int g = (int)(within / ((size_t)d * eb));
    const int de = (int)(within % ((size_t)d * eb));
    const int i = de / eb, byte = de % eb;
    const int j = i < half ? 2 * i : 2 * (i - half) + 1;
    const int pos = row0 + r;
    const int32_t blk = bt[pos >> 4];
    const size_t tile = (size_t)DFLASH_KV_BLOCK * d * eb;
    const size_t kbase = ((((size_t)blk * L + layer) * 2 + 0) * n_kv + g) * tile;
    const size_t vbase = ((((size_t)blk * L + layer) * 2 + 1) * n_kv + g) * tile;
    // K tile [16][d] (dims in RoPE pair order), V tile transposed [d][16]
    if (k_out) k_out[e] = pool[kbase + ((size_t)(pos & 15) * d + j) * eb + byte];
    if (v_out) v_out[e] = pool[vbase + ((size_t)i * DFLASH_KV_BLOCK + (pos & 15)) * eb + byte];
  }
}

// Zero n 32-bit words (a fill kernel rather than a memset, so the launch can
// sit in a captured graph).
__global__ void k_zero_u32(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

int grid_for(size_t total, int block) {
  size_t b = (total + block - 1) / block;
  if (b > 65535) b = 65535;
  return b < 1 ? 1 : (int)b;
}

}  // namespace

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  if (bytes % 4 != 0 || ((uintptr_t)p & 3u) != 0) return hipErrorInvalidValue;
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3(std::min(grid_for(n, 256), 1024)), dim3(256), 0, s, (uint32_t *)p, n);
  return hipGetLastError();
}

hipError_t launch_setup(const SetupArgs &a, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_setup, dim3(M), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_convert_rows(uint16_t *dst, const void *src, const void *src2, int rows, int cols, bool src_f32,
                               int order, int head_dim, hipStream_t s) {
  hipLaunchKernelGGL(k_convert_rows, dim3(grid_for((size_t)rows * cols, 256)), dim3(256), 0, s, dst, src, src2, rows,
                     cols, (int)src_f32, order, head_dim);
  return hipGetLastError();
}

size_t tiled_elems(int rows, int cols) { return (size_t)((rows + 15) / 16) * 16 * (size_t)((cols + 127) / 128) * 128; }

hipError_t launch_tile_rows(uint16_t *dst, int dst_row0, const void *src, const void *src2, int rows, int cols,
                            bool src_f32, int order, int head_dim, hipStream_t s) {
  if (dst_row0 % 16) return hipErrorInvalidValue;
  const size_t chunks = (size_t)((rows + 15) / 16) * ((cols + 127) / 128) * 256;
  hipLaunchKernelGGL(k_tile_rows, dim3(grid_for(chunks, 256)), dim3(256), 0, s, dst, dst_row0 / 16, src, src2, rows,
                     cols, (int)src_f32, order, head_dim);
  return hipGetLastError();
}

hipError_t launch_tile_fp8(uint8_t *dst, const uint8_t *src, int rows, int cols, hipStream_t s) {
  const size_t chunks = (size_t)((rows + 15) / 16) * ((cols + 127) / 128) * 128;
  hipLaunchKernelGGL(k_tile_fp8, dim3(grid_for(chunks, 256)), dim3(256), 0, s, dst, src, rows, cols, 0);
  return hipGetLastError();
}

hipError_t launch_untile_fp8(uint8_t *dst, const uint8_t *src, int rows, int cols, hipStream_t s) {
  const size_t chunks = (size_t)((rows + 15) / 16) * ((cols + 127) / 128) * 128;
  hipLaunchKernelGGL(k_tile_fp8, dim3(grid_for(chunks, 256)), dim3(256), 0, s, dst, src, rows, cols, 1);
  return hipGetLastError();
}

hipError_t launch_to_f32(float *dst, const void *src, int n, bool src_f32, hipStream_t s) {
  hipLaunchKernelGGL(k_to_f32, dim3(grid_for(n, 256)), dim3(256), 0, s, dst, src, n, (int)src_f32);
  return hipGetLastError();
}

hipError_t launch_fp8_mirror(const uint16_t *src, int V, int h, uint8_t *codes, float *scale, hipStream_t s) {
  hipLaunchKernelGGL(k_fp8_mirror, dim3(V), dim3(256), 0, s, src, h, codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_rows_a8(const uint16_t *src, int M, int h, uint8_t *codes, float *scale, hipStream_t s) {
  if (M < 1 || h % 128 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_rows_a8, dim3(M), dim3(256), 0, s, src, h, codes, scale);
  return hipGetLastError();
}

hipError_t launch_read_kv(const void *pool, const int32_t *bt, int L, int layer, int n_kv, int d, int elem_bytes,
                          int row0, int n_rows, void *k_out, void *v_out, hipStream_t s) {
  const size_t total = (size_t)n_rows * n_kv * d * elem_bytes;
  hipLaunchKernelGGL(k_read_kv, dim3(grid_for(total, 256)), dim3(256), 0, s, (const uint8_t *)pool, bt, L, layer, n_kv,
                     d, elem_bytes, row0, n_rows, (uint8_t *)k_out, (uint8_t *)v_out);
  return hipGetLastError();
}

}  // namespace dflash
