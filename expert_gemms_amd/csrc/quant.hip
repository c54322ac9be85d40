// Block quantisers: dispatch quantisation of x and the weight casts.
//
// MX (DeepGEMM MegaMoE experts page, module docstring: one UE8M0 scale per
// 1x32 block; Qwen4-Exp MegaMoE page, _requantize: power-of-two float32
// scales whose exponent byte is the code): the scale is the smallest power of
// two that keeps the block's largest magnitude within the element format, the
// elements are value / scale rounded to nearest even.
// NVFP4 (same module docstring: E4M3 scale per 1x16 block plus an FP32 global
// scale; dispatch scales each token by its own FP32 scale): global g, block
// scale bs = E4M3(amax16 / (6 g)), elements E2M1(v * (1 / (bs g))), all in
// float32 arithmetic.  The token scale is amax_t / (6 * 448).
#include "common.h"
#include "l2input.h"
#include "launch.h"

namespace moe {

// One thread per 32-element MX block (the block body is quant_mx_block).
template <bool F32, bool FP4>
__global__ void __launch_bounds__(256) k_quant_mx(const void* __restrict__ src, int64_t nblocks,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b < nblocks) quant_mx_block<F32, FP4>(src, b, codes, scales);
}

// NVFP4: one workgroup per row.  The row's global scale is either given
// (fixed_g[row / rows_per_g]) or computed from the row's amax and written to
// row_g[row].  Codes are packed two per byte.
template <bool F32>
__global__ void __launch_bounds__(256) k_quant_nv(const void* __restrict__ src, int cols,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float* __restrict__ row_g, const float* __restrict__ fixed_g,
                                                  int rows_per_g) {
#pragma clang fp contract(off)
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int64_t base = row * cols;
  float g;
  if (fixed_g) {
    g = fixed_g[row / rows_per_g];
  } else {
    float amax = 0.0f;
    if constexpr (F32) {
      for (int i = threadIdx.x; i < cols; i += 256) amax = __builtin_fmaxf(amax, __builtin_fabsf(load_elem<F32>(src, base + i)));
    } else {
      // BF16 rows: 8 values (16 bytes) per load
      for (int i = threadIdx.x * 8; i < cols; i += 256 * 8) {
        const uint4 u = *(const uint4*)((const uint16_t*)src + base + i);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(u2f(wd[j] << 16)),
                                                       __builtin_fabsf(u2f(wd[j] & 0xFFFF0000u))));
      }
    }
    amax = group_max<6>(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    g = amax > 0.0f ? amax / 2688.0f : 1.0f;
    if (threadIdx.x == 0) row_g[row] = g;
  }
  const float six_g = 6.0f * g;
  for (int blk = threadIdx.x; blk < cols / 16; blk += 256) {
    float v[16];
    float amax = 0.0f;
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = load_elem<F32>(src, base + blk * 16 + i);
    } else {
      const uint4* p = (const uint4*)((const uint16_t*)src + base + blk * 16);
      const uint4 u0 = p[0], u1 = p[1];
      const uint32_t wd[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = u2f(wd[j] << 16);
        v[2 * j + 1] = u2f(wd[j] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    const float t = amax / six_g;
    const uint32_t bs = e4m3_encode(t);
    const float bsv = e4m3_decode(bs);
    uint32_t w[2] = {0, 0};
    if (bsv != 0.0f) {
      const float r = 1.0f / (bsv * g);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        w[h] = e2m1_x4(v[8 * h] * r, v[8 * h + 1] * r, v[8 * h + 2] * r, v[8 * h + 3] * r) |
               (e2m1_x4(v[8 * h + 4] * r, v[8 * h + 5] * r, v[8 * h + 6] * r, v[8 * h + 7] * r) << 16);
    }
    scales[row * (cols / 16) + blk] = (uint8_t)bs;
    *(uint2*)(codes + (base + blk * 16) / 2) = make_uint2(w[0], w[1]);
  }
}

// NVFP4 dispatch quantisation of BF16 rows, each with its own global scale
// from its amax: the arithmetic of k_quant_nv, one wave per row (four rows
// per workgroup, no workgroup barrier) and lane l holding 32 consecutive
// values, two 16-element blocks, of each 2048-column chunk.  The row is read
// twice, for its amax and for its codes; the second read finds it in cache.
__global__ void __launch_bounds__(256) k_quant_nv_rows(const uint16_t* __restrict__ src, int64_t rows, int cols,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       float* __restrict__ row_g) {
#pragma clang fp contract(off)
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* p = src + row * cols;
  auto load32 = [&](int c, float (&v)[32]) __attribute__((always_inline)) {
    const uint4* q = (const uint4*)(p + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = q[i];
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = u2f(wd[j] << 16);
        v[8 * i + 2 * j + 1] = u2f(wd[j] & 0xFFFF0000u);
      }
    }
  };
  float amax = 0.0f;
  for (int c = l * 32; c < cols; c += 64 * 32) {
    float v[32];
    load32(c, v);
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
  amax = group_max<6>(amax);
  const float g = amax > 0.0f ? amax / 2688.0f : 1.0f;
  if (l == 0) row_g[row] = g;
  const float six_g = 6.0f * g;
  for (int c = l * 32; c < cols; c += 64 * 32) {
    float v[32];
    load32(c, v);
    uint32_t w[4] = {0, 0, 0, 0}, bs2 = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* b = v + 16 * h;
      float bmax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) bmax = __builtin_fmaxf(bmax, __builtin_fabsf(b[i]));
      const uint32_t bs = e4m3_encode(bmax / six_g);
      const float bsv = e4m3_decode(bs);
      if (bsv != 0.0f) {
        const float r = 1.0f / (bsv * g);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          w[2 * h + q] = e2m1_x4(b[8 * q] * r, b[8 * q + 1] * r, b[8 * q + 2] * r, b[8 * q + 3] * r) |
                         (e2m1_x4(b[8 * q + 4] * r, b[8 * q + 5] * r, b[8 * q + 6] * r, b[8 * q + 7] * r) << 16);
      }
      bs2 |= bs << (8 * h);
    }
    *(uint16_t*)(scales + row * (cols / 16) + c / 16) = (uint16_t)bs2;
    *(uint4*)(codes + (row * cols + c) / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Per-expert amax -> NVFP4 global scale amax / (6 * 448) (1 if zero).
__global__ void __launch_bounds__(256) k_weight_gscale(const float* __restrict__ src, int64_t per_expert,
                                                       float* __restrict__ gscale) {
  __shared__ float red[4];
  const float* p = src + (int64_t)blockIdx.x * per_expert;
  float amax = 0.0f;
  for (int64_t i = threadIdx.x; i < per_expert; i += 256) amax = __builtin_fmaxf(amax, __builtin_fabsf(p[i]));
  amax = group_max<6>(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    gscale[blockIdx.x] = m > 0.0f ? m / 2688.0f : 1.0f;
  }
}

void launch_weight_gscale(int E, int64_t per_expert, const float* src, float* gscale, hipStream_t st) {
  hipLaunchKernelGGL(k_weight_gscale, dim3(E), dim3(256), 0, st, src, per_expert, gscale);
}

void launch_quant_mx(bool fp4, bool f32, int64_t rows, int cols, const void* src, uint8_t* codes, uint8_t* scales,
                     hipStream_t st) {
  const int64_t nblocks = rows * (cols / 32);
  const dim3 grid((unsigned)((nblocks + 255) / 256));
  if (f32) {
    if (fp4) hipLaunchKernelGGL((k_quant_mx<true, true>), grid, dim3(256), 0, st, src, nblocks, codes, scales);
    else hipLaunchKernelGGL((k_quant_mx<true, false>), grid, dim3(256), 0, st, src, nblocks, codes, scales);
  } else {
    if (fp4) hipLaunchKernelGGL((k_quant_mx<false, true>), grid, dim3(256), 0, st, src, nblocks, codes, scales);
    else hipLaunchKernelGGL((k_quant_mx<false, false>), grid, dim3(256), 0, st, src, nblocks, codes, scales);
  }
}

void launch_quant_nv(bool f32, int64_t rows, int cols, const void* src, uint8_t* codes, uint8_t* scales,
                     float* row_g, const float* fixed_g, int rows_per_g, hipStream_t st) {
  if (f32)
    hipLaunchKernelGGL((k_quant_nv<true>), dim3((unsigned)rows), dim3(256), 0, st, src, cols, codes, scales, row_g,
                       fixed_g, rows_per_g);
  else if (!fixed_g)
    hipLaunchKernelGGL(k_quant_nv_rows, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, (const uint16_t*)src, rows,
                       cols, codes, scales, row_g);
  else
    hipLaunchKernelGGL((k_quant_nv<false>), dim3((unsigned)rows), dim3(256), 0, st, src, cols, codes, scales, row_g,
                       fixed_g, rows_per_g);
}

}  // namespace moe
