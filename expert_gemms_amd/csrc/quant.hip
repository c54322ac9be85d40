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
  else
    hipLaunchKernelGGL((k_quant_nv<false>), dim3((unsigned)rows), dim3(256), 0, st, src, cols, codes, scales, row_g,
                       fixed_g, rows_per_g);
}

}  // namespace moe
