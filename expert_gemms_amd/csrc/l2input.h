// The gated activation and the quantisation of the L2 input, shared by the L1
// GEMM epilogue and the kernel that finishes a K-split L1 GEMM, so both
// write identical codes for identical activations.
//
// Activation (MegaMoEActivation on the DeepGEMM MegaMoE experts page): with a
// clamp c, gate <- min(gate, c) and up <- clamp(up, -c, c); then
// gate * sigmoid(alpha * gate) * (up + beta), float32 with the hardware exp
// and reciprocal.  L2-input quantisation (the per-group quantisation between
// the two GEMMs in the "fused_moe" page's DeepGemmExperts.apply): BF16 RNE;
// MXFP8 one UE8M0 scale per 32 intermediate columns; NVFP4 one E4M3 scale
// per 16 columns with the one global scale g2, E2M1 codes two per byte.
// Scales go to planes of one byte per sorted row (plane stride c_sf_ld).
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

// Element codes by the gfx950 converts, which round to nearest even (ties to
// the even code) like e2m1_encode / e4m3_encode and equal them code for code
// (checked on the hardware over a dense sweep, every midpoint and both
// signs): E2M1 saturates to 6 as e2m1_encode does; E4M3 equals e4m3_encode
// for |x| <= 448, which the MX scale choice guarantees here (the block's
// amax / 2^(c - 127) <= 448).  Element i of the result takes bits 4i (E2M1)
// or 8i (E4M3).
__device__ __forceinline__ uint32_t e2m1_x4(float a0, float a1, float a2, float a3) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a0, a1, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, a2, a3, 1.0f, 1);
  return r & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e2m1_x1(float a) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, 0.0f, 1.0f, 0) & 0xFu;
}
__device__ __forceinline__ uint32_t e4m3_x4_mx(float a0, float a1, float a2, float a3) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
  return (uint32_t)r;
}
__device__ __forceinline__ uint32_t e4m3_x1_mx(float a) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false) & 0xFFu;
}

// CLAMP: whether the clamp applies (p.has_clamp), fixed at compile time by
// callers that evaluate many activations per branch.
template <bool CLAMP>
__device__ __forceinline__ float act_swiglu_c(float g, float u, const GemmArgs& p) {
  if constexpr (CLAMP) {
    g = __builtin_fminf(g, p.clamp);
    u = __builtin_fminf(__builtin_fmaxf(u, -p.clamp), p.clamp);
  }
  float s = __builtin_amdgcn_rcpf(1.0f + __expf(-p.alpha * g));
  return g * s * (u + p.beta);
}

__device__ __forceinline__ float act_swiglu(float g, float u, const GemmArgs& p) {
  return p.has_clamp ? act_swiglu_c<true>(g, u, p) : act_swiglu_c<false>(g, u, p);
}

// Activation value a of sorted row `row`, intermediate column icol.  The 32
// lanes of a half-wave hold 32 consecutive columns (icol % 32 == l32) of one
// row: the MX scale group is the half-wave, the NVFP4 group 16 lanes.
template <int FMT>
__device__ __forceinline__ void store_l2_input(float a, int64_t row, int icol, int l32, const GemmArgs& p) {
  if constexpr (FMT == F_NVFP4) {
#pragma clang fp contract(off)
    const float amax = group_max<4>(__builtin_fabsf(a));
    const float six_g = 6.0f * p.l2_scale;
    const uint32_t bs = e4m3_encode(amax / six_g);
    const float bsv = e4m3_decode(bs);
    uint32_t q = 0;
    if (bsv != 0.0f) {
      const float r = 1.0f / (bsv * p.l2_scale);
      q = e2m1_x1(a * r);
    }
    const uint32_t qn = (uint32_t)shfl_xor((int)q, 1);
    if ((l32 & 1) == 0) p.c[row * p.c_ld + (icol >> 1)] = (uint8_t)(q | (qn << 4));
    if ((l32 & 15) == 0) p.c_sf[(int64_t)(icol >> 4) * p.c_sf_ld + row] = (uint8_t)bs;
  } else if constexpr (FMT == F_BF16) {
    // stage-blocked: [M / bm][I / 32][bm][32]
    ((uint16_t*)p.c)[((row / p.bm) * (p.inter / 32) + icol / 32) * p.bm * 32 + (row % p.bm) * 32 + icol % 32] = bf16_rne(a);
  } else {
    const float amax = group_max<5>(__builtin_fabsf(a));
    uint32_t q = 0;
    int c = 0;
    if (amax > 0.0f) {
      c = mx_scale_code<false>(amax);
      q = e4m3_x1_mx(__builtin_ldexpf(a, 127 - c));
    }
    p.c[row * p.c_ld + icol] = (uint8_t)q;
    if (l32 == 0) p.c_sf[(int64_t)(icol >> 5) * p.c_sf_ld + row] = (uint8_t)c;
  }
}

// The same quantisation for the L1 epilogue's layout: the lane holds
// activations a[4j + i] of sorted row `row`, intermediate columns
// icol0 + 8j + 4g + i (g = lane / 32), and lane l ^ 32 holds the rest of the
// 32 columns from icol0 on.  Block maxima: the lane's values, then the
// partner's; codes and scales are those store_l2_input writes for the same
// activations.  Stores: 4 consecutive columns at a time.
template <int FMT>
__device__ __forceinline__ void store_l2_input_rows(const float (&a)[16], int64_t row, int icol0, int g,
                                                    const GemmArgs& p) {
  if constexpr (FMT == F_NVFP4) {
#pragma clang fp contract(off)
    const float six_g = 6.0f * p.l2_scale;
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // 16-column block h: values 8h .. 8h+7
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(a[8 * h + i]));
      amax = __builtin_fmaxf(amax, shfl_xor(amax, 32));
      const uint32_t bs = e4m3_encode(amax / six_g);
      const float bsv = e4m3_decode(bs);
      const float r = bsv != 0.0f ? 1.0f / (bsv * p.l2_scale) : 0.0f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * h + jj;
        uint32_t q = 0;
        if (bsv != 0.0f) q = e2m1_x4(a[4 * j] * r, a[4 * j + 1] * r, a[4 * j + 2] * r, a[4 * j + 3] * r);
        *(uint16_t*)(p.c + row * p.c_ld + ((icol0 + 8 * j + 4 * g) >> 1)) = (uint16_t)q;
      }
      if (g == h) p.c_sf[(int64_t)((icol0 >> 4) + h) * p.c_sf_ld + row] = (uint8_t)bs;
    }
  } else if constexpr (FMT == F_BF16) {
    // stage-blocked: [M / bm][I / 32][bm][32]; the 32 columns from icol0 on
    // are one stage
    uint16_t* out = (uint16_t*)p.c + ((row / p.bm) * (p.inter / 32) + icol0 / 32) * p.bm * 32 + (row % p.bm) * 32 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(uint2*)(out + 8 * j) = make_uint2((uint32_t)bf16_rne(a[4 * j]) | ((uint32_t)bf16_rne(a[4 * j + 1]) << 16),
                                          (uint32_t)bf16_rne(a[4 * j + 2]) | ((uint32_t)bf16_rne(a[4 * j + 3]) << 16));
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) amax = __builtin_fmaxf(amax, __builtin_fabsf(a[v]));
    amax = __builtin_fmaxf(amax, shfl_xor(amax, 32));
    int c = 0;
    if (amax > 0.0f) c = mx_scale_code<false>(amax);
    uint8_t* out = p.c + row * p.c_ld + icol0 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t q = 0;
      if (amax > 0.0f)
        q = e4m3_x4_mx(__builtin_ldexpf(a[4 * j], 127 - c), __builtin_ldexpf(a[4 * j + 1], 127 - c),
                       __builtin_ldexpf(a[4 * j + 2], 127 - c), __builtin_ldexpf(a[4 * j + 3], 127 - c));
      *(uint32_t*)(out + 8 * j) = q;
    }
    if (g == 0) p.c_sf[(int64_t)(icol0 >> 5) * p.c_sf_ld + row] = (uint8_t)c;
  }
}

template <bool F32>
__device__ __forceinline__ float load_elem(const void* src, int64_t i) {
  if (F32) return ((const float*)src)[i];
  uint32_t b = (uint32_t)((const uint16_t*)src)[i] << 16;
  return u2f(b);
}

// MX block b (32 elements of src): its UE8M0 scale and element codes,
// written unpacked for E4M3 and two per byte for E2M1, by the hardware
// converts (equal to the software encoders here: the scaled block maximum is
// at most the format's largest value).  Returns the scale code.
template <bool F32, bool FP4>
__device__ __forceinline__ int quant_mx_block(const void* __restrict__ src, int64_t b, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
#pragma clang fp contract(off)
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = load_elem<F32>(src, b * 32 + i);
    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
  int c = 0;
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (amax > 0.0f) {
    c = mx_scale_code<FP4>(amax);
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_ldexpf(v[i], 127 - c);
#pragma unroll
    for (int j = 0; j < (FP4 ? 4 : 8); ++j) {
      if constexpr (FP4)
        w[j] = e2m1_x4(x[8 * j], x[8 * j + 1], x[8 * j + 2], x[8 * j + 3]) |
               (e2m1_x4(x[8 * j + 4], x[8 * j + 5], x[8 * j + 6], x[8 * j + 7]) << 16);
      else
        w[j] = e4m3_x4_mx(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
    }
  }
  scales[b] = (uint8_t)c;
  if (FP4) {
    *(uint4*)(codes + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *(uint4*)(codes + b * 32) = make_uint4(w[0], w[1], w[2], w[3]);
    *(uint4*)(codes + b * 32 + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  }
  return c;
}

}  // namespace moe
