// Top-k combine: y[t] = sum_j w[t, j] * O[t * k' + j], one round to BF16.
// When the L2 GEMM split K, O[slot] is the sum of its parts, added in part
// order before the weighting.  The rows are float32 for BF16 layers and split
// L2s, BF16 for the block-scaled formats (the L2 output in the activation
// dtype, as the unfused decomposition keeps it); the sum is float32 either way.
//
// The weighted un-permute-and-reduce of the "fused_moe" page's
// DeepGemmExperts.apply (deepgemm_unpermute_and_reduce; CutlassExpertsFp8
// notes the top-k weights and the reduction fused in one unpermute kernel),
// into BF16 [T, H] as DeepGemmMegaMoEExperts.forward returns it.  The L2
// epilogue stores O by slot, so each token's k' rows are contiguous and the
// gather is a stream.  Shared-expert slots carry weight 1; dropped slots
// (slot_row < 0) contribute nothing.  The float32 sum runs in slot order.
#include "common.h"
#include "launch.h"

namespace moe {

// Columns h .. h+3 of slot row s: float32 rows (with K split, the parts
// added in part order) or BF16 rows (one part).  Slot rows are read once, so
// their loads are non-temporal.
template <bool O16>
__device__ __forceinline__ f32x4 slot_cols(const float* __restrict__ o, int nsplit, int64_t o_split, int64_t s,
                                           int H, int h) {
  if constexpr (O16) {
    const uint2 b = *(const uint2*)((const uint16_t*)o + s * H + h);
    return (f32x4){u2f(b.x << 16), u2f(b.x & 0xFFFF0000u), u2f(b.y << 16), u2f(b.y & 0xFFFF0000u)};
  } else {
    f32x4 v = __builtin_nontemporal_load((const f32x4*)(o + s * H + h));
    for (int q = 1; q < nsplit; ++q) v += __builtin_nontemporal_load((const f32x4*)(o + q * o_split + s * H + h));
    return v;
  }
}

// Columns h .. h+3 of slot s after an L2 with a split tail (TailSplit ts):
// the slot's row in the tile that computed those columns (BLOCK_M block of
// its sorted row m, 256-column block of h, numbered as the GEMM numbers its
// tiles) is a whole tile's row in o, or a tail tile's parts in o_tail, added
// in part order.  A dropped slot (m < 0) gives zeros.
__device__ __forceinline__ f32x4 slot_cols_tail(const float* __restrict__ o, const CombineTail& tl, TailSplit ts,
                                                const int32_t* __restrict__ slot_row, int64_t s, int H, int h) {
  const int m = slot_row[s];
  if (m < 0) return (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  const int mb = m / tl.bm;
  const int4 ti = *(const int4*)(tl.tile_info + 4 * mb);   // expert, its first block, its block count
  const int u = ti.y * (H / GEMM_BN) + (h / GEMM_BN) * ti.z + (mb - ti.y);
  if (u < ts.full) return __builtin_nontemporal_load((const f32x4*)(o + s * H + h));
  const float* p = tl.o_tail + ((int64_t)(u - ts.full) * ts.kt * tl.bm + m % tl.bm) * GEMM_BN + h % GEMM_BN;
  f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  for (int q = 1; q < ts.kt; ++q) v += __builtin_nontemporal_load((const f32x4*)(p + (int64_t)q * tl.bm * GEMM_BN));
  return v;
}

// Weighted sum of token t's slot rows at columns h .. h+3, in slot order.
// The rows are loaded 8 slots at a time before any is added, so a thread
// keeps 8 loads in flight; a dropped slot's row (never written) is loaded
// but not added.  TL: float32 rows of an L2 with a split tail.
template <bool O16, bool TL = false>
__device__ __forceinline__ f32x4 token_sum(const float* __restrict__ o, int nsplit, int64_t o_split,
                                           const int32_t* __restrict__ slot_row,
                                           const float* __restrict__ topk_w, int t, int k, int kk, int H, int h,
                                           const CombineTail& tl = CombineTail{}) {
  const int64_t s0 = (int64_t)t * kk;
  TailSplit ts = {0, 0, 1};
  if constexpr (TL) ts = tail_split(tl.meta[0] * (H / GEMM_BN), tl.nw, tl.kmax, tl.cap, tl.nst);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < kk; j0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (j0 + i < kk) {
        if constexpr (TL)
          v[i] = slot_cols_tail(o, tl, ts, slot_row, s0 + j0 + i, H, h);
        else
          v[i] = slot_cols<O16>(o, nsplit, o_split, s0 + j0 + i, H, h);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      if (j < kk && slot_row[s0 + j] >= 0) {
        const float wt = j < k && topk_w ? topk_w[(int64_t)t * k + j] : 1.0f;
        acc[0] += wt * v[i][0];
        acc[1] += wt * v[i][1];
        acc[2] += wt * v[i][2];
        acc[3] += wt * v[i][3];
      }
    }
  }
  return acc;
}

// The same sum over BF16 slot rows at columns h .. h+7: one 16-byte load per
// row, the additions of each column in the same order and form as token_sum.
__device__ __forceinline__ void token_sum8(const uint16_t* __restrict__ o16, const int32_t* __restrict__ slot_row,
                                           const float* __restrict__ topk_w, int t, int k, int kk, int H, int h,
                                           float (&acc)[8]) {
  const int64_t s0 = (int64_t)t * kk;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  for (int j0 = 0; j0 < kk; j0 += 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (j0 + i < kk) {
        const i32x4 q = __builtin_nontemporal_load((const i32x4*)(o16 + (s0 + j0 + i) * H + h));
        v[i] = make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      if (j < kk && slot_row[s0 + j] >= 0) {
        const float wt = j < k && topk_w ? topk_w[(int64_t)t * k + j] : 1.0f;
        const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += wt * u2f((c & 1) ? (wd[c >> 1] & 0xFFFF0000u) : (wd[c >> 1] << 16));
      }
    }
  }
}

// BF16 slot rows: workgroup (t, c) takes token t, columns [8 B c, 8 B (c + 1))
// for B = blockDim.x threads, 8 per thread (one workgroup per token up to
// H = 8192, so no column block is left partly idle).
__global__ void __launch_bounds__(1024) k_combine16(const uint16_t* __restrict__ o16,
                                                    const int32_t* __restrict__ slot_row,
                                                    const float* __restrict__ topk_w, int k, int kk, int H,
                                                    uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (h >= H) return;
  float acc[8];
  token_sum8(o16, slot_row, topk_w, t, k, kk, H, h, acc);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)bf16_rne(acc[2 * i]) | ((uint32_t)bf16_rne(acc[2 * i + 1]) << 16);
  *(uint4*)(out + (int64_t)t * H + h) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Workgroup (t, c): token t, columns [1024 c, 1024 c + 1024), 4 per thread.
template <bool O16, bool TL>
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ o, int nsplit, int64_t o_split,
                                                 const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ topk_w, int k, int kk, int H,
                                                 CombineTail tl, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 1024 + threadIdx.x * 4;
  if (h >= H) return;
  const f32x4 acc = token_sum<O16, TL>(o, nsplit, o_split, slot_row, topk_w, t, k, kk, H, h, tl);
  uint2 packed;
  packed.x = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
  packed.y = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
  *(uint2*)(out + (int64_t)t * H + h) = packed;
}

// With the post-expert RMSNorm: one workgroup per token keeps the float32 row
// in LDS, sums its squares, then writes y / sqrt(mean(y^2) + eps) * gamma.
// The weighting matches k_combine element for element.
template <bool O16, bool TL>
__global__ void __launch_bounds__(256) k_combine_norm(const float* __restrict__ o, int nsplit, int64_t o_split,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w, int k, int kk, int H,
                                                      const float* __restrict__ gamma, float eps, CombineTail tl,
                                                      uint16_t* __restrict__ out) {
  extern __shared__ f32x4 rowv[];   // H / 4
  __shared__ float red[4];
  const int t = blockIdx.x;
  float ss = 0.0f;
  for (int h = threadIdx.x * 4; h < H; h += 1024) {
    const f32x4 acc = token_sum<O16, TL>(o, nsplit, o_split, slot_row, topk_w, t, k, kk, H, h, tl);
    rowv[h >> 2] = acc;
    ss += acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] + acc[3] * acc[3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / __builtin_sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int h = threadIdx.x * 4; h < H; h += 1024) {
    const f32x4 acc = rowv[h >> 2];
    const f32x4 g = *(const f32x4*)(gamma + h);
    uint2 packed;
    packed.x = (uint32_t)bf16_rne(acc[0] * r * g[0]) | ((uint32_t)bf16_rne(acc[1] * r * g[1]) << 16);
    packed.y = (uint32_t)bf16_rne(acc[2] * r * g[2]) | ((uint32_t)bf16_rne(acc[3] * r * g[3]) << 16);
    *(uint2*)(out + (int64_t)t * H + h) = packed;
  }
}

// apply_router_weight_on_input: xw[t] = BF16(x[t] * w[t]) (top_k = 1), float32
// product, one round to nearest even.
__global__ void __launch_bounds__(256) k_scale_rows(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                    int H, uint16_t* __restrict__ xw) {
  const int t = blockIdx.x;
  const float s = w[t];
  for (int h = threadIdx.x * 4; h < H; h += 1024) {
    const uint2 v = *(const uint2*)(x + (int64_t)t * H + h);
    const float a = u2f(v.x << 16) * s, b = u2f(v.x & 0xFFFF0000u) * s;
    const float c = u2f(v.y << 16) * s, d = u2f(v.y & 0xFFFF0000u) * s;
    uint2 r;
    r.x = (uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16);
    r.y = (uint32_t)bf16_rne(c) | ((uint32_t)bf16_rne(d) << 16);
    *(uint2*)(xw + (int64_t)t * H + h) = r;
  }
}

void launch_combine(const float* o, int o_bf16, int nsplit, int64_t o_split, const int32_t* slot_row,
                    const float* topk_w, int T, int k, int kk, int H, const float* gamma, float eps,
                    const CombineTail& tl, uint16_t* out, hipStream_t stream) {
  const dim3 grid(T, (H + 1023) / 1024);
  const bool tail = !o_bf16 && tl.o_tail;
  if (gamma && o_bf16)
    hipLaunchKernelGGL((k_combine_norm<true, false>), dim3(T), dim3(256), (size_t)H * 4, stream, o, nsplit, o_split,
                       slot_row, topk_w, k, kk, H, gamma, eps, tl, out);
  else if (gamma && tail)
    hipLaunchKernelGGL((k_combine_norm<false, true>), dim3(T), dim3(256), (size_t)H * 4, stream, o, nsplit, o_split,
                       slot_row, topk_w, k, kk, H, gamma, eps, tl, out);
  else if (gamma)
    hipLaunchKernelGGL((k_combine_norm<false, false>), dim3(T), dim3(256), (size_t)H * 4, stream, o, nsplit, o_split,
                       slot_row, topk_w, k, kk, H, gamma, eps, tl, out);
  else if (o_bf16) {
    // H / 8 threads (a multiple of 16, as H is of 128), at most 1024
    const int threads = H / 8 <= 1024 ? H / 8 : 1024;
    hipLaunchKernelGGL(k_combine16, dim3(T, (H / 8 + threads - 1) / threads), dim3(threads), 0, stream,
                       (const uint16_t*)o, slot_row, topk_w, k, kk, H, out);
  } else if (tail)
    hipLaunchKernelGGL((k_combine<false, true>), grid, dim3(256), 0, stream, o, nsplit, o_split, slot_row, topk_w, k,
                       kk, H, tl, out);
  else
    hipLaunchKernelGGL((k_combine<false, false>), grid, dim3(256), 0, stream, o, nsplit, o_split, slot_row, topk_w, k,
                       kk, H, tl, out);
}

void launch_scale_rows(const uint16_t* x, const float* w, int T, int H, uint16_t* xw, hipStream_t stream) {
  hipLaunchKernelGGL(k_scale_rows, dim3(T), dim3(256), 0, stream, x, w, H, xw);
}

}  // namespace moe
