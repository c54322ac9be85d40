// Top-k combine: y[t] = sum_j w[t, j] * O[t * k' + j], one round to BF16.
// When the L2 GEMM split K, O[slot] is the sum of its parts, added in part
// order before the weighting.
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

// Workgroup (t, c): token t, columns [1024 c, 1024 c + 1024), 4 per thread;
// every load of a thread is independent, so a token's k' x nsplit rows stream
// in together.
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ o, int nsplit, int64_t o_split,
                                                 const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ topk_w, int k, int kk, int H,
                                                 uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 1024 + threadIdx.x * 4;
  if (h >= H) return;
  const int64_t s0 = (int64_t)t * kk;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < kk; ++j) {
    if (slot_row[s0 + j] < 0) continue;
    const float wt = j < k ? topk_w[(int64_t)t * k + j] : 1.0f;
    f32x4 v = *(const f32x4*)(o + (s0 + j) * H + h);
    for (int q = 1; q < nsplit; ++q) v += *(const f32x4*)(o + q * o_split + (s0 + j) * H + h);
    acc[0] += wt * v[0];
    acc[1] += wt * v[1];
    acc[2] += wt * v[2];
    acc[3] += wt * v[3];
  }
  uint2 packed;
  packed.x = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
  packed.y = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
  *(uint2*)(out + (int64_t)t * H + h) = packed;
}

void launch_combine(const float* o, int nsplit, int64_t o_split, const int32_t* slot_row, const float* topk_w,
                    int T, int k, int kk, int H, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_combine, dim3(T, (H + 1023) / 1024), dim3(256), 0, stream, o, nsplit, o_split, slot_row,
                     topk_w, k, kk, H, out);
}

}  // namespace moe
