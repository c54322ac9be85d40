// Router top-k: router logits [T, E] -> topk_ids [T, k], topk_weights [T, k].
//
// The routing functions the "fused_moe" page's FusedMoE.select_experts picks
// from (fused_topk: softmax scores, top-k, renormalise; fused_topk_bias: a
// per-expert correction bias on the choice, weights times
// routed_scaling_factor; grouped_topk: num_expert_group groups of which
// topk_group are kept, softmax or sigmoid scores), and the padding-token skip
// of the DeepGEMM MegaMoE experts page's forward (a padding token's slots
// are all dropped: ids -1, weights 0).  Scores are float32; the choice score
// is score + bias; a group ranks by its best choice score; ties go to the
// lower expert (or group) id; ids are listed best first; the weights are the
// unbiased scores of the chosen experts, divided by their sum when
// renormalising, then times the scaling factor.
//
// One wave per token; lane l holds experts l, l + 64, ... (NJ per lane), so
// every reduction is six DPP lane moves inside the wave and each of the k
// picks is one wave-wide (value, id) argmax.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

template <int V> using IC = std::integral_constant<int, V>;

// Wave-wide reductions with DPP lane moves (no LDS round trips): quad
// swaps, half-row and row mirrors, then the row broadcasts carry rows 0-2
// into lane 63, which holds the result; readlane makes it uniform.  Lanes a
// move does not reach keep their own value (old = src).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}

template <typename F>
__device__ __forceinline__ void dpp_reduce(F&& step) {
  step(IC<0xB1>{}, IC<0xF>{});    // quad_perm [1,0,3,2]
  step(IC<0x4E>{}, IC<0xF>{});    // quad_perm [2,3,0,1]
  step(IC<0x141>{}, IC<0xF>{});   // row_half_mirror
  step(IC<0x140>{}, IC<0xF>{});   // row_mirror
  step(IC<0x142>{}, IC<0xA>{});   // row_bcast:15 into rows 1, 3
  step(IC<0x143>{}, IC<0xC>{});   // row_bcast:31 into rows 2, 3
}

__device__ __forceinline__ float wave_max(float v) {
  dpp_reduce([&](auto c, auto r) {
    const float o = __builtin_bit_cast(float, dpp<decltype(c)::value, decltype(r)::value>(__builtin_bit_cast(int, v)));
    v = __builtin_fmaxf(v, o);
  });
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  // the mirrors pair each lane with another one, so every lane's value is
  // counted once in lane 63's running sum
  dpp_reduce([&](auto c, auto r) {
    constexpr int C = decltype(c)::value, R = decltype(r)::value;
    const float o = __builtin_bit_cast(float, dpp<C, R>(__builtin_bit_cast(int, v)));
    if constexpr (R == 0xF) {
      v = v + o;
    } else {
      // row broadcasts: only the receiving rows add (others got their own value back)
      const int row = lane_id() >> 4;
      if ((R >> row) & 1) v = v + o;
    }
  });
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// (value, id) of the best candidate across the wave: larger value, then lower
// id; uniform on return
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  dpp_reduce([&](auto c, auto r) {
    constexpr int C = decltype(c)::value, R = decltype(r)::value;
    const float ov = __builtin_bit_cast(float, dpp<C, R>(__builtin_bit_cast(int, v)));
    const int oi = dpp<C, R>(id);
    if (ov > v || (ov == v && oi < id)) {
      v = ov;
      id = oi;
    }
  });
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  id = __builtin_amdgcn_readlane(id, 63);
}

template <int NJ>
__global__ void __launch_bounds__(256) k_route(const float* __restrict__ logits, const float* __restrict__ bias, int T,
                                               int E, int k, int sigmoid, int G, int TG, int renorm, float scaling,
                                               const uint8_t* __restrict__ is_padding, int32_t* __restrict__ ids,
                                               float* __restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // uniform over the wave
  int32_t* out_id = ids + (int64_t)t * k;
  float* out_w = wts + (int64_t)t * k;
  if (is_padding && is_padding[t]) {
    for (int r = lane; r < k; r += 64) {
      out_id[r] = -1;
      out_w[r] = 0.0f;
    }
    return;
  }
  const float NEG = -__builtin_huge_valf();
  const float* row = logits + (int64_t)t * E;
  float s[NJ], c[NJ];
  float mx = NEG;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    s[j] = e < E ? row[e] : NEG;
    mx = __builtin_fmaxf(mx, s[j]);
  }
  if (!sigmoid) {
    mx = wave_max(mx);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      s[j] = lane + 64 * j < E ? __expf(s[j] - mx) : 0.0f;
      sum += s[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < NJ; ++j) s[j] = s[j] / sum;
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) s[j] = lane + 64 * j < E ? 1.0f / (1.0f + __expf(-s[j])) : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    c[j] = e < E ? s[j] + (bias ? bias[e] : 0.0f) : NEG;
  }
  if (G > 1) {
    // lane g < G holds group g's rank: its best choice score
    const int gs = E / G;
    float gscore = NEG;
    for (int g = 0; g < G; ++g) {
      float m = NEG;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if ((lane + 64 * j) / gs == g) m = __builtin_fmaxf(m, c[j]);
      m = wave_max(m);
      if (lane == g) gscore = m;
    }
    uint64_t keep = 0;
    for (int r = 0; r < TG; ++r) {
      float v = lane < G && !((keep >> lane) & 1) ? gscore : NEG;
      int id = lane < G && !((keep >> lane) & 1) ? lane : 0x7FFFFFFF;
      wave_argmax(v, id);
      keep |= 1ull << id;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((keep >> (e / gs)) & 1)) c[j] = NEG;
    }
  }
  int my_id = -1;
  float my_w = 0.0f, wsum = 0.0f;
  for (int r = 0; r < k; ++r) {
    float v = NEG;
    int id = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < E && c[j] != NEG && (c[j] > v || id == 0x7FFFFFFF)) {
        v = c[j];
        id = e;
      }
    }
    wave_argmax(v, id);
    // the winner's unbiased score, from its lane; the winner leaves the race
    const int wl = id & 63, wj = id >> 6;
    float sc = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (j == wj) sc = s[j];
    sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), wl));
    if (lane == wl) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (j == wj) c[j] = NEG;
    }
    if (lane == r) {
      my_id = id;
      my_w = sc;
    }
    wsum += sc;
  }
  if (lane < k) {
    float w = renorm ? my_w / wsum : my_w;
    out_id[lane] = my_id;
    out_w[lane] = w * scaling;
  }
}

void launch_route(const float* logits, const float* bias, int T, int E, int k, int sigmoid, int G, int TG,
                  int renorm, float scaling, const uint8_t* is_padding, int32_t* ids, float* wts,
                  hipStream_t stream) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  const int nj = (E + 63) / 64;
  if (nj <= 1)
    hipLaunchKernelGGL(k_route<1>, grid, block, 0, stream, logits, bias, T, E, k, sigmoid, G, TG, renorm, scaling,
                       is_padding, ids, wts);
  else if (nj <= 2)
    hipLaunchKernelGGL(k_route<2>, grid, block, 0, stream, logits, bias, T, E, k, sigmoid, G, TG, renorm, scaling,
                       is_padding, ids, wts);
  else if (nj <= 4)
    hipLaunchKernelGGL(k_route<4>, grid, block, 0, stream, logits, bias, T, E, k, sigmoid, G, TG, renorm, scaling,
                       is_padding, ids, wts);
  else if (nj <= 8)
    hipLaunchKernelGGL(k_route<8>, grid, block, 0, stream, logits, bias, T, E, k, sigmoid, G, TG, renorm, scaling,
                       is_padding, ids, wts);
  else
    hipLaunchKernelGGL(k_route<16>, grid, block, 0, stream, logits, bias, T, E, k, sigmoid, G, TG, renorm, scaling,
                       is_padding, ids, wts);
}

}  // namespace moe
