// Canonical weights -> the kernel layout the grouped GEMMs read.
//
// The page's own kernel layout (DeepGEMM MegaMoE experts page,
// _kernel_layout_shard / _pack_scale; Muse-Spark page,
// transform_weights_for_mega_moe) interleaves gate and up rows so one L1
// output tile holds matching columns, and repacks block scales for its
// hardware's loads.  This layout keeps that idea for gfx950: gate and up rows
// alternate in 32-row blocks (the width of one 32x32 MFMA tile, so SiLU(g)*u
// pairs accumulators of the same lane), and each 32-row x K-step fragment is
// stored in the exact order of the MFMA operand registers:
//   BF16 (32x32x16):  1 KiB, lane l = row l%32, bytes [32ks + 16(l/32), +16)
//   FP8  (32x32x64):  2 KiB, half j: lane l = row l%32, bytes
//                     [64ks + 32j + 16(l/32), +16)  (8-bit operands hold K
//                     [16g,16g+16) in register bytes 0-15 and [32+16g, ..)
//                     in bytes 16-31 of lane group g)
//   FP4  (32x32x64):  1 KiB, lane l = row l%32, bytes [32ks + 16(l/32), +16)
//                     (4-bit operands hold K [32g, 32g+32) contiguously)
// BF16 fragments are ordered [256-row N block][64-K stage][32-row block of
// the 8][K-step within the stage], so the weights one 256-column tile streams
// over all of K are one contiguous run (measured 2.5 % faster for the
// MFMA-bound BF16 GEMMs).  The other formats keep [128-K stage][32-row block]
// [K-step within the stage]: the blocks of the tiles that run side by side
// are adjacent (measured faster for weight-streaming launches).  UE8M0 scales
// become [128-K stage][32-row block][lane][2]: byte j of lane l is the scale
// of row l%32, block 4*stage + 2j + l/32, the byte the scaled MFMA of K-step
// j takes from that lane.
#include "common.h"
#include "launch.h"

namespace moe {

// One thread per 16-byte destination chunk of one matrix (all experts).
template <int FMT, bool W13>
__global__ void __launch_bounds__(256) k_transform_codes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int N, int K, int inter, int64_t chunks_per_expert,
                                                         int64_t total) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int64_t e = c / chunks_per_expert, ce = c % chunks_per_expert;
  int n, kbyte;
  int64_t row_bytes;
  const int nls = FMT == F_BF16 ? K / 64 : K / 128;   // K stages
  // BF16: rest = (N block * nls + stage) * 8 + block within the N block;
  // others: rest = stage * (N / 32) + block
  auto split = [&](int64_t rest, int& nf, int& stage) {
    if (FMT == F_BF16) {
      const int64_t t2 = rest >> 3;
      nf = (int)((t2 / nls) * 8 + (rest & 7));
      stage = (int)(t2 % nls);
    } else {
      nf = (int)(rest % (N / 32));
      stage = (int)(rest / (N / 32));
    }
  };
  int nf, stage;
  if (FMT == F_BF16) {
    const int64_t f = ce >> 6;                  // [.. block][4 K-steps of 16]
    const int l = (int)(ce & 63);
    split(f >> 2, nf, stage);
    const int ks = stage * 4 + (int)(f & 3);
    n = nf * 32 + (l & 31);
    kbyte = ks * 32 + (l >> 5) * 16;
    row_bytes = (int64_t)K * 2;
  } else if (FMT == F_MXFP8) {
    const int64_t f = ce >> 7;                  // [.. block][2 K-steps of 64]
    const int within = (int)(ce & 127), j = within >> 6, l = within & 63;
    split(f >> 1, nf, stage);
    const int ks = stage * 2 + (int)(f & 1);
    n = nf * 32 + (l & 31);
    kbyte = ks * 64 + 32 * j + 16 * (l >> 5);
    row_bytes = K;
  } else {  // FP4
    const int64_t f = ce >> 6;                  // [.. block][2 K-steps of 64]
    const int l = (int)(ce & 63);
    split(f >> 1, nf, stage);
    const int ks = stage * 2 + (int)(f & 1);
    n = nf * 32 + (l & 31);
    kbyte = ks * 32 + 16 * (l >> 5);
    row_bytes = K / 2;
  }
  const int srow = W13 ? w13_canonical_row(n, inter) : n;
  const uint8_t* s = src + e * (int64_t)N * row_bytes + (int64_t)srow * row_bytes + kbyte;
  *(uint4*)(dst + c * 16) = *(const uint4*)s;
}

// UE8M0 scales: one thread per destination byte.
template <bool W13>
__global__ void __launch_bounds__(256) k_transform_mx_scales(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                             int N, int K, int inter, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t per_expert = (int64_t)N * (K / 32);
  const int64_t e = i / per_expert, r = i % per_expert;
  const int64_t blk = r / 128;             // (stage, nf) block of 128 bytes
  const int within = (int)(r % 128), l = within >> 1, j = within & 1;
  const int nf = (int)(blk % (N / 32)), stage = (int)(blk / (N / 32));
  const int n = nf * 32 + (l & 31);
  const int kb = stage * 4 + 2 * j + (l >> 5);
  const int srow = W13 ? w13_canonical_row(n, inter) : n;
  dst[i] = src[e * per_expert + (int64_t)srow * (K / 32) + kb];
}

// NVFP4 E4M3 scales: [128-K stage][32-row block][lane][4]: byte 2*kg + i of
// lane l is the scale of row l%32, 16-block 8*stage + 4*kg + 2*(l/32) + i,
// i.e. the blocks of the 32 values lane group l/32 holds in 64-K group kg.
template <bool W13>
__global__ void __launch_bounds__(256) k_transform_nv_scales(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                             int N, int K, int inter, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t per_expert = (int64_t)N * (K / 16);
  const int64_t e = i / per_expert, r = i % per_expert;
  const int64_t blk = r / 256;             // (stage, nf) block of 256 bytes
  const int within = (int)(r % 256), l = within >> 2, b = within & 3;
  const int nf = (int)(blk % (N / 32)), stage = (int)(blk / (N / 32));
  const int n = nf * 32 + (l & 31);
  const int kb = stage * 8 + (b >> 1) * 4 + 2 * (l >> 5) + (b & 1);
  const int srow = W13 ? w13_canonical_row(n, inter) : n;
  dst[i] = src[e * per_expert + (int64_t)srow * (K / 16) + kb];
}

template <int FMT>
static void transform_codes(int E, int N, int K, int inter, bool w13, const uint8_t* src, uint8_t* dst,
                            hipStream_t st) {
  const int64_t bytes = FMT == F_BF16 ? (int64_t)N * K * 2 : (FMT == F_MXFP8 ? (int64_t)N * K : (int64_t)N * K / 2);
  const int64_t cpe = bytes / 16, total = cpe * E;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (w13)
    hipLaunchKernelGGL((k_transform_codes<FMT, true>), grid, dim3(256), 0, st, src, dst, N, K, inter, cpe, total);
  else
    hipLaunchKernelGGL((k_transform_codes<FMT, false>), grid, dim3(256), 0, st, src, dst, N, K, inter, cpe, total);
}

void launch_transform(int fmt, int E, int H, int I, const uint8_t* w13, const uint8_t* w13_sf, const uint8_t* w2,
                      const uint8_t* w2_sf, uint8_t* w13_k, uint8_t* w13_sf_k, uint8_t* w2_k, uint8_t* w2_sf_k,
                      hipStream_t st) {
  switch (fmt) {
    case F_BF16:
      transform_codes<F_BF16>(E, 2 * I, H, I, true, w13, w13_k, st);
      transform_codes<F_BF16>(E, H, I, I, false, w2, w2_k, st);
      return;
    case F_MXFP8:
      transform_codes<F_MXFP8>(E, 2 * I, H, I, true, w13, w13_k, st);
      transform_codes<F_MXFP8>(E, H, I, I, false, w2, w2_k, st);
      break;
    case F_MXFP4:
      transform_codes<F_MXFP4>(E, 2 * I, H, I, true, w13, w13_k, st);
      transform_codes<F_MXFP4>(E, H, I, I, false, w2, w2_k, st);
      break;
    case F_NVFP4: {
      // E2M1 codes share the MXFP4 fragment layout; the E4M3 scales get their own
      transform_codes<F_MXFP4>(E, 2 * I, H, I, true, w13, w13_k, st);
      transform_codes<F_MXFP4>(E, H, I, I, false, w2, w2_k, st);
      const int64_t n13 = (int64_t)E * 2 * I * (H / 16), n2 = (int64_t)E * H * (I / 16);
      hipLaunchKernelGGL((k_transform_nv_scales<true>), dim3((unsigned)((n13 + 255) / 256)), dim3(256), 0, st, w13_sf,
                         w13_sf_k, 2 * I, H, I, n13);
      hipLaunchKernelGGL((k_transform_nv_scales<false>), dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st, w2_sf,
                         w2_sf_k, H, I, I, n2);
      return;
    }
    default:
      return;
  }
  const int64_t t13 = (int64_t)E * 2 * I * (H / 32), t2 = (int64_t)E * H * (I / 32);
  hipLaunchKernelGGL((k_transform_mx_scales<true>), dim3((unsigned)((t13 + 255) / 256)), dim3(256), 0, st, w13_sf,
                     w13_sf_k, 2 * I, H, I, t13);
  hipLaunchKernelGGL((k_transform_mx_scales<false>), dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, st, w2_sf,
                     w2_sf_k, H, I, I, t2);
}

}  // namespace moe
