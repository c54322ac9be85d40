// Shared device/host definitions of the MI355X (gfx950) fused-MoE library.
//
// Number formats (DeepGEMM MegaMoE experts page, module docstring and
// MegaMoEWeightSpec; element encodings of the OCP FP8 and OCP MX v1.0
// specifications): BF16; FP8 E4M3 (bias 7, max 448, no inf); FP4 E2M1
// (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; two per byte, even element in the
// low nibble); UE8M0 block scales (a biased exponent; the Qwen4-Exp MegaMoE
// page's _requantize moves it into / out of the float32 exponent field);
// E4M3 block scales with a float32 global scale (NVFP4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- vectors
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int WAVE = 64;

// ---------------------------------------------------------------- shapes
// Layer-level constants of the formats.
constexpr int MX_GROUP = 32;   // UE8M0 scale per 32 values along K
constexpr int NV_GROUP = 16;   // E4M3 scale per 16 values along K

// Kernel-layout fragment geometry.  A weight fragment is 32 rows (N) x one
// MFMA K-step, stored as 64 lanes x 16 bytes in the order the MFMA operand
// registers want them (lane l: row l % 32, second K-half when l >= 32).
//   BF16: 32x32x16 MFMA, K-step 16 elements = 32 bytes per row, 1 KiB/frag.
//   FP8:  32x32x64 scaled MFMA, K-step 64 elements = 64 bytes/row, 2 KiB.
//   FP4:  32x32x64 scaled MFMA, K-step 64 elements = 32 bytes/row, 1 KiB.
// w13 rows are interleaved in 32-row blocks: kernel row n -> pair p = n / 64,
// half h = (n / 32) % 2 (0 gate, 1 up), canonical row h * I + p * 32 + n % 32.
__host__ __device__ inline int w13_canonical_row(int n, int inter) {
  return ((n >> 5) & 1) * inter + (n >> 6) * 32 + (n & 31);
}

// ---------------------------------------------------------------- bits
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// float32 -> bf16 bits, round to nearest even: gfx950's conversion
// (v_cvt_pk_bf16_f32), the same bits as adding 0x7FFF plus the kept lsb and
// truncating, for finite inputs.
__device__ __forceinline__ uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---------------------------------------------------------------- E4M3 / E2M1
// Round-to-nearest-even, saturating to the largest finite magnitude; the
// code's sign bit is the input's sign bit.  All steps are exact in float32:
// a power-of-two scaling, an exact subtraction, and rint (ties to even).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
#pragma clang fp contract(off)
  uint32_t sign = (f2u(x) >> 24) & 0x80u;
  float a = __builtin_fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                         // below 2^-6: step 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int e = (int)((f2u(a) >> 23) & 0xFF) - 127;  // 2^-6 <= a < 448 -> e in [-6, 8]
  float m = __builtin_ldexpf(a, -e);           // [1, 2)
  uint32_t q = (uint32_t)__builtin_rintf((m - 1.0f) * 8.0f);
  if (q == 8u) { q = 0; e += 1; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | q;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ uint32_t e2m1_encode(float x) {
#pragma clang fp contract(off)
  uint32_t sign = (f2u(x) >> 28) & 0x8u;
  float a = __builtin_fabsf(x);
  if (!(a < 8.0f)) return sign | 0x7u;
  if (a < 1.0f) return sign | (uint32_t)__builtin_rintf(a * 2.0f);  // 0, 0.5, 1
  int e = (int)((f2u(a) >> 23) & 0xFF) - 127;  // 0..2
  float m = __builtin_ldexpf(a, -e);
  uint32_t q = (uint32_t)__builtin_rintf((m - 1.0f) * 2.0f);
  if (q == 2u) { q = 0; e += 1; }
  if (e > 2) return sign | 0x7u;
  return sign | ((uint32_t)(e + 1) << 1) | q;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t E = (c >> 3) & 0xF, M = c & 7;
  float mag = E == 0 ? (float)M * 0.001953125f : __builtin_ldexpf(1.0f + (float)M * 0.125f, (int)E - 7);
  return (c & 0x80) ? -mag : mag;
}

// E4M3 byte -> float32: the exponent and mantissa fields moved into the
// float32 fields and rebiased by 2^120 (subnormal codes land on float32
// subnormals first, so every code is exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return u2f(((c & 0x80u) << 24) | ((c & 0x7Fu) << 20)) * 0x1p120f;
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Two E4M3 block scales (bytes 2 W and 2 W + 1 of c) as FP16 by the
// hardware convert: every E4M3 value, subnormals included (down to 2^-9),
// is an FP16 normal number, so this is exact.
template <bool W>
__device__ __forceinline__ f16x2 nv_scales(uint32_t c) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, W);
}

// Eight packed E2M1 values (one dword, two per byte, element 2b in the low
// nibble of byte b) times an E4M3 block scale s (both halves of s hold it)
// -> eight FP16 values: the convert gives the E2M1 values, the packed FP16
// multiply the products.  E2M1 x E4M3 has at most 6 significant bits and
// magnitudes in [2^-10, 2688], so both steps are exact in FP16.  (The
// multiply takes s from one half of a pair of scales through its op_sel.)
// The vector is assembled by bit casts of whole dwords.
__device__ __forceinline__ f16x8 nvfp4_to_f16x8(int packed, f16x2 s) {
  const uint32_t v = (uint32_t)packed;
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3) * s;
  const i32x4 w = {__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1), __builtin_bit_cast(int, p2),
                   __builtin_bit_cast(int, p3)};
  return __builtin_bit_cast(f16x8, w);
}

// UE8M0 code of an MX block from its float32 amax (> 0): the smallest e with
// amax <= fmax * 2^e, code 127 + e clamped to [1, 254].  With amax = m * 2^p:
// E4M3 (fmax = 1.75 * 2^8): e = p - 8 + [m > 1.75];  E2M1 (1.5 * 2^2):
// e = p - 2 + [m > 1.5].  A subnormal amax always clamps to 1.
template <bool FP4>
__device__ __forceinline__ int mx_scale_code(float amax) {
  uint32_t u = f2u(amax);
  int E = (int)(u >> 23);
  uint32_t M = u & 0x7FFFFFu;
  if (E == 0) return 1;
  int c = FP4 ? E - 2 + (M > 0x400000u) : E - 8 + (M > 0x600000u);
  return c < 1 ? 1 : (c > 254 ? 254 : c);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Scalar (SMEM) loads of wave-uniform addresses, waited for on lgkmcnt.  A
// kernel that keeps LDS-DMA copies in flight reads its metadata this way: the
// use of a vector load makes the compiler wait for vmcnt(0), which would also
// wait for every copy in flight.  (Loads only; nothing is written through the
// scalar cache.)
// The address is made scalar explicitly (it is wave-uniform; the compiler
// may otherwise keep it in VGPRs, which an SMEM load cannot take).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int sload(const void* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}
__device__ __forceinline__ i32x4 sload4(const void* p) {
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}
__device__ __forceinline__ i32x8 sload8(const void* p) {
  i32x8 v;
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}
__device__ __forceinline__ i32x16 sload16(const void* p) {
  i32x16 v;
  asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

// max over the 2^LOG lanes of a lane group (group = lanes with equal l >> LOG)
template <int LOG>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < (1 << LOG); m <<= 1) v = __builtin_fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-offs whose copies the caller has already
// waited for with wait_vmcnt: this wave's LDS reads complete, then s_barrier.
// (__syncthreads' release fence would also wait for every LDS-DMA copy still
// in flight, including those of later stages.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte global -> LDS copy without a register round trip: lane l's 16
// bytes land at `lds_base + 16 * l` (lds_base is uniform over the wave).
__device__ __forceinline__ void g2lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 16, 0, 0);
}

// The same copy with the non-temporal cache policy (the `nt` bit): for data
// that one workgroup reads once and no other is about to read.
__device__ __forceinline__ void g2lds16_nt(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 16, 0, 2);
}

// A raw buffer resource over the bytes from `base` on (no range limit, no
// stride: the gfx9 dword-3 word), for copies addressed by 32-bit offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// 16-byte buffer -> LDS copy: lane l's 16 bytes at byte voff (per lane) +
// soff (uniform) of the buffer land at `lds_base + 16 * l`, the same as
// g2lds16, with the offset sum done by the load itself rather than by 64-bit
// address arithmetic per copy.  NT: the non-temporal cache policy.
template <bool NT = false>
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, NT ? 2 : 0);
}

}  // namespace moe
