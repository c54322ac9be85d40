// C ABI of the fused MoE layer (declared in include/moe.h).
//
// Argument rules follow the DeepGEMM MegaMoE experts page:
// check_deep_gemm_mega_moe_supported (hidden and intermediate multiples of
// 128, else ValueError; unsupported device, NotImplementedError),
// MegaMoEActivation (finite alpha/beta, clamp >= 0; unsupported activation,
// NotImplementedError), DeepGemmMegaMoEExperts.forward (more tokens than the
// buffer was sized for, ValueError).  Every check runs before anything is
// enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include <cmath>

#include "common.h"
#include "launch.h"

// The intermediate buffers of moe_forward_noalloc: one fixed array per GPU
// (the device code object's own storage, held until the process ends).  In
// host code its name is a host-side stand-in: only the address
// hipGetSymbolAddress returns for a device is ever used.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

struct DeviceInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
  bool gemm_ready = false;
  void* scratch = nullptr;   // this device's address of `scratch`
};
constexpr int MAX_DEVICES = 64;
DeviceInfo g_dev[MAX_DEVICES];
std::mutex g_mu;
thread_local hipError_t g_last_hip = hipSuccess;

// Returns MOE_OK and fills *info for the current device, or an error.
int device_info(DeviceInfo** info) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { g_last_hip = e; return MOE_E_UNSUPPORTED; }
  if (dev < 0 || dev >= MAX_DEVICES) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) { g_last_hip = e; return MOE_E_UNSUPPORTED; }
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950) return MOE_E_UNSUPPORTED;
  if (!d.gemm_ready) {
    e = gemm_init(dev);
    if (e != hipSuccess) { g_last_hip = e; return MOE_E_HIP; }
    d.gemm_ready = true;
  }
  *info = &d;
  return MOE_OK;
}

// This device's address of the no-allocation scratch, looked up on first use
// (with the device current).
int scratch_of(DeviceInfo* d, void** ptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!d->scratch) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip = e == hipSuccess ? hipErrorInvalidSymbol : e;
      return MOE_E_HIP;
    }
    d->scratch = p;
  }
  *ptr = d->scratch;
  return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace carve-up of moe_forward.
struct Workspace {
  int32_t* counts;
  int32_t* offsets;
  int32_t* meta;
  int32_t* sorted_slot;
  int32_t* slot_row;
  int32_t* tile_expert;
  int32_t* tile_info;      // GemmArgs::tile_info
  int32_t* block_counts;   // the many-workgroup dispatch's per-chunk counts
  uint8_t* xq;        // dispatch-quantised x codes
  uint8_t* xq_sf;     // its block scales, [T, H / block]
  uint8_t* a1_sf;     // the same in sorted-row planes (one per K block)
  int64_t sf_plane;   // bytes per scale plane (a1_sf, a2_sf)
  float* x_tok;
  float* row_tok;     // NVFP4: token scale of each sorted row       // NVFP4 per-token scale
  uint8_t* a2;        // L2 input codes
  uint8_t* a2_sf;     // L2 input block scales, planes of sorted rows
  float* p1;          // K parts of a split L1 GEMM, float32 [ksplit1, S, 2I]
  float* o;           // L2 output rows per slot
  float* o_tail;      // split-tail L2: the tail tiles' K parts (TAIL_UNITS units)
  uint16_t* xw;       // BF16 input rows scaled by their routing weight
  uint16_t* xs;       // BF16: sorted x rows, stage-blocked (the L1 A operand)
  size_t bytes;
};

// Work units a split-tail L2's parts buffer holds (one round of the 256-CU
// grid); the GEMM splits no more of its tail than fit.
constexpr int TAIL_UNITS = 256;

Workspace plan(int fmt, int64_t T, int64_t H, int64_t I, int64_t n_loc, int64_t n_sh, int64_t k, int64_t bm,
               int64_t ksplit, int64_t ksplit1, int64_t tail_kmax, uint8_t* base) {
  const int64_t E = n_loc + n_sh, S = T * (k + n_sh), M = S + E * (bm - 1);
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t n) { uint8_t* p = base ? base + off : nullptr; off += align_up(n); return p; };
  w.counts = (int32_t*)take(E * 4);
  w.offsets = (int32_t*)take((E + 1) * 4);
  w.meta = (int32_t*)take(16);
  w.sorted_slot = (int32_t*)take(M * 4);
  w.slot_row = (int32_t*)take(S * 4);
  w.tile_expert = (int32_t*)take(M / bm * 4 + 4);
  w.tile_info = (int32_t*)take(M / bm * 16 + 16);
  w.block_counts = (int32_t*)take(dispatch_scratch_ints(S, (int)E) * 4);
  w.xq = w.xq_sf = w.a1_sf = w.a2 = w.a2_sf = nullptr;
  w.xs = nullptr;
  w.x_tok = w.row_tok = nullptr;
  // a scale plane holds every sorted row plus 256 bytes, so a tile's
  // 256-byte plane copy from its first row stays inside
  w.sf_plane = (M + 256 + 255) / 256 * 256;
  if (fmt == F_MXFP8 || fmt == F_MXFP4) {
    w.xq = take(T * H);
    w.xq_sf = take(T * H / 32);
    w.a1_sf = take(H / 32 * w.sf_plane);
    w.a2 = take(M * I);
    w.a2_sf = take(I / 32 * w.sf_plane);
  } else if (fmt == F_NVFP4) {
    w.xq = take(T * H / 2);
    w.xq_sf = take(T * H / 16);
    w.a1_sf = take(H / 16 * w.sf_plane);
    w.x_tok = (float*)take(T * 4);
    w.row_tok = (float*)take(M * 4);
    w.a2 = take(M * I / 2);
    w.a2_sf = take(I / 16 * w.sf_plane);
  } else {
    // stage-blocked [M / bm][K / 32][bm][32]: whole blocks of bm rows
    const int64_t Mb = (M + bm - 1) / bm * bm;
    w.a2 = take(Mb * I * 2);
    w.xs = (uint16_t*)take(Mb * H * 2);
  }
  w.o = (float*)take(S * H * 4 * ksplit);
  w.o_tail = tail_kmax > 1 ? (float*)take((int64_t)TAIL_UNITS * bm * GEMM_BN * 4) : nullptr;
  w.p1 = ksplit1 > 1 ? (float*)take(S * 2 * I * 4 * ksplit1) : nullptr;
  w.xw = (uint16_t*)take(T * H * 2);
  w.bytes = off;
  return w;
}

bool valid_fmt(int f) { return f == MOE_FMT_BF16 || f == MOE_FMT_MXFP8 || f == MOE_FMT_MXFP4 || f == MOE_FMT_NVFP4; }

// Formats whose grouped GEMMs this build implements.
bool gemm_fmt(int f) { return valid_fmt(f); }

// Expected padded rows of one group whose row count c is near-Poisson with
// mean m: E[ceil(c / bm)] * bm = bm * sum_j P(c > j bm).  The Poisson tail is
// summed directly below a mean of 64 (decode batches, where most experts get
// no row and the normal approximation miscounts the experts that get one),
// and approximated by the normal distribution above.
double expected_padded(double m, int bm) {
  if (m <= 0.0) return 0.0;
  if (m < 64.0) {
    double tiles = 0.0, pmf = std::exp(-m), cdf = 0.0;   // pmf: P(c = n)
    int n = 0;
    for (int j = 0;; ++j) {
      for (; n <= j * bm; ++n) {
        cdf += pmf;
        pmf *= m / (n + 1);
      }
      const double tail = 1.0 - cdf;
      if (tail < 1e-12 || n > 4096) break;   // (the tail is negligible long before n = 4096 for m < 64)
      tiles += tail;
    }
    return tiles * bm;
  }
  const double sd = std::sqrt(m);
  double tiles = 0.0;
  for (int j = 0;; ++j) {
    const double x = (double)j * bm + 0.5;
    if (x > m + 8.0 * sd + 1.0) break;
    tiles += 0.5 * std::erfc((x - m) / (sd * 1.4142135623730951));
  }
  return tiles * bm;
}

// BLOCK_M from the expected group sizes (routed experts T*k/n_loc rows,
// shared experts T): each candidate's expected padded row count is weighed by
// the tile's relative efficiency (smaller tiles re-read more operand bytes
// per FLOP); the cheapest wins.  The block-scaled formats stop at 128 (their
// 256-row tiles run out of registers).  NVFP4 is measured apart: its GEMMs
// convert every E2M1 fragment to FP16 in registers, and 64-row tiles, which
// run two workgroups per CU, overlap one workgroup's conversions with the
// other's MFMAs (64 rows: 1.13 ms for both GEMMs of the 16384-token layer,
// 128 rows: 1.24 ms, 32 rows: 1.53 ms).
int block_m_rule(int T, int n_loc, int n_sh, int k, int fmt) {
  const double routed = (double)T * k / n_loc;
  const int cand[4] = {32, 64, 128, 256};
  const double eff_mfma[4] = {0.35, 0.55, 0.85, 1.0};
  const double eff_nv[4] = {0.70, 1.0, 0.90, 0.0};
  const double* eff = fmt == MOE_FMT_NVFP4 ? eff_nv : eff_mfma;
  const int nc = fmt == MOE_FMT_BF16 ? 4 : 3;
  int best = 32;
  double best_cost = -1.0;
  for (int i = 0; i < nc; ++i) {
    const double padded = n_loc * expected_padded(routed, cand[i]) + n_sh * (double)((T + cand[i] - 1) / cand[i]) * cand[i];
    const double cost = padded / eff[i];
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = cand[i];
    }
  }
  return best;
}

// The split rule counts rounds on a 256-CU part (MI355X); a host-only
// constant, so workspace sizing and launches agree without a device query.
constexpr int SPLIT_RULE_CUS = 256;

// K splits of the L2 GEMM.  Its tiles (expected count at the rule's BLOCK_M)
// run in rounds of one per CU; when the last round is partly empty, splitting
// K into ks parts (each part's float32 result in its own buffer, added by the
// combine) fills it at the price of (ks - 1) extra O writes and reads.  The
// estimate takes the tile time from a nominal per-format MFMA rate; ks must
// divide the stage count.  The choice does not depend on the BLOCK_M a caller
// passes, so every BLOCK_M sums in the same order.
int l2_ksplit(int fmt, int64_t T, int64_t H, int64_t I, int n_loc, int n_sh, int k, int cus) {
  if (T <= 0 || cus <= 0) return 1;
  const int bm = block_m_rule((int)T, n_loc, n_sh, k, fmt);
  const double mtiles = n_loc * expected_padded((double)T * k / n_loc, bm) / bm +
                        n_sh * (double)((T + bm - 1) / bm);
  const double tiles = mtiles * (double)(H / GEMM_BN);
  const int kst = fmt == MOE_FMT_BF16 ? 32 : 128;
  const int64_t nst = I / kst;
  const double rate = (fmt == MOE_FMT_BF16 ? 1.0e15 : (fmt == MOE_FMT_NVFP4 ? 0.6e15 : 1.6e15)) / cus;
  const double t_tile = 2.0 * bm * GEMM_BN * (double)I / rate;
  const double S = (double)T * (k + n_sh);
  int best = 1;
  double best_t = 0.0;
  for (int ks = 1; ks <= 4; ++ks) {
    if (nst % ks) continue;
    const double t = std::ceil(tiles * ks / cus) * t_tile / ks + (ks - 1) * S * (double)H * 8.0 / 5.0e12;
    if (ks == 1 || t < 0.97 * best_t) {   // a split must win by 3 %
      best = ks;
      best_t = t;
    }
  }
  return best;
}

// BF16 L2s (float32 rows) with at least as many tiles as the rule's CUs
// split only the persistent grid's partial last round (TailSplit; the
// largest kmax of 4, 2 that divides the stage count) instead of every tile:
// whole tiles keep one part and one epilogue.  0: no split tail.
int l2_tail_kmax(int fmt, int64_t T, int64_t H, int64_t I, int n_loc, int n_sh, int k, int cus) {
  if (fmt != MOE_FMT_BF16 || T <= 0 || cus <= 0) return 0;
  const int bm = block_m_rule((int)T, n_loc, n_sh, k, fmt);
  const double mtiles = n_loc * expected_padded((double)T * k / n_loc, bm) / bm +
                        n_sh * (double)((T + bm - 1) / bm);
  if (mtiles * (double)(H / GEMM_BN) < cus) return 0;
  for (int km = 4; km >= 2; km >>= 1)
    if ((I / 32) % km == 0) return km;
  return 0;
}

// K splits of the L1 GEMM, for launches with few tiles (decode batches):
// when the tiles leave work slots idle (two per CU for the small tiles such
// launches use), each tile's K is cut into ks parts that run as separate work
// units; the float32 parts (per slot) are summed by the finish kernel before
// the activation.  A tile's time is its MFMA work at a nominal per-format
// rate or the streaming of its weight block at the slot's share of 6 TB/s,
// whichever is longer; a split pays the parts' write and read at 5 TB/s and
// the finish launch, and must win by 3 %.  ks divides the stage count;
// BLOCK_M-independent like the L2 rule.
int l1_ksplit(int fmt, int64_t T, int64_t H, int64_t I, int n_loc, int n_sh, int k, int cus) {
  if (T <= 0 || cus <= 0) return 1;
  const int bm = block_m_rule((int)T, n_loc, n_sh, k, fmt);
  const double mtiles = n_loc * expected_padded((double)T * k / n_loc, bm) / bm +
                        n_sh * (double)((T + bm - 1) / bm);
  const double tiles = std::max(1.0, mtiles * (double)(2 * I / GEMM_BN));
  const double slots = (bm <= 64 ? 2.0 : 1.0) * cus;
  const double rate = (fmt == MOE_FMT_BF16 ? 1.0e15 : (fmt == MOE_FMT_NVFP4 ? 0.6e15 : 1.6e15)) / slots;
  const double elem = fmt == MOE_FMT_BF16 ? 2.0 : (fmt == MOE_FMT_MXFP8 ? 1.0 : 0.5);
  const double t_tile = std::max(2.0 * bm * GEMM_BN * (double)H / rate, GEMM_BN * (double)H * elem / (6.0e12 / slots));
  const double S = (double)T * (k + n_sh);
  const int kst = fmt == MOE_FMT_BF16 ? 32 : 128;
  const int64_t nst = H / kst;
  int best = 1;
  double best_t = 0.0;
  for (int ks = 1; ks <= 4; ++ks) {
    if (nst % ks) continue;
    double t = std::ceil(tiles * ks / slots) * t_tile / ks;
    if (ks > 1) t += ks * S * 2.0 * (double)I * 8.0 / 5.0e12 + 3.0e-6;
    if (ks == 1 || t < 0.97 * best_t) {
      best = ks;
      best_t = t;
    }
  }
  return best;
}

// The checks of moe_forward on the layer's shape (no pointers): MOE_OK or
// MOE_E_INVALID.
int check_shape(int fmt, int num_tokens, int hidden, int inter, int top_k, int num_local_experts, int num_shared,
                int block_m) {
  if (!valid_fmt(fmt)) return MOE_E_INVALID;
  if (num_tokens < 0 || hidden <= 0 || inter <= 0 || hidden % 128 || inter % 128) return MOE_E_INVALID;
  if (top_k < 1 || num_local_experts < 1 || num_shared < 0 || num_local_experts + num_shared > MAX_LOCAL_EXPERTS)
    return MOE_E_INVALID;
  if ((int64_t)num_tokens * (top_k + num_shared) > (int64_t)1 << 30) return MOE_E_INVALID;
  if (block_m != 0 && block_m != 32 && block_m != 64 && block_m != 128 && block_m != 256) return MOE_E_INVALID;
  // the GEMMs copy each expert's weights and the quantised x through buffer
  // resources with 32-bit offsets: both stay below 4 GiB (a 1 MiB margin for
  // the offsets within a row).  w13 holds 2 I H elements per expert, of 2
  // (BF16), 1 (MXFP8) or 1/2 bytes; x's codes are 1 byte (MX) or 1/2 (NVFP4).
  const int64_t lim = ((int64_t)1 << 32) - ((int64_t)1 << 20);
  const int64_t w13_bytes = (int64_t)inter * hidden * (fmt == MOE_FMT_BF16 ? 4 : fmt == MOE_FMT_MXFP8 ? 2 : 1);
  const int64_t x_bytes = (int64_t)num_tokens * hidden / (fmt == MOE_FMT_NVFP4 ? 2 : 1);
  if (w13_bytes >= lim || (fmt != MOE_FMT_BF16 && x_bytes >= lim)) return MOE_E_INVALID;
  return MOE_OK;
}

// BLOCK_M, K splits and workspace carve-up of one forward call (host only):
// the rule's BLOCK_M when block_m is 0; the K splits the rules pick, each
// dropped (L1 first) while the workspace cannot hold its float32 parts.
struct Resolved {
  int bm, ks, ks1, tail;   // tail: the L2's split-tail kmax (0: none)
  Workspace w;
};
int resolve(int fmt, int num_tokens, int hidden, int inter, int top_k, int num_local_experts, int num_shared,
            int block_m, size_t workspace_bytes, uint8_t* base, Resolved* r) {
  const int bm = block_m ? block_m : block_m_rule(num_tokens, num_local_experts, num_shared, top_k, fmt);
  const int64_t T = num_tokens, H = hidden, I = inter;
  int tail = l2_tail_kmax(fmt, T, H, I, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  int ks = tail ? 1 : l2_ksplit(fmt, T, H, I, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  int ks1 = l1_ksplit(fmt, T, H, I, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  auto need = [&]() {
    return plan(fmt, T, H, I, num_local_experts, num_shared, top_k, bm, ks, ks1, tail, nullptr).bytes;
  };
  if (need() > workspace_bytes) ks1 = 1;
  if (need() > workspace_bytes) ks = 1;
  if (need() > workspace_bytes) tail = 0;
  if (need() > workspace_bytes) return MOE_E_WORKSPACE;
  r->bm = bm;
  r->ks = ks;
  r->ks1 = ks1;
  r->tail = tail;
  r->w = plan(fmt, T, H, I, num_local_experts, num_shared, top_k, bm, ks, ks1, tail, base);
  return MOE_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_E_HIP;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_E_INVALID: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported device, format or activation";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_HIP: return g_last_hip == hipSuccess ? "HIP error" : hipGetErrorString(g_last_hip);
    case MOE_E_TOO_LARGE: return "the layer needs more intermediate memory than the fixed no-allocation scratch holds";
    default: return "unknown status";
  }
}

int moe_get_block_m(int num_tokens, int num_local_experts, int num_shared, int top_k, moe_format_t fmt) {
  if (num_tokens < 0 || num_local_experts < 1 || num_shared < 0 || top_k < 1 || !valid_fmt(fmt)) return MOE_E_INVALID;
  return block_m_rule(num_tokens, num_local_experts, num_shared, top_k, fmt);
}

size_t moe_workspace_bytes(moe_format_t fmt, int max_tokens, int hidden, int inter, int num_local_experts,
                           int num_shared, int top_k, int block_m) {
  if (!valid_fmt(fmt) || max_tokens < 0 || hidden <= 0 || inter <= 0 || hidden % 128 || inter % 128 ||
      num_local_experts < 1 || num_shared < 0 || top_k < 1)
    return 0;
  if (block_m == 0) block_m = 256;
  if (block_m != 32 && block_m != 64 && block_m != 128 && block_m != 256) return 0;
  const int tail = l2_tail_kmax(fmt, max_tokens, hidden, inter, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  const int ks =
      tail ? 1 : l2_ksplit(fmt, max_tokens, hidden, inter, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  const int ks1 = l1_ksplit(fmt, max_tokens, hidden, inter, num_local_experts, num_shared, top_k, SPLIT_RULE_CUS);
  return plan(fmt, max_tokens, hidden, inter, num_local_experts, num_shared, top_k, block_m, ks, ks1, tail, nullptr)
      .bytes;
}

int moe_transform_weights(moe_format_t fmt, int num_experts, int hidden, int inter, const void* w13,
                          const void* w13_sf, const void* w2, const void* w2_sf, void* w13_k, void* w13_sf_k,
                          void* w2_k, void* w2_sf_k, void* stream) {
  if (!valid_fmt(fmt) || num_experts < 1 || hidden <= 0 || inter <= 0 || hidden % 128 || inter % 128)
    return MOE_E_INVALID;
  if (!w13 || !w2 || !w13_k || !w2_k || !aligned16(w13) || !aligned16(w2) || !aligned16(w13_k) || !aligned16(w2_k))
    return MOE_E_INVALID;
  const bool scaled = fmt != MOE_FMT_BF16;
  if (scaled && (!w13_sf || !w2_sf || !w13_sf_k || !w2_sf_k)) return MOE_E_INVALID;
  if (!gemm_fmt(fmt)) return MOE_E_UNSUPPORTED;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  launch_transform(fmt, num_experts, hidden, inter, (const uint8_t*)w13, (const uint8_t*)w13_sf, (const uint8_t*)w2,
                   (const uint8_t*)w2_sf, (uint8_t*)w13_k, (uint8_t*)w13_sf_k, (uint8_t*)w2_k, (uint8_t*)w2_sf_k,
                   (hipStream_t)stream);
  return hip_status(hipGetLastError());
}

int moe_quantize_weights(moe_format_t fmt, int num_experts, int rows, int cols, const float* src, void* codes,
                         void* scales, float* gscale, void* stream) {
  if (!(fmt == MOE_FMT_MXFP8 || fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_NVFP4)) return MOE_E_INVALID;
  if (num_experts < 1 || rows < 1 || cols < 32 || cols % 32) return MOE_E_INVALID;
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes)) return MOE_E_INVALID;
  if (fmt == MOE_FMT_NVFP4 && !gscale) return MOE_E_INVALID;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = (int64_t)num_experts * rows;
  if (fmt == MOE_FMT_NVFP4) {
    launch_weight_gscale(num_experts, (int64_t)rows * cols, src, gscale, s);
    launch_quant_nv(true, R, cols, src, (uint8_t*)codes, (uint8_t*)scales, nullptr, gscale, rows, s);
  } else {
    launch_quant_mx(fmt == MOE_FMT_MXFP4, true, R, cols, src, (uint8_t*)codes, (uint8_t*)scales, s);
  }
  return hip_status(hipGetLastError());
}

int moe_quantize_x(moe_format_t fmt, int num_tokens, int hidden, const void* x, void* codes, void* scales,
                   float* token_scale, void* stream) {
  if (!(fmt == MOE_FMT_MXFP8 || fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_NVFP4)) return MOE_E_INVALID;
  if (num_tokens < 0 || hidden < 32 || hidden % 32) return MOE_E_INVALID;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_E_INVALID;
  if (fmt == MOE_FMT_NVFP4 && !token_scale) return MOE_E_INVALID;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (fmt == MOE_FMT_NVFP4)
    launch_quant_nv(false, num_tokens, hidden, x, (uint8_t*)codes, (uint8_t*)scales, token_scale, nullptr, 1, s);
  else
    launch_quant_mx(false, false, num_tokens, hidden, x, (uint8_t*)codes, (uint8_t*)scales, s);
  return hip_status(hipGetLastError());
}

int moe_dispatch(int num_tokens, int top_k, int num_shared, int expert_start, int num_local_experts, int block_m,
                 const int32_t* topk_ids, int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                 int32_t* tile_expert, int32_t* block_counts, void* stream) {
  if (num_tokens < 0 || top_k < 1 || num_shared < 0 || num_local_experts < 1 ||
      num_local_experts + num_shared > MAX_LOCAL_EXPERTS)
    return MOE_E_INVALID;
  if (block_m != 32 && block_m != 64 && block_m != 128 && block_m != 256) return MOE_E_INVALID;
  if ((num_tokens > 0 && top_k > 0 && !topk_ids) || !counts || !offsets || !sorted_slot || !slot_row || !tile_expert)
    return MOE_E_INVALID;
  if ((int64_t)num_tokens * (top_k + num_shared) > (int64_t)1 << 30) return MOE_E_INVALID;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  launch_dispatch(topk_ids, num_tokens, top_k, num_shared, expert_start, num_local_experts, block_m, counts, offsets,
                  sorted_slot, slot_row, tile_expert, nullptr, nullptr, block_counts, (hipStream_t)stream);
  return hip_status(hipGetLastError());
}

int moe_route(int num_tokens, int num_experts, int top_k, const float* logits, const float* bias, int scoring,
              int num_groups, int topk_groups, int renormalize, float routed_scaling_factor,
              const uint8_t* is_padding, int32_t* topk_ids, float* topk_weights, void* stream) {
  if (num_tokens < 0 || num_experts < 1 || num_experts > 1024 || top_k < 1 || top_k > 64 || top_k > num_experts)
    return MOE_E_INVALID;
  if (scoring != MOE_SCORE_SOFTMAX && scoring != MOE_SCORE_SIGMOID) return MOE_E_INVALID;
  if (num_groups < 1 || num_groups > 64 || num_experts % num_groups || topk_groups < 1 || topk_groups > num_groups)
    return MOE_E_INVALID;
  if (num_groups > 1 && (int64_t)topk_groups * (num_experts / num_groups) < top_k) return MOE_E_INVALID;
  if (!isfinite(routed_scaling_factor)) return MOE_E_INVALID;
  if (num_tokens == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_E_INVALID;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  launch_route(logits, bias, num_tokens, num_experts, top_k, scoring == MOE_SCORE_SIGMOID, num_groups, topk_groups,
               renormalize != 0, routed_scaling_factor, is_padding, topk_ids, topk_weights, (hipStream_t)stream);
  return hip_status(hipGetLastError());
}

int64_t moe_dispatch_scratch_ints(int num_tokens, int top_k, int num_shared, int num_local_experts) {
  if (num_tokens < 0 || top_k < 1 || num_shared < 0 || num_local_experts < 1) return -1;
  return dispatch_scratch_ints((int64_t)num_tokens * (top_k + num_shared), num_local_experts + num_shared);
}

int moe_workspace_layout(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k, int num_local_experts,
                         int num_shared, int block_m, size_t workspace_bytes, moe_workspace_layout_t* layout) {
  if (!layout) return MOE_E_INVALID;
  const int sst = check_shape(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, block_m);
  if (sst != MOE_OK) return sst;
  Resolved rs;
  // carve from a non-null base so that absent buffers stay distinguishable
  uint8_t* const base = (uint8_t*)(uintptr_t)4096;
  const int rst = resolve(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, block_m,
                          workspace_bytes, base, &rs);
  if (rst != MOE_OK) return rst;
  auto off = [&](const void* p) -> int64_t { return p ? (int64_t)((const uint8_t*)p - base) : -1; };
  const Workspace& w = rs.w;
  moe_workspace_layout_t& L = *layout;
  L.block_m = rs.bm;
  L.l1_ksplit = rs.ks1;
  L.l2_ksplit = rs.ks;
  L.l2_rows_bf16 = fmt != MOE_FMT_BF16 && rs.ks == 1;
  L.sf_plane = fmt == MOE_FMT_BF16 ? 0 : w.sf_plane;
  L.a2_ld = fmt == MOE_FMT_BF16 ? (int64_t)inter * 2 : (fmt == MOE_FMT_NVFP4 ? inter / 2 : inter);
  L.counts = off(w.counts);
  L.offsets = off(w.offsets);
  L.sorted_slot = off(w.sorted_slot);
  L.slot_row = off(w.slot_row);
  L.tile_expert = off(w.tile_expert);
  L.xq = off(w.xq);
  L.xq_sf = off(w.xq_sf);
  L.x_tok = off(w.x_tok);
  L.a1_sf = off(w.a1_sf);
  L.a2 = off(w.a2);
  L.a2_sf = off(w.a2_sf);
  L.o = off(w.o);
  L.bytes = (int64_t)w.bytes;
  return MOE_OK;
}

}  // extern "C"

namespace {

// moe_forward_profiled, and with noalloc the no-allocation variant (the
// workspace arguments are ignored; the device's scratch array is used).
int forward_impl(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k, int expert_start,
                 int num_local_experts, int num_shared, int block_m, const moe_activation_t* act,
                 const moe_options_t* opts, const void* x, const int32_t* topk_ids, const float* topk_weights,
                 const void* w13_k, const void* w13_sf_k, const void* w2_k, const void* w2_sf_k,
                 const float* w13_gscale, const float* w2_gscale, float l2_activation_scale, void* out,
                 void* workspace, size_t workspace_bytes, void* stream, void* const* ev, bool noalloc) {
  // ---- shapes and parameters
  const int shape_status = check_shape(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, block_m);
  if (shape_status != MOE_OK) return shape_status;
  moe_activation_t a = {MOE_ACT_SWIGLU, 0, 0.0f, 1.0f, 0.0f};
  if (act) a = *act;
  if (a.kind != MOE_ACT_SWIGLU) return MOE_E_UNSUPPORTED;
  moe_options_t o = {nullptr, 0.0f, 0};
  if (opts) o = *opts;
  if (o.post_expert_norm_gamma &&
      (!aligned16(o.post_expert_norm_gamma) || hidden > 16384 || !(o.post_expert_norm_eps >= 0.0f) ||
       !isfinite(o.post_expert_norm_eps)))
    return MOE_E_INVALID;
  if (o.apply_router_weight_on_input && (top_k != 1 || num_shared != 0)) return MOE_E_INVALID;
  if (!isfinite(a.alpha) || !isfinite(a.beta) || (a.has_clamp && !(a.clamp >= 0.0f))) return MOE_E_INVALID;
  if (fmt == MOE_FMT_NVFP4 && (!(l2_activation_scale > 0.0f) || !isfinite(l2_activation_scale)))
    return MOE_E_INVALID;
  if (num_tokens == 0) return MOE_OK;
  // ---- pointers
  const bool scaled = fmt != MOE_FMT_BF16;
  if (noalloc) {
    workspace = nullptr;
    workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  }
  if (!x || !topk_ids || !topk_weights || !w13_k || !w2_k || !out || (!noalloc && !workspace)) return MOE_E_INVALID;
  if (!aligned16(x) || !aligned16(w13_k) || !aligned16(w2_k) || !aligned16(out) || !aligned16(workspace))
    return MOE_E_INVALID;
  if (scaled && (!w13_sf_k || !w2_sf_k || !aligned16(w13_sf_k) || !aligned16(w2_sf_k))) return MOE_E_INVALID;
  if (fmt == MOE_FMT_NVFP4 && (!w13_gscale || !w2_gscale)) return MOE_E_INVALID;
  if (!gemm_fmt(fmt) || hidden % 256) return MOE_E_UNSUPPORTED;
  Resolved rs;
  const int rst = resolve(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, block_m,
                          workspace_bytes, nullptr, &rs);
  if (rst != MOE_OK) return noalloc && rst == MOE_E_WORKSPACE ? MOE_E_TOO_LARGE : rst;
  DeviceInfo* d;
  int st = device_info(&d);
  if (st != MOE_OK) return st;
  if (noalloc && (st = scratch_of(d, &workspace)) != MOE_OK) return st;
  rs.w = plan(fmt, num_tokens, hidden, inter, num_local_experts, num_shared, top_k, rs.bm, rs.ks, rs.ks1, rs.tail,
              (uint8_t*)workspace);
  const int bm = rs.bm, ks = rs.ks, ks1 = rs.ks1;
  const Workspace& w = rs.w;
  const int64_t T = num_tokens, H = hidden, I = inter, kk = top_k + num_shared;
  const int E = num_local_experts + num_shared;
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], s);
  };

  // a1: dispatch quantisation (with the routing weight on the input, of the
  // scaled rows)
  mark(2 * MOE_STEP_QUANT_X);
  const void* xin = x;
  if (o.apply_router_weight_on_input) {
    launch_scale_rows((const uint16_t*)x, topk_weights, num_tokens, (int)H, w.xw, s);
    xin = w.xw;
  }
  // MX formats with the single-workgroup dispatch: quantisation and routing
  // metadata (a2) in one launch, timed as the quantisation step
  const bool mx = fmt == MOE_FMT_MXFP8 || fmt == MOE_FMT_MXFP4;
  const bool fused = mx && (!w.block_counts || dispatch_single_wg(num_tokens, top_k, num_shared));
  bool planes = false;   // the fused launch also wrote the L1 scale planes
  if (fused)
    planes = launch_dispatch_quant_mx(topk_ids, num_tokens, top_k, num_shared, expert_start, num_local_experts, bm,
                                      w.counts, w.offsets, w.sorted_slot, w.slot_row, w.tile_expert, w.tile_info,
                                      w.meta, xin,
                                      (int)H, w.xq, w.xq_sf, w.a1_sf, w.sf_plane, s);
  else if (mx)
    launch_quant_mx(false, false, T, (int)H, xin, w.xq, w.xq_sf, s);
  else if (fmt == MOE_FMT_NVFP4)
    launch_quant_nv(false, T, (int)H, xin, w.xq, w.xq_sf, w.x_tok, nullptr, 1, s);
  mark(2 * MOE_STEP_QUANT_X + 1);
  // a2: routing metadata
  mark(2 * MOE_STEP_DISPATCH);
  if (!fused)
    launch_dispatch(topk_ids, num_tokens, top_k, num_shared, expert_start, num_local_experts, bm, w.counts,
                    w.offsets, w.sorted_slot, w.slot_row, w.tile_expert, w.tile_info, w.meta, w.block_counts, s);
  const bool nv = fmt == MOE_FMT_NVFP4, fp4 = fmt == MOE_FMT_MXFP4 || nv;
  const int64_t grp = nv ? 16 : 32;          // elements per block scale
  if (scaled && !planes) {
    // the dispatch-quantised x scales in the sorted rows' plane layout
    // (padding rows: scale 1)
    const int64_t M = T * kk + (int64_t)E * (bm - 1);
    launch_gather_sf(w.sorted_slot, w.offsets, E, (int)kk, w.xq_sf, (int)(H / grp), w.sf_plane, M,
                     nv ? 0x38 : 127, w.a1_sf, nv ? w.x_tok : nullptr, w.row_tok, s);
  }
  if (fmt == MOE_FMT_BF16) {
    const int64_t M = T * kk + (int64_t)E * (bm - 1);
    launch_block_rows_bf16((const uint16_t*)xin, w.sorted_slot, w.offsets, E, (int)kk, (int)H, bm, M, w.xs, s);
  }
  mark(2 * MOE_STEP_DISPATCH + 1);
  const int grid = (d->cus >= 8 ? d->cus : 8) / 8 * 8;

  // a3-a5: L1 GEMM + activation + L2-input quantisation
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  const int64_t ebytes = fmt == MOE_FMT_BF16 ? 2 : 1;  // bytes per element (codes); FP4 below
  g.bm = bm;
  if (fmt == MOE_FMT_BF16) {
    g.a = (const uint8_t*)w.xs;   // stage-blocked sorted rows
    g.a_ld = H * 2;
  } else {
    g.a = w.xq;
    g.a_ld = nv ? H / 2 : H;
    g.a_sf = w.a1_sf;
    g.a_sf_ld = w.sf_plane;
    g.a_tok = w.x_tok;
  }
  g.w = (const uint8_t*)w13_k;
  g.w_sf = (const uint8_t*)w13_sf_k;
  g.w_gs = w13_gscale;
  const int64_t w13_elems = 2 * I * H, w2_elems = H * I;
  g.w_expert_bytes = fp4 ? w13_elems / 2 : w13_elems * ebytes;
  g.w_sf_expert_bytes = scaled ? w13_elems / grp : 0;
  g.N = (int)(2 * I);
  g.K = (int)H;
  g.sorted_slot = w.sorted_slot;
  g.offsets = w.offsets;
  g.tile_expert = w.tile_expert;
  g.tile_info = w.tile_info;
  g.row_scale = w.row_tok;
  g.meta = w.meta;
  g.kk = (int)kk;
  g.c = w.a2;
  g.c_sf = w.a2_sf;
  g.c_ld = fmt == MOE_FMT_BF16 ? I * 2 : (nv ? I / 2 : I);
  g.c_sf_ld = w.sf_plane;
  g.inter = (int)I;
  g.has_clamp = a.has_clamp;
  g.clamp = a.clamp;
  g.alpha = a.alpha;
  g.beta = a.beta;
  g.l2_scale = l2_activation_scale;
  g.ksplit = ks1;
  g.o = w.p1;
  g.o_split = T * kk * 2 * I;
  mark(2 * MOE_STEP_L1);
  hipError_t e = launch_gemm(fmt, 1, bm, g, grid, s);
  if (e != hipSuccess) return hip_status(e);
  if (ks1 > 1) launch_l1_finish(fmt, g, w.slot_row, w.tile_expert, bm, (int)(T * kk), s);
  mark(2 * MOE_STEP_L1 + 1);

  // a6: L2 GEMM
  GemmArgs g2 = g;
  g2.a = w.a2;
  g2.a_ld = g.c_ld;
  g2.a_sf = w.a2_sf;
  g2.a_sf_ld = w.sf_plane;
  g2.a_tok = nullptr;
  g2.w = (const uint8_t*)w2_k;
  g2.w_sf = (const uint8_t*)w2_sf_k;
  g2.w_gs = w2_gscale;
  g2.w_expert_bytes = fp4 ? w2_elems / 2 : w2_elems * ebytes;
  g2.w_sf_expert_bytes = scaled ? w2_elems / grp : 0;
  g2.N = (int)H;
  g2.K = (int)I;
  g2.o = w.o;
  g2.ksplit = ks;
  g2.o_bf16 = scaled && ks == 1;
  g2.o_split = (int64_t)T * kk * H;
  g2.o_tail = w.o_tail;
  g2.tail_kmax = rs.tail;
  g2.tail_units = TAIL_UNITS;
  mark(2 * MOE_STEP_L2);
  e = launch_gemm(fmt, 2, bm, g2, grid, s);
  if (e != hipSuccess) return hip_status(e);
  mark(2 * MOE_STEP_L2 + 1);

  // a7: weighted combine
  mark(2 * MOE_STEP_COMBINE);
  const CombineTail tl = {rs.tail > 1 ? w.o_tail : nullptr, w.tile_info, w.meta, bm,
                          gemm_workgroups(fmt, bm, grid), rs.tail, TAIL_UNITS, (int)(I / 32)};
  launch_combine(w.o, g2.o_bf16, ks, (int64_t)T * kk * H, w.slot_row,
                 o.apply_router_weight_on_input ? nullptr : topk_weights, num_tokens, top_k, (int)kk, (int)H,
                 o.post_expert_norm_gamma, o.post_expert_norm_eps, tl, (uint16_t*)out, s);
  mark(2 * MOE_STEP_COMBINE + 1);
  return hip_status(hipGetLastError());
}

}  // namespace

extern "C" {

int moe_forward_profiled(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k, int expert_start,
                         int num_local_experts, int num_shared, int block_m, const moe_activation_t* act,
                         const moe_options_t* opts, const void* x, const int32_t* topk_ids, const float* topk_weights, const void* w13_k,
                         const void* w13_sf_k, const void* w2_k, const void* w2_sf_k, const float* w13_gscale,
                         const float* w2_gscale, float l2_activation_scale, void* out, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* ev) {
  return forward_impl(fmt, num_tokens, hidden, inter, top_k, expert_start, num_local_experts, num_shared, block_m,
                      act, opts, x, topk_ids, topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale,
                      l2_activation_scale, out, workspace, workspace_bytes, stream, ev, false);
}

int moe_forward(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k, int expert_start,
                int num_local_experts, int num_shared, int block_m, const moe_activation_t* act,
                const moe_options_t* opts, const void* x, const int32_t* topk_ids, const float* topk_weights, const void* w13_k, const void* w13_sf_k,
                const void* w2_k, const void* w2_sf_k, const float* w13_gscale, const float* w2_gscale,
                float l2_activation_scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(fmt, num_tokens, hidden, inter, top_k, expert_start, num_local_experts, num_shared, block_m,
                      act, opts, x, topk_ids, topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale,
                      l2_activation_scale, out, workspace, workspace_bytes, stream, nullptr, false);
}

int moe_forward_noalloc(moe_format_t fmt, int num_tokens, int hidden, int inter, int top_k, int expert_start,
                        int num_local_experts, int num_shared, int block_m, const moe_activation_t* act,
                        const moe_options_t* opts, const void* x, const int32_t* topk_ids, const float* topk_weights,
                        const void* w13_k, const void* w13_sf_k, const void* w2_k, const void* w2_sf_k,
                        const float* w13_gscale, const float* w2_gscale, float l2_activation_scale, void* out,
                        void* stream) {
  return forward_impl(fmt, num_tokens, hidden, inter, top_k, expert_start, num_local_experts, num_shared, block_m,
                      act, opts, x, topk_ids, topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale,
                      l2_activation_scale, out, nullptr, 0, stream, nullptr, true);
}

}  // extern "C"
