// Host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int MAX_LOCAL_EXPERTS = 1000;  // E' = local + shared experts
constexpr int GEMM_THREADS = 256;        // 4 waves per workgroup
constexpr int GEMM_BN = 256;             // N columns per tile

// Arguments of one grouped GEMM launch (L1 or L2).
struct GemmArgs {
  // A operand: rows of x (L1, gathered through sorted_slot / k') or of the
  // L2 input (L2, already in sorted order).
  const uint8_t* a;        // element codes (BF16 / E4M3 / packed E2M1)
  const uint8_t* a_sf;     // block scales (UE8M0 or E4M3), NULL for BF16: one
                           // plane per K block, a byte per sorted row
  const float* a_tok;      // NVFP4 L1: per-token global scale
  int64_t a_ld;            // bytes per A row
  int64_t a_sf_ld;         // bytes per A-scale plane (a multiple of 256; rows
                           // up to the last tile's start + 255 are readable)
  // B operand: kernel-layout weights of all local experts.
  const uint8_t* w;
  const uint8_t* w_sf;
  const float* w_gs;       // NVFP4 per-expert global scale
  int64_t w_expert_bytes;
  int64_t w_sf_expert_bytes;
  int N, K;                // GEMM N (2I for L1, H for L2) and K (H or I)
  // routing
  const int32_t* sorted_slot;
  const int32_t* offsets;  // [E'+1], multiples of BLOCK_M
  const int32_t* tile_expert;   // [M / BLOCK_M] expert of each BLOCK_M block
  // [M / BLOCK_M] int4 per BLOCK_M block: its expert, the expert's first
  // block and its number of blocks (what tile_expert and offsets give, in
  // one 16-byte record, so a tile's set-up waits out one load, not three)
  const int32_t* tile_info;
  const float* row_scale;  // NVFP4 L1: token scale of each sorted row (1 if padding)
  const int32_t* meta;     // meta[0] = number of BLOCK_M tiles
  int kk;                  // slots per token (top_k + shared)
  // L1 epilogue: activation + L2-input quantisation into (c, c_sf)
  uint8_t* c;
  uint8_t* c_sf;
  int64_t c_ld, c_sf_ld;   // c_sf: planes of c_sf_ld bytes, as a_sf
  int inter;
  int has_clamp;
  float clamp, alpha, beta;
  float l2_scale;          // NVFP4 global scale of the L2 input
  // float32 rows per slot [S, N]: the L2 output, and the parts of an L1
  // whose K is split; with K split in ksplit parts, part ks goes to
  // o + ks * o_split
  float* o;
  int ksplit;
  int64_t o_split;
  // L2 of a block-scaled layer with K unsplit: the rows of o are BF16 (RNE of
  // the float32 accumulators), [S, N] uint16
  int o_bf16;
  // L2 with a split tail (tail_kmax > 1, float32 rows, ksplit 1): the tiles
  // of the persistent grid's partial last round run as K parts (tail_split);
  // their parts go to o_tail as [tail tile][part][bm rows][256 columns], the
  // other tiles' rows to o.  o_tail holds tail_units such units.
  float* o_tail;
  int tail_kmax;
  int tail_units;
  // BLOCK_M.  BF16 layers keep both GEMMs' A operand (the sorted x rows, the
  // L2 input) stage-blocked: [M / bm][K / 32][bm rows][32 values], so a
  // tile's 32-K stage of A is one contiguous run of bm * 64 bytes
  int bm;
};

enum Fmt { F_BF16 = 0, F_MXFP8 = 1, F_MXFP4 = 2, F_NVFP4 = 3 };

// The split tail of an L2 launch over `tiles` whole tiles with nw work slots
// (the persistent grid's workgroups): when tiles >= nw leaves a partial last
// round of tail = tiles % nw tiles, those (the last in the grid's order) run
// as kt K parts each, kt the largest power of two <= kmax with tail * kt <=
// min(nw, cap) that divides the nst K stages, so the parts fill that round;
// the first `full` tiles run whole.  kt = 1, tail = 0 when nothing splits.
// The GEMM and the combine both derive it from the same routing count.
struct TailSplit {
  int full, tail, kt;
};
__host__ __device__ inline TailSplit tail_split(int tiles, int nw, int kmax, int cap, int nst) {
  TailSplit r = {tiles, 0, 1};
  if (kmax < 2 || nw < 1 || tiles < nw || tiles % nw == 0) return r;
  const int tail = tiles % nw, lim = nw < cap ? nw : cap;
  for (int kt = kmax; kt >= 2; kt >>= 1) {
    if (tail * kt <= lim && nst % kt == 0) {
      r.full = tiles - tail;
      r.tail = tail;
      r.kt = kt;
      return r;
    }
  }
  return r;
}

// Routing metadata; with block_counts (dispatch_scratch_ints(S, E) int32
// values) and at least DISPATCH_MANY_MIN_SLOTS slots, the many-workgroup
// kernels (same result), else one workgroup.
constexpr int64_t DISPATCH_MANY_MIN_SLOTS = 16384;
int64_t dispatch_scratch_ints(int64_t S, int E);
// With tile_info, also the GemmArgs::tile_info records.
void launch_dispatch(const int32_t* topk_ids, int T, int k, int n_sh, int start, int n_loc, int bm,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                     int32_t* tile_expert, int32_t* tile_info, int32_t* meta, int32_t* block_counts,
                     hipStream_t stream);
// True when launch_dispatch runs the single-workgroup kernel.
bool dispatch_single_wg(int T, int k, int n_sh);
// That kernel and the MX dispatch quantisation of BF16 x [T, H] (E4M3 codes,
// UE8M0 scales, as launch_quant_mx(false, false, ...)) in one launch; with
// a1_sf, the same launch also writes the scale planes launch_gather_sf would
// (fill 127) when the slots of a quantising workgroup's tokens fit its LDS,
// and returns whether it did.
bool launch_dispatch_quant_mx(const int32_t* topk_ids, int T, int k, int n_sh, int start, int n_loc, int bm,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                              int32_t* tile_expert, int32_t* tile_info, int32_t* meta, const void* x, int H,
                              uint8_t* codes,
                              uint8_t* scales, uint8_t* a1_sf, int64_t plane, hipStream_t stream);

// Sum of the K parts of a split L1 GEMM (a.o, a.ksplit, a.o_split), then its
// activation and L2-input quantisation into (a.c, a.c_sf).
void launch_l1_finish(int fmt, const GemmArgs& a, const int32_t* slot_row, const int32_t* tile_expert, int bm,
                      int S, hipStream_t st);

hipError_t launch_gemm(int fmt, int layer, int bm, const GemmArgs& args, int grid, hipStream_t stream);
// Workgroups of that launch: grid times the tile's workgroups per CU.
int gemm_workgroups(int fmt, int bm, int grid);
hipError_t gemm_init(int device);

// Combine (topk_w NULL: every slot weighs 1); gamma non-NULL adds the
// post-expert RMSNorm.
// The split tail of the L2 that wrote the rows (o_tail NULL: none): the
// GemmArgs fields and the L2 launch's work slots, from which the combine
// derives the same TailSplit as the GEMM.
struct CombineTail {
  const float* o_tail;
  const int32_t* tile_info;
  const int32_t* meta;
  int bm, nw, kmax, cap, nst;
};
void launch_combine(const float* o, int o_bf16, int nsplit, int64_t o_split, const int32_t* slot_row,
                    const float* topk_w, int T, int k, int kk, int H, const float* gamma, float eps,
                    const CombineTail& tail, uint16_t* out, hipStream_t stream);
// L1 A-operand block scales x_sf [T, sf_ld] -> block-major planes of the
// sorted rows: out[kb * plane + m] (rows m < offsets[E]); with a_tok, also
// row_scale[m] = a_tok of the row's token (1 for padding).
void launch_gather_sf(const int32_t* sorted_slot, const int32_t* offsets, int E, int kk, const uint8_t* x_sf,
                      int sf_ld, int64_t plane, int64_t max_rows, uint8_t fill, uint8_t* out, const float* a_tok,
                      float* row_scale, hipStream_t stream);

void launch_scale_rows(const uint16_t* x, const float* w, int T, int H, uint16_t* xw, hipStream_t stream);

// BF16 x rows in sorted order, stage-blocked for the L1 GEMM (GemmArgs::bm):
// sorted row m < offsets[E] takes x[sorted_slot[m] / kk], a padding row zeros.
void launch_block_rows_bf16(const uint16_t* x, const int32_t* sorted_slot, const int32_t* offsets, int E, int kk,
                            int H, int bm, int64_t max_rows, uint16_t* xs, hipStream_t stream);

void launch_transform(int fmt, int E, int H, int I, const uint8_t* w13, const uint8_t* w13_sf,
                      const uint8_t* w2, const uint8_t* w2_sf, uint8_t* w13_k, uint8_t* w13_sf_k,
                      uint8_t* w2_k, uint8_t* w2_sf_k, hipStream_t stream);

// MX quantiser: rows x cols (cols % 32 == 0), BF16 or float32 source;
// fp4 selects E2M1 elements (two per byte), else E4M3.
void launch_quant_mx(bool fp4, bool f32, int64_t rows, int cols, const void* src, uint8_t* codes, uint8_t* scales,
                     hipStream_t stream);

// NVFP4 quantiser, one row per workgroup.  fixed_g != NULL: row r uses
// fixed_g[r / rows_per_g]; else the row's own amax / (6 * 448) is used and
// written to row_g[r].
void launch_quant_nv(bool f32, int64_t rows, int cols, const void* src, uint8_t* codes, uint8_t* scales,
                     float* row_g, const float* fixed_g, int rows_per_g, hipStream_t stream);

void launch_route(const float* logits, const float* bias, int T, int E, int k, int sigmoid, int G, int TG,
                  int renorm, float scaling, const uint8_t* is_padding, int32_t* ids, float* wts,
                  hipStream_t stream);

void launch_weight_gscale(int E, int64_t per_expert, const float* src, float* gscale, hipStream_t stream);

}  // namespace moe
