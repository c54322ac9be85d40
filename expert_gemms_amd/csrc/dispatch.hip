// Token dispatch: routing metadata for the grouped GEMMs.
//
// The contiguous layout of the "fused_moe" page's DeepGemmExperts.apply:
// rows of every local expert are gathered into one group padded to BLOCK_M
// (compute_aligned_M), permuted there and un-permuted after the L2 GEMM.
// Slot s = t * k' + j (k' = top_k + num_shared); shared choices are always
// selected (DeepGEMM MegaMoE experts page: a fused shared expert runs inside
// the launch as an always-selected expert); routed ids outside this GPU's
// expert range are dropped.
//
// One workgroup of 16 waves.  Wave w owns a contiguous run of slots.  Pass 1
// counts each expert's slots per wave: inside a 64-slot batch the lanes that
// hold the same expert find each other with one ballot per expert-id bit, and
// the lowest such lane adds the group size, so no two lanes of a wave touch
// one counter and no order-dependent atomics are needed.  Pass 2 scans the
// per-wave counts (per expert) and the BLOCK_M-padded totals (over experts).
// Pass 3 walks the batches again in order and scatters every slot to
// offset + (earlier slots of its expert), which is the stable order.
#include <type_traits>

#include "common.h"
#include "l2input.h"
#include "launch.h"

namespace moe {

constexpr int DISPATCH_WAVES = 16;
constexpr int DISPATCH_THREADS = DISPATCH_WAVES * WAVE;

__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ topk_ids, int s, int kk, int k,
                                           int start, int n_loc) {
  int t = s / kk, j = s - t * kk;
  if (j >= k) return n_loc + (j - k);
  int e = topk_ids[(size_t)t * k + j] - start;
  return (e >= 0 && e < n_loc) ? e : -1;
}

// Lanes of this wave whose expert equals mine (bit-sliced compare).
__device__ __forceinline__ uint64_t match_mask(int e, int nbits) {
  uint64_t m = ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    bool bit = (e >> b) & 1;
    uint64_t bb = ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return e >= 0 ? m : 0ull;
}

// Experts of lane l's slots in G consecutive 64-slot batches from b (-1:
// past s1 or dropped).  All G loads are issued before any is used, so a pass
// over a wave's slots waits out one load latency per G batches, not one per
// batch.  The many-workgroup passes take 8 batches at a time; the
// single-workgroup dispatch one (at decode sizes, where a wave has one batch
// or none, the wider form measured slower).
template <int G>
__device__ __forceinline__ void group_experts(const int32_t* __restrict__ topk_ids, int b, int s1, int kk, int k,
                                              int start, int n_loc, int l, int (&e)[G]) {
#pragma unroll
  for (int i = 0; i < G; ++i) {
    e[i] = -1;
    if (b + i * WAVE < s1) {   // uniform: no work for batches past the end
      const int s = b + i * WAVE + l;
      if (s < s1) e[i] = slot_expert(topk_ids, s, kk, k, start, n_loc);
    }
  }
}

// Counting pass over one wave's slots [s0, s1): hist_w[e] += its slots of
// expert e (the lowest lane of each group of equal experts adds the group).
template <int G>
__device__ __forceinline__ void wave_count(const int32_t* __restrict__ topk_ids, int s0, int s1, int kk, int k,
                                           int start, int n_loc, int nbits, int* hist_w, int l) {
  for (int b = s0; b < s1; b += G * WAVE) {
    int eg[G];
    group_experts<G>(topk_ids, b, s1, kk, k, start, n_loc, l, eg);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (b + i * WAVE >= s1) break;
      const int e = eg[i];
      uint64_t m = match_mask(e, nbits);
      if (e >= 0 && (__builtin_ctzll(m) == l)) hist_w[e] += __builtin_popcountll(m);
    }
  }
}

// Scatter pass over one wave's slots [s0, s1) in order: slot s of expert e
// goes to row hist_w[e] + (earlier slots of e in its batch), then the group
// leader advances hist_w[e]; a dropped slot gets slot_row -1.
template <int G>
__device__ __forceinline__ void wave_scatter(const int32_t* __restrict__ topk_ids, int s0, int s1, int kk, int k,
                                             int start, int n_loc, int nbits, int* hist_w, int l,
                                             int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row) {
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  for (int b0 = s0; b0 < s1; b0 += G * WAVE) {
    int eg[G];
    group_experts<G>(topk_ids, b0, s1, kk, k, start, n_loc, l, eg);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int b = b0 + i * WAVE;
      if (b >= s1) break;
      const int s = b + l;
      const bool live = s < s1;
      const int e = eg[i];
      uint64_t m = match_mask(e, nbits);
      if (e >= 0) {
        int pos = hist_w[e] + __builtin_popcountll(m & lt_mask);
        sorted_slot[pos] = s;
        slot_row[s] = pos;
      } else if (live) {
        slot_row[s] = -1;
      }
      // every lane has read its base before the group leader bumps it
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && __builtin_ctzll(m) == l) hist_w[e] += __builtin_popcountll(m);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// The tile -> expert tables for BLOCK_M blocks [0, nblocks), the blocks
// spread over the workgroup's threads: block tb belongs to the last expert
// whose group starts at or before row tb * bm (empty groups share their
// start with the next group and come before it).  s_off: the groups' first
// rows [E + 1] in LDS.
__device__ __forceinline__ void tile_tables(const int* s_off, int E, int bm, int nblocks,
                                            int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_info) {
  for (int tb = threadIdx.x; tb < nblocks; tb += DISPATCH_THREADS) {
    const int r = tb * bm;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    tile_expert[tb] = lo;
    if (tile_info) *(int4*)(tile_info + 4 * tb) = make_int4(lo, s_off[lo] / bm, (s_off[lo + 1] - s_off[lo]) / bm, 0);
  }
}

__device__ __forceinline__ void dispatch_wg(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start,
                                            int n_loc, int bm, int nbits, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                                            int32_t* __restrict__ slot_row, int32_t* __restrict__ tile_expert,
                                            int32_t* __restrict__ tile_info, int32_t* __restrict__ meta) {
  __shared__ int hist[DISPATCH_WAVES][MAX_LOCAL_EXPERTS];
  __shared__ int wave_tot[DISPATCH_WAVES];
  __shared__ int s_off[MAX_LOCAL_EXPERTS + 1];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE;
  const int kk = k + n_sh, E = n_loc + n_sh, S = T * kk;

  for (int i = tid; i < DISPATCH_WAVES * MAX_LOCAL_EXPERTS; i += DISPATCH_THREADS) (&hist[0][0])[i] = 0;
  __syncthreads();

  // slots of wave w: [s0, s1), s0 a multiple of 64
  const int per = ((S + DISPATCH_WAVES - 1) / DISPATCH_WAVES + WAVE - 1) / WAVE * WAVE;
  const int s0 = min(w * per, S), s1 = min(s0 + per, S);

  // pass 1: per-wave histogram
  wave_count<1>(topk_ids, s0, s1, kk, k, start, n_loc, nbits, hist[w], l);
  __syncthreads();

  // pass 2a: expert tid: exclusive scan of its per-wave counts; padded size
  static_assert(MAX_LOCAL_EXPERTS <= DISPATCH_THREADS, "one expert per thread");
  int run = 0;
  if (tid < E) {
    for (int ww = 0; ww < DISPATCH_WAVES; ++ww) { int c = hist[ww][tid]; hist[ww][tid] = run; run += c; }
    counts[tid] = run;
  }
  const int v = tid < E ? (run + bm - 1) / bm * bm : 0;
  // pass 2b: exclusive scan of padded sizes over experts (one per thread)
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    int o = __shfl_up(incl, d, 64);
    if (l >= d) incl += o;
  }
  if (l == WAVE - 1) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int ww = 0; ww < w; ++ww) wbase += wave_tot[ww];
  const int off = wbase + incl - v;                 // exclusive offset of expert tid
  int total = 0;
  for (int ww = 0; ww < DISPATCH_WAVES; ++ww) total += wave_tot[ww];
  if (tid < E) {
    offsets[tid] = off;
    s_off[tid] = off;
    for (int ww = 0; ww < DISPATCH_WAVES; ++ww) hist[ww][tid] += off;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = total;
    if (meta) {
      meta[0] = total / bm;   // number of BLOCK_M tiles
      meta[1] = total;        // padded rows
    }
  }
  __syncthreads();

  // pass 3: stable scatter
  wave_scatter<1>(topk_ids, s0, s1, kk, k, start, n_loc, nbits, hist[w], l, sorted_slot, slot_row);

  // padding rows and the tile -> expert tables
  if (tid < E)
    for (int r = off + run; r < off + v; ++r) sorted_slot[r] = -1;
  tile_tables(s_off, E, bm, total / bm, tile_expert, tile_info);
}

__global__ void __launch_bounds__(DISPATCH_THREADS)
k_dispatch(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start, int n_loc,
           int bm, int nbits, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
           int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row,
           int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_info, int32_t* __restrict__ meta) {
  dispatch_wg(topk_ids, T, k, n_sh, start, n_loc, bm, nbits, counts, offsets, sorted_slot, slot_row, tile_expert,
              tile_info, meta);
}

// Sorted rows of the slots [s0, s1) (whole tokens) without the routing
// metadata, for a workgroup that needs them but does not build them: every
// slot's expert is counted (LDS atomics; cnt_before counts the slots before
// s0), the BLOCK_M-padded groups are laid out as dispatch_wg lays them out
// (gstart: each group's first row), and the slots of [s0, s1) are ranked in
// slot order from gstart + cnt_before, the same stable order, so row_of[s -
// s0] equals the slot_row[s] the dispatch writes (-1: dropped).
constexpr int LOCAL_SLOTS = 4096;

__device__ __forceinline__ void local_rows(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start,
                                           int n_loc, int bm, int nbits, int s0, int s1, int* cnt_all,
                                           int* cnt_before, int* gstart, int* row_of) {
  __shared__ int wave_tot[DISPATCH_WAVES];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE;
  const int kk = k + n_sh, E = n_loc + n_sh, S = T * kk;
  for (int e = tid; e < E; e += DISPATCH_THREADS) cnt_all[e] = cnt_before[e] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += DISPATCH_THREADS) {
    const int e = slot_expert(topk_ids, s, kk, k, start, n_loc);
    if (e >= 0) {
      atomicAdd(&cnt_all[e], 1);
      if (s < s0) atomicAdd(&cnt_before[e], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the padded group sizes over experts (one per thread)
  const int v = tid < E ? (cnt_all[tid] + bm - 1) / bm * bm : 0;
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (l >= d) incl += o;
  }
  if (l == WAVE - 1) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int ww = 0; ww < w; ++ww) wbase += wave_tot[ww];
  if (tid < E) {
    gstart[tid] = wbase + incl - v;
    cnt_before[tid] += wbase + incl - v;      // next row of expert tid for the slots from s0 on
  }
  __syncthreads();
  // wave 0 ranks [s0, s1) in 64-slot batches (as wave_scatter does)
  if (w == 0) {
    const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
    for (int b = s0; b < s1; b += WAVE) {
      const int s = b + l;
      const bool live = s < s1;
      const int e = live ? slot_expert(topk_ids, s, kk, k, start, n_loc) : -1;
      const uint64_t m = match_mask(e, nbits);
      if (e >= 0) row_of[s - s0] = cnt_before[e] + __builtin_popcountll(m & lt_mask);
      else if (live) row_of[s - s0] = -1;
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && __builtin_ctzll(m) == l) cnt_before[e] += __builtin_popcountll(m);
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
}

// The single-workgroup dispatch and the MX dispatch quantisation of x (E4M3
// codes, BF16 input) in one launch: workgroup 0 builds the routing metadata
// while workgroups 1 .. nq quantise x, one MX block per thread (QB blocks
// per workgroup with a1_sf, which spreads the scale scatter over more CUs;
// the rest of the workgroup's threads only help to count).  With a1_sf
// the launch also writes the L1 GEMM's scale planes that launch_gather_sf
// would: the quantising workgroups place each block scale at a1_sf[kb *
// plane + row] for every sorted row of its token (rows from local_rows), and
// workgroups nq + 1 .. each fill the padding rows of FILL_PLANES planes with
// UE8M0 1.0, lanes on consecutive rows.  Real and padding rows are disjoint,
// so no two workgroups write one byte.  This saves two launches on
// decode-sized batches.
constexpr int FILL_PLANES = 4;
constexpr int QB = 256;

__global__ void __launch_bounds__(DISPATCH_THREADS)
k_dispatch_quant_mx(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start, int n_loc, int bm,
                    int nbits, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row,
                    int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_info, int32_t* __restrict__ meta,
                    const void* __restrict__ x,
                    int nkb, int64_t nblocks, int nq, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                    uint8_t* __restrict__ a1_sf, int64_t plane) {
  if (blockIdx.x == 0) {
    dispatch_wg(topk_ids, T, k, n_sh, start, n_loc, bm, nbits, counts, offsets, sorted_slot, slot_row, tile_expert,
                tile_info, meta);
    return;
  }
  const int q = blockIdx.x - 1, tid = threadIdx.x;
  if (!a1_sf) {
    const int64_t b = (int64_t)q * DISPATCH_THREADS + tid;
    if (b < nblocks) quant_mx_block<false, false>(x, b, codes, scales);
    return;
  }
  const int64_t b0 = (int64_t)q * QB, b = b0 + tid;
  __shared__ int cnt_all[MAX_LOCAL_EXPERTS], next_row[MAX_LOCAL_EXPERTS], gstart[MAX_LOCAL_EXPERTS];
  __shared__ int row_of[LOCAL_SLOTS];
  const int kk = k + n_sh, E = n_loc + n_sh;
  if (q < nq) {
    // this workgroup's tokens [t0, t1)
    const int t0 = (int)(b0 / nkb);
    const int t1 = (int)min<int64_t>((b0 + QB - 1) / nkb + 1, T);
    local_rows(topk_ids, T, k, n_sh, start, n_loc, bm, nbits, t0 * kk, t1 * kk, cnt_all, next_row, gstart, row_of);
    if (tid < QB && b < nblocks) {
      const int c = quant_mx_block<false, false>(x, b, codes, scales);
      const int t = (int)(b / nkb), kb = (int)(b % nkb);
      for (int j = 0; j < kk; ++j) {
        const int r = row_of[(t - t0) * kk + j];
        if (r >= 0) a1_sf[kb * plane + r] = (uint8_t)c;
      }
    }
    return;
  }
  // padding rows of planes [kb0, kb1): expert e pads rows [gstart + count,
  // gstart + padded); pad_end (in row_of) is the inclusive scan of the
  // padding counts, and padding row i of the plane belongs to the first
  // expert whose pad_end exceeds i
  __shared__ int wave_tot[DISPATCH_WAVES];
  local_rows(topk_ids, T, k, n_sh, start, n_loc, bm, nbits, 0, 0, cnt_all, next_row, gstart, row_of);
  const int w = tid / WAVE, l = tid % WAVE;
  const int pad = tid < E ? (cnt_all[tid] + bm - 1) / bm * bm - cnt_all[tid] : 0;
  int incl = pad;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (l >= d) incl += o;
  }
  if (l == WAVE - 1) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0, P = 0;
  for (int ww = 0; ww < DISPATCH_WAVES; ++ww) {
    if (ww < w) wbase += wave_tot[ww];
    P += wave_tot[ww];
  }
  if (tid < E) row_of[tid] = wbase + incl;
  __syncthreads();
  const int kb0 = (q - nq) * FILL_PLANES, kb1 = min(kb0 + FILL_PLANES, nkb);
  for (int i = tid; i < P; i += DISPATCH_THREADS) {
    int lo = 0, hi = E - 1;                    // first e with pad_end[e] > i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (row_of[mid] > i) hi = mid;
      else lo = mid + 1;
    }
    const int n = cnt_all[lo], pad_lo = (n + bm - 1) / bm * bm - n;
    const int r = gstart[lo] + n + (i - (row_of[lo] - pad_lo));
    for (int kb = kb0; kb < kb1; ++kb) a1_sf[kb * plane + r] = 127;
  }
}

// Many-workgroup dispatch for large slot counts: the same metadata in three
// launches.  The slots are cut into chunks of DCHUNK (4 waves of 512): a
// counting launch writes each chunk's per-expert counts to block_counts
// [chunks, E]; one workgroup scans them per expert (chunk order), lays out
// the BLOCK_M-padded groups and turns block_counts into each chunk's first
// row per expert; a scatter launch recounts each chunk per wave and places
// its slots in order.  Chunks, and waves inside a chunk, are in slot order,
// so the result equals the single-workgroup kernel's row for row.
constexpr int DCHUNK = 2048;
constexpr int DC_WAVES = 4;
constexpr int DC_PER_WAVE = DCHUNK / DC_WAVES;

__global__ void __launch_bounds__(DC_WAVES * WAVE)
k_dispatch_count(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start, int n_loc, int nbits,
                 int32_t* __restrict__ block_counts) {
  __shared__ int hist[DC_WAVES][MAX_LOCAL_EXPERTS];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE;
  const int kk = k + n_sh, E = n_loc + n_sh, S = T * kk;
  for (int i = tid; i < DC_WAVES * MAX_LOCAL_EXPERTS; i += DC_WAVES * WAVE) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int s0 = min(blockIdx.x * DCHUNK + w * DC_PER_WAVE, S), s1 = min(s0 + DC_PER_WAVE, S);
  wave_count<8>(topk_ids, s0, s1, kk, k, start, n_loc, nbits, hist[w], l);
  __syncthreads();
  for (int e = tid; e < E; e += DC_WAVES * WAVE) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < DC_WAVES; ++ww) c += hist[ww][e];
    block_counts[(int64_t)blockIdx.x * E + e] = c;
  }
}

__global__ void __launch_bounds__(DISPATCH_THREADS)
k_dispatch_scan(int nchunks, int E, int bm, int32_t* __restrict__ block_counts, int32_t* __restrict__ counts,
                int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_info, int32_t* __restrict__ meta) {
  __shared__ int wave_tot[DISPATCH_WAVES];
  __shared__ int s_off[MAX_LOCAL_EXPERTS + 1];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE;
  // the chunks' counts of expert tid: up to RCHUNKS chunks all loaded at
  // once and kept in registers (one load latency, then one round of
  // stores); more chunks 16 loads at a time, with a second pass adding the
  // offset (a load-add-store chain per chunk would wait out each load)
  constexpr int RCHUNKS = 64, BATCH = 16;
  const bool in_regs = nchunks <= RCHUNKS;
  int n[RCHUNKS];
  int run = 0;
  if (tid < E) {
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < RCHUNKS; ++i) n[i] = i < nchunks ? block_counts[(int64_t)i * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < RCHUNKS; ++i) {
        const int c = n[i];
        n[i] = run;
        run += c;
      }
    } else {
      for (int c0 = 0; c0 < nchunks; c0 += BATCH) {
        int nb[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) nb[i] = c0 + i < nchunks ? block_counts[(int64_t)(c0 + i) * E + tid] : 0;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          if (c0 + i < nchunks) block_counts[(int64_t)(c0 + i) * E + tid] = run;
          run += nb[i];
        }
      }
    }
    counts[tid] = run;
  }
  const int v = tid < E ? (run + bm - 1) / bm * bm : 0;
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    int o = __shfl_up(incl, d, 64);
    if (l >= d) incl += o;
  }
  if (l == WAVE - 1) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int ww = 0; ww < w; ++ww) wbase += wave_tot[ww];
  const int off = wbase + incl - v;
  int total = 0;
  for (int ww = 0; ww < DISPATCH_WAVES; ++ww) total += wave_tot[ww];
  if (tid < E) {
    offsets[tid] = off;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < RCHUNKS; ++i)
        if (i < nchunks) block_counts[(int64_t)i * E + tid] = n[i] + off;
    } else {
      for (int c0 = 0; c0 < nchunks; c0 += BATCH) {
        int b[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) b[i] = c0 + i < nchunks ? block_counts[(int64_t)(c0 + i) * E + tid] : 0;
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          if (c0 + i < nchunks) block_counts[(int64_t)(c0 + i) * E + tid] = b[i] + off;
      }
    }
    for (int r = off + run; r < off + v; ++r) sorted_slot[r] = -1;
    s_off[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = total;
    if (meta) {
      meta[0] = total / bm;
      meta[1] = total;
    }
  }
  __syncthreads();
  tile_tables(s_off, E, bm, total / bm, tile_expert, tile_info);
}

__global__ void __launch_bounds__(DC_WAVES * WAVE)
k_dispatch_scatter(const int32_t* __restrict__ topk_ids, int T, int k, int n_sh, int start, int n_loc, int nbits,
                   const int32_t* __restrict__ block_counts, int32_t* __restrict__ sorted_slot,
                   int32_t* __restrict__ slot_row) {
  __shared__ int hist[DC_WAVES][MAX_LOCAL_EXPERTS];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE;
  const int kk = k + n_sh, E = n_loc + n_sh, S = T * kk;
  for (int i = tid; i < DC_WAVES * MAX_LOCAL_EXPERTS; i += DC_WAVES * WAVE) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int s0 = min(blockIdx.x * DCHUNK + w * DC_PER_WAVE, S), s1 = min(s0 + DC_PER_WAVE, S);
  wave_count<8>(topk_ids, s0, s1, kk, k, start, n_loc, nbits, hist[w], l);
  __syncthreads();
  // each wave's first row per expert: the chunk's base plus the earlier waves
  for (int e = tid; e < E; e += DC_WAVES * WAVE) {
    int base = block_counts[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int ww = 0; ww < DC_WAVES; ++ww) {
      const int c = hist[ww][e];
      hist[ww][e] = base;
      base += c;
    }
  }
  __syncthreads();
  wave_scatter<8>(topk_ids, s0, s1, kk, k, start, n_loc, nbits, hist[w], l, sorted_slot, slot_row);
}

int64_t dispatch_scratch_ints(int64_t S, int E) { return (S + DCHUNK - 1) / DCHUNK * E; }

void launch_dispatch(const int32_t* topk_ids, int T, int k, int n_sh, int start, int n_loc, int bm,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                     int32_t* tile_expert, int32_t* tile_info, int32_t* meta, int32_t* block_counts,
                     hipStream_t stream) {
  int E = n_loc + n_sh;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int64_t S = (int64_t)T * (k + n_sh);
  if (block_counts && S >= DISPATCH_MANY_MIN_SLOTS) {
    const int nchunks = (int)((S + DCHUNK - 1) / DCHUNK);
    hipLaunchKernelGGL(k_dispatch_count, dim3(nchunks), dim3(DC_WAVES * WAVE), 0, stream, topk_ids, T, k, n_sh, start,
                       n_loc, nbits, block_counts);
    hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(DISPATCH_THREADS), 0, stream, nchunks, E, bm, block_counts,
                       counts, offsets, sorted_slot, tile_expert, tile_info, meta);
    hipLaunchKernelGGL(k_dispatch_scatter, dim3(nchunks), dim3(DC_WAVES * WAVE), 0, stream, topk_ids, T, k, n_sh,
                       start, n_loc, nbits, block_counts, sorted_slot, slot_row);
    return;
  }
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(DISPATCH_THREADS), 0, stream, topk_ids, T, k, n_sh, start,
                     n_loc, bm, nbits, counts, offsets, sorted_slot, slot_row, tile_expert, tile_info, meta);
}

bool dispatch_single_wg(int T, int k, int n_sh) { return (int64_t)T * (k + n_sh) < DISPATCH_MANY_MIN_SLOTS; }

bool launch_dispatch_quant_mx(const int32_t* topk_ids, int T, int k, int n_sh, int start, int n_loc, int bm,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                              int32_t* tile_expert, int32_t* tile_info, int32_t* meta, const void* x, int H,
                              uint8_t* codes,
                              uint8_t* scales, uint8_t* a1_sf, int64_t plane, hipStream_t stream) {
  const int E = n_loc + n_sh;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int nkb = H / 32;
  const int64_t nblocks = (int64_t)T * nkb;
  // a workgroup's QB blocks touch at most (QB - 1) / nkb + 2 tokens
  const bool planes = a1_sf && ((QB - 1) / nkb + 2) * (k + n_sh) <= LOCAL_SLOTS;
  const int per = planes ? QB : DISPATCH_THREADS;
  const unsigned nq = (unsigned)((nblocks + per - 1) / per);
  const unsigned nf = planes ? (unsigned)((nkb + FILL_PLANES - 1) / FILL_PLANES) : 0;
  hipLaunchKernelGGL(k_dispatch_quant_mx, dim3(1 + nq + nf), dim3(DISPATCH_THREADS), 0, stream, topk_ids, T, k,
                     n_sh, start, n_loc, bm, nbits, counts, offsets, sorted_slot, slot_row, tile_expert, tile_info, meta,
                     x, nkb,
                     nblocks, (int)nq, codes, scales, planes ? a1_sf : nullptr, plane);
  return planes;
}

// Block scales of the L1 A operand in the GEMM's layout: one plane per
// K block (plane kb holds the scale of every sorted row, row-contiguous), so
// a tile's scales for one K block are BLOCK_M consecutive bytes.  Row m of
// the sorted order takes the scale row of token sorted_slot[m] / kk; a
// padding row, and the rows from offsets[E] to the next multiple of 4, take
// `fill`.  A thread takes 4 rows and P planes (blockIdx.y: the plane group;
// P = 16 where the rows' scale bytes split into 16-byte pieces, else 8) and
// stores a dword of 4 rows per plane (256 consecutive bytes per wave).
// With a_tok (NVFP4), the first plane group also writes each row's token
// scale to row_scale (1 for a padding row).
template <int P>
__global__ void __launch_bounds__(256) k_gather_sf(const int32_t* __restrict__ sorted_slot,
                                                   const int32_t* __restrict__ offsets, int E, int kk,
                                                   const uint8_t* __restrict__ x_sf, int sf_ld, int64_t plane,
                                                   uint8_t fill, uint8_t* __restrict__ out,
                                                   const float* __restrict__ a_tok, float* __restrict__ row_scale) {
  static_assert(P == 8 || P == 16, "8 or 16 planes per thread");
  using V = typename std::conditional<P == 16, uint4, uint2>::type;
  const int m = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int M = offsets[E];
  if (m >= M) return;
  const uint8_t* src[4];
  bool real[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = m + i < M ? sorted_slot[m + i] : -1;
    real[i] = sl >= 0;
    src[i] = x_sf + (int64_t)(real[i] ? sl / kk : 0) * sf_ld;
    if (a_tok && blockIdx.y == 0 && m + i < M) row_scale[m + i] = real[i] ? a_tok[sl / kk] : 1.0f;
  }
  const int kb = blockIdx.y * P;
  uint32_t v[4][P / 4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const V x = *(const V*)(src[i] + kb);
    v[i][0] = x.x;
    v[i][1] = x.y;
    if constexpr (P == 16) {
      v[i][2] = x.z;
      v[i][3] = x.w;
    }
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = real[i] ? (v[i][j / 4] >> (8 * (j & 3))) & 0xFF : fill;
      word |= b << (8 * i);
    }
    *(uint32_t*)(out + (int64_t)(kb + j) * plane + m) = word;
  }
}

void launch_gather_sf(const int32_t* sorted_slot, const int32_t* offsets, int E, int kk, const uint8_t* x_sf,
                      int sf_ld, int64_t plane, int64_t max_rows, uint8_t fill, uint8_t* out, const float* a_tok,
                      float* row_scale, hipStream_t stream) {
  const unsigned blocks = (unsigned)((max_rows + 1023) / 1024);
  if (blocks == 0 || sf_ld < 8) return;
  if (sf_ld % 16 == 0)
    hipLaunchKernelGGL(k_gather_sf<16>, dim3(blocks, (unsigned)(sf_ld / 16)), dim3(256), 0, stream, sorted_slot,
                       offsets, E, kk, x_sf, sf_ld, plane, fill, out, a_tok, row_scale);
  else
    hipLaunchKernelGGL(k_gather_sf<8>, dim3(blocks, (unsigned)(sf_ld / 8)), dim3(256), 0, stream, sorted_slot,
                       offsets, E, kk, x_sf, sf_ld, plane, fill, out, a_tok, row_scale);
}

// BF16 layers: the L1 GEMM's A rows in sorted order and stage-blocked
// ([M / bm][H / 32][bm][32 values]), so a tile's stage is one contiguous run
// of full cache lines.  Workgroup m copies sorted row m (x of its token, or
// zeros for a padding row) in 16-byte chunks.
__global__ void __launch_bounds__(256) k_block_rows_bf16(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ sorted_slot,
                                                         const int32_t* __restrict__ offsets, int E, int kk, int H,
                                                         int bm, uint16_t* __restrict__ xs) {
  const int m = blockIdx.x;
  if (m >= offsets[E]) return;
  const int sl = sorted_slot[m];
  const uint16_t* src = x + (int64_t)(sl >= 0 ? sl / kk : 0) * H;
  uint16_t* dst = xs + (int64_t)(m / bm) * H * bm + (m % bm) * 32;
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    const uint4 v = sl >= 0 ? *(const uint4*)(src + c * 8) : make_uint4(0, 0, 0, 0);
    // element 8c: stage 8c / 32, column 8c % 32 of that stage's 32
    *(uint4*)(dst + (int64_t)(c / 4) * bm * 32 + (c % 4) * 8) = v;
  }
}

void launch_block_rows_bf16(const uint16_t* x, const int32_t* sorted_slot, const int32_t* offsets, int E, int kk,
                            int H, int bm, int64_t max_rows, uint16_t* xs, hipStream_t stream) {
  if (max_rows <= 0) return;
  hipLaunchKernelGGL(k_block_rows_bf16, dim3((unsigned)max_rows), dim3(256), 0, stream, x, sorted_slot, offsets, E, kk,
                     H, bm, xs);
}

}  // namespace moe
