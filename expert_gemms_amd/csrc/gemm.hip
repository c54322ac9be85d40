// Grouped expert GEMMs on gfx950 MFMA: L1 (x * W13^T, gated activation and
// L2-input quantisation in the epilogue) and L2 (A2 * W2^T -> float32 rows
// per slot).
//
// What is computed: the two expert GEMMs of the DeepGEMM MegaMoE experts page
// (one launch runs L1, the activation of MegaMoEActivation, the L2-input
// quantisation and L2), in the step order of the "fused_moe" page's
// DeepGemmExperts.apply (grouped GEMM, activation, per-group quantisation,
// grouped GEMM).  Weight formats: BF16 (32x32x16 bf16 MFMA), MXFP8 and MXFP4
// (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4 consuming the UE8M0 block scales
// directly; MXFP4 weights against MXFP8 activations), NVFP4 (E2M1 operands
// with E4M3 block scales, dequantised to exact FP16 in registers and fed to
// the 32x32x16 f16 MFMA; per-token and per-expert FP32 scales in the
// epilogues).
//
// Work decomposition: a persistent grid of (#CUs) workgroups walks the tiles
// (BLOCK_M rows of one expert x 256 output columns).  Every tile has the same
// cost, so skewed routing only changes how many tiles an expert owns, and the
// static round-robin stays balanced.  Tiles are ordered expert-major, then by
// N block, then by M block, and each XCD takes a contiguous run of tiles per
// round, so the M blocks of one expert that share a weight block run on the
// same XCD at the same time and read it through that XCD's L2.
//
// Per tile: 4 waves, each owning a (BLOCK_M / WM) x (256 / WN) sub-tile of
// 32x32 MFMA accumulators.  K advances in stages; each stage's A rows, weight
// fragments and block scales are copied global -> LDS by the LDS-DMA path
// (global_load_lds_dwordx4) into a ring of LDS buffers, several stages ahead
// of the MFMAs.  A rows sit in LDS as 64- or 128-byte rows whose 16-byte
// chunks are XOR-swizzled (see swz) so each ds_read_b128 phase is bank-
// conflict free.
// Fragments of K-step ks+1 are read into a second register set while the
// MFMAs of K-step ks run.  Weights arrive in the kernel layout written by
// moe_transform_weights: each 32-row x K-step fragment is 1 KiB (or 2 KiB)
// in register order, so the weight copy and its LDS reads are linear.
#include <type_traits>

#include "common.h"
#include "l2input.h"
#include "launch.h"

namespace moe {

template <int FMT> struct FmtCfg;
// KSTAGE: K elements per LDS stage; A_ROW / B_ROW: bytes per row per stage;
// STEPS: register-fragment steps per stage (an MFMA K-step, or for NVFP4 a
// 64-K group of four 16-wide K-steps); NBUF: LDS stage buffers (NBUF - 1
// stages are in flight while one is computed).  Weight fragments are FRAG
// bytes and sit in the weight layout as [layout stage][32-row block][KS_PER_L
// K-steps], independent of how many K-steps a kernel stage takes.
template <> struct FmtCfg<F_BF16> {
  static constexpr int KSTAGE = 32, A_ROW = 64, B_ROW = 64, STEPS = 2, NBUF = 4;
  static constexpr int FRAG = 1024, KS_PER_L = 4;
  static constexpr bool SCALED = false, NV = false;
};
// MX formats: a stage is one 128-K block-scale layout stage, two 64-K
// scaled-MFMA steps (K-step j takes A-scale byte 2j + lane group and B-scale
// byte j of the layout stage); fewer, longer stages amortise each stage's
// wait, barrier and scale reads.
template <> struct FmtCfg<F_MXFP8> {
  static constexpr int KSTAGE = 128, A_ROW = 128, B_ROW = 128, STEPS = 2, NBUF = 3;
  static constexpr int FRAG = 2048, KS_PER_L = 2;
  static constexpr bool SCALED = true, NV = false;
};
template <> struct FmtCfg<F_MXFP4> {
  static constexpr int KSTAGE = 128, A_ROW = 128, B_ROW = 64, STEPS = 2, NBUF = 4;
  static constexpr int FRAG = 1024, KS_PER_L = 2;
  static constexpr bool SCALED = true, NV = false;
};
template <> struct FmtCfg<F_NVFP4> {
  static constexpr int KSTAGE = 128, A_ROW = 64, B_ROW = 64, STEPS = 2, NBUF = 4;
  static constexpr int FRAG = 1024, KS_PER_L = 2;
  static constexpr bool SCALED = true, NV = true;
};

// Configuration per tile height: the format's, except MXFP8 with 256-row
// tiles, whose 128-K stages would not fit three times in LDS.  Those take
// 64-K stages of one scaled K-step, whose scales are one half of the 128-K
// layout stage's, chosen by the stage's parity.
template <int FMT, int BM> struct Cfg : FmtCfg<FMT> {};
template <> struct Cfg<F_MXFP8, 256> : FmtCfg<F_MXFP8> {
  static constexpr int KSTAGE = 64, A_ROW = 64, B_ROW = 64, STEPS = 1, NBUF = 4;
};

template <int FMT, int BM>
struct TileGeom {
  using C = Cfg<FMT, BM>;
  static constexpr int WM = BM >= 128 ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = GEMM_BN / WN / 32;
  // every wave issues at least one A copy (rows wrap modulo BM)
  static constexpr int A_STAGE = BM * C::A_ROW < 4096 ? 4096 : BM * C::A_ROW;
  static constexpr int B_STAGE = GEMM_BN * C::B_ROW;
  // A scales: 256 bytes (one K block's plane from the tile's first row on)
  // per copy, one copy per wave (MX: a 128-K stage's 4 blocks, a 64-K
  // stage's 2 blocks twice), two for NVFP4 (8 blocks); B scales: every wave
  // copies its own, so the copy code has no wave branches
  static constexpr int A_SF_STAGE = C::SCALED ? (C::NV ? 2 : 1) * 4 * 256 : 0;
  // B scales: MX 1 KiB per stage (the 8 column blocks' 128 bytes, a quarter
  // per wave), NVFP4 1 KiB per wave (its column blocks)
  static constexpr int B_SF_STAGE = C::SCALED ? (C::NV ? 4 : 1) * 1024 : 0;
  static constexpr int STAGE = A_STAGE + B_STAGE + A_SF_STAGE + B_SF_STAGE;
  // workgroups per CU: two for the small tiles of weight-streaming launches
  // when three stage buffers each fit in half the LDS (while one workgroup
  // waits at a stage boundary the other computes or issues copies), else
  // one (the MFMA-bound tiles also need every register)
  // per-row data of two tiles (the current one and the next), 4 bytes per row:
  // NVFP4 L1 token scales, L2 (and K-split L1) slots
  static constexpr int ROWBUF = 2 * 1024;
  static constexpr int OCC = BM <= 64 && 3 * STAGE + ROWBUF <= 80 * 1024 ? 2 : 1;
  // LDS stage buffers: the format's ring depth (or as many as fit) for the
  // large (MFMA-bound) tiles; as many as fit, up to 8, for the small tiles of
  // weight-streaming launches, whose stages are short and need more copies in
  // flight.
  static constexpr int NBUF_FIT = (160 * 1024 / OCC - ROWBUF) / STAGE;
  static constexpr int NBUF = BM >= 128 ? (C::NBUF < NBUF_FIT ? C::NBUF : NBUF_FIT) : (NBUF_FIT < 8 ? NBUF_FIT : 8);
  static constexpr int ROWS_OFF = NBUF * STAGE;      // the row buffers
  static constexpr int LDS = NBUF * STAGE + ROWBUF;
  // A rows one wave copies per stage (contiguous; they wrap modulo BM)
  static constexpr int A_WROWS = A_STAGE / 4 / C::A_ROW;
  static constexpr int A_INSTR = A_STAGE / 1024 / 4;   // per wave
  static constexpr int B_INSTR = B_STAGE / 1024 / 4;   // per wave
  static constexpr int A_RPI = 1024 / C::A_ROW;         // A rows per copy instruction
  static constexpr int A_CPR = C::A_ROW / 16;           // 16-byte chunks per A row
  static constexpr int B_FRAGS_PER_NF = C::B_ROW * 32 / 1024;   // 1 KiB copies per 32-row block
  // copy instructions per wave per stage (the in-flight count of the ring)
  static constexpr int CPS = A_INSTR + B_INSTR + (C::SCALED ? (C::NV ? 3 : 2) : 0);
  static_assert((NBUF - 2) * CPS < 64, "vmcnt holds 6 bits");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small");
  static_assert(NBUF >= 3, "the copies of stage s + NBUF - 1 are spread over stage s");
  static_assert(LDS * OCC <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
  // kernel stages per 128-K stage of the block-scale layouts
  static constexpr int SPL = 128 / C::KSTAGE;
  static_assert(!C::SCALED || C::NV || (SPL == 2 && C::STEPS == 1) || (SPL == 1 && C::STEPS == 2),
                "MX stages are one 128-K layout stage or one half of it");
  static_assert(TN % 2 == 0, "gate/up pairs need an even number of N fragments");
};

// LDS A rows are 128 bytes (8 chunks of 16 bytes: MX 128-K stages) or 64
// bytes (4 chunks: BF16, NVFP4, MXFP8 256-row tiles).  gfx950 LDS serves 16 lanes x 16 bytes per cycle from 64 banks,
// so the 16 rows a ds_read_b128 phase touches must land on 16 distinct
// 16-byte bank groups: the chunk index is XORed with (r >> 1) & 7 for
// 128-byte rows (rows r, r+1 already differ by 128 bytes) and with
// (r >> 2) & 3 for 64-byte rows.
template <int A_ROW>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (A_ROW == 128) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);
}

// MFMA operand fragments of one K-step.
template <int FMT> struct Frag;
template <> struct Frag<F_BF16> { using A = bf16x8; using B = bf16x8; };
template <> struct Frag<F_MXFP8> { using A = i32x8; using B = i32x8; };
template <> struct Frag<F_MXFP4> { using A = i32x8; using B = i32x8; };
template <> struct Frag<F_NVFP4> { using A = i32x4; using B = i32x4; };   // raw E2M1, 32 values

template <int FMT, int TM, int TN, typename C>
__device__ __forceinline__ void load_frags(const uint8_t* As, const uint8_t* Bs, int ks, int wm, int wn, int lane,
                                           typename Frag<FMT>::A (&af)[TM], typename Frag<FMT>::B (&bf)[TN]) {
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * TM * 32 + tm * 32 + l32;
    if constexpr (FMT == F_BF16) {
      af[tm] = *(const bf16x8*)(As + r * C::A_ROW + (swz<C::A_ROW>(r, ks * 2 + g) << 4));
    } else if constexpr (FMT == F_NVFP4) {
      // 64-K group ks: lane group g holds K [32g, 32g+32) of the group
      af[tm] = *(const i32x4*)(As + r * C::A_ROW + (swz<C::A_ROW>(r, ks * 2 + g) << 4));
    } else {
      // 8-bit A operand: register bytes 0-15 hold K [16g, 16g+16) of the
      // 64-wide K-step, bytes 16-31 hold K [32+16g, +16)
      const i32x4 lo = *(const i32x4*)(As + r * C::A_ROW + (swz<C::A_ROW>(r, ks * 4 + g) << 4));
      const i32x4 hi = *(const i32x4*)(As + r * C::A_ROW + (swz<C::A_ROW>(r, ks * 4 + 2 + g) << 4));
      af[tm] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int nf = wn * TN + tn;
    if constexpr (FMT == F_BF16) {
      bf[tn] = *(const bf16x8*)(Bs + (nf * C::STEPS + ks) * 1024 + lane * 16);
    } else if constexpr (FMT == F_MXFP8) {
      const uint8_t* f = Bs + (nf * C::STEPS + ks) * C::FRAG + lane * 16;
      const i32x4 lo = *(const i32x4*)f, hi = *(const i32x4*)(f + 1024);
      bf[tn] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else if constexpr (FMT == F_NVFP4) {
      bf[tn] = *(const i32x4*)(Bs + (nf * C::STEPS + ks) * C::FRAG + lane * 16);
    } else {
      const i32x4 v = *(const i32x4*)(Bs + (nf * C::STEPS + ks) * C::FRAG + lane * 16);
      bf[tn] = (i32x8){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    }
  }
}

template <int V> using IC = std::integral_constant<int, V>;

// f(IC<I>) for I = LO .. HI-1, unrolled at compile time.
template <int LO, int HI, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (LO < HI) {
    f(IC<LO>{});
    static_for<LO + 1, HI>(f);
  }
}

// Scheduling hints.  interleave_hint: READS LDS reads spread between MFMAS
// MFMAs, one read followed by its share of the MFMAs.
template <int I, int READS, int MFMAS>
__device__ __forceinline__ void interleave_hint() {
  if constexpr (I < READS) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    constexpr int q = ((I + 1) * MFMAS) / READS - (I * MFMAS) / READS;
    if constexpr (q > 0) __builtin_amdgcn_sched_group_barrier(0x008, q, 0);
    interleave_hint<I + 1, READS, MFMAS>();
  }
}

// boundary_hint: after the barrier, the next stage's first reads are spread
// over the first half of the last K-step's MFMAs and the copies of stage s+2
// over the second half.
template <int I, int READS, int MFMAS, int VMEM>
__device__ __forceinline__ void boundary_mfma_hint() {
  if constexpr (I < MFMAS) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int H = MFMAS / 2 > 0 ? MFMAS / 2 : 1;
    if constexpr (I < H) {
      constexpr int r = ((I + 1) * READS) / H - (I * READS) / H;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    } else {
      constexpr int J = I - H, H2 = MFMAS - H > 0 ? MFMAS - H : 1;
      constexpr int v = ((J + 1) * VMEM) / H2 - (J * VMEM) / H2;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);
    }
    boundary_mfma_hint<I + 1, READS, MFMAS, VMEM>();
  }
}

template <int READS, int MFMAS, int VMEM>
__device__ __forceinline__ void boundary_hint() {
  boundary_mfma_hint<0, READS, MFMAS, VMEM>();
}

// LAYER 1: the L1 GEMM (A rows gathered from x through sorted_slot; the
// activation and L2-input quantisation in the epilogue); 2: the L2 GEMM;
// 3: one K part of a split L1 GEMM (gathered A rows, raw float32 output).
template <int FMT, int BM, int LAYER>
__global__ void __launch_bounds__(GEMM_THREADS, (TileGeom<FMT, BM>::OCC))
    __attribute__((amdgpu_waves_per_eu((TileGeom<FMT, BM>::OCC), (TileGeom<FMT, BM>::OCC)))) k_gemm(const GemmArgs p) {
  using G = TileGeom<FMT, BM>;
  using C = typename G::C;
  using FA = typename Frag<FMT>::A;
  using FB = typename Frag<FMT>::B;
  constexpr int TM = G::TM, TN = G::TN;
  constexpr int READS = FMT == F_NVFP4 ? TM + TN : TM * (FMT == F_BF16 ? 1 : 2) + TN * (FMT == F_MXFP8 ? 2 : 1);
  // scale registers held per stage: NVFP4 two dwords of 4 E4M3 A scales per
  // row block and one dword of B scales per column block; MX one UE8M0 byte
  // per row block and K-step (A), and per column block one 16-bit word with
  // the bytes of both K-steps of its 128-K layout stage (B), the byte chosen
  // by the MFMA's scale op_sel, so no VALU work splits the word
  constexpr int SA_N = C::NV ? 2 * TM : C::STEPS * TM;
  constexpr int SB_N = TN;
  // L1 passes the weights as the MFMA's first operand: accumulator element v
  // of lane l is then intermediate column 8 (v / 4) + 4 (l / 32) + v % 4 of
  // its 32-column block for sorted row l % 32, so a row's 32 columns sit in
  // two lanes and the L2-input quantiser's block maxima need one cross-lane
  // step per 16 values.  L2 and the K-split L1 keep the rows on the first
  // operand (a lane's 16 values lie in one column, stored as runs of a row).
  constexpr bool WFIRST = LAYER == 1;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  // the wave index as a wave-uniform (scalar) value
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5,
            l32 = lane & 31;
  const int wm = w / G::WN, wn = w % G::WN;
  const int NB = p.N / GEMM_BN;
  // Work units: the first `full` tiles whole, then `tail` tiles as kt K
  // parts each (unit full + ks * tail + i: part ks of tile full + i, stages
  // [ks * nst / kt, (ks + 1) * nst / kt)).  A uniform K split (ksplit) has
  // full = 0, tail = tiles; an L2 with a split tail splits only the
  // persistent grid's partial last round (tail_split).
  const int nst = p.K / C::KSTAGE;   // stages of a whole tile
  const int tiles = p.meta[0] * NB;
  constexpr bool TAILBUF = LAYER == 2 && FMT == F_BF16;   // float32 rows: a split tail is possible
  int full = 0, tail = tiles, kt = p.ksplit;
  if (TAILBUF && p.tail_kmax > 1) {
    const TailSplit ts = tail_split(tiles, (int)gridDim.x, p.tail_kmax, p.tail_units, nst);
    full = ts.full;
    tail = ts.tail;
    kt = ts.kt;
  }
  const int total = full + tail * kt;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xj = blockIdx.x >> 3;

  // A rows and weight fragments are copied through buffer resources with
  // 32-bit offsets (a per-lane offset and a per-stage uniform one), so a copy
  // needs no 64-bit address arithmetic.  A rows gathered from x (L1, K-split
  // L1) are addressed from x itself; the L2's rows and the BF16 stage-blocked
  // rows from the tile's first row.  The host keeps x and each expert's
  // weights below 4 GiB.
  constexpr bool BLOCKED = FMT == F_BF16;               // A rows stage-blocked, in sorted order
  constexpr bool TILE_A = BLOCKED || LAYER == 2;        // A resource per tile
  const __amdgpu_buffer_rsrc_t ra_x = buf_rsrc(p.a);

  // One tile: an expert, a 256-column block and a BLOCK_M-row block, with the
  // per-lane source offsets of its A rows.
  struct TileCtx {
    int e, nb, m0;
    int s0;                 // first K stage of the work unit
    int ks;                 // its K split
    int par;                // its row buffer
    int ns;                 // its K stages
    int tidx;               // split tail: its tile's index in the tail, else -1
    uint32_t a_off[G::A_INSTR];
    __amdgpu_buffer_rsrc_t ra;   // TILE_A: the tile's A rows
    __amdgpu_buffer_rsrc_t rw;   // the tile's N block of the weights (layout stage 0)
    const uint8_t* wsf;
    const uint8_t* asf;     // MX: the wave's A-scale plane at the tile's first row (stage 0)
    const uint8_t* bsf;     // MX: the wave's B-scale column blocks (layout stage 0)
  };
  auto make_tile = [&](int uu) __attribute__((always_inline)) -> TileCtx {
    TileCtx t;
    int u;
    if (uu < full) {
      u = uu;
      t.ks = 0;
      t.ns = nst;
      t.tidx = -1;
    } else {
      const int v = uu - full;
      t.ks = v / tail;
      const int i = v - t.ks * tail;
      u = full + i;
      t.ns = nst / kt;
      t.tidx = TAILBUF && p.tail_kmax > 1 ? i : -1;
    }
    t.s0 = t.ks * t.ns;
    // tile -> (expert, n block, m block).  The tiles of expert e are
    // [mb0 * NB, mb1 * NB) with [mb0, mb1) its BLOCK_M blocks, so u / NB is
    // one of e's blocks, whose tile_info record names e, mb0 and mb1 - mb0.
    // Scalar loads: the copies in flight are not waited for.
    const i32x4 ti = sload4(p.tile_info + 4 * (u / NB));
    const int e = ti[0], mb0 = ti[1], mcount = ti[2];
    const int local = u - mb0 * NB;
    t.e = e;
    t.nb = local / mcount;
    t.m0 = (mb0 + local % mcount) * BM;
    // per-lane A row offsets for the LDS-DMA copies: lane l of copy i fills
    // LDS row r = A_RPI * (copy index) + l / A_CPR, physical chunk l % A_CPR
    // (rows wrap modulo BM when a wave has more lanes than rows).  L1: the
    // wave's A_WROWS contiguous rows' slots come in by scalar loads and each
    // lane picks its rows' token.
    int sv[G::A_WROWS];
    if constexpr (LAYER != 2 && !BLOCKED) {
      const int32_t* base = p.sorted_slot + t.m0 + (w * G::A_WROWS) % BM;
      if constexpr (G::A_WROWS == 8) {
        const i32x8 v = sload8(base);
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = v[j];
      } else {
#pragma unroll
        for (int h = 0; h < G::A_WROWS / 16; ++h) {
          const i32x16 v = sload16(base + 16 * h);
#pragma unroll
          for (int j = 0; j < 16; ++j) sv[16 * h + j] = v[j];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G::A_INSTR; ++i) {
      const int rl = (w * G::A_INSTR + i) * G::A_RPI + lane / G::A_CPR;
      const int r = rl % BM;
      const uint32_t chunk = (uint32_t)swz<C::A_ROW>(rl, lane % G::A_CPR) << 4;
      if constexpr (BLOCKED) {
        // row r of the tile's block of the [M / BM][K / 32][BM][64 B] layout
        t.a_off[i] = (uint32_t)r * 64 + chunk;
      } else if constexpr (LAYER != 2) {
        int sl = sv[i * G::A_RPI];
#pragma unroll
        for (int k = 1; k < G::A_RPI; ++k)
          if (lane / G::A_CPR == k) sl = sv[i * G::A_RPI + k];
        t.a_off[i] = (uint32_t)(sl >= 0 ? sl / p.kk : 0) * (uint32_t)p.a_ld + chunk;
      } else {
        t.a_off[i] = (uint32_t)r * (uint32_t)p.a_ld + chunk;
      }
    }
    if constexpr (BLOCKED)
      t.ra = buf_rsrc(p.a + (int64_t)(t.m0 / BM) * (p.K / 32) * BM * 64);
    else if constexpr (LAYER == 2)
      t.ra = buf_rsrc(p.a + (int64_t)t.m0 * p.a_ld);
    {
      constexpr int LSK = C::KSTAGE / C::STEPS * C::KS_PER_L;   // K per layout stage
      t.rw = buf_rsrc(p.w + (int64_t)e * p.w_expert_bytes +
                      (FMT == F_BF16 ? (int64_t)t.nb * (p.K / LSK) * 8 * (C::KS_PER_L * C::FRAG)
                                     : (int64_t)t.nb * 8 * (C::KS_PER_L * C::FRAG)));
    }
    t.wsf = C::SCALED ? p.w_sf + (int64_t)e * p.w_sf_expert_bytes : nullptr;
    if constexpr (C::SCALED && !C::NV) {
      t.asf = p.a_sf + t.m0 + (int64_t)(w % (C::KSTAGE / 32)) * p.a_sf_ld;
      t.bsf = t.wsf + (int64_t)(t.nb * 8 + 2 * w) * 128;
    }
    return t;
  };

  // Copy instruction c (0 <= c < CPS) of stage s into LDS stage buffer st:
  // A rows, then weight fragments, then block scales.
  auto copy = [&](auto ci, const TileCtx t, int s, uint8_t* st) __attribute__((always_inline)) {
    constexpr int c = decltype(ci)::value;
    constexpr int SC = G::A_INSTR + G::B_INSTR;   // first scale copy
    if constexpr (c < G::A_INSTR) {
      constexpr uint32_t SSTRIDE = FMT == F_BF16 ? BM * C::A_ROW : C::A_ROW;   // bytes per stage of a row
      buf2lds16(TILE_A ? t.ra : ra_x, t.a_off[c], (uint32_t)(t.s0 + s) * SSTRIDE, st + (w * G::A_INSTR + c) * 1024);
    } else if constexpr (c < SC) {
      // weight fragments: LDS [32-row block][K-step of the stage][FRAG];
      // global BF16 [N block][layout stage][32-row block of 8][KS_PER_L
      // K-steps][FRAG], others [layout stage][32-row block][KS_PER_L][FRAG]
      // the tile's weight resource (t.rw), a term per stage (layout stage
      // S / R of the tile's N block, K-step (S % R) * STEPS within it) and a
      // term per copy (32-row block nf, K-step ksl of the stage, 1 KiB piece)
      const int q = w * G::B_INSTR + (c - G::A_INSTR);
      const int nf = q / G::B_FRAGS_PER_NF, piece = q % G::B_FRAGS_PER_NF;
      const int ksl = piece / (C::FRAG / 1024), sub = piece % (C::FRAG / 1024);
      constexpr unsigned R = C::KS_PER_L / C::STEPS;   // kernel stages per layout stage
      const unsigned S = (unsigned)(t.s0 + s);
      const uint32_t lstride = FMT == F_BF16 ? 8u * C::KS_PER_L * C::FRAG
                                             : (uint32_t)(p.N / 32) * (C::KS_PER_L * C::FRAG);
      const uint32_t sterm = (S / R) * lstride + (S % R) * (C::STEPS * C::FRAG);
      const uint32_t cterm = nf * (C::KS_PER_L * C::FRAG) + ksl * C::FRAG + sub * 1024;
      // 32-row tiles (the BLOCK_M of decode-sized batches, where an expert
      // rarely has more than one M block) stream their weights: each line is
      // read by one workgroup once, so it is copied non-temporally and does
      // not displace lines that are still to be read.  Taller tiles share
      // weight blocks between an expert's M blocks and keep them cached.
      buf2lds16<(BM <= 32)>(t.rw, cterm + (uint32_t)lane * 16, sterm, st + G::A_STAGE + q * 1024);
    } else if constexpr (!C::NV && c == SC) {
      // A scales: K block w % (blocks per stage) of this stage, the plane's
      // bytes of rows m0 .. m0+255 (rows past the tile are not read)
      // (the tile's base t.asf plus NBLK planes per stage; plane strides fit
      // 32 bits)
      constexpr unsigned NBLK = C::KSTAGE / 32;
      const uint64_t soff = (uint64_t)(unsigned)(t.s0 + s) * (NBLK * (unsigned)p.a_sf_ld);
      __builtin_amdgcn_global_load_lds(t.asf + soff + lane * 4,
                                       (lds_void*)(st + G::A_STAGE + G::B_STAGE + w * 256), 4, 0, 0);
    } else if constexpr (!C::NV) {
      // B scales: [layout stage][32-row block][64 lanes x 2 K-steps]; wave w
      // copies column blocks 2w and 2w + 1 (256 contiguous bytes)
      const uint64_t soff = (uint64_t)((unsigned)(t.s0 + s) / G::SPL) * ((unsigned)(p.N / 32) * 128u);
      __builtin_amdgcn_global_load_lds(t.bsf + soff + lane * 4,
                                       (lds_void*)(st + G::A_STAGE + G::B_STAGE + G::A_SF_STAGE + w * 256), 4, 0,
                                       0);
    } else if constexpr (c < SC + 2) {
      // NVFP4 A scales: K blocks w and w + 4 of this stage's 8, the planes'
      // bytes of rows m0 .. m0+255
      constexpr int h = c - SC;
      const int64_t blk = (int64_t)(t.s0 + s) * 8 + w + 4 * h;
      __builtin_amdgcn_global_load_lds(p.a_sf + blk * p.a_sf_ld + t.m0 + lane * 4,
                                       (lds_void*)(st + G::A_STAGE + G::B_STAGE + (w + 4 * h) * 256), 4, 0, 0);
    } else {
      // NVFP4 B scales of this wave's TN blocks: [stage][32-row block][64 lanes x 4]
      const int byte = (lane * 16) % (TN * 256);
      const uint8_t* src = t.wsf + ((int64_t)(t.s0 + s) * (p.N / 32) + t.nb * 8 + wn * TN + byte / 256) * 256 + byte % 256;
      g2lds16(src, st + G::A_STAGE + G::B_STAGE + G::A_SF_STAGE + w * 1024);
    }
  };
  // copies [LO, HI) of stage s of tile t into buffer buf
  auto issue = [&](auto lo, auto hi, const TileCtx t, int s, int buf) __attribute__((always_inline)) {
    uint8_t* st = smem + buf * G::STAGE;
    static_for<decltype(lo)::value, decltype(hi)::value>([&](auto ci) __attribute__((always_inline)) { copy(ci, t, s, st); });
  };

  f32x16 acc[TM][TN];   // the tile's accumulators (AGPRs)
  // Block scales of a stage (in buffer st).  MX: for each K-step, the one
  // UE8M0 byte each lane hands its scaled MFMA for A: the byte of the lane's
  // row in K block 2 * (K-step) + g of the stage, read as a byte so no VALU
  // work waits on the LDS read; for B the lane's 16-bit word of its 128-K
  // layout stage, whose byte kl (the K-step, or for 64-K stages the stage
  // parity) the MFMA selects.  NVFP4: two E4M3 A scales per row and 64-K
  // group, a dword of four B scales per column block.
  auto read_scales = [&](const uint8_t* st, uint32_t (&sa)[SA_N], uint32_t (&sb)[SB_N])
      __attribute__((always_inline)) {
    if constexpr (C::SCALED) {
      const uint8_t* Asf = st + G::A_STAGE + G::B_STAGE;
      const uint8_t* Bsf = Asf + G::A_SF_STAGE;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = wm * TM * 32 + tm * 32 + l32;
        if constexpr (C::NV) {
          // 64-K group ks: lane group g takes K blocks 4ks + 2g and + 1
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            sa[ks * TM + tm] = (uint32_t)Asf[(4 * ks + 2 * g) * 256 + r] |
                               ((uint32_t)Asf[(4 * ks + 2 * g + 1) * 256 + r] << 8);
        } else {
          // K-step ks takes K block 2ks + g of the stage
#pragma unroll
          for (int ks = 0; ks < C::STEPS; ++ks) sa[ks * TM + tm] = Asf[(2 * ks + g) * 256 + r];
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if constexpr (C::NV) {
          sb[tn] = *(const uint32_t*)(Bsf + w * 1024 + tn * 256 + lane * 4);
        } else {
          sb[tn] = *(const uint16_t*)(Bsf + (wn * TN + tn) * 128 + lane * 2);
        }
      }
    }
  };
  // MFMAs of K-step ks of a stage; kl: the byte of the B-scale words the MX
  // K-step takes (op_sel of the weights' scale)
  auto mfmas = [&](auto ksc, auto klc, const FA (&af)[TM], const FB (&bf)[TN], const uint32_t (&sa)[SA_N],
                   const uint32_t (&sb)[SB_N]) __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
    constexpr int kl = decltype(klc)::value;
    if constexpr (C::NV) {
      // 64-K group ks: four 16-wide K-steps; sub-step j takes the lane's
      // values [8j, 8j+8) (K = 32g + 8j + i), in block 2g + j/2 of the
      // group: byte 2g + j/2 of the row's A-scale dword, byte 2ks + j/2 of
      // the lane's B-scale dword
      // the row's (column's) two block scales of the group as FP16, one
      // convert each: A bytes 0, 1 of its dword, B bytes 2ks, 2ks + 1
      f16x2 pa[TM], pb[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) pa[tm] = nv_scales<false>(sa[ks * TM + tm]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) pb[tn] = nv_scales<ks == 1>(sb[tn]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {            // the two 16-blocks of the lane's 32 values
        f16x2 ssa[TM], ssb[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) ssa[tm] = h ? pa[tm].yy : pa[tm].xx;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) ssb[tn] = h ? pb[tn].yy : pb[tn].xx;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * h + jj;
          f16x8 a8[TM], b8[TN];
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) a8[tm] = nvfp4_to_f16x8(af[tm][j], ssa[tm]);
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) b8[tn] = nvfp4_to_f16x8(bf[tn][j], ssb[tn]);
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
              acc[tm][tn] = WFIRST ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b8[tn], a8[tm], acc[tm][tn], 0, 0, 0)
                                   : __builtin_amdgcn_mfma_f32_32x32x16_f16(a8[tm], b8[tn], acc[tm][tn], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if constexpr (FMT == F_BF16 && WFIRST) {
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[tn], af[tm], acc[tm][tn], 0, 0, 0);
          } else if constexpr (FMT == F_BF16) {
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
          } else if constexpr (WFIRST) {
            // operand formats: weights FP4 (MXFP4) or FP8, activations FP8
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[tn], af[tm], acc[tm][tn], FMT == F_MXFP4 ? 4 : 0, 0, kl, (int)sb[tn], 0,
                (int)sa[ks * TM + tm]);
          } else {
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[tm], bf[tn], acc[tm][tn], 0, FMT == F_MXFP4 ? 4 : 0, 0, (int)sa[ks * TM + tm], kl,
                (int)sb[tn]);
          }
        }
      }
    }
  };

  // Stages rotate through NBUF LDS buffers.  Each stage's wait + barrier
  // sits just before its last K-step, so the next stage's first fragments
  // are read while the last K-step's MFMAs run; by that barrier every wave
  // has read all of the stage's buffer.  A stage's copies go out in two
  // windows of about half the copies each, spread over the MFMAs: the K-step
  // window of stage s (its K-steps before the barrier) and the boundary
  // window (the last K-step, after the barrier).  Two schedules:
  // - late: stage s+NBUF-1 is copied into the buffer stage s-1 left, its
  //   copies [0, LAST) in stage s's K-step window, [LAST, CPS) in its
  //   boundary window;
  // - early (EARLY): the buffer is refilled right after its barrier: copies
  //   [0, PA) of stage s+NBUF go into stage s's buffer in stage s's boundary
  //   window, the rest [PA, CPS) in stage s+1's K-step window.  Each copy
  //   has half a stage longer to land, with the same copies per window.
  // The 128- and 256-row MXFP8 tiles, whose weight stream waits on HBM
  // (the M blocks of an expert share each weight line in L2, so few
  // distinct lines are in flight), run early; the others measured faster
  // late.  The last stages of a tile issue the first stages of the
  // workgroup's next tile (when K has enough stages), so the next tile
  // starts without a pipeline fill and its copies overlap this tile's
  // epilogue; with no next tile, the copies re-copy the last stage into a
  // buffer that is not read again (stage indices clamped), which keeps the
  // copy count per window fixed for the vmcnt bookkeeping.
  constexpr bool EARLY = FMT == F_MXFP8 && BM >= 128;
  constexpr int LAST = (C::STEPS - 1) * G::CPS / C::STEPS;   // copies in a K-step window
  constexpr int PA = G::CPS - LAST;                          // copies in a boundary window
  static_assert((G::NBUF - 1) * G::CPS < 64, "vmcnt holds 6 bits");
  constexpr int CHAIN_MIN = G::NBUF - 1 + (EARLY ? 1 : 0);   // stages a tile needs to hand over
  // work unit of round r: in a full round each XCD takes a contiguous run
  // (M blocks sharing a weight block meet in one L2); a partial last round
  // is dealt out across the XCDs in turn, so a small launch uses them all
  const int NW = (int)gridDim.x;
  auto unit = [&](int r) __attribute__((always_inline)) -> int {
    const int base = r * NW;
    return base + NW <= total ? base + xcd * per_xcd + xj : base + (int)blockIdx.x;
  };
  // Per-row data of tile t into its row buffer, 4 bytes per row, 64 rows per
  // wave: NVFP4 L1 token scales, L2 (and K-split L1) slots, read by the
  // tile's epilogue.  Issued a tile ahead, so it is older than that tile's
  // first copies and the waits before its K loop cover it.
  constexpr bool ROWDMA = LAYER != 1 || C::NV;
  auto row_dma = [&](const TileCtx& t) __attribute__((always_inline)) {
    if constexpr (ROWDMA) {
      const uint8_t* src = LAYER == 1 ? (const uint8_t*)p.row_scale : (const uint8_t*)p.sorted_slot;
      if (w * 64 < BM && (BM >= 64 || lane < BM))
        __builtin_amdgcn_global_load_lds(src + ((int64_t)t.m0 + w * 64 + lane) * 4,
                                         (lds_void*)(smem + G::ROWS_OFF + t.par * 1024 + w * 256), 4, 0, 0);
    }
  };
  const int u0 = unit(0);
  TileCtx ta, tb;
  int cur = 0;           // LDS buffer of the current stage
  bool primed = false;   // the current tile's first NBUF-1 stages are issued
  if (u0 < total) {
    ta = make_tile(u0);
    ta.par = 0;
    row_dma(ta);
  }
  for (int r = 0; unit(r) < total; ++r) {
    const int un = unit(r + 1);
    const bool has_next = un < total;
    if (has_next) {
      tb = make_tile(un);
      tb.par = ta.par ^ 1;
    }
    // the next tile's first stages are copied during this one's last
    const bool chain_next = has_next && ta.ns >= CHAIN_MIN && tb.ns >= CHAIN_MIN;
    const int nstages = ta.ns;
    lds_barrier();        // every wave is done with the previous tile's LDS
    if (has_next) row_dma(tb);
    if (!primed) {
      // a tile the previous one could not prefetch: drain that tile's
      // clamped re-copies, then issue stages 0 .. NBUF-2 (early: and the
      // boundary-window copies of stage NBUF-1)
      wait_vmcnt0();
#pragma unroll
      for (int i = 0; i + 1 < G::NBUF; ++i) {
        const int bi = cur + i < G::NBUF ? cur + i : cur + i - G::NBUF;
        issue(IC<0>{}, IC<G::CPS>{}, ta, i < nstages ? i : nstages - 1, bi);
      }
      if constexpr (EARLY) {
        constexpr int i = G::NBUF - 1;
        issue(IC<0>{}, IC<PA>{}, ta, i < nstages ? i : nstages - 1, cur == 0 ? i : cur - 1);
      }
    }
    // stage 0 has landed
    wait_vmcnt<(G::NBUF - 2) * G::CPS + (EARLY ? PA : 0)>();
    lds_barrier();

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    FA af[2][TM];
    FB bfr[2][TN];
    uint32_t sa4[SA_N] = {}, sb2[SB_N] = {}, sa4n[SA_N] = {}, sb2n[SB_N] = {};
    {
      const uint8_t* st0 = smem + cur * G::STAGE;
      read_scales(st0, sa4, sb2);
      load_frags<FMT, TM, TN, C>(st0, st0 + G::A_STAGE, 0, wm, wn, lane, af[0], bfr[0]);
    }
    constexpr int MF = TM * TN * (C::NV ? 4 : 1);   // MFMAs per K-step
    // One stage.  RB: register set holding the stage's first K-step
    // fragments (K-step ks uses set (RB + ks) & 1; the next stage's first
    // fragments go to set (RB + STEPS) & 1).  LASTC: the tile's last stage
    // (no next stage to wait for or read).  K-step window: copies of stage
    // s + NBUF - 1 (tf / js: of this tile, else of the next) into the buffer
    // stage s - 1 left; boundary window: the same stage's into the same
    // buffer (late), or stage s + NBUF's (tfb / jsb) into this stage's
    // buffer (early).
    // CURC: the stage's buffer when known at compile time (else -1: cur).
    auto stage_body = [&](auto rbc, auto lastc, auto curc, const TileCtx& tf, int js, const TileCtx& tfb, int jsb)
        __attribute__((always_inline)) {
      constexpr int RB = decltype(rbc)::value;
      constexpr bool LASTS = decltype(lastc)::value;
      constexpr int CURC = decltype(curc)::value;
      const int cb = CURC >= 0 ? CURC : cur;
      const uint8_t* st = smem + cb * G::STAGE;
      const int fill = CURC >= 0 ? (CURC == 0 ? G::NBUF - 1 : CURC - 1) : (cur == 0 ? G::NBUF - 1 : cur - 1);
      static_for<0, C::STEPS - 1>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value;
        constexpr int K0 = EARLY ? PA : 0;
        constexpr int lo = K0 + ks * LAST / (C::STEPS - 1), hi = K0 + (ks + 1) * LAST / (C::STEPS - 1);
        constexpr int r0 = (RB + ks) & 1, r1 = (RB + ks + 1) & 1;
        load_frags<FMT, TM, TN, C>(st, st + G::A_STAGE, ks + 1, wm, wn, lane, af[r1], bfr[r1]);
        issue(IC<lo>{}, IC<hi>{}, tf, js, fill);
        mfmas(IC<ks>{}, IC<ks>{}, af[r0], bfr[r0], sa4, sb2);
        boundary_hint<READS, MF, hi - lo>();
      });
      constexpr int rl = (RB + C::STEPS - 1) & 1, rn = (RB + C::STEPS) & 1;
      const int nxt = CURC >= 0 ? (CURC + 1) % G::NBUF : (cur + 1 == G::NBUF ? 0 : cur + 1);
      // stage boundary: stage s+1 has landed (this wave's later copies may
      // still be in flight: late, stages s+2 .. s+NBUF-2 and the K-step
      // window's part of s+NBUF-1; early, stages s+2 .. s+NBUF-1) and every
      // wave is done reading stage s.  Early, the last stage also needs the
      // barrier: its boundary window writes its own buffer.
      if constexpr (!LASTS) wait_vmcnt<EARLY ? (G::NBUF - 2) * G::CPS : (G::NBUF - 3) * G::CPS + LAST>();
      if constexpr (!LASTS || EARLY) lds_barrier();
      if constexpr (!LASTS) {
        const uint8_t* nx = smem + nxt * G::STAGE;
        read_scales(nx, sa4n, sb2n);
        load_frags<FMT, TM, TN, C>(nx, nx + G::A_STAGE, 0, wm, wn, lane, af[rn], bfr[rn]);
      }
      if constexpr (EARLY)
        issue(IC<0>{}, IC<PA>{}, tfb, jsb, cb);
      else
        issue(IC<LAST>{}, IC<G::CPS>{}, tf, js, fill);
      // with one K-step per stage, RB is the stage's parity: the half of
      // the 128-K layout stage whose B-scale byte the K-step takes
      mfmas(IC<C::STEPS - 1>{}, IC<C::STEPS == 1 ? (RB & 1) : C::STEPS - 1>{}, af[rl], bfr[rl], sa4, sb2);
      boundary_hint<LASTS ? 0 : READS + (C::SCALED ? SA_N + SB_N : 0), MF, PA>();
      if constexpr (!LASTS) {
#pragma unroll
        for (int tm = 0; tm < SA_N; ++tm) sa4[tm] = sa4n[tm];
#pragma unroll
        for (int tn = 0; tn < SB_N; ++tn) sb2[tn] = sb2n[tn];
      }
      cur = nxt;
    };
    // Stage s.  TAILC: it may copy stages past this tile's last (the next
    // tile's, or clamped re-copies); the stages before nt copy only this
    // tile's own stages, with no selects.
    auto stage = [&](auto rbc, auto lastc, auto tailc, int s, auto curc) __attribute__((always_inline)) {
      const int sf = s + G::NBUF - 1;
      const int sfb = sf + (EARLY ? 1 : 0);
      if constexpr (decltype(tailc)::value) {
        const bool own = sf < nstages;
        const int js = own ? sf : (chain_next ? sf - nstages : nstages - 1);
        // copy source (a uniform branch: selects would make the tiles addressable)
        TileCtx tf = ta;
        if (!own && chain_next) tf = tb;
        const bool ownb = sfb < nstages;
        const int jsb = ownb ? sfb : (chain_next ? sfb - nstages : nstages - 1);
        TileCtx tfb = ta;
        if (!ownb && chain_next) tfb = tb;
        stage_body(rbc, lastc, curc, tf, js, tfb, jsb);
      } else {
        stage_body(rbc, lastc, curc, ta, sf, ta, sfb);
      }
    };
    const int nt = nstages - (G::NBUF - 1 + (EARLY ? 1 : 0));
    using F_ = std::false_type;
    using T_ = std::true_type;
    using RT_ = IC<-1>;   // buffer index at run time
    if constexpr (C::STEPS % 2 == 0) {
      // own-tile stages: until the ring is back at buffer 0, then in groups
      // of NBUF whose buffers are compile-time constants (no ring-index or
      // LDS-address arithmetic per stage), then the rest
      int s = 0;
      for (; s < nt && cur != 0; ++s) stage(IC<0>{}, F_{}, F_{}, s, RT_{});
      for (; s + G::NBUF <= nt; s += G::NBUF)
        static_for<0, G::NBUF>([&](auto jc) __attribute__((always_inline)) {
          stage(IC<0>{}, F_{}, F_{}, s + decltype(jc)::value, jc);
        });
      for (; s < nt && s + 1 < nstages; ++s) stage(IC<0>{}, F_{}, F_{}, s, RT_{});
      for (; s + 1 < nstages; ++s) stage(IC<0>{}, F_{}, T_{}, s, RT_{});
      stage(IC<0>{}, T_{}, T_{}, nstages - 1, RT_{});
    } else {
      int s = 0;
      for (; s + 1 < nt && s + 2 < nstages; s += 2) {
        stage(IC<0>{}, F_{}, F_{}, s, RT_{});
        stage(IC<1>{}, F_{}, F_{}, s + 1, RT_{});
      }
      for (; s + 2 < nstages; s += 2) {
        stage(IC<0>{}, F_{}, T_{}, s, RT_{});
        stage(IC<1>{}, F_{}, T_{}, s + 1, RT_{});
      }
      if (s + 1 < nstages) {
        stage(IC<0>{}, F_{}, T_{}, s, RT_{});
        stage(IC<1>{}, T_{}, T_{}, s + 1, RT_{});
      } else {
        stage(IC<0>{}, T_{}, T_{}, s, RT_{});
      }
    }
    primed = chain_next;
    const int e = ta.e, nb = ta.nb, m0 = ta.m0;

    // ---- epilogue.  Accumulator element v of lane l is row
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 and column l % 32 of its 32x32 tile.
    // L1: activation and L2-input quantisation here.  L2, and L1 with K
    // split (LAYER 3): float32 rows per slot (LAYER 3: raw accumulators in
    // the kernel's column order, summed and activated by k_l1_finish).
    if constexpr (LAYER == 1) {
      const float wgs = C::NV ? __builtin_bit_cast(float, sload(p.w_gs + e)) : 1.0f;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = m0 + wm * TM * 32 + tm * 32 + l32;   // the lane's sorted row
        // NVFP4 accumulators carry neither the token nor the expert scale
        const float alpha = C::NV ? ((const float*)(smem + G::ROWS_OFF + ta.par * 1024))[row - m0] * wgs : 1.0f;
#pragma unroll
        for (int pp = 0; pp < TN / 2; ++pp) {
          const int icol0 = nb * (GEMM_BN / 2) + (wn * (TN / 2) + pp) * 32;
          float a[16];
          // the clamp's presence is chosen once per 16 activations
          auto act16 = [&](auto clampc) __attribute__((always_inline)) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float gv = acc[tm][2 * pp][v], uv = acc[tm][2 * pp + 1][v];
              if constexpr (C::NV) {
                gv *= alpha;
                uv *= alpha;
              }
              a[v] = act_swiglu_c<decltype(clampc)::value>(gv, uv, p);
            }
          };
          if (p.has_clamp)
            act16(std::true_type{});
          else
            act16(std::false_type{});
          store_l2_input_rows<FMT>(a, row, icol0, g, p);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // NVFP4 L2: w2's expert scale times the L2 input's global scale
      const float alpha2 = C::NV && LAYER == 2 ? __builtin_bit_cast(float, sload(p.w_gs + e)) * p.l2_scale : 1.0f;
      // the slots of the lane's 16 rows of each row block, from the row
      // buffer (one row block at a time)
      const int32_t* rslot = (const int32_t*)(smem + G::ROWS_OFF + ta.par * 1024);
      // block-scaled L2 with K unsplit: BF16 rows (the output dtype the
      // combine reads), stored non-temporally (written once, read once by
      // the combine, so they need not displace the weights from the
      // caches); else float32 rows (BF16 layers, K parts, split L1).  MODE
      // 0: float32, 1: BF16, 2: chosen per row (BF16 layers and the 256-row
      // NVFP4 L2), 3: BF16 with fewer than 2^32 elements in o, so a row's
      // offset is a 24-bit product (slot < 2^24 as N >= 256), not a 64-bit
      // one.  The other block-scaled L2s choose once per tile
      auto l2_epilogue = [&](auto modec) __attribute__((always_inline)) {
        constexpr int MODE = decltype(modec)::value;
        const bool o16 = MODE == 2 ? FMT != F_BF16 && LAYER == 2 && p.o_bf16 : MODE == 1 || MODE == 3;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          // split tail: this row block's rows in the tile's part
          float* const tail_base =
              TAILBUF && ta.tidx >= 0
                  ? p.o_tail + ((int64_t)(ta.tidx * kt + ta.ks) * BM + wm * TM * 32 + tm * 32) * GEMM_BN +
                        wn * TN * 32 + l32
                  : nullptr;
          int slots[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int4 s4 = *(const int4*)(rslot + wm * TM * 32 + tm * 32 + 8 * q + 4 * g);
            slots[4 * q] = s4.x;
            slots[4 * q + 1] = s4.y;
            slots[4 * q + 2] = s4.z;
            slots[4 * q + 3] = s4.w;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int slot = slots[v];
            if (slot < 0) continue;
            const int64_t col = (int64_t)slot * p.N + nb * GEMM_BN + wn * TN * 32 + l32;
            if (o16) {
              uint16_t* orow =
                  MODE == 3 ? (uint16_t*)p.o + (__umul24((uint32_t)slot, (uint32_t)p.N) +
                                                (uint32_t)(nb * GEMM_BN + wn * TN * 32 + l32))
                            : (uint16_t*)p.o + col;
#pragma unroll
              for (int tn = 0; tn < TN; ++tn)
                __builtin_nontemporal_store(bf16_rne(C::NV ? acc[tm][tn][v] * alpha2 : acc[tm][tn][v]),
                                            orow + tn * 32);
            } else {
              // by slot; a part of a split-tail tile: [tail tile][part][row][column]
              float* orow = p.o + ta.ks * p.o_split + col;
              if (TAILBUF && ta.tidx >= 0)
                orow = tail_base + (8 * (v / 4) + 4 * g + v % 4) * GEMM_BN;
#pragma unroll
              for (int tn = 0; tn < TN; ++tn)
                orow[tn * 32] = C::NV && LAYER == 2 ? acc[tm][tn][v] * alpha2 : acc[tm][tn][v];
            }
          }
        }
      };
      // (the 256-row NVFP4 L2 has no registers to spare for the extra copies)
      if constexpr (FMT != F_BF16 && LAYER == 2 && !(C::NV && BM == 256)) {
        if (p.o_bf16 && p.o_split < (int64_t{1} << 32))
          l2_epilogue(IC<3>{});
        else if (p.o_bf16)
          l2_epilogue(IC<1>{});
        else
          l2_epilogue(IC<0>{});
      } else {
        l2_epilogue(IC<2>{});
      }
    }
    if (has_next) ta = tb;
  }
  wait_vmcnt0();   // no LDS-DMA copy outlives the workgroup
}

// Finish of a K-split L1 GEMM: per slot, the float32 parts of its gate and up
// columns summed in part order (NVFP4: times the token and expert scales, as
// the unsplit epilogue does), then the same activation and L2-input
// quantisation as the unsplit epilogue, into the slot's sorted row.  One wave
// per (slot, 64 intermediate columns); a dropped slot has no row.
template <int FMT>
__global__ void __launch_bounds__(64) k_l1_finish(const GemmArgs p, const int32_t* __restrict__ slot_row,
                                                  const int32_t* __restrict__ tile_expert, int bm) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x, l32 = lane & 31;
  const int icol = blockIdx.y * 64 + lane;
  const int nc = (icol >> 5) * 64 + (icol & 31);   // gate column; up is 32 further
  // the parts (at most 4, the split rule's limit) are loaded together with
  // the slot's row, so the launch waits out one load latency, not two; a
  // dropped slot's parts, never written, are loaded and not used
  float gp[4], up[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < p.ksplit) {
      const float* row = p.o + ks * p.o_split + (int64_t)s * p.N;
      gp[ks] = row[nc];
      up[ks] = row[nc + 32];
    }
  }
  const int m = slot_row[s];
  if (m < 0) return;
  float g = 0.0f, u = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < p.ksplit) {
      g += gp[ks];
      u += up[ks];
    }
  }
  if constexpr (FMT == F_NVFP4) {
    const float alpha = p.a_tok[s / p.kk] * p.w_gs[tile_expert[m / bm]];
    g *= alpha;
    u *= alpha;
  }
  store_l2_input<FMT>(act_swiglu(g, u, p), m, icol, l32, p);
}

void launch_l1_finish(int fmt, const GemmArgs& a, const int32_t* slot_row, const int32_t* tile_expert, int bm,
                      int S, hipStream_t st) {
  const dim3 grid((unsigned)S, (unsigned)(a.inter / 64));
  switch (fmt) {
    case F_BF16: hipLaunchKernelGGL(k_l1_finish<F_BF16>, grid, dim3(64), 0, st, a, slot_row, tile_expert, bm); break;
    case F_MXFP8: hipLaunchKernelGGL(k_l1_finish<F_MXFP8>, grid, dim3(64), 0, st, a, slot_row, tile_expert, bm); break;
    case F_MXFP4: hipLaunchKernelGGL(k_l1_finish<F_MXFP4>, grid, dim3(64), 0, st, a, slot_row, tile_expert, bm); break;
    default: hipLaunchKernelGGL(k_l1_finish<F_NVFP4>, grid, dim3(64), 0, st, a, slot_row, tile_expert, bm); break;
  }
}

// ------------------------------------------------------------------ host side
template <int FMT, int BM, int LAYER>
static hipError_t set_lds_attr() {
  return hipFuncSetAttribute((const void*)k_gemm<FMT, BM, LAYER>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             TileGeom<FMT, BM>::LDS);
}

template <int FMT, int BM>
static hipError_t init_fmt_bm() {
  hipError_t e = set_lds_attr<FMT, BM, 1>();
  if (e != hipSuccess) return e;
  if ((e = set_lds_attr<FMT, BM, 3>()) != hipSuccess) return e;
  return set_lds_attr<FMT, BM, 2>();
}

template <int FMT>
static hipError_t init_fmt() {
  hipError_t e;
  if ((e = init_fmt_bm<FMT, 32>()) != hipSuccess) return e;
  if ((e = init_fmt_bm<FMT, 64>()) != hipSuccess) return e;
  if ((e = init_fmt_bm<FMT, 128>()) != hipSuccess) return e;
  return init_fmt_bm<FMT, 256>();
}

hipError_t gemm_init(int /*device*/) {
  hipError_t e;
  if ((e = init_fmt<F_BF16>()) != hipSuccess) return e;
  if ((e = init_fmt<F_MXFP8>()) != hipSuccess) return e;
  if ((e = init_fmt<F_MXFP4>()) != hipSuccess) return e;
  return init_fmt<F_NVFP4>();
}

template <int FMT, int BM>
static hipError_t launch_fmt_bm(int layer, const GemmArgs& a, int grid, hipStream_t st) {
  constexpr int lds = TileGeom<FMT, BM>::LDS;
  // the persistent grid: OCC workgroups per CU (grid is a multiple of 8, so
  // the XCD round-robin of workgroups stays exact)
  const int g = grid * TileGeom<FMT, BM>::OCC;
  if (layer == 1 && a.ksplit > 1)
    hipLaunchKernelGGL((k_gemm<FMT, BM, 3>), dim3(g), dim3(GEMM_THREADS), lds, st, a);
  else if (layer == 1)
    hipLaunchKernelGGL((k_gemm<FMT, BM, 1>), dim3(g), dim3(GEMM_THREADS), lds, st, a);
  else
    hipLaunchKernelGGL((k_gemm<FMT, BM, 2>), dim3(g), dim3(GEMM_THREADS), lds, st, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(int layer, int bm, const GemmArgs& a, int grid, hipStream_t st) {
  switch (bm) {
    case 32: return launch_fmt_bm<FMT, 32>(layer, a, grid, st);
    case 64: return launch_fmt_bm<FMT, 64>(layer, a, grid, st);
    case 128: return launch_fmt_bm<FMT, 128>(layer, a, grid, st);
    default: return launch_fmt_bm<FMT, 256>(layer, a, grid, st);
  }
}

template <int FMT>
static int workgroups_fmt(int bm, int grid) {
  switch (bm) {
    case 32: return grid * TileGeom<FMT, 32>::OCC;
    case 64: return grid * TileGeom<FMT, 64>::OCC;
    case 128: return grid * TileGeom<FMT, 128>::OCC;
    default: return grid * TileGeom<FMT, 256>::OCC;
  }
}

int gemm_workgroups(int fmt, int bm, int grid) {
  switch (fmt) {
    case F_BF16: return workgroups_fmt<F_BF16>(bm, grid);
    case F_MXFP8: return workgroups_fmt<F_MXFP8>(bm, grid);
    case F_MXFP4: return workgroups_fmt<F_MXFP4>(bm, grid);
    default: return workgroups_fmt<F_NVFP4>(bm, grid);
  }
}

hipError_t launch_gemm(int fmt, int layer, int bm, const GemmArgs& a, int grid, hipStream_t st) {
  switch (fmt) {
    case F_BF16: return launch_fmt<F_BF16>(layer, bm, a, grid, st);
    case F_MXFP8: return launch_fmt<F_MXFP8>(layer, bm, a, grid, st);
    case F_MXFP4: return launch_fmt<F_MXFP4>(layer, bm, a, grid, st);
    case F_NVFP4: return launch_fmt<F_NVFP4>(layer, bm, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
