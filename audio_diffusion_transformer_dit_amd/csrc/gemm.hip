// Projections of the H3 DiT block on gfx950 MFMA: out = A W^T with A [M][K] (tokens x in),
// W [N][K] (out x in) ([DD] "h3.c 的核心设计" and "int8 量化": QKV, attention output, FC1, FC2
// in bf16 or int8 with per-token / per-channel / per-1024-group scales).
//
// Tiling: a workgroup owns a BM x BN output tile split over a WGM x WGN grid of waves, each
// wave a grid of 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16 or v_mfma_i32_32x32x32_i8; both
// read 16 bytes of K per lane, so one LDS layout serves both).  K advances in 128-byte slices
// (full cache lines per row) that travel global -> VGPR -> LDS.  Chunk c of row r sits at LDS
// slot c ^ ((r >> 1) & 7): the 16 lanes of one LDS read phase (16 rows, one chunk) cover all
// 64 banks.  Fragment reads of the next 16-byte K step overlap the MFMAs of the current one.
// The main shape is 256 x 256, in one of two forms:
//  * bf16: 4 waves (one per SIMD) of 128 x 128, accumulators in AGPRs.  Measured on gfx950 the
//    fragment reads out of LDS are what holds the matrix pipe back, and a 128 x 128 wave tile
//    reads a third fewer LDS bytes per MFMA than 128 x 64.  With no second wave to cover
//    stalls the schedule is explicit: slice k+1's LDS stores and slice k+2's loads are spread
//    between the MFMAs of slice k, and the per-slice barrier sits before the last K step so
//    that the next slice's first fragments are read under that step's MFMAs.
//  * int8 (and the 256 x 128 shape): 8 waves (two per SIMD) of 128 x 64 (the grouped int8
//    FC2: 4-wave 128 x 128 tiles of 64 x 64, two workgroups per CU); while slice k is
//    multiplied, slice k+1 is stored to the other LDS stage at the top of the iteration and
//    the loads of slice k+3 are spread between the MFMAs, so each load has more than a whole
//    iteration to arrive.
// Rows past M read as zeros (buffer range check).  The epilogue stages the bf16 tile in LDS
// and writes 16-byte row chunks (or, for V, 16-byte token chunks of V^T).  Workgroups are
// dealt round-robin to the 8 XCDs; the tile order is remapped so that each XCD sweeps a
// contiguous band of tiles, 8 tile-rows at a time, sharing A and W in its L2.
#include "common.hpp"

namespace h3 {

constexpr int GKB = 128;        // bytes of K per slice and row

struct GemmP {
  const uint8_t *a;
  const uint8_t *w;
  int64_t M, N, K;
  int hm_hd;
  const float *a_scale;
  int a_group;
  const float *w_scale;
  void *out;
  const float *cos_t, *sin_t;
  int heads, hd;
  uint16_t *oq, *ok, *ov;
  int ldv;
  int tiles_m, tiles_n;
  // split-K of the last, partial round: tiles [n_dp, tiles_m*tiles_n) are computed as `split`
  // K segments of kt_seg slices each, whose fp32 / int32 partial tiles go to `part`; a second
  // launch (the FIX instantiation, one workgroup per split tile) sums them in segment order
  // and runs the epilogue
  int n_dp, split, kt_seg;
  uint8_t *part;
};

template <int BM, int BN, int WGM, int WGN>
struct GemmCfg {
  static constexpr int NW = WGM * WGN;                  // waves
  static constexpr int NT = NW * 64;                    // threads
  static constexpr int FM = BM / WGM / 32;              // 32-row MFMA blocks per wave
  static constexpr int FN = BN / WGN / 32;              // 32-col MFMA blocks per wave
  static constexpr int STAGE = (BM + BN) * GKB;         // bytes per LDS slice
  static constexpr int LA = BM / (8 * NW);              // loads per lane per slice (A)
  static constexpr int LW = BN / (8 * NW);              // loads per lane per slice (W)
  static constexpr int CPITCH = BN * 2 + 16;            // bytes per row of the staged C tile
  static constexpr int CTILE = BM * CPITCH;
  static constexpr int LDS = (2 * STAGE > CTILE) ? 2 * STAGE : CTILE;
  static_assert(LA >= 1 && LW >= 1 && FM >= 1 && FN >= 1, "tile shape");
};

// Workgroups are dealt round-robin to the 8 XCDs: renumber a range of n launch indices so that
// each XCD gets a contiguous run of work items.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  return (n & 7) == 0 ? (b & 7) * (n >> 3) + (b >> 3) : b;
}

// tile index -> (tile row, tile column), 8 tile rows at a time
__device__ __forceinline__ void tile_coords(int b, int &tm, int &tn, int tiles_m, int tiles_n) {
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = b / per_group;
  const int first = g * GROUP;
  const int gsize = min(tiles_m - first, GROUP);
  const int r = b - g * per_group;
  tm = first + r % gsize;
  tn = r / gsize;
}

__device__ __forceinline__ u32x4 lds_frag(const uint8_t *base, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(base + row * GKB + ((chunk ^ ((row >> 1) & 7)) << 4));
}

// out_kind: H3DIT_OUT_*.  GROUPED: int8 FC2 with per-(row, group) activation scales.
// HM: A is the head-major attention output [K/hd][M][hd] (bf16 only).  FIX: the split-K fixup
// launch (sums partial tiles and runs the epilogue; its own kernel so that profiles separate it).
template <int BM, int BN, int WGM, int WGN, bool INT8, int OUT, bool GROUPED, bool HM, bool FIX>
__global__ __launch_bounds__(64 * WGM * WGN, (GROUPED && WGM * WGN == 4) ? 2 : 1) void k_gemm(GemmP p) {
  using C = GemmCfg<BM, BN, WGM, WGN>;
  constexpr int FM = C::FM, FN = C::FN, NW = C::NW, NT = C::NT, LA = C::LA, LW = C::LW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];

  // work item: a whole tile, one K segment of a split tile, or (fixup) the sum of a split tile
  int tile, seg = -1;
  const int KT = (int)(p.K * (INT8 ? 1 : 2) / GKB);
  int kt0 = 0, kt1 = KT;
  if (FIX) {
    tile = p.n_dp + (int)blockIdx.x;
  } else if ((int)blockIdx.x < p.n_dp) {
    tile = xcd_remap((int)blockIdx.x, p.n_dp);
  } else {
    const int n_units = (int)gridDim.x - p.n_dp;
    const int u = xcd_remap((int)blockIdx.x - p.n_dp, n_units);
    tile = p.n_dp + u / p.split;
    seg = u % p.split;
    kt0 = seg * p.kt_seg;
    kt1 = kt0 + p.kt_seg;
  }
  int tm, tn;
  tile_coords(tile, tm, tn, p.tiles_m, p.tiles_n);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  constexpr int esz = INT8 ? 1 : 2;
  const uint32_t a_bytes = (uint32_t)(p.M * p.K * esz), w_bytes = (uint32_t)(p.N * p.K * esz);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, a_bytes), rw = make_rsrc(p.w, w_bytes);

  // Per-lane load offsets.  A slice of the tile is (BM + BN) rows x 128 B; lanes take it in
  // 1 KiB blocks of 8 rows (8 consecutive lanes = one row's 8 chunks), so every global load
  // instruction reads whole 128-byte lines.  Block i of wave w covers rows (i*NW + w)*8 .. +7.
  // Within a lane all blocks share the row-in-block and chunk, and (NW even) the
  // swizzle too, so each operand needs one per-lane offset; the block stride and the slice
  // offset go into the scalar offset of the buffer load.
  static_assert(NW % 2 == 0, "blocks of one lane share the swizzle when the block stride is a multiple of 16 rows");
  const int rl = lane >> 3, cl = lane & 7;
  static_assert(!(HM && INT8), "head-major input is bf16");
  constexpr bool hm = HM;
  const int r0 = wid * 8 + rl;                         // row of block 0
  const int sw = (cl ^ ((r0 >> 1) & 7)) << 4;          // swizzled 16-byte slot (same for every block)
  const uint32_t a_voff = hm ? (uint32_t)((m0 + r0) * p.hm_hd * 2 + cl * 16) : (uint32_t)((m0 + r0) * p.K * esz + cl * 16);
  const uint32_t w_voff = (uint32_t)((n0 + r0) * p.K * esz + cl * 16);
  const uint32_t a_bstride = hm ? (uint32_t)(NW * 8 * p.hm_hd * 2) : (uint32_t)(NW * 8 * p.K * esz);
  const uint32_t w_bstride = (uint32_t)(NW * 8 * p.K * esz);
  const uint32_t lds0 = (uint32_t)(r0 * GKB + sw);     // LDS byte offset of block 0 (A); blocks step NW*1 KiB
  // Offset of K slice kt inside an A row, without branches: head-major bf16 input places
  // element k at (k / hd) * (M*hd*2) + (k % hd) * 2 bytes past the row start; token-major is
  // the same formula with shift 31, head stride 0 and a full mask (k * 2 bytes).
  const uint32_t hm_head = hm ? (uint32_t)(p.M * p.hm_hd * 2) : 0u;
  const uint32_t hm_shift = hm ? (p.hm_hd == 128 ? 7u : 6u) : 31u;
  const uint32_t hm_mask = hm ? (uint32_t)(p.hm_hd - 1) : 0xFFFFFFFFu;

  // Slices travel global -> registers -> LDS through two register sets (the loop forms below
  // say which slices they hold when).
  constexpr int NL = LA + LW;                       // 16-byte loads per lane per slice
  u32x4 stage_reg[2][NL];
  auto load_one = [&](u32x4 *dst, int kt, int li) {
    const uint32_t kb = (uint32_t)kt * GKB;   // byte offset of the slice inside a W row
    if (li < LA) {
      const uint32_t kel = kb >> 1;           // a slice never crosses a head
      const uint32_t ka = INT8 ? kb : (kel >> hm_shift) * hm_head + ((kel & hm_mask) << 1);
      dst[li] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff, ka + li * a_bstride, 0));
    } else {
      dst[li] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff, kb + (li - LA) * w_bstride, 0));
    }
  };
  auto store_slice = [&](const u32x4 *src, int kt) {
    uint8_t *st = smem + (kt & 1) * C::STAGE + lds0;
#pragma unroll
    for (int li = 0; li < NL; li++)
      *reinterpret_cast<u32x4 *>(st + (li < LA ? li * NW * 1024 : BM * GKB + (li - LA) * NW * 1024)) = src[li];
  };

  using AccT = typename std::conditional<INT8, i32x16, f32x16>::type;
  AccT acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = AccT{0};
  f32x16 sum[GROUPED ? FM : 1][GROUPED ? FN : 1];
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++) sum[i][j] = f32x16{0};
  }
  const int kt_per_group = GROUPED ? p.a_group * esz / GKB : 0;
  const int n_groups = GROUPED ? (int)(p.K / p.a_group) : 0;
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(p.a_scale, GROUPED ? (uint32_t)(p.M * n_groups * 4) : 0u);
  const uint32_t sc_voff =
      (uint32_t)((m0 + wm * (BM / WGM) + 4 * (lane >> 5)) * n_groups * 4);   // this lane's first row

  const int arow0 = wm * (BM / WGM) + (lane & 31);
  const int brow0 = wn * (BN / WGN) + (lane & 31);
  const int hsel = lane >> 5;
  auto read_step = [&](const uint8_t *sa, int ks, u32x4 *fa, u32x4 *fb) {
    const uint8_t *sb = sa + BM * GKB;
#pragma unroll
    for (int i = 0; i < FM; i++) fa[i] = lds_frag(sa, arow0 + 32 * i, 2 * ks + hsel);
#pragma unroll
    for (int j = 0; j < FN; j++) fb[j] = lds_frag(sb, brow0 + 32 * j, 2 * ks + hsel);
  };

  // partial tile of (split tile, segment): each lane's 16 accumulators of block (i, j) are 64
  // contiguous bytes; a wave's block is 4 KiB
  auto part_ptr = [&](int sg, int i, int j) {
    const int64_t slot = (int64_t)(tile - p.n_dp) * p.split + sg;
    return reinterpret_cast<i32x4 *>(p.part + slot * (BM * BN * 4) + ((wid * FM + i) * FN + j) * 4096 + lane * 64);
  };
  if constexpr (!GROUPED && FIX) {
    // sum of the segments' partial tiles, in segment order.  (Vectors are reinterpreted
    // whole: clang's __builtin_bit_cast of a single ext_vector element reads element 0.)
    for (int sg = 0; sg < p.split; sg++)
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
          const i32x4 *src = part_ptr(sg, i, j);
          i32x16 bits;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const i32x4 v = src[q];
#pragma unroll
            for (int e = 0; e < 4; e++) bits[4 * q + e] = v[e];
          }
          const AccT val = __builtin_bit_cast(AccT, bits);
          acc[i][j] = sg == 0 ? val : acc[i][j] + val;
        }
  } else {
  if constexpr (NW == 4 && !GROUPED) {
    // One wave per SIMD, 128 x 128 each (accumulators in AGPRs): a third fewer LDS bytes per
    // MFMA than 8 waves of 128 x 64.  Iteration kt: MFMA steps 0..3 of slice kt from stage
    // kt&1 with fragments read one step ahead; the register set holding slice kt+1 goes to
    // stage (kt+1)&1 during steps 0 and 1, and the loads of slice kt+2 into the other set are
    // spread over the iteration.
    // The barrier sits before step 3, whose fragments are already in registers; the step-0
    // fragments of slice kt+1 are read right after it, under step 3's MFMAs.
    // LDS store li follows MFMA 2 li of the iteration (steps 0 and 1), global load li follows
    // MFMA 4 li + 1 (spread over all four steps)
    constexpr int NSTEP = FM * FN;
    static_assert(2 * (NL - 1) < 3 * NSTEP && 4 * (NL - 1) + 1 < 4 * NSTEP, "store / load placement");
    u32x4 fa[2][FM], fb[2][FN];
    auto store_one = [&](const u32x4 *src, int kt, int li) {
      uint8_t *st = smem + (kt & 1) * C::STAGE + lds0;
      *reinterpret_cast<u32x4 *>(st + (li < LA ? li * NW * 1024 : BM * GKB + (li - LA) * NW * 1024)) = src[li];
    };
#pragma unroll
    for (int li = 0; li < NL; li++) load_one(stage_reg[0], kt0, li);
    store_slice(stage_reg[0], kt0);
#pragma unroll
    for (int li = 0; li < NL; li++) load_one(stage_reg[1], kt0 + 1 < kt1 ? kt0 + 1 : kt1 - 1, li);
    __syncthreads();
    read_step(smem + (kt0 & 1) * C::STAGE, 0, fa[0], fb[0]);
    auto iter1 = [&](int kt, const u32x4 *cur, u32x4 *nxt, auto steady) {
      constexpr bool STEADY = decltype(steady)::value;
      const bool more = STEADY || kt + 1 < kt1;
      const int ktl = kt + 2 < kt1 ? kt + 2 : kt1 - 1;
      const uint8_t *sa = smem + (kt & 1) * C::STAGE;
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        if (ks < 3) {
          read_step(sa, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        } else {
          __syncthreads();
          if (more) read_step(smem + ((kt + 1) & 1) * C::STAGE, 0, fa[0], fb[0]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
          for (int j = 0; j < FN; j++) {
            const int g = ks * NSTEP + i * FN + j;
            if constexpr (INT8)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa[ks & 1][i]),
                                                                __builtin_bit_cast(i32x4, fb[ks & 1][j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[ks & 1][i]),
                                                                  __builtin_bit_cast(bf16x8, fb[ks & 1][j]), acc[i][j], 0, 0, 0);
#pragma unroll
            for (int li = 0; li < NL; li++) {
              if (g == 2 * li && more) {
                __builtin_amdgcn_sched_barrier(0);
                store_one(cur, kt + 1, li);
                __builtin_amdgcn_sched_barrier(0);
              }
              if (STEADY && g == 4 * li + 1) {
                __builtin_amdgcn_sched_barrier(0);
                load_one(nxt, ktl, li);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
      }
    };
    using Steady = std::integral_constant<bool, true>;
    using Tail = std::integral_constant<bool, false>;
    int kt = kt0;
    for (; kt + 2 < kt1; kt += 2) {
      iter1(kt, stage_reg[1], stage_reg[0], Steady{});
      iter1(kt + 1, stage_reg[0], stage_reg[1], Steady{});
    }
    if (kt < kt1) iter1(kt, stage_reg[1], stage_reg[0], Tail{});
    if (kt + 1 < kt1) iter1(kt + 1, stage_reg[0], stage_reg[1], Tail{});
  } else {
  // prologue: slice kt0 into its LDS stage, slices kt0+1 and kt0+2 in the two register sets
#pragma unroll
  for (int li = 0; li < NL; li++) load_one(stage_reg[0], kt0, li);
  store_slice(stage_reg[0], kt0);
#pragma unroll
  for (int li = 0; li < NL; li++) load_one(stage_reg[1], kt0 + 1 < kt1 ? kt0 + 1 : kt1 - 1, li);
#pragma unroll
  for (int li = 0; li < NL; li++) load_one(stage_reg[0], kt0 + 2 < kt1 ? kt0 + 2 : kt1 - 1, li);
  __syncthreads();

  // Iteration kt: the register set holding slice kt+1 -> LDS stage (kt+1)&1 (last read in
  // iteration kt-1), then the same set receives slice kt+3, its loads spread between the MFMAs
  // of slice kt; the other set (slice kt+2) stays in flight for the whole iteration; barrier.
  // Past the end the loads repeat the last slice (in range, never stored).  sched_barrier
  // fixes the issue order.
  constexpr int NMMA = 4 * FM * FN;                 // MFMAs per slice; load li follows MFMA li*NMMA/NL
  auto iteration = [&](int kt, const u32x4 *cur, u32x4 *nxt, auto steady) {
    constexpr bool STEADY = decltype(steady)::value;
    if (STEADY || kt + 1 < kt1) store_slice(cur, kt + 1);
    const int ktl = kt + 3 < kt1 ? kt + 3 : kt1 - 1;
    const uint8_t *sa = smem + (kt & 1) * C::STAGE;
    u32x4 fa[2][FM], fb[2][FN];
    read_step(sa, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      if (ks < 3) read_step(sa, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
          const int m = (ks * FM + i) * FN + j;
          if constexpr (INT8)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa[ks & 1][i]),
                                                              __builtin_bit_cast(i32x4, fb[ks & 1][j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[ks & 1][i]),
                                                                __builtin_bit_cast(bf16x8, fb[ks & 1][j]), acc[i][j], 0, 0, 0);
#pragma unroll
          for (int li = 0; li < NL; li++)
            if (STEADY && li * NMMA / NL == m) {
              __builtin_amdgcn_sched_barrier(0);
              load_one(nxt, ktl, li);
              __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if constexpr (GROUPED) {
      if ((kt + 1) % kt_per_group == 0) {
        const int g = kt / kt_per_group;
        // one 32-row block at a time, so that only 16 row scales are live; scales are read
        // through a buffer resource (rows past M read 0): per-lane row base in the vector
        // offset, row-in-block and group in the scalar offset
#pragma unroll
        for (int i = 0; i < FM; i++) {
          float sc[16];
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const uint32_t soff = (uint32_t)(((32 * i + 8 * (r / 4) + (r % 4)) * n_groups + g) * 4);
            sc[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, sc_voff, soff, 0));
          }
#pragma unroll
          for (int r = 0; r < 16; r++)
#pragma unroll
            for (int j = 0; j < FN; j++) {
              sum[i][j][r] = sum[i][j][r] + (float)acc[i][j][r] * sc[r];
              acc[i][j][r] = 0;
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __syncthreads();
  };
  // two iterations per trip so that each register set is addressed statically
  using Steady = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  int kt = kt0;
  for (; kt + 2 < kt1; kt += 2) {
    iteration(kt, stage_reg[1], stage_reg[1], Steady{});
    iteration(kt + 1, stage_reg[0], stage_reg[0], Steady{});
  }
  if (kt < kt1) iteration(kt, stage_reg[1], stage_reg[1], Tail{});
  if (kt + 1 < kt1) iteration(kt + 1, stage_reg[0], stage_reg[0], Tail{});
  }
  wait_vmem();   // the register loads past the end
  if (!GROUPED && seg >= 0) {
    // one K segment of a split tile: store the raw partial, the fixup launch finishes it
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++) {
        i32x4 *dst = part_ptr(seg, i, j);
        const i32x16 bits = __builtin_bit_cast(i32x16, acc[i][j]);
#pragma unroll
        for (int q = 0; q < 4; q++) {
          i32x4 v;
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = bits[4 * q + e];
          dst[q] = v;
        }
      }
    return;
  }
  }

  // ---------------------------------------------------------------- epilogue
  // value of accumulator (i, j, r): row = m0 + wm*BM/WGM + 32 i + 8 (r/4) + 4 hsel + r%4,
  //                                 col = n0 + wn*BN/WGN + 32 j + lane%32
  const int rbase = wm * (BM / WGM) + 4 * hsel;
  const int cbase = wn * (BN / WGN) + (lane & 31);
  if constexpr (OUT == H3DIT_OUT_F32 || OUT == H3DIT_OUT_I32) {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int64_t row = m0 + rbase + 32 * i + 8 * (r / 4) + (r % 4);
          const int64_t col = n0 + cbase + 32 * j;
          if (row < p.M) {
            if constexpr (OUT == H3DIT_OUT_F32)
              reinterpret_cast<float *>(p.out)[row * p.N + col] = acc[i][j][r];
            else
              reinterpret_cast<int32_t *>(p.out)[row * p.N + col] = acc[i][j][r];
          }
        }
    return;
  } else {
    // registers -> bf16 tile in LDS
#pragma unroll
    for (int i = 0; i < FM; i++) {
      float sa_r[16];
      if constexpr (INT8 && !GROUPED) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int64_t row = m0 + rbase + 32 * i + 8 * (r / 4) + (r % 4);
          sa_r[r] = row < p.M ? p.a_scale[row] : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < FN; j++) {
        float sw = 0.0f;
        if constexpr (INT8) sw = p.w_scale[n0 + cbase + 32 * j];
#pragma unroll
        for (int r = 0; r < 16; r++) {
          float v;
          if constexpr (GROUPED)
            v = sum[i][j][r] * sw;
          else if constexpr (INT8)
            v = ((float)acc[i][j][r] * sa_r[r]) * sw;
          else
            v = acc[i][j][r];
          const int row = rbase + 32 * i + 8 * (r / 4) + (r % 4);
          const int col = cbase + 32 * j;
          *reinterpret_cast<uint16_t *>(smem + row * C::CPITCH + col * 2) = f2bf(v);
        }
      }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    constexpr int CH = BN / 8;  // 16-byte chunks per tile row
    // A thread stores chunk column tid % CH of rows tid / CH, + NT / CH, ... (NT is a multiple
    // of CH), so its column, and everything derived from it, is computed once.
    static_assert(NT % CH == 0, "whole tile rows per pass");
    const int c = tid % CH;
    if constexpr (OUT == H3DIT_OUT_QKV) {
      const int d = p.heads * p.hd;
      const int part = (int)(n0 / d);
      if (part < 2) {
        const int half = p.hd / 2;
        const int col = (int)(n0 % d) + c * 8;
        const int h = col / p.hd, i0 = col % p.hd;
        uint16_t *dst = (part == 0 ? p.oq : p.ok) + (int64_t)h * p.M * p.hd + i0;
        const float *cos_c = p.cos_t + i0 / 2, *sin_c = p.sin_t + i0 / 2;
        for (int r = tid / CH; r < BM; r += NT / CH) {
          const int64_t row = m0 + r;
          if (row >= p.M) break;   // later rows are past the end too
          float f[8], o[8];
          unpack8(*reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + c * 16), f);
          const float4 cs = *reinterpret_cast<const float4 *>(cos_c + row * half);
          const float4 sn = *reinterpret_cast<const float4 *>(sin_c + row * half);
          const float cc[4] = {cs.x, cs.y, cs.z, cs.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            o[2 * e] = f[2 * e] * cc[e] - f[2 * e + 1] * ss[e];
            o[2 * e + 1] = f[2 * e] * ss[e] + f[2 * e + 1] * cc[e];
          }
          *reinterpret_cast<u32x4 *>(dst + row * p.hd) = pack8(o);
        }
      } else {
        // V^T[h][i][vt_pos(m)]: one lane per (feature column, group of 16 tokens); inside a
        // group, tokens 0-3 | 8-11 | 4-7 | 12-15 land at slots 0-15 (two 16-byte stores)
        // (a thread keeps one feature column: NT is a multiple of BN)
        static_assert(NT % BN == 0, "whole feature columns per pass");
        const int cv = tid % BN;
        const int col = (int)(n0 % d) + cv;
        const int h = col / p.hd, i = col % p.hd;
        uint16_t *dst_c = p.ov + ((int64_t)h * p.hd + i) * p.ldv;
        for (int rb = tid / BN; rb < BM / 16; rb += NT / BN) {
          const int64_t row = m0 + rb * 16;
          if (row >= p.M) break;   // later groups are past the end too
          uint16_t v16[16];
#pragma unroll
          for (int e = 0; e < 16; e++)
            v16[vt_pos(e)] = *reinterpret_cast<const uint16_t *>(smem + (rb * 16 + e) * C::CPITCH + cv * 2);
          uint16_t *dst = dst_c + row;
          if (row + 16 <= p.M) {
            u32x4 v0, v1;
#pragma unroll
            for (int e = 0; e < 4; e++) {
              v0[e] = (uint32_t)v16[2 * e] | ((uint32_t)v16[2 * e + 1] << 16);
              v1[e] = (uint32_t)v16[8 + 2 * e] | ((uint32_t)v16[8 + 2 * e + 1] << 16);
            }
            reinterpret_cast<u32x4 *>(dst)[0] = v0;
            reinterpret_cast<u32x4 *>(dst)[1] = v1;
          } else {
#pragma unroll
            for (int e = 0; e < 16; e++)
              if (row + e < p.M) dst[vt_pos(e)] = v16[vt_pos(e)];
          }
        }
      }
    } else {
      uint16_t *out = reinterpret_cast<uint16_t *>(p.out) + n0 + c * 8;
      for (int r = tid / CH; r < BM; r += NT / CH) {
        const int64_t row = m0 + r;
        if (row >= p.M) break;   // later rows are past the end too
        u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + c * 16);
        if constexpr (OUT == H3DIT_OUT_GELU) {
          float f[8];
          unpack8(v, f);
#pragma unroll
          for (int e = 0; e < 8; e++) f[e] = gelu_tanh(f[e]);
          v = pack8(f);
        }
        *reinterpret_cast<u32x4 *>(out + row * p.N) = v;
      }
    }
  }
}

// Split-K sum for the bf16 output of the 4-wave 256 x 256 tile: the same segment-order fp32
// sums and bf16 rounding as the fixup instantiation of k_gemm, spread over one thread per
// 64-byte partial chunk (a lane's 16 accumulators of one 32 x 32 block) instead of one
// workgroup per tile, so that the partial tiles are read by the whole chip.
constexpr int SK_THREADS = 256;
__global__ __launch_bounds__(SK_THREADS) void k_splitk_bf16(GemmP p, int n_split) {
  constexpr int FM = 4, FN = 4, PER_TILE = 4 * FM * FN * 64;   // chunks per 256 x 256 tile
  const int64_t t = (int64_t)blockIdx.x * SK_THREADS + threadIdx.x;
  if (t >= (int64_t)n_split * PER_TILE) return;
  const int ti = (int)(t / PER_TILE), rem = (int)(t % PER_TILE);
  const int wid = rem / (FM * FN * 64), blk = (rem / 64) % (FM * FN), lane = rem % 64;
  const int i = blk / FN, j = blk % FN;
  float acc[16];
  for (int sg = 0; sg < p.split; sg++) {
    const int64_t slot = (int64_t)ti * p.split + sg;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.part + slot * (256 * 256 * 4) + (int64_t)blk * 4096 +
                                                       (int64_t)wid * FM * FN * 4096 + lane * 64);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const f32x4 v = src[q];
#pragma unroll
      for (int e = 0; e < 4; e++) acc[4 * q + e] = sg == 0 ? v[e] : acc[4 * q + e] + v[e];
    }
  }
  int tm, tn;
  tile_coords(p.n_dp + ti, tm, tn, p.tiles_m, p.tiles_n);
  const int wm = wid / 2, wn = wid % 2, hsel = lane >> 5;
  const int64_t col = (int64_t)tn * 256 + wn * 128 + 32 * j + (lane & 31);
  uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int64_t row = (int64_t)tm * 256 + wm * 128 + 32 * i + 8 * (r / 4) + 4 * hsel + (r % 4);
    if (row < p.M) out[row * p.N + col] = f2bf(acc[r]);
  }
}

// Final head with its AdaLN applied while the A tiles are loaded ([DD] "DiT 融合内核": the bf16
// head applies AdaLN as it loads its projection tiles, so no normalised copy of the rows is
// stored).  A 128 x 128 output tile per workgroup, 4 waves of 64 x 64, K in 64-element slices
// through one LDS stage.  Each A chunk of 8 values becomes bf16(((x - mean) * rstd) *
// (1 + scale) + shift) with the row statistics of launch_row_stats, exactly the values the
// row kernel would store, and the K order of the MFMAs is that of k_gemm, so the output
// equals the two-kernel form byte for byte.  The head is a small GEMM (N = latent channels).
constexpr int HT = 128;
__global__ __launch_bounds__(256) void k_head_gemm(int64_t M, int N, int K, const uint16_t *__restrict__ x,
                                                   const float *__restrict__ stats,
                                                   const uint16_t *__restrict__ shift,
                                                   const uint16_t *__restrict__ scale,
                                                   const uint16_t *__restrict__ w, uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[HT * GKB];
  __shared__ __attribute__((aligned(16))) uint8_t sb[HT * GKB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wm = wid >> 1, wn = wid & 1, hsel = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * HT;
  const int64_t n0 = (int64_t)blockIdx.y * HT;
  // loads: thread = (row r = tid / 8 + 32 i, 16-byte chunk c = tid % 8) of the slice, i < 4
  const int c = tid & 7, rb = tid >> 3;
  float mu[4], rs[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = m0 + rb + 32 * i;
    mu[i] = row < M ? stats[2 * row] : 0.0f;
    rs[i] = row < M ? stats[2 * row + 1] : 0.0f;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16{0};
  const int KT = K / 64;
  for (int kt = 0; kt < KT; kt++) {
    const int64_t k0 = (int64_t)kt * 64 + c * 8;
    u32x4 av[4], wv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t row = m0 + rb + 32 * i;
      av[i] = row < M ? *reinterpret_cast<const u32x4 *>(x + row * K + k0) : u32x4{0, 0, 0, 0};
      wv[i] = *reinterpret_cast<const u32x4 *>(w + (n0 + rb + 32 * i) * K + k0);
    }
    float sh[8], sc[8];
    unpack8(*reinterpret_cast<const u32x4 *>(shift + k0), sh);
    unpack8(*reinterpret_cast<const u32x4 *>(scale + k0), sc);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float v[8];
      unpack8(av[i], v);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float t = (v[e] - mu[i]) * rs[i];
        t = t * (1.0f + sc[e]) + sh[e];
        v[e] = t;
      }
      av[i] = pack8(v);
    }
    __syncthreads();   // the previous slice's fragments have been read
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = rb + 32 * i;
      const int slot = (c ^ ((r >> 1) & 7)) << 4;
      *reinterpret_cast<u32x4 *>(sa + r * GKB + slot) = av[i];
      *reinterpret_cast<u32x4 *>(sb + r * GKB + slot) = wv[i];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; i++) fa[i] = lds_frag(sa, wm * 64 + 32 * i + (lane & 31), 2 * ks + hsel);
#pragma unroll
      for (int j = 0; j < 2; j++) fb[j] = lds_frag(sb, wn * 64 + 32 * j + (lane & 31), 2 * ks + hsel);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                              __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r / 4) + 4 * hsel + (r % 4);
        const int64_t col = n0 + wn * 64 + 32 * j + (lane & 31);
        if (row < M) out[row * N + col] = f2bf(acc[i][j][r]);
      }
}

hipError_t launch_head_gemm(int64_t n, int c, int d, const uint16_t *x, const float *stats, const uint16_t *shift,
                            const uint16_t *scale, const uint16_t *w, uint16_t *out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (d % 64 || c % HT) return hipErrorInvalidValue;
  dim3 grid((unsigned)((n + HT - 1) / HT), (unsigned)(c / HT));
  k_head_gemm<<<grid, 256, 0, st>>>(n, c, d, x, stats, shift, scale, w, out);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, bool INT8, int OUT, bool GROUPED, bool HM>
static hipError_t run_gemm(GemmP p, const LinearPlan &pl, hipStream_t st) {
  p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)(p.N / BN);
  p.n_dp = pl.n_dp;
  p.split = pl.split;
  p.kt_seg = pl.kt_seg;
  const unsigned grid = (unsigned)(pl.n_dp + pl.n_split * pl.split);
  k_gemm<BM, BN, WGM, WGN, INT8, OUT, GROUPED, HM, false><<<grid, GemmCfg<BM, BN, WGM, WGN>::NT, 0, st>>>(p);
  if constexpr (!GROUPED && BN == 256) {
    if (pl.n_split > 0) {
      if constexpr (!INT8 && OUT == H3DIT_OUT_BF16 && WGM == 2 && WGN == 2) {
        const int64_t chunks = (int64_t)pl.n_split * 4 * 16 * 64;
        k_splitk_bf16<<<(unsigned)((chunks + SK_THREADS - 1) / SK_THREADS), SK_THREADS, 0, st>>>(p, pl.n_split);
      } else {
        k_gemm<BM, BN, WGM, WGN, INT8, OUT, GROUPED, HM, true>
            <<<(unsigned)pl.n_split, GemmCfg<BM, BN, WGM, WGN>::NT, 0, st>>>(p);
      }
    }
  }
  return hipGetLastError();
}

// Work plan of one projection on a chip of kCUs compute units holding one workgroup each.
// Candidates, costed in units of one 256 x 256 tile over the whole K (about K * 28 ps per
// byte of K row on gfx950):
//   256 x 256 tiles: rounds = ceil(tiles / kCUs);
//   256 x 128 tiles: rounds of half tiles, each ~0.52 of a whole one;
//   256 x 256 with the last partial round cut into `split` K segments: full rounds +
//     ceil(segments / kCUs) / split, plus the partial tiles: 16 us per round of segments
//     for their fp32 stores, then the sum.  A fixup launch of one workgroup per split tile
//     (measured on MI355X: ~50 us in all for 64 tiles x 4 segments) is modelled as 10 us +
//     6 us per segment; the chip-wide sum of the bf16 4-wave form reads the partials at
//     about 5 TB/s (13.6 us for 64 x 4 segments), modelled as 3 us + 0.05 us per segment.
//     Every bf16 plan is costed with the chip-wide sum, whatever the output form, so that the
//     plan depends only on shape and precision: a fused epilogue and its unfused sequence
//     accumulate K in the same segments.  Where the per-tile fixup runs instead (fp32, GELU
//     and rotary outputs) this under-costs it; at the block's shapes (2048-8192 tokens) it
//     selects the same plans as costing that fixup would.
// The grouped int8 FC2 uses 128 x 128 tiles (its second accumulator set does not fit 256 wide).
constexpr int kCUs = 256;

LinearPlan plan_linear(const h3dit_linear_args &a) {
  LinearPlan pl{};
  const bool i8 = a.precision == H3DIT_INT8;
  const bool grouped = i8 && a.a_group > 0;
  const int64_t d = (int64_t)a.heads * a.head_dim;
  const int KT = (int)(a.K * (i8 ? 1 : 2) / 128);
  bool wide = a.N % 256 == 0 && !grouped;
  if (a.out_kind == H3DIT_OUT_QKV && d % 256) wide = false;
  const int64_t tm = (a.M + 255) / 256;
  pl.split = 1;
  pl.kt_seg = KT;
  pl.n_split = 0;
  pl.part_bytes = 0;
  pl.bn = 128;
  pl.n_dp = (int)(tm * (a.N / 128));
  if (grouped) pl.n_dp = (int)((a.M + 127) / 128 * (a.N / 128));   // 128 x 128 tiles
  if (!wide) return pl;
  const int64_t tiles = tm * (a.N / 256), full = tiles / kCUs, rem = tiles % kCUs;
  const double t_tile_us = (double)KT * 128 * 0.0277 / 2;   // one 256 x 256 tile over the whole K
  const double c256 = (double)(full + (rem ? 1 : 0));
  const double c128 = (double)((2 * tiles + kCUs - 1) / kCUs) * 0.52;
  const bool chip_sum = !i8;
  double best = c256;
  int best_s = 1;
  for (int sp = 2; sp <= 8 && rem; sp++) {
    if (KT % sp || KT / sp < 2) continue;
    const int64_t seg_rounds = (rem * sp + kCUs - 1) / kCUs;
    const double sum_us = chip_sum ? 3.0 + 0.05 * (double)(rem * sp) : 10.0 + 6.0 * sp;
    const double cost = (double)full + (double)seg_rounds / sp + (16.0 * seg_rounds + sum_us) / t_tile_us;
    if (cost < best - 1e-9) {
      best = cost;
      best_s = sp;
    }
  }
  if (c128 < best - 1e-9) return pl;
  pl.bn = 256;
  pl.n_dp = (int)tiles;
  if (best_s == 1) return pl;
  pl.split = best_s;
  pl.kt_seg = KT / best_s;
  pl.n_split = (int)rem;
  pl.n_dp = (int)(tiles - rem);
  pl.part_bytes = (size_t)rem * best_s * 256 * 256 * 4;
  return pl;
}

template <bool INT8, int OUT, bool GROUPED, bool HM = false>
static hipError_t dispatch(const GemmP &p, const LinearPlan &pl, hipStream_t st) {
  if constexpr (GROUPED) {
    // two accumulator sets (int32 per group, fp32 across groups) per lane: 128 x 128 tiles of
    // 4 waves of 64 x 64, two workgroups per CU (1280 tiles at 4096 x 5120: whole rounds)
    return run_gemm<128, 128, 2, 2, INT8, OUT, GROUPED, false>(p, pl, st);
  } else {
    // bf16: four waves of 128 x 128; int8: eight waves of 128 x 64 (measured faster for int8)
    if (pl.bn == 256) {
      if constexpr (INT8) return run_gemm<256, 256, 2, 4, INT8, OUT, GROUPED, HM>(p, pl, st);
      else return run_gemm<256, 256, 2, 2, INT8, OUT, GROUPED, HM>(p, pl, st);
    }
    return run_gemm<256, 128, 4, 2, INT8, OUT, GROUPED, HM>(p, pl, st);
  }
}

size_t linear_workspace(const h3dit_linear_args &a) { return plan_linear(a).part_bytes; }

hipError_t launch_linear(const h3dit_linear_args &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const LinearPlan pl = plan_linear(a);
  if (pl.part_bytes > 0 && (a.workspace == nullptr || a.workspace_bytes < pl.part_bytes)) return hipErrorInvalidValue;
  GemmP p{};
  p.a = reinterpret_cast<const uint8_t *>(a.a);
  p.w = reinterpret_cast<const uint8_t *>(a.w);
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  p.hm_hd = a.a_headmajor_hd;
  p.a_scale = a.a_scale;
  p.a_group = a.a_group;
  p.w_scale = a.w_scale;
  p.out = a.out;
  p.cos_t = a.cos_t;
  p.sin_t = a.sin_t;
  p.heads = a.heads;
  p.hd = a.head_dim;
  p.oq = a.out_q;
  p.ok = a.out_k;
  p.ov = a.out_v;
  p.ldv = (int)vt_pitch(a.M);
  p.part = reinterpret_cast<uint8_t *>(a.workspace);
  const bool i8 = a.precision == H3DIT_INT8;
  if (i8 && a.a_group > 0) return dispatch<true, H3DIT_OUT_BF16, true>(p, pl, st);
  if (a.a_headmajor_hd > 0) {
    if (i8) return hipErrorInvalidValue;
    if (a.out_kind == H3DIT_OUT_BF16) return dispatch<false, H3DIT_OUT_BF16, false, true>(p, pl, st);
    if (a.out_kind == H3DIT_OUT_F32) return dispatch<false, H3DIT_OUT_F32, false, true>(p, pl, st);
    return hipErrorInvalidValue;
  }
  switch (a.out_kind) {
    case H3DIT_OUT_BF16:
      return i8 ? dispatch<true, H3DIT_OUT_BF16, false>(p, pl, st) : dispatch<false, H3DIT_OUT_BF16, false>(p, pl, st);
    case H3DIT_OUT_F32:
      return dispatch<false, H3DIT_OUT_F32, false>(p, pl, st);
    case H3DIT_OUT_I32:
      return dispatch<true, H3DIT_OUT_I32, false>(p, pl, st);
    case H3DIT_OUT_GELU:
      return i8 ? dispatch<true, H3DIT_OUT_GELU, false>(p, pl, st) : dispatch<false, H3DIT_OUT_GELU, false>(p, pl, st);
    case H3DIT_OUT_QKV:
      return i8 ? dispatch<true, H3DIT_OUT_QKV, false>(p, pl, st) : dispatch<false, H3DIT_OUT_QKV, false>(p, pl, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace h3
