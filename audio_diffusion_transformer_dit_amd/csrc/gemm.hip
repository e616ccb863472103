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
// The main shape is 256 x 256, in one of two wave layouts:
//  * bf16: 4 waves (one per SIMD) of 128 x 128, accumulators in AGPRs.  Measured on gfx950 the
//    fragment reads out of LDS are what holds the matrix pipe back, and a 128 x 128 wave tile
//    reads a third fewer LDS bytes per MFMA than 128 x 64.
//  * int8 (and the 256 x 128 shape): 8 waves (two per SIMD) of 128 x 64 (256 x 128: 64 x 64,
//    also the grouped int8 FC2).
// Where whole rounds of those tiles would leave the chip partly idle, the int8 projections can
// hand their last columns to a second launch of 128 x 128 tiles (8 waves of 64 x 32).
// One loop serves both, its schedule explicit: slice k+1's LDS stores and slice k+2's loads
// are spread between the MFMAs of slice k, and the per-slice barrier sits before the last K
// step so that the next slice's first fragments are read under that step's MFMAs.
// Rows past M read as zeros (buffer range check, see a_load).  The epilogue stages the bf16 tile in LDS
// and writes 16-byte row chunks (or, for V, 16-byte token chunks of V^T).  Workgroups are
// dealt round-robin to the 8 XCDs; the tile order is remapped so that each XCD sweeps a
// contiguous band of tiles, 8 tile-rows at a time, sharing A and W in its L2.
#include "common.hpp"

namespace h3 {

constexpr int GKB = 128;        // bytes of K per slice and row
// Tiles of the grouped int8 FC2 (two accumulator sets per lane: int32 within a group, fp32
// across groups): G_BM x G_BN, a G_WGM x G_WGN grid of waves of 64 x 64, one workgroup
// per CU; and the small GS_BM x GS_BN tile of eight waves of 64 x 32, which covers the last
// columns where whole rounds of the large tile would leave the chip partly idle (also for the
// ungrouped int8 projections after 256 x 256 tiles).  (Four waves of 64 x 64 on that tile, one
// per SIMD, took as long as a large tile.)
constexpr int G_BM = 256, G_BN = 128, G_WGM = G_BM / 64, G_WGN = 2;
constexpr int GS_BM = 128, GS_BN = 128, GS_WGM = GS_BM / 64, GS_WGN = 4;
// s_waitcnt immediate that waits for lgkmcnt == 0 only (gfx9 encoding: vmcnt bits 3:0 and 15:14
// at their maximum, expcnt bits 6:4 at 7, lgkmcnt bits 11:8 at 0)
constexpr int kLgkmZero = 0xC07F;

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
  int64_t n_lo;   // first output column of this launch (its tiles cover columns n_lo ..)
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

// Byte addressing of one 16-byte load of the A operand: block li of a lane whose block-0 row
// is tile row r0, 16-byte chunk cl, K slice kt.  The range check of a raw buffer load covers
// the vector offset (plus the instruction offset), not the scalar offset, so everything that
// depends on the row sits in the vector offset or in the resource: block li reads through a
// resource based li block strides further on with its record count shortened to match.
// Token-major A: a load returns zeros exactly when its row is >= M (voff >= nrec).  Head-major
// A (the attention output [K/hd][M][hd]): the slice's head offset goes into the vector offset
// too (one add per slice), so a row >= M of head h reads row (row - M) of head h + 1 (its sums
// are never stored) and past the last head the range check returns zeros.  Every load that is
// not masked stays inside [base, base + nrec), i.e. inside A.
struct ALoad {
  int64_t base;   // byte offset of the resource base from A
  int64_t nrec;   // bytes the resource covers (>= 0)
  uint32_t voff;  // per-lane vector offset
  uint32_t soff;  // wave-uniform scalar offset (the K position inside a row)
};
__host__ __device__ __forceinline__ ALoad a_load(int64_t M, int64_t K, int esz, int hm_hd, int nw, int64_t m0,
                                                 int r0, int cl, int li, int kt) {
  ALoad L;
  const int64_t rows_before = (int64_t)nw * 8 * li;   // rows of the blocks before block li
  const int64_t left = M - rows_before > 0 ? M - rows_before : 0;
  if (hm_hd) {
    const int64_t kel = (int64_t)kt * (GKB / 2);         // first element of the slice (bf16)
    const int64_t head = kel / hm_hd;
    const int64_t total = M * K * 2;
    L.base = rows_before * hm_hd * 2;
    L.nrec = total - L.base > 0 ? total - L.base : 0;
    L.voff = (uint32_t)((m0 + r0) * hm_hd * 2 + cl * 16 + head * M * hm_hd * 2);
    L.soff = (uint32_t)((kel % hm_hd) * 2);
  } else {
    L.base = rows_before * K * esz;
    L.nrec = left * K * esz;
    L.voff = (uint32_t)((m0 + r0) * K * esz + cl * 16);
    L.soff = (uint32_t)kt * GKB;
  }
  return L;
}

// Addressing of the group scale of grouped-FC2 accumulator row u + v + e, group g: u = m0 +
// 32 i + 8 q (the tile's part, wave-uniform), v = the wave's and lane's row offset, e < 4.
// The resource starts at scale (u, g) and holds (M - u) * n_groups - g scales; v + e goes into
// the vector offset.  A row >= M reads 0 (its sums are never stored); no read leaves the
// [M][n_groups] scale array.
struct ScLoad {
  int64_t base;   // first scale (element index) of the resource
  int64_t nrec;   // bytes the resource covers (>= 0)
  uint32_t voff;  // per-lane vector offset (bytes)
};
__host__ __device__ __forceinline__ ScLoad sc_load(int64_t M, int n_groups, int64_t u, int v, int e, int g) {
  ScLoad L;
  const int64_t left = (M - u) * n_groups - g;
  L.base = u * n_groups + g;
  L.nrec = left > 0 ? left * 4 : 0;
  L.voff = (uint32_t)((v + e) * n_groups * 4);
  return L;
}

__device__ __forceinline__ u32x4 lds_frag(const uint8_t *base, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(base + row * GKB + ((chunk ^ ((row >> 1) & 7)) << 4));
}

// out_kind: H3DIT_OUT_*.  GROUPED: int8 FC2 with per-(row, group) activation scales.
// HM: A is the head-major attention output [K/hd][M][hd] (bf16 only).  FIX: the split-K fixup
// launch (sums partial tiles and runs the epilogue; its own kernel so that profiles separate it).
template <int BM, int BN, int WGM, int WGN, bool INT8, int OUT, bool GROUPED, bool HM, bool FIX>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void k_gemm(GemmP p) {
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
  const int64_t m0 = (int64_t)tm * BM, n0 = p.n_lo + (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  constexpr int esz = INT8 ? 1 : 2;
  const uint32_t w_bytes = (uint32_t)(p.N * p.K * esz);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, w_bytes);

  // Per-lane load offsets.  A slice of the tile is (BM + BN) rows x 128 B; lanes take it in
  // 1 KiB blocks of 8 rows (8 consecutive lanes = one row's 8 chunks), so every global load
  // instruction reads whole 128-byte lines.  Block i of wave w covers rows (i*NW + w)*8 .. +7.
  // Within a lane all blocks share the row-in-block and chunk, and (NW even) the swizzle
  // too, so each operand needs one per-lane offset.  W rows are all inside the matrix (N is a
  // multiple of BN): the block stride and the slice offset go into the scalar offset.  A rows
  // may run past M: each block of A reads through its own resource (a_load).
  static_assert(NW % 2 == 0, "blocks of one lane share the swizzle when the block stride is a multiple of 16 rows");
  const int rl = lane >> 3, cl = lane & 7;
  static_assert(!(HM && INT8), "head-major input is bf16");
  constexpr bool hm = HM;
  const int hm_hd = hm ? p.hm_hd : 0;
  const int r0 = wid * 8 + rl;                         // row of block 0
  const int sw = (cl ^ ((r0 >> 1) & 7)) << 4;          // swizzled 16-byte slot (same for every block)
  const uint32_t a_voff = a_load(p.M, p.K, esz, hm_hd, NW, m0, r0, cl, 0, 0).voff;   // every block, head 0
  const uint32_t hm_head = hm ? (uint32_t)(p.M * p.hm_hd * 2) : 0u;                    // bytes per head
  const uint32_t hm_shift = hm ? (p.hm_hd == 128 ? 7u : 6u) : 0u;
  const uint32_t hm_mask = hm ? (uint32_t)(p.hm_hd - 1) : 0u;
  const uint32_t w_voff = (uint32_t)((n0 + r0) * p.K * esz + cl * 16);
  const uint32_t w_bstride = (uint32_t)(NW * 8 * p.K * esz);
  const uint32_t lds0 = (uint32_t)(r0 * GKB + sw);     // LDS byte offset of block 0 (A); blocks step NW*1 KiB
  auto a_rsrc = [&](int li, int kt) {
    const ALoad L = a_load(p.M, p.K, esz, hm_hd, NW, m0, r0, cl, li, kt);
    return make_rsrc(p.a + L.base, (uint32_t)L.nrec);
  };
  // the block resources do not depend on the slice (built once, scalar registers)
  __amdgpu_buffer_rsrc_t ra[LA];
#pragma unroll
  for (int li = 0; li < LA; li++) ra[li] = a_rsrc(li, 0);

  // Slices travel global -> registers -> LDS through two register sets (the loop below says
  // which slices they hold when).
  constexpr int NL = LA + LW;                       // 16-byte loads per lane per slice
  u32x4 stage_reg[2][NL];
  auto load_one = [&](u32x4 *dst, int kt, int li) {
    const uint32_t kb = (uint32_t)kt * GKB;   // byte offset of the slice inside a W row
    if (li < LA) {
      if constexpr (hm) {
        // head-major: the slice's head moves the vector offset (a slice never crosses a head);
        // the same arithmetic as a_load
        const uint32_t kel = kb >> 1;
        dst[li] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra[li], a_voff + (kel >> hm_shift) * hm_head,
                                                         (kel & hm_mask) << 1, 0));
      } else {
        dst[li] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra[li], a_voff, kb, 0));
      }
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
  const int sc_v = wm * (BM / WGM) + 4 * (lane >> 5);   // the wave's and lane's part of an accumulator row

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
  // close group g: sum += (float)acc * row scale, acc = 0; one 32-row block at a time, so that
  // only 16 row scales are live; accumulator r of block i sits at row
  // (m0 + 32 i + 8 (r / 4)) + sc_v + r % 4 (sc_load)
  auto fold = [&](int g) {
    if constexpr (GROUPED) {
#pragma unroll
      for (int i = 0; i < FM; i++) {
        float sc[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int64_t u = m0 + 32 * i + 8 * q4;
          const ScLoad L0 = sc_load(p.M, n_groups, u, sc_v, 0, g);
          const __amdgpu_buffer_rsrc_t rsc = make_rsrc(p.a_scale + L0.base, (uint32_t)L0.nrec);
#pragma unroll
          for (int e = 0; e < 4; e++)
            sc[4 * q4 + e] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsc, sc_load(p.M, n_groups, u, sc_v, e, g).voff, 0, 0));
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
    // bf16 256 x 256: one wave per SIMD, 128 x 128 each (accumulators in AGPRs), a third fewer
    // LDS bytes per MFMA than 8 waves of 128 x 64.  int8, the grouped int8 FC2 and the 256 x 128
    // tiles: 8 waves, two per SIMD, of the same workgroup.
    // Iteration kt: MFMA steps 0..3 of slice kt from stage kt&1 with fragments read one step
    // ahead; the register set holding slice kt+1 goes to stage (kt+1)&1 during steps 0 to 2,
    // and the loads of slice kt+2 into the other set are spread over the iteration.
    // The barrier sits before step 3, whose fragments are already in registers; the step-0
    // fragments of slice kt+1 are read right after it, under step 3's MFMAs (with the stores
    // and the barrier at the top of the iteration instead, the two waves of a SIMD reach the
    // slice boundary together and both wait for the first fragments: int8 QKV and FC1 ran
    // 6-7% slower, the int8 out-projection 4%).
    // LDS store li follows MFMA SSTEP li of the iteration (2 li where that fits), global load li
    // follows MFMA LSTEP li + 1 (4 li + 1 where that fits: spread over all four steps).  The
    // grouped FC2 closes a group at the end of the iteration that finishes it.
    constexpr int NSTEP = FM * FN;
    constexpr int LSTEP = (4 * NSTEP - 2) / (NL - 1) < 4 ? (4 * NSTEP - 2) / (NL - 1) : 4;
    constexpr int SSTEP = (3 * NSTEP - 1) / (NL - 1) < 2 ? (3 * NSTEP - 1) / (NL - 1) : 2;
    static_assert(SSTEP * (NL - 1) < 3 * NSTEP && LSTEP * (NL - 1) + 1 < 4 * NSTEP && LSTEP >= 1 && SSTEP >= 1,
                  "store / load placement");
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
    // No LDS or scalar-memory operation is left pending where the loop is entered or repeated
    // (the step-0 fragments of the next slice are read a whole K step earlier), which lets the
    // wait-count insertion see that the first MFMAs of an iteration need no wait, instead of
    // waiting for every LDS read issued so far at the loop header.
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
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
              if (g == SSTEP * li && more) {
                __builtin_amdgcn_sched_barrier(0);
                store_one(cur, kt + 1, li);
                __builtin_amdgcn_sched_barrier(0);
              }
              if (STEADY && g == LSTEP * li + 1) {
                __builtin_amdgcn_sched_barrier(0);
                load_one(nxt, ktl, li);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
      }
      __builtin_amdgcn_s_waitcnt(kLgkmZero);   // the next slice's step-0 reads, issued 16 MFMAs ago
      if constexpr (GROUPED) {
        if ((kt + 1) % kt_per_group == 0) fold(kt / kt_per_group);
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
    // registers -> bf16 tile in LDS.  int8: every row and column scale the lane needs is
    // loaded before any is used (one round trip): rows m0 + rbase + 32 i + 8 q .. + 3 as one
    // 16-byte load through a resource that ends with the scale array; the range check is per
    // dword, so rows >= M read 0 while the rows before them in the same load read their scales
    // (the ragged int8 QKV case M = 130 checks it bit for bit)
    float4 sa4[INT8 && !GROUPED ? FM : 1][4];
    float swj[INT8 ? FN : 1];
    if constexpr (INT8 && !GROUPED) {
      const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.a_scale, (uint32_t)(p.M * 4));
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
          sa4[i][q4] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(rsa, (uint32_t)((m0 + rbase + 32 * i + 8 * q4) * 4), 0, 0));
    }
    if constexpr (INT8) {
#pragma unroll
      for (int j = 0; j < FN; j++) swj[j] = p.w_scale[n0 + cbase + 32 * j];
    }
#pragma unroll
    for (int i = 0; i < FM; i++) {
      float sa_r[16];
      if constexpr (INT8 && !GROUPED) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          sa_r[4 * q4] = sa4[i][q4].x;
          sa_r[4 * q4 + 1] = sa4[i][q4].y;
          sa_r[4 * q4 + 2] = sa4[i][q4].z;
          sa_r[4 * q4 + 3] = sa4[i][q4].w;
        }
      }
#pragma unroll
      for (int j = 0; j < FN; j++) {
        float sw = 0.0f;
        if constexpr (INT8) sw = swj[j];
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
        // A thread takes one 8-element chunk ci of a head row and does it for every head of the
        // tile (the heads of one token share its rotary table entries), rows tid / cph, +
        // NT / cph, ... (head rows of at least 8 chunks: hd >= 64)
        const int cph = p.hd / 8;              // chunks per head row
        const int hpt = BN / p.hd;             // heads per tile
        const int ci = tid % cph, i0 = ci * 8;
        const int h0 = (int)(n0 % d) / p.hd;   // first head of the tile
        uint16_t *dst0 = (part == 0 ? p.oq : p.ok) + (int64_t)h0 * p.M * p.hd + i0;
        const int half = p.hd / 2;
        const float *cos_c = p.cos_t + i0 / 2, *sin_c = p.sin_t + i0 / 2;
        // the table entries of all the thread's rows (BM * cph / NT of them; cph <= 16) are
        // loaded first, so that their latencies overlap
        constexpr int MAXR = BM * 16 / NT;
        const int r0 = tid / cph, rstep = NT / cph;
        float4 tcos[MAXR], tsin[MAXR];
#pragma unroll
        for (int k = 0; k < MAXR; k++) {
          const int r = r0 + k * rstep;
          if (r < BM && m0 + r < p.M) {
            tcos[k] = *reinterpret_cast<const float4 *>(cos_c + (m0 + r) * half);
            tsin[k] = *reinterpret_cast<const float4 *>(sin_c + (m0 + r) * half);
          }
        }
        auto rope = [&](u32x4 v, int k) {
          const float cc[4] = {tcos[k].x, tcos[k].y, tcos[k].z, tcos[k].w};
          const float ss[4] = {tsin[k].x, tsin[k].y, tsin[k].z, tsin[k].w};
          float f[8], o[8];
          unpack8(v, f);
#pragma unroll
          for (int e = 0; e < 4; e++) {
            o[2 * e] = f[2 * e] * cc[e] - f[2 * e + 1] * ss[e];
            o[2 * e + 1] = f[2 * e] * ss[e] + f[2 * e + 1] * cc[e];
          }
          return pack8(o);
        };
        if (hpt == 2 && m0 + BM <= p.M && MAXR * rstep == BM) {
          // whole tile, two heads per tile: every row of the thread is in the tile and inside M,
          // and the LDS reads of a batch of rows (both heads) go out together
          constexpr int RB = 4;
          static_assert(MAXR % RB == 0, "whole batches");
#pragma unroll
          for (int k0 = 0; k0 < MAXR; k0 += RB) {
            u32x4 x[RB][2];
#pragma unroll
            for (int u = 0; u < RB; u++)
#pragma unroll
              for (int hh = 0; hh < 2; hh++)
                x[u][hh] = *reinterpret_cast<const u32x4 *>(smem + (r0 + (k0 + u) * rstep) * C::CPITCH +
                                                            (hh * cph + ci) * 16);
#pragma unroll
            for (int u = 0; u < RB; u++)
#pragma unroll
              for (int hh = 0; hh < 2; hh++)
                *reinterpret_cast<u32x4 *>(dst0 + (int64_t)hh * p.M * p.hd + (m0 + r0 + (k0 + u) * rstep) * p.hd) =
                    rope(x[u][hh], k0 + u);
          }
        } else {
#pragma unroll
          for (int k = 0; k < MAXR; k++) {
            const int r = r0 + k * rstep;
            const int64_t row = m0 + r;
            if (r >= BM || row >= p.M) break;   // later rows are past the tile or the end too
            for (int hh = 0; hh < hpt; hh++)
              *reinterpret_cast<u32x4 *>(dst0 + (int64_t)hh * p.M * p.hd + row * p.hd) =
                  rope(*reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + (hh * cph + ci) * 16), k);
          }
        }
      } else {
        // V^T[h][i][vt_pos(m)].  Inside a 16-token group, positions 0-7 hold tokens 0-3 and
        // 8-11, positions 8-15 tokens 4-7 and 12-15.  A unit is (group rb, half hh, 8-feature
        // chunk fc): the half's 8 tokens are read as 16-byte rows of the staged tile (the
        // chunk's 8 features each), transposed in registers and stored as one 16-byte piece
        // of each of the chunk's 8 V^T rows.
        constexpr int FCH = BN / 8;                   // feature chunks per tile
        constexpr int UNITS = (BM / 16) * 2 * FCH;
        static_assert(UNITS % NT == 0, "whole passes");
        const int fc = tid % FCH;
        const int col = (int)(n0 % d) + fc * 8;       // first feature of the chunk
        const int h = col / p.hd, i = col % p.hd;     // the chunk's 8 features share the head
        uint16_t *dst_c = p.ov + ((int64_t)h * p.hd + i) * p.ldv;
        for (int gh = tid / FCH; gh < (BM / 16) * 2; gh += NT / FCH) {
          const int rb = gh >> 1, hh = gh & 1;
          const int64_t row0 = m0 + rb * 16;
          if (row0 >= p.M) break;   // later groups are past the end too
          u32x4 x[8];
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const int tok = (j & 3) + 4 * hh + 8 * (j >> 2);
            x[j] = *reinterpret_cast<const u32x4 *>(smem + (rb * 16 + tok) * C::CPITCH + fc * 16);
          }
          // word w of feature e's piece: tokens 2w (low half) and 2w + 1 (high half)
          u32x4 y[8];
#pragma unroll
          for (int e = 0; e < 8; e++)
#pragma unroll
            for (int w = 0; w < 4; w++)
              y[e][w] = __builtin_amdgcn_perm(x[2 * w + 1][e >> 1], x[2 * w][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
          uint16_t *dst = dst_c + row0 + 8 * hh;
          if (row0 + 16 <= p.M) {
#pragma unroll
            for (int e = 0; e < 8; e++) *reinterpret_cast<u32x4 *>(dst + (int64_t)e * p.ldv) = y[e];
          } else {
#pragma unroll
            for (int j = 0; j < 8; j++) {
              const int tok = (j & 3) + 4 * hh + 8 * (j >> 2);
              if (row0 + tok < p.M) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                  dst[(int64_t)e * p.ldv + j] = (uint16_t)(y[e][j >> 1] >> (16 * (j & 1)));
              }
            }
          }
        }
      }
    } else {
      uint16_t *out = reinterpret_cast<uint16_t *>(p.out) + n0 + c * 8;
      auto finish = [&](u32x4 v) {
        if constexpr (OUT == H3DIT_OUT_GELU) {
          float f[8];
          unpack8(v, f);
#pragma unroll
          for (int e = 0; e < 8; e++) f[e] = gelu_tanh(f[e]);
          v = pack8(f);
        }
        return v;
      };
      constexpr int RSTEP = NT / CH, RPT = BM / RSTEP, UB = RPT < 8 ? RPT : 8;   // rows per pass / thread / batch
      static_assert(RPT % UB == 0, "whole batches");
      if (m0 + BM <= p.M) {
        // whole tile: the LDS reads of a batch of rows go out together, so that their latency
        // is paid once per batch and not once per row
        for (int k0 = 0; k0 < RPT; k0 += UB) {
          u32x4 v[UB];
#pragma unroll
          for (int u = 0; u < UB; u++)
            v[u] = *reinterpret_cast<const u32x4 *>(smem + (tid / CH + (k0 + u) * RSTEP) * C::CPITCH + c * 16);
#pragma unroll
          for (int u = 0; u < UB; u++)
            *reinterpret_cast<u32x4 *>(out + (m0 + tid / CH + (k0 + u) * RSTEP) * p.N) = finish(v[u]);
        }
      } else {
        for (int r = tid / CH; r < BM; r += RSTEP) {
          const int64_t row = m0 + r;
          if (row >= p.M) break;   // later rows are past the end too
          *reinterpret_cast<u32x4 *>(out + row * p.N) =
              finish(*reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + c * 16));
        }
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
  const int64_t col = p.n_lo + (int64_t)tn * 256 + wn * 128 + 32 * j + (lane & 31);
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

// One launch over the output columns [n_lo, n_hi): pl.n_dp whole tiles, then pl.n_split
// tiles in pl.split K segments.
template <int BM, int BN, int WGM, int WGN, bool INT8, int OUT, bool GROUPED, bool HM>
static hipError_t run_gemm(GemmP p, const LinearPlan &pl, int64_t n_lo, int64_t n_hi, hipStream_t st) {
  p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)((n_hi - n_lo) / BN);
  p.n_lo = n_lo;
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
//   int8 (not the QKV epilogue, whose V^T pass is laid out for the wider tiles): 256 x 256
//     tiles over the first columns and a second launch
//     of 128 x 128 tiles (eight waves of 64 x 32) over the rest, a round of those ~0.43 of a
//     round of whole tiles (measured at 4096 x 5120 x 5120: one round of each, 118-121 us,
//     against 131-132 us for 2.5 rounds of 256 x 128 tiles).  int8 sums are exact, so the
//     output does not depend on the plan.
// The grouped int8 FC2 uses 256 x 128 tiles (its second accumulator set does not fit 256 wide)
// over its first n_big columns and 128 x 128 tiles over the rest, n_big chosen to fill whole
// rounds: a round of large tiles costs 1, a round of 256 small tiles 0.86 (measured at 4096
// tokens: eight waves of 64 x 32, two per SIMD, half a large tile's MFMAs but three quarters
// of its LDS fragment reads).  No K is split: every element sums its groups in ascending
// order within one workgroup, whichever tile holds it.
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
  pl.n_big = a.N;
  pl.n_small = 0;
  if (grouped) {
    const int64_t tmb = (a.M + G_BM - 1) / G_BM, tms = (a.M + GS_BM - 1) / GS_BM, nc = a.N / G_BN;
    int64_t best_c = nc;
    double best = (double)((tmb * nc + kCUs - 1) / kCUs);
    for (int64_t c = nc - 1; c >= 0; c--) {
      const int64_t nb = tmb * c, ns = tms * (nc - c) * (G_BN / GS_BN);
      const double cost = (double)((nb + kCUs - 1) / kCUs) + 0.86 * (double)((ns + kCUs - 1) / kCUs);
      if (cost < best - 0.01) {
        best = cost;
        best_c = c;
      }
    }
    pl.n_big = best_c * G_BN;
    pl.n_dp = (int)(tmb * best_c);
    pl.n_small = (int)(tms * (nc - best_c) * (G_BN / GS_BN));
    return pl;
  }
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
  // int8 (exact whatever the plan): whole 256 x 256 tiles over the first c * 256 columns,
  // 128 x 128 tiles over the rest
  int64_t mix_c = -1;
  if (i8 && a.out_kind != H3DIT_OUT_QKV) {
    const int64_t tms = (a.M + 127) / 128, nc = a.N / 256;
    for (int64_t c = nc - 1; c >= 1; c--) {
      const int64_t nb = tm * c, ns = tms * (a.N - 256 * c) / 128;
      const double cost = (double)((nb + kCUs - 1) / kCUs) + 0.43 * (double)((ns + kCUs - 1) / kCUs);
      if (cost < best - 1e-9 && cost < c128 - 1e-9) {
        best = cost;
        best_s = 1;
        mix_c = c;
      }
    }
  }
  if (mix_c > 0) {
    pl.bn = 256;
    pl.n_dp = (int)(tm * mix_c);
    pl.n_big = mix_c * 256;
    pl.n_small = (int)((a.M + 127) / 128 * (a.N - 256 * mix_c) / 128);
    return pl;
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
    // two accumulator sets (int32 per group, fp32 across groups) per lane: 256 x 128 tiles of
    // 8 waves of 64 x 64 over columns [0, n_big), 128 x 128 tiles of 8 waves of 64 x 32 after them
    hipError_t e = hipSuccess;
    if (pl.n_big > 0) e = run_gemm<G_BM, G_BN, G_WGM, G_WGN, INT8, OUT, GROUPED, false>(p, pl, 0, pl.n_big, st);
    if (e == hipSuccess && pl.n_small > 0) {
      LinearPlan sp = pl;
      sp.n_dp = pl.n_small;
      e = run_gemm<GS_BM, GS_BN, GS_WGM, GS_WGN, INT8, OUT, GROUPED, false>(p, sp, pl.n_big, p.N, st);
    }
    return e;
  } else {
    // bf16: four waves of 128 x 128; int8: eight waves of 128 x 64 (measured faster for int8)
    if (pl.bn == 256) {
      if constexpr (INT8 && OUT != H3DIT_OUT_QKV) {
        if (pl.n_small > 0) {
          hipError_t e = run_gemm<256, 256, 2, 4, INT8, OUT, GROUPED, HM>(p, pl, 0, pl.n_big, st);
          LinearPlan sp = pl;
          sp.n_dp = pl.n_small;
          if (e == hipSuccess) e = run_gemm<GS_BM, GS_BN, GS_WGM, GS_WGN, INT8, OUT, GROUPED, HM>(p, sp, pl.n_big, p.N, st);
          return e;
        }
      }
      if constexpr (INT8) return run_gemm<256, 256, 2, 4, INT8, OUT, GROUPED, HM>(p, pl, 0, p.N, st);
      else return run_gemm<256, 256, 2, 2, INT8, OUT, GROUPED, HM>(p, pl, 0, p.N, st);
    }
    return run_gemm<256, 128, 4, 2, INT8, OUT, GROUPED, HM>(p, pl, 0, p.N, st);
  }
}

size_t linear_workspace(const h3dit_linear_args &a) { return plan_linear(a).part_bytes; }

// Host walk over every A load of the launch plan_linear chooses (all tiles, waves, lanes,
// blocks and K slices), with the kernel's own addressing (a_load): the largest byte end of
// a load the range check lets through, and the number of loads whose masking is wrong (a row
// < M returning zeros, a row >= M reading memory, or a load that straddles its resource end).
void linear_a_extent(const h3dit_linear_args &a, uint64_t *max_end, uint64_t *bad) {
  const LinearPlan pl = plan_linear(a);
  const bool i8 = a.precision == H3DIT_INT8;
  const bool grouped = i8 && a.a_group > 0;
  const int esz = i8 ? 1 : 2;
  const int KT = (int)(a.K * esz / GKB);
  const int hm_hd = i8 ? 0 : a.a_headmajor_hd;
  uint64_t top = 0, nbad = 0;
  // one tile form: BM rows, NW waves in a WGM-row grid
  auto walk = [&](int BM, int NW, int WGM) {
    const int LA = BM / (8 * NW);
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    for (int64_t tm = 0; tm < tiles_m; tm++)
      for (int r0 = 0; r0 < NW * 8; r0++)
        for (int cl = 0; cl < 8; cl++)
          for (int li = 0; li < LA; li++)
            for (int kt = 0; kt < KT; kt++) {
              const int64_t m0 = tm * BM;
              const ALoad L = a_load(a.M, a.K, esz, hm_hd, NW, m0, r0, cl, li, kt);
              const int64_t row = m0 + r0 + (int64_t)NW * 8 * li;
              const bool masked = (int64_t)L.voff >= L.nrec;
              // a row < M is always read; a row >= M reads zeros (token-major A) or, head-major,
              // a row of the next head inside A, masked only past the last head
              if ((row < a.M && masked) || (!hm_hd && row >= a.M && !masked)) nbad++;
              if (!masked) {
                if ((int64_t)L.voff + L.soff + 16 > L.nrec) nbad++;
                const uint64_t end = (uint64_t)(L.base + L.voff + L.soff + 16);
                if (end > top) top = end;
              }
            }
    if (grouped) {
      // the group scales [M][K / a_group] fp32 of the grouped FC2 (waves 64 rows high, WGM rows
      // of them, two 32-row blocks each)
      const int ng = (int)(a.K / a.a_group);
      uint64_t stop = 0;
      for (int64_t tm = 0; tm < tiles_m; tm++)
        for (int wm = 0; wm < WGM; wm++)
          for (int hsel = 0; hsel < 2; hsel++)
            for (int i = 0; i < 2; i++)
              for (int q4 = 0; q4 < 4; q4++)
                for (int e = 0; e < 4; e++)
                  for (int g = 0; g < ng; g++) {
                    const int64_t u = tm * BM + 32 * i + 8 * q4;
                    const int v = wm * 64 + 4 * hsel;
                    const ScLoad L = sc_load(a.M, ng, u, v, e, g);
                    const bool masked = (int64_t)L.voff >= L.nrec;
                    if (masked != (u + v + e >= a.M)) nbad++;
                    if (!masked) {
                      if ((int64_t)L.voff + 4 > L.nrec) nbad++;
                      const uint64_t end = (uint64_t)(L.base * 4 + L.voff + 4);
                      if (end > stop) stop = end;
                    }
                  }
      if (stop > (uint64_t)a.M * ng * 4) nbad++;
    }
  };
  if (grouped) {
    if (pl.n_dp > 0) walk(G_BM, G_WGM * G_WGN, G_WGM);
    if (pl.n_small > 0) walk(GS_BM, GS_WGM * GS_WGN, GS_WGM);
  } else if (pl.bn == 256) {
    walk(256, i8 ? 8 : 4, 2);
    if (pl.n_small > 0) walk(GS_BM, GS_WGM * GS_WGN, GS_WGM);
  } else {
    walk(256, 8, 4);
  }
  *max_end = top;
  *bad = nbad;
}

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
