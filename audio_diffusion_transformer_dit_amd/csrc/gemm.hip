// Projections of the H3 DiT block on gfx950 MFMA: out = A W^T with A [M][K] (tokens x in),
// W [N][K] (out x in) ([DD] "h3.c 的核心设计" and "int8 量化": QKV, attention output, FC1, FC2
// in bf16 or int8 with per-token / per-channel / per-1024-group scales).
//
// Tiling: a workgroup of 4 waves owns a 256 x BN output tile (BN = 256 or 128); waves are
// 2 x 2, each owning 128 x BN/2 as a grid of 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16 or
// v_mfma_i32_32x32x32_i8; both read 16 bytes of K per lane, so one LDS layout serves both).
// K advances 128 bytes per step: every row of a step is 8 chunks of 16 B.  Both operands go
// global -> LDS with buffer_load ... lds (no VGPR staging), double-buffered, chunk c of row r
// stored at slot c ^ (r & 7) so that the 8 lanes of an LDS read phase hit 8 distinct bank
// groups.  Rows past M read as zeros (buffer range check).  The epilogue stages the bf16 tile
// in LDS and writes 16-byte row chunks (or, for V, 16-byte token chunks of V^T).
// Workgroups are dealt round-robin to the 8 XCDs; the tile order is remapped so that each
// XCD sweeps a contiguous band of tiles, 8 tile-rows at a time, sharing A and W in its L2.
#include "common.hpp"

namespace h3 {

constexpr int GKB = 128;        // bytes of K per step and row
constexpr int GTHREADS = 256;   // 4 waves

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
};

template <int BM, int BN>
struct GemmCfg {
  static constexpr int FM = BM / 64;                    // 32-row MFMA blocks per wave
  static constexpr int FN = BN / 64;                    // 32-col MFMA blocks per wave
  static constexpr int STAGE = (BM + BN) * GKB;         // bytes per LDS stage
  static constexpr int CPITCH = BN * 2 + 16;            // bytes per row of the staged C tile
  static constexpr int CTILE = BM * CPITCH;
  static constexpr int LDS = (2 * STAGE > CTILE) ? 2 * STAGE : CTILE;
};

__device__ __forceinline__ void tile_coords(int &tm, int &tn, int tiles_m, int tiles_n) {
  const int nwg = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((nwg & 7) == 0) b = (b & 7) * (nwg >> 3) + (b >> 3);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = b / per_group;
  const int first = g * GROUP;
  const int gsize = min(tiles_m - first, GROUP);
  const int r = b - g * per_group;
  tm = first + r % gsize;
  tn = r / gsize;
}

// Issues the loads of one K step (rows m0.. of A, n0.. of W) into LDS stage `st`.
template <int BM, int BN, bool INT8>
__device__ __forceinline__ void load_stage(const GemmP &p, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rw,
                                           uint8_t *st, int64_t m0, int64_t n0, int kt) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int rl = lane >> 3;           // row within the 8-row group of this instruction
  const int slot = lane & 7;          // LDS slot of this lane
  const int chunk = slot ^ rl;        // global chunk it fetches
  const int64_t esz = INT8 ? 1 : 2;
  const int64_t kel = (int64_t)kt * (GKB / esz) + chunk * (16 / esz);   // K element index
#pragma unroll
  for (int i = 0; i < BM / 32; i++) {
    const int rb = i * 4 + wid;                 // 8-row block
    const int64_t m = m0 + rb * 8 + rl;
    uint32_t off;
    if (!INT8 && p.hm_hd > 0)
      off = (uint32_t)((((kel / p.hm_hd) * p.M + m) * p.hm_hd + kel % p.hm_hd) * 2);
    else
      off = (uint32_t)((m * p.K + kel) * esz);
    buffer_load_lds16(ra, (lds_void *)(st + rb * 8 * GKB), off);
  }
#pragma unroll
  for (int i = 0; i < BN / 32; i++) {
    const int rb = i * 4 + wid;
    const int64_t n = n0 + rb * 8 + rl;
    const uint32_t off = (uint32_t)((n * p.K + kel) * esz);
    buffer_load_lds16(rw, (lds_void *)(st + BM * GKB + rb * 8 * GKB), off);
  }
}

__device__ __forceinline__ u32x4 lds_frag(const uint8_t *base, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(base + row * GKB + ((chunk ^ (row & 7)) << 4));
}

// out_kind: H3DIT_OUT_*.  GROUPED: int8 FC2 with per-(row, group) activation scales.
template <int BM, int BN, bool INT8, int OUT, bool GROUPED>
__global__ __launch_bounds__(GTHREADS, 1) void k_gemm(GemmP p) {
  using C = GemmCfg<BM, BN>;
  constexpr int FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];

  int tm, tn;
  tile_coords(tm, tn, p.tiles_m, p.tiles_n);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int esz = INT8 ? 1 : 2;
  const uint32_t a_bytes = (uint32_t)(p.M * p.K * esz), w_bytes = (uint32_t)(p.N * p.K * esz);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, a_bytes), rw = make_rsrc(p.w, w_bytes);
  const int KT = (int)(p.K * esz / GKB);

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
  const int kt_per_group = GROUPED ? p.a_group / GKB : 0;
  const int n_groups = GROUPED ? (int)(p.K / p.a_group) : 0;

  load_stage<BM, BN, INT8>(p, ra, rw, smem, m0, n0, 0);
  wait_vmem();
  __syncthreads();

  const int arow0 = wm * (BM / 2) + (lane & 31);
  const int brow0 = wn * (BN / 2) + (lane & 31);
  const int hsel = lane >> 5;
  for (int kt = 0; kt < KT; kt++) {
    uint8_t *cur = smem + (kt & 1) * C::STAGE;
    if (kt + 1 < KT) load_stage<BM, BN, INT8>(p, ra, rw, smem + ((kt + 1) & 1) * C::STAGE, m0, n0, kt + 1);
    const uint8_t *sa = cur, *sb = cur + BM * GKB;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) af[i] = lds_frag(sa, arow0 + 32 * i, 2 * ks + hsel);
#pragma unroll
      for (int j = 0; j < FN; j++) bfr[j] = lds_frag(sb, brow0 + 32 * j, 2 * ks + hsel);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
          if constexpr (INT8)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, af[i]),
                                                              __builtin_bit_cast(i32x4, bfr[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                                __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (GROUPED) {
      if ((kt + 1) % kt_per_group == 0) {
        const int g = kt / kt_per_group;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int64_t row = m0 + wm * (BM / 2) + 32 * i + 8 * (r / 4) + 4 * hsel + (r % 4);
            const float s = row < p.M ? p.a_scale[row * n_groups + g] : 0.0f;
#pragma unroll
            for (int j = 0; j < FN; j++) {
              sum[i][j][r] = sum[i][j][r] + (float)acc[i][j][r] * s;
              acc[i][j][r] = 0;
            }
          }
      }
    }
    wait_vmem();
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // value of accumulator (i, j, r): row = m0 + wm*BM/2 + 32 i + 8 (r/4) + 4 hsel + r%4,
  //                                 col = n0 + wn*BN/2 + 32 j + lane%32
  const int rbase = wm * (BM / 2) + 4 * hsel;
  const int cbase = wn * (BN / 2) + (lane & 31);
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
    if constexpr (OUT == H3DIT_OUT_QKV) {
      const int d = p.heads * p.hd;
      const int part = (int)(n0 / d);
      if (part < 2) {
        uint16_t *dst = part == 0 ? p.oq : p.ok;
        const int half = p.hd / 2;
        for (int idx = tid; idx < BM * CH; idx += GTHREADS) {
          const int r = idx / CH, c = idx % CH;
          const int64_t row = m0 + r;
          if (row >= p.M) continue;
          const int col = (int)(n0 % d) + c * 8;
          const int h = col / p.hd, i0 = col % p.hd;
          float f[8], o[8];
          unpack8(*reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + c * 16), f);
          const float4 cs = *reinterpret_cast<const float4 *>(p.cos_t + row * half + i0 / 2);
          const float4 sn = *reinterpret_cast<const float4 *>(p.sin_t + row * half + i0 / 2);
          const float cc[4] = {cs.x, cs.y, cs.z, cs.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            o[2 * e] = f[2 * e] * cc[e] - f[2 * e + 1] * ss[e];
            o[2 * e + 1] = f[2 * e] * ss[e] + f[2 * e + 1] * cc[e];
          }
          *reinterpret_cast<u32x4 *>(dst + ((int64_t)h * p.M + row) * p.hd + i0) = pack8(o);
        }
      } else {
        // V^T[h][i][m]: one lane per (feature column, block of 8 tokens)
        const bool vec = (p.ldv % 8) == 0;
        for (int idx = tid; idx < BN * (BM / 8); idx += GTHREADS) {
          const int c = idx % BN, rb = idx / BN;
          const int col = (int)(n0 % d) + c;
          const int h = col / p.hd, i = col % p.hd;
          uint16_t v8[8];
#pragma unroll
          for (int e = 0; e < 8; e++) v8[e] = *reinterpret_cast<const uint16_t *>(smem + (rb * 8 + e) * C::CPITCH + c * 2);
          const int64_t row = m0 + rb * 8;
          uint16_t *dst = p.ov + ((int64_t)h * p.hd + i) * p.ldv + row;
          if (vec && row + 8 <= p.M) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] = (uint32_t)v8[2 * e] | ((uint32_t)v8[2 * e + 1] << 16);
            *reinterpret_cast<u32x4 *>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
              if (row + e < p.M) dst[e] = v8[e];
          }
        }
      }
    } else {
      uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
      for (int idx = tid; idx < BM * CH; idx += GTHREADS) {
        const int r = idx / CH, c = idx % CH;
        const int64_t row = m0 + r;
        if (row >= p.M) continue;
        u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * C::CPITCH + c * 16);
        if constexpr (OUT == H3DIT_OUT_GELU) {
          float f[8];
          unpack8(v, f);
#pragma unroll
          for (int e = 0; e < 8; e++) f[e] = gelu_tanh(f[e]);
          v = pack8(f);
        }
        *reinterpret_cast<u32x4 *>(out + row * p.N + n0 + c * 8) = v;
      }
    }
  }
}

template <int BM, int BN, bool INT8, int OUT, bool GROUPED>
static hipError_t run_gemm(GemmP p, hipStream_t st) {
  p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)(p.N / BN);
  const unsigned nwg = (unsigned)p.tiles_m * p.tiles_n;
  k_gemm<BM, BN, INT8, OUT, GROUPED><<<nwg, GTHREADS, 0, st>>>(p);
  return hipGetLastError();
}

// Tile width: 256 when that still gives every CU work for about two rounds, else 128.
static int pick_bn(int64_t M, int64_t N) {
  if (N % 256 != 0) return 128;
  const int64_t tiles256 = ((M + 255) / 256) * (N / 256);
  return tiles256 >= 512 ? 256 : 128;
}

template <bool INT8, int OUT, bool GROUPED>
static hipError_t dispatch_bn(const GemmP &p, int bn, hipStream_t st) {
  if constexpr (GROUPED) {
    // two accumulator sets (int32 per group, fp32 across groups) per lane: 128 x 128 tiles
    return run_gemm<128, 128, INT8, OUT, GROUPED>(p, st);
  } else {
    if (bn == 256) return run_gemm<256, 256, INT8, OUT, GROUPED>(p, st);
    return run_gemm<256, 128, INT8, OUT, GROUPED>(p, st);
  }
}

hipError_t launch_linear(const h3dit_linear_args &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
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
  p.ldv = (int)((a.M + 7) / 8 * 8);
  int bn = pick_bn(a.M, a.N);
  if (a.out_kind == H3DIT_OUT_QKV) {
    const int64_t d = (int64_t)a.heads * a.head_dim;
    if (d % bn) bn = 128;
  }
  const bool i8 = a.precision == H3DIT_INT8;
  if (i8 && a.a_group > 0) return dispatch_bn<true, H3DIT_OUT_BF16, true>(p, bn, st);
  switch (a.out_kind) {
    case H3DIT_OUT_BF16:
      return i8 ? dispatch_bn<true, H3DIT_OUT_BF16, false>(p, bn, st) : dispatch_bn<false, H3DIT_OUT_BF16, false>(p, bn, st);
    case H3DIT_OUT_F32:
      return dispatch_bn<false, H3DIT_OUT_F32, false>(p, bn, st);
    case H3DIT_OUT_I32:
      return dispatch_bn<true, H3DIT_OUT_I32, false>(p, bn, st);
    case H3DIT_OUT_GELU:
      return i8 ? dispatch_bn<true, H3DIT_OUT_GELU, false>(p, bn, st) : dispatch_bn<false, H3DIT_OUT_GELU, false>(p, bn, st);
    case H3DIT_OUT_QKV:
      return i8 ? dispatch_bn<true, H3DIT_OUT_QKV, false>(p, bn, st) : dispatch_bn<false, H3DIT_OUT_QKV, false>(p, bn, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace h3
