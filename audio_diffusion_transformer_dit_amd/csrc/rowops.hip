// HBM-bound row kernels of the H3 DiT block on gfx950: gated residual + AdaLN (+ int8 code),
// int8 row/group codes, GELU, rotary tables and head split, token pair / restore.
//
// Memory pattern: one workgroup of 128 lanes owns one token row; every lane moves 16-byte
// chunks (8 bf16) so a wave touches 1 KiB contiguous per access.  Loads are ordinary
// (cached): the rows were usually just written by the previous kernel and are served from
// the 256 MB last-level cache; nontemporal loads measured 25-30% slower here.  The row stays in registers
// between the gated residual and the normalisation ([DD] "DiT 融合内核": the rounded residual
// is written exactly while the same row is normalised without a global re-read).
#include "common.hpp"

namespace h3 {

constexpr int ROW_THREADS = 128;   // workgroup of the two-pass kernel for spans past 32768
constexpr int RW_WAVES = 4;        // rows (one per wave) per workgroup of the row kernels

template <int NW>
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; w++) t = fmaxf(t, red[w]);
  __syncthreads();
  return t;
}

// Gated residual and/or AdaLN, one token row per wave (four rows per workgroup): lane l holds
// the 16-byte chunks l, l + 64, ... of its row in registers (MAXJ of them), so the row is read
// once and every reduction is a wave reduction (no LDS, no barrier).  GATE: x_out = bf16(x +
// g*y).  NORM: LN of the rounded row (mean, then the variance about it, both over the
// registers), modulation, bf16 rounding, and optionally the row's int8 code.  The LN part is
// the same code whether or not GATE ran in this kernel, so the fused and the two-kernel
// sequences give the same bytes.
// Modulation sets: rows [0, seg1) use gate/shift/scale as given, rows [seg1, seg2) the vectors
// set_stride elements further, rows from seg2 on 2*set_stride further (set_stride 0: one set).
// x_out may equal x (the residual updated in place): neither is marked __restrict__; a row's
// loads all precede its stores and each wave touches only its own row.
template <bool GATE, bool NORM, bool STATS, int MAXJ>
__global__ __launch_bounds__(64 * RW_WAVES) void k_row(int64_t n, int d, float eps, const uint16_t *x,
                                                       const uint16_t *__restrict__ gate,
                                                       const uint16_t *__restrict__ y, uint16_t *x_out,
                                                       const uint16_t *__restrict__ shift,
                                                       const uint16_t *__restrict__ scale, uint16_t *__restrict__ h,
                                                       int8_t *__restrict__ q, float *__restrict__ s, int64_t seg1,
                                                       int64_t seg2, int64_t set_stride) {
  const int64_t row = (int64_t)blockIdx.x * RW_WAVES + (threadIdx.x >> 6);
  if (row >= n) return;   // whole waves
  const int64_t mset = (int64_t)(row >= seg1) + (int64_t)(row >= seg2);
  gate += mset * set_stride;
  shift += mset * set_stride;
  scale += mset * set_stride;
  const int nch = d >> 3;
  const int lane = threadIdx.x & 63;
  // the row stays packed (8 bf16 per 16-byte chunk): every value it holds is a bf16 already
  u32x4 xv[MAXJ];
  const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * d);
#pragma unroll
  for (int j = 0; j < MAXJ; j++) {
    const int c = lane + 64 * j;
    if (c < nch) xv[j] = xr[c];
  }
  if constexpr (GATE) {
    const u32x4 *yr = reinterpret_cast<const u32x4 *>(y + row * d);
    const u32x4 *gr = reinterpret_cast<const u32x4 *>(gate);
    u32x4 yw[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; j++) {
      const int c = lane + 64 * j;
      if (c < nch) yw[j] = yr[c];
    }
    u32x4 *xo = reinterpret_cast<u32x4 *>(x_out + row * d);
#pragma unroll
    for (int j = 0; j < MAXJ; j++) {
      const int c = lane + 64 * j;
      if (c < nch) {
        float a[8], yv[8], gv[8];
        unpack8(xv[j], a);
        unpack8(yw[j], yv);
        unpack8(gr[c], gv);
#pragma unroll
        for (int e = 0; e < 8; e++) a[e] = a[e] + gv[e] * yv[e];
        xv[j] = pack8(a);
        xo[c] = xv[j];
      }
    }
  }
  if constexpr (NORM) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXJ; j++)
      if (lane + 64 * j < nch) {
        float a[8];
        unpack8(xv[j], a);
#pragma unroll
        for (int e = 0; e < 8; e++) part += a[e];
      }
    const float mu = wave_sum(part) / (float)d;
    part = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXJ; j++)
      if (lane + 64 * j < nch) {
        float a[8];
        unpack8(xv[j], a);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float c = a[e] - mu;
          part += c * c;
        }
      }
    const float var = wave_sum(part) / (float)d;
    const float rs = 1.0f / sqrtf(var + eps);
    if constexpr (STATS) {
      // statistics only (for a consumer that applies the modulation itself): s[2 row] = mean,
      // s[2 row + 1] = 1 / sqrt(var + eps), the very values the modulation below uses
      if (lane == 0) {
        s[2 * row] = mu;
        s[2 * row + 1] = rs;
      }
      return;
    }
    const u32x4 *shr = reinterpret_cast<const u32x4 *>(shift);
    const u32x4 *scr = reinterpret_cast<const u32x4 *>(scale);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXJ; j++) {
      const int c = lane + 64 * j;
      if (c < nch) {
        float a[8], sh[8], sc[8];
        unpack8(xv[j], a);
        unpack8(shr[c], sh);
        unpack8(scr[c], sc);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          float t = (a[e] - mu) * rs;
          t = t * (1.0f + sc[e]) + sh[e];
          a[e] = t;
        }
        xv[j] = pack8(a);   // the normalised row, rounded to bf16
        if (h) reinterpret_cast<u32x4 *>(h + row * d)[c] = xv[j];
        float r[8];
        unpack8(xv[j], r);
#pragma unroll
        for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(r[e]));
      }
    }
    if (q) {
      const float sa = wave_max(amax) / 127.0f, inv = 1.0f / sa;
      if (lane == 0) s[row] = sa;
#pragma unroll
      for (int j = 0; j < MAXJ; j++) {
        const int c = lane + 64 * j;
        if (c < nch) {
          float r[8];
          unpack8(xv[j], r);
          reinterpret_cast<uint2 *>(q + row * d)[c] = q8_pack8(r, sa, inv);
        }
      }
    }
  }
}

// chunks per lane of a d-wide row: the smallest instantiated count >= ceil(d / 512)
static int row_maxj(int d) {
  const int need = (d / 8 + 63) / 64;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 10 ? 10 : 16;
}

template <bool GATE, bool NORM, bool STATS>
static void row_dispatch(int64_t n, int d, float eps, const uint16_t *x, const uint16_t *gate, const uint16_t *y,
                         uint16_t *x_out, const uint16_t *shift, const uint16_t *scale, uint16_t *h, int8_t *q,
                         float *s, hipStream_t st, int64_t seg1, int64_t seg2, int64_t set_stride) {
  const dim3 grid((unsigned)((n + RW_WAVES - 1) / RW_WAVES)), block(64 * RW_WAVES);
#define H3_ROW(J)                                                                                                   \
  k_row<GATE, NORM, STATS, J><<<grid, block, 0, st>>>(n, d, eps, x, gate, y, x_out, shift, scale, h, q, s, seg1, seg2, \
                                                       set_stride)
  switch (row_maxj(d)) {
    case 1: H3_ROW(1); break;
    case 2: H3_ROW(2); break;
    case 4: H3_ROW(4); break;
    case 8: H3_ROW(8); break;
    case 10: H3_ROW(10); break;
    default: H3_ROW(16); break;
  }
#undef H3_ROW
}

hipError_t launch_row(int64_t n, int d, float eps, const uint16_t *x, const uint16_t *gate, const uint16_t *y,
                      uint16_t *x_out, const uint16_t *shift, const uint16_t *scale, uint16_t *h, int8_t *q,
                      float *s, hipStream_t st, int64_t seg1, int64_t seg2, int64_t set_stride) {
  if (n == 0) return hipSuccess;
  if (gate && shift)
    row_dispatch<true, true, false>(n, d, eps, x, gate, y, x_out, shift, scale, h, q, s, st, seg1, seg2, set_stride);
  else if (gate)
    row_dispatch<true, false, false>(n, d, eps, x, gate, y, x_out, shift, scale, h, q, s, st, seg1, seg2, set_stride);
  else
    row_dispatch<false, true, false>(n, d, eps, x, gate, y, x_out, shift, scale, h, q, s, st, seg1, seg2, set_stride);
  return hipGetLastError();
}

hipError_t launch_row_stats(int64_t n, int d, float eps, const uint16_t *x, float *stats, hipStream_t st) {
  if (n == 0) return hipSuccess;
  row_dispatch<false, true, true>(n, d, eps, x, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, stats,
                                  st, n, n, 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------- int8 codes of spans

// Spans of up to 8192 columns (the per-token codes of a d-wide row, the 1024-channel groups of
// the FC2 input): one wave per GPW consecutive spans of one row, lane l holding chunks l, l + 64,
// ... of each span (CPL per span), so that a lane has several 16-byte loads in flight and every
// absmax is a wave reduction.  Waves are numbered across rows (wave w: row w / upr, spans from
// (w % upr) * GPW, upr = ceil(spans per row / GPW)), so that every wave of a workgroup has work
// even where a row has fewer units than a workgroup has waves.  Head-major input (hm_hd > 0):
// element (r, c) of the token-major view sits at ((c / hd) * rows + r) * hd + c % hd; a chunk of
// 8 never crosses a head.
template <int CPL, int GPW>
__global__ __launch_bounds__(64 * RW_WAVES) void k_quant_span(int64_t rows, int64_t cols, int group,
                                                              const uint16_t *__restrict__ v, int hm_hd,
                                                              int8_t *__restrict__ q, float *__restrict__ s) {
  const int64_t ng = cols / group;
  const int64_t upr = (ng + GPW - 1) / GPW;   // wave units per row
  const int64_t w = (int64_t)blockIdx.x * RW_WAVES + (threadIdx.x >> 6);
  if (w >= rows * upr) return;   // whole waves
  const int64_t r = w / upr;
  const int64_t g0 = (w % upr) * GPW;
  const int lane = threadIdx.x & 63;
  const int nch = group >> 3;
  u32x4 raw[GPW][CPL];
#pragma unroll
  for (int k = 0; k < GPW; k++)
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const int c = lane + 64 * j;
      if (g0 + k < ng && c < nch) {
        const int64_t col = (g0 + k) * group + 8 * c;
        int64_t off = r * cols + col;
        if (hm_hd > 0) off = ((col / hm_hd) * rows + r) * hm_hd + col % hm_hd;
        raw[k][j] = *reinterpret_cast<const u32x4 *>(v + off);
      }
    }
#pragma unroll
  for (int k = 0; k < GPW; k++) {
    if (g0 + k >= ng) break;   // wave-uniform
    float val[CPL][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; j++)
      if (lane + 64 * j < nch) {
        unpack8(raw[k][j], val[j]);
#pragma unroll
        for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(val[j][e]));
      }
    const float sa = wave_max(amax) / 127.0f, inv = 1.0f / sa;
    if (lane == 0) s[r * ng + g0 + k] = sa;
    uint2 *dst = reinterpret_cast<uint2 *>(q + r * cols + (g0 + k) * group);
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const int c = lane + 64 * j;
      if (c < nch) dst[c] = q8_pack8(val[j], sa, inv);
    }
  }
}

// Token-major spans of 8193..32768 columns (a whole FC2-input row of 20480 channels, the
// 20480-wide weight rows): one 256-lane workgroup per span, values in registers, one pass
// over global memory.  Same arithmetic as k_quant_span.
constexpr int QWIDE_THREADS = 256;
constexpr int QWIDE_MAXJ = 16;
__global__ __launch_bounds__(QWIDE_THREADS) void k_quant_wide(int64_t cols, int group, const uint16_t *__restrict__ v,
                                                              int8_t *__restrict__ q, float *__restrict__ s) {
  __shared__ float red[QWIDE_THREADS / 64];
  const int64_t r = blockIdx.x;
  const int64_t g = blockIdx.y;
  const int nch = group >> 3;
  const int tid = threadIdx.x;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(v + r * cols + g * group);
  float val[QWIDE_MAXJ][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < QWIDE_MAXJ; j++) {
    const int c = tid + j * QWIDE_THREADS;
    if (c < nch) {
      unpack8(src[c], val[j]);
#pragma unroll
      for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(val[j][e]));
    }
  }
  const float sa = block_max<QWIDE_THREADS / 64>(amax, red) / 127.0f, inv = 1.0f / sa;
  if (tid == 0) s[r * (cols / group) + g] = sa;
  uint2 *dst = reinterpret_cast<uint2 *>(q + r * cols + g * group);
#pragma unroll
  for (int j = 0; j < QWIDE_MAXJ; j++) {
    const int c = tid + j * QWIDE_THREADS;
    if (c < nch) dst[c] = q8_pack8(val[j], sa, inv);
  }
}

// Spans longer than the register-resident kernels hold (weight rows of the FC2 matrix, 20480
// wide): one workgroup per span, absmax in a first pass over global memory, codes in a second.
__global__ __launch_bounds__(ROW_THREADS) void k_quant_long(int64_t cols, int64_t group, const uint16_t *__restrict__ v,
                                                            int8_t *__restrict__ q, float *__restrict__ s) {
  __shared__ float red[ROW_THREADS / 64];
  const int64_t r = blockIdx.x;
  const int64_t g = blockIdx.y;
  const int64_t nch = group >> 3;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(v + r * cols + g * group);
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < nch; c += ROW_THREADS) {
    float f[8];
    unpack8(src[c], f);
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(f[e]));
  }
  const float sa = block_max<ROW_THREADS / 64>(amax, red) / 127.0f, inv = 1.0f / sa;
  if (threadIdx.x == 0) s[r * (cols / group) + g] = sa;
  uint2 *dst = reinterpret_cast<uint2 *>(q + r * cols + g * group);
  for (int64_t c = threadIdx.x; c < nch; c += ROW_THREADS) {
    float f[8];
    unpack8(src[c], f);
    dst[c] = q8_pack8(f, sa, inv);
  }
}

hipError_t launch_quant_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v, int hm_hd, int8_t *q,
                             float *s, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t ng = cols / group;
  if (group > 8192) {
    if (hm_hd > 0) return hipErrorInvalidValue;
    dim3 grid((unsigned)rows, (unsigned)ng);
    if (group <= (int64_t)QWIDE_THREADS * QWIDE_MAXJ * 8)
      k_quant_wide<<<grid, QWIDE_THREADS, 0, st>>>(cols, (int)group, v, q, s);
    else
      k_quant_long<<<grid, ROW_THREADS, 0, st>>>(cols, group, v, q, s);
    return hipGetLastError();
  }
  // chunks per lane and span, and spans per wave (at least about eight 16-byte loads per lane);
  // one wave per unit of GPW spans, numbered across rows (grid of at most 2^30 workgroups)
  if (rows * ng > ((int64_t)1 << 32)) return hipErrorInvalidValue;
  const int need = (int)((group / 8 + 63) / 64);
#define H3_QS(CPL, GPW)                                                                                           k_quant_span<CPL, GPW><<<(unsigned)((rows * ((ng + GPW - 1) / GPW) + RW_WAVES - 1) / RW_WAVES),                  64 * RW_WAVES, 0, st>>>(rows, cols, (int)group, v, hm_hd, q, s)
  if (need <= 1) H3_QS(1, 8);
  else if (need <= 2) H3_QS(2, 4);
  else if (need <= 4) H3_QS(4, 2);
  else if (need <= 8) H3_QS(8, 1);
  else if (need <= 10) H3_QS(10, 1);
  else H3_QS(16, 1);
#undef H3_QS
  return hipGetLastError();
}

// ---------------------------------------------------------------- GELU (unfused form)

__global__ void k_gelu(int64_t nch, const uint16_t *__restrict__ u, uint16_t *__restrict__ gl) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  float f[8];
  unpack8(reinterpret_cast<const u32x4 *>(u)[c], f);
#pragma unroll
  for (int e = 0; e < 8; e++) f[e] = gelu_tanh(f[e]);
  reinterpret_cast<u32x4 *>(gl)[c] = pack8(f);
}

hipError_t launch_gelu(int64_t count, const uint16_t *u, uint16_t *gl, hipStream_t st) {
  const int64_t nch = count / 8;
  if (nch == 0) return hipSuccess;
  k_gelu<<<(unsigned)((nch + 255) / 256), 256, 0, st>>>(nch, u, gl);
  return hipGetLastError();
}

// ---------------------------------------------------------------- velocity step

// z = bf16(z + dt * v): one Euler transition, product and sum each rounded in fp32.
__global__ void k_velocity_step(int64_t nch, float dt, const uint16_t *__restrict__ v, uint16_t *__restrict__ z) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  float fz[8], fv[8];
  unpack8(reinterpret_cast<const u32x4 *>(z)[c], fz);
  unpack8(reinterpret_cast<const u32x4 *>(v)[c], fv);
#pragma unroll
  for (int e = 0; e < 8; e++) fz[e] = __fadd_rn(fz[e], __fmul_rn(dt, fv[e]));
  reinterpret_cast<u32x4 *>(z)[c] = pack8(fz);
}

hipError_t launch_velocity_step(int64_t count, float dt, const uint16_t *v, uint16_t *z, hipStream_t st) {
  const int64_t nch = count / 8;
  if (nch == 0) return hipSuccess;
  k_velocity_step<<<(unsigned)((nch + 255) / 256), 256, 0, st>>>(nch, dt, v, z);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotary tables

// Position of token n along each axis.  Video token (t, h, w) rotates the first rope_t/2
// pairs by t, the next rope_h/2 by h, the last rope_w/2 by w, each section with
// frequencies theta^(-2j/section); text and audio use 1-D rotary over the head dim at their
// index in their own segment.  In the reduced layout pair token (t, h, k) sits at w = 2k+0.5.
__global__ void k_rope_tables(h3dit_layout L, int hd, int reduced, int64_t n_tok, float *__restrict__ cos_t,
                              float *__restrict__ sin_t) {
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_tok * half) return;
  const int64_t n = idx / half;
  const int j = (int)(idx % half);
  const int W = L.video_w;
  const int wr = reduced ? (W / 2 + W % 2) : W;
  const int64_t nv = (int64_t)L.video_t * L.video_h * wr;
  double pos, sec;
  int jj;
  if (n < nv) {
    const int64_t th = n / wr;
    const int c = (int)(n % wr);
    const int t = (int)(th / L.video_h), hh = (int)(th % L.video_h);
    double wpos = c;
    if (reduced) wpos = (c < W / 2) ? 2.0 * c + 0.5 : (double)(W - 1);
    if (j < L.rope_t / 2) {
      pos = t; sec = L.rope_t; jj = j;
    } else if (j < (L.rope_t + L.rope_h) / 2) {
      pos = hh; sec = L.rope_h; jj = j - L.rope_t / 2;
    } else {
      pos = wpos; sec = L.rope_w; jj = j - (L.rope_t + L.rope_h) / 2;
    }
  } else {
    int64_t p = n - nv;
    if (p >= L.n_text) p -= L.n_text;
    pos = (double)p;
    sec = hd;
    jj = j;
  }
  const double ang = pos * pow((double)L.rope_theta, -2.0 * jj / sec);
  cos_t[idx] = (float)cos(ang);
  sin_t[idx] = (float)sin(ang);
}

hipError_t launch_rope_tables(const h3dit_layout &L, int hd, int reduced, float *cos_t, float *sin_t,
                              hipStream_t st) {
  const int W = L.video_w;
  const int wr = reduced ? (W / 2 + W % 2) : W;
  const int64_t n_tok = (int64_t)L.video_t * L.video_h * wr + L.n_text + L.n_audio;
  const int64_t total = n_tok * (hd / 2);
  if (total == 0) return hipSuccess;
  k_rope_tables<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(L, hd, reduced, n_tok, cos_t, sin_t);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotary + head split (unfused form)

// One lane per (token, chunk of 8 features) of t[n][3d].  q and k: pairs (2j, 2j+1) become
// (a c - b s, a s + b c); v goes to V^T[h][i][vt_pos(tok)] (row pitch vt_pitch(n)).
__global__ void k_rope_split(int64_t n, int heads, int hd, const uint16_t *__restrict__ t,
                             const float *__restrict__ cos_t, const float *__restrict__ sin_t,
                             uint16_t *__restrict__ q, uint16_t *__restrict__ k, uint16_t *__restrict__ vt) {
  const int d = heads * hd;
  const int nch = 3 * d / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * nch) return;
  const int64_t tok = idx / nch;
  const int col = (int)(idx % nch) * 8;
  const int part = col / d, h = (col % d) / hd, i = col % hd;
  float f[8];
  unpack8(reinterpret_cast<const u32x4 *>(t + tok * 3 * d)[col / 8], f);
  if (part < 2) {
    const int half = hd / 2;
    float o[8];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const float c = cos_t[tok * half + i / 2 + p], s = sin_t[tok * half + i / 2 + p];
      const float a = f[2 * p], b = f[2 * p + 1];
      o[2 * p] = a * c - b * s;
      o[2 * p + 1] = a * s + b * c;
    }
    uint16_t *dst = part == 0 ? q : k;
    *reinterpret_cast<u32x4 *>(dst + ((int64_t)h * n + tok) * hd + i) = pack8(o);
  } else {
    const int64_t ldv = vt_pitch(n), pos = vt_pos(tok);
#pragma unroll
    for (int e = 0; e < 8; e++) vt[((int64_t)h * hd + i + e) * ldv + pos] = f2bf(f[e]);
  }
}

hipError_t launch_rope_split(int64_t n, int heads, int hd, const uint16_t *t, const float *cos_t,
                             const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *vt, hipStream_t st) {
  const int64_t total = n * (3 * heads * hd / 8);
  if (total == 0) return hipSuccess;
  k_rope_split<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(n, heads, hd, t, cos_t, sin_t, q, k, vt);
  return hipGetLastError();
}

// ---------------------------------------------------------------- token pair / restore

// One lane per (reduced token, chunk of 8).  Pair token (t,h,k) = bf16((x[2k] + x[2k+1]) * 0.5);
// the odd last column, text and audio are copied.
__global__ void k_token_pair(int rows, int W, int64_t rest, int d, const uint16_t *__restrict__ x,
                             uint16_t *__restrict__ r, uint16_t *__restrict__ r_in) {
  const int pairs = W / 2, wr = W / 2 + W % 2;
  const int nch = d / 8;
  const int64_t n_red = (int64_t)rows * wr + rest;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_red * nch) return;
  const int64_t p = idx / nch;
  const int c = (int)(idx % nch);
  u32x4 out;
  if (p < (int64_t)rows * wr) {
    const int64_t row = p / wr;
    const int col = (int)(p % wr);
    if (col < pairs) {
      float a[8], b[8], m[8];
      unpack8(reinterpret_cast<const u32x4 *>(x + (row * W + 2 * col) * d)[c], a);
      unpack8(reinterpret_cast<const u32x4 *>(x + (row * W + 2 * col + 1) * d)[c], b);
#pragma unroll
      for (int e = 0; e < 8; e++) m[e] = (a[e] + b[e]) * 0.5f;
      out = pack8(m);
    } else {
      out = reinterpret_cast<const u32x4 *>(x + (row * W + W - 1) * d)[c];
    }
  } else {
    out = reinterpret_cast<const u32x4 *>(x + ((int64_t)rows * W + (p - (int64_t)rows * wr)) * d)[c];
  }
  reinterpret_cast<u32x4 *>(r + p * d)[c] = out;
  if (r_in) reinterpret_cast<u32x4 *>(r_in + p * d)[c] = out;
}

// One lane per (full token, chunk of 8).  Paired token: bf16(bypass + (y - r_in)) of its pair;
// others: the reduced output.
__global__ void k_token_restore(int rows, int W, int64_t rest, int d, uint16_t *x, const uint16_t *__restrict__ y,
                                const uint16_t *__restrict__ r_in) {
  const int pairs = W / 2, wr = W / 2 + W % 2;
  const int nch = d / 8;
  const int64_t n_full = (int64_t)rows * W + rest;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_full * nch) return;
  const int64_t i = idx / nch;
  const int c = (int)(idx % nch);
  u32x4 *xi = reinterpret_cast<u32x4 *>(x + i * d) + c;
  if (i < (int64_t)rows * W) {
    const int64_t row = i / W;
    const int col = (int)(i % W);
    const int64_t p = row * wr + (col / 2 < pairs ? col / 2 : wr - 1);
    if (col / 2 < pairs) {
      float b[8], yy[8], ri[8], o[8];
      unpack8(*xi, b);
      unpack8(reinterpret_cast<const u32x4 *>(y + p * d)[c], yy);
      unpack8(reinterpret_cast<const u32x4 *>(r_in + p * d)[c], ri);
#pragma unroll
      for (int e = 0; e < 8; e++) o[e] = b[e] + (yy[e] - ri[e]);
      *xi = pack8(o);
    } else {
      *xi = reinterpret_cast<const u32x4 *>(y + p * d)[c];
    }
  } else {
    *xi = reinterpret_cast<const u32x4 *>(y + ((int64_t)rows * wr + (i - (int64_t)rows * W)) * d)[c];
  }
}

hipError_t launch_token_pair(const h3dit_layout &L, int d, const uint16_t *x, uint16_t *r, uint16_t *r_in,
                             hipStream_t st) {
  const int rows = L.video_t * L.video_h, W = L.video_w;
  const int64_t rest = (int64_t)L.n_text + L.n_audio;
  const int64_t total = ((int64_t)rows * (W / 2 + W % 2) + rest) * (d / 8);
  if (total == 0) return hipSuccess;
  k_token_pair<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(rows, W, rest, d, x, r, r_in);
  return hipGetLastError();
}

hipError_t launch_token_restore(const h3dit_layout &L, int d, uint16_t *x, const uint16_t *y, const uint16_t *r_in,
                                hipStream_t st) {
  const int rows = L.video_t * L.video_h, W = L.video_w;
  const int64_t rest = (int64_t)L.n_text + L.n_audio;
  const int64_t total = ((int64_t)rows * W + rest) * (d / 8);
  if (total == 0) return hipSuccess;
  k_token_restore<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(rows, W, rest, d, x, y, r_in);
  return hipGetLastError();
}

}  // namespace h3
