// Shared device helpers of the gfx950 H3 DiT kernels: vector types, bf16 conversion,
// buffer resources for direct-to-LDS loads, wave reductions and the launch table shared by
// the host orchestration.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/h3dit.h"
#include "../../include/h3dit_stages.h"

namespace h3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// two fp32 -> two bf16 (lo in the low half), round to nearest even: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// 8 bf16 held in a 16-byte vector
__device__ __forceinline__ void unpack8(u32x4 v, float *f) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const float *f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
  return v;
}

// raw buffer resource over `bytes` bytes: loads past the end return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer byte offset `voff` into LDS at lds_base + lane*16
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, lds_void *lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_base, 16, (int)voff, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// V^T layout: row pitch (tokens rounded up to 16) and the position of token n in a row.  Keys
// are permuted inside each group of 16 (bits 2 and 3 of the index swapped) so that the 8 keys
// one lane contributes to a 16-key MFMA step of the attention value product - keys
// 4h..4h+3 and 8+4h..8+4h+3 of the step - are adjacent (one 16-byte LDS read).
__host__ __device__ __forceinline__ int64_t vt_pitch(int64_t n) { return (n + 15) / 16 * 16; }
__host__ __device__ __forceinline__ int64_t vt_pos(int64_t n) {
  return (n & ~(int64_t)15) | (n & 3) | ((n & 4) << 1) | ((n & 8) >> 1);
}

// GELU, tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), evaluated through
// the identity 0.5 (1 + tanh z) = 1 / (1 + e^(-2z)) with the hardware exp2 and reciprocal:
// u / (1 + 2^(-2 z log2 e)).  Large negative u gives exp2 = inf and an exact (signed) zero, large
// positive u gives u.  Agrees with the tanh form to a few fp32 ulps away from the far tail.
__device__ __forceinline__ float gelu_tanh(float u) {
  const float u3 = u * u * u;
  const float k = -2.0f * 0.7978845608f * 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(k * (u + 0.044715f * u3));
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// int8 codes of 8 values of one span with scale s: round-half-even(v / s) of the correctly
// rounded quotient, clamped to +-127, 0 when s == 0; packed little-endian into two words.
// inv = 1/s (correctly rounded, once per span).  The quotient is first approximated by
// t = v * inv: with |v / s| <= 127 (s is the span's absmax / 127), t and the correctly rounded
// v / s differ by at most |v/s| (2^-23 + 2^-24) < 2.3e-5, so they round to the same integer
// unless a half-integer lies within that distance of t.  Values within 4e-5 of a half-integer
// (and non-finite t) take the true division, for the whole wave at once (a uniform branch
// taken for a few percent of the 8-value chunks), so the codes are those of rintf(v / s).
// Rounding: y = t + 1.5 * 2^23 is rintf(t) + 1.5 * 2^23 exactly for |t| < 2^22 (the sum has an
// ulp of 1 and rounds to nearest even), so the low byte of y's bits is the two's complement
// code, and y - 1.5 * 2^23 is rintf(t).  |t - rintf(t)| <= 1/2, so the tie test is one
// comparison.  |t| <= 127 (1 + 2^-22) needs no clamp; the true-division path clamps.
__device__ __forceinline__ uint2 q8_pack8(const float *v, float s, float inv) {
  if (s == 0.0f) return make_uint2(0u, 0u);   // the span is all zeros
  constexpr float MAGIC = 12582912.0f;         // 1.5 * 2^23
  float y[8];
  bool exact = false;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float t = v[e] * inv;
    y[e] = t + MAGIC;
    const float d = t - (y[e] - MAGIC);
    exact |= !(fabsf(t) < 128.0f) || fabsf(d) >= 0.5f - 4e-5f;
  }
  if (__any(exact)) {
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = fminf(fmaxf(rintf(v[e] / s), -127.0f), 127.0f) + MAGIC;
  }
  // low bytes of y[0..3] and y[4..7]: two byte pairs per v_perm, then the pairs into a word
  const uint32_t p01 = __builtin_amdgcn_perm(__float_as_uint(y[1]), __float_as_uint(y[0]), 0x0c0c0400u);
  const uint32_t p23 = __builtin_amdgcn_perm(__float_as_uint(y[3]), __float_as_uint(y[2]), 0x0c0c0400u);
  const uint32_t p45 = __builtin_amdgcn_perm(__float_as_uint(y[5]), __float_as_uint(y[4]), 0x0c0c0400u);
  const uint32_t p67 = __builtin_amdgcn_perm(__float_as_uint(y[7]), __float_as_uint(y[6]), 0x0c0c0400u);
  return make_uint2(__builtin_amdgcn_perm(p23, p01, 0x05040100u), __builtin_amdgcn_perm(p67, p45, 0x05040100u));
}

}  // namespace h3

// ---------------------------------------------------------------- launchers (internal)
namespace h3 {

hipError_t launch_rope_tables(const h3dit_layout &L, int hd, int reduced, float *cos_t, float *sin_t,
                              hipStream_t st);
// one modulation set (seg1 = seg2 = n, set_stride = 0), or three sets by row segment
hipError_t launch_row(int64_t n, int d, float eps, const uint16_t *x, const uint16_t *gate,
                      const uint16_t *y, uint16_t *x_out, const uint16_t *shift, const uint16_t *scale,
                      uint16_t *h, int8_t *q, float *s, hipStream_t st, int64_t seg1 = 0, int64_t seg2 = 0,
                      int64_t set_stride = 0);
// LayerNorm statistics of n rows: stats[2 r] = mean, stats[2 r + 1] = 1/sqrt(var + eps), as
// launch_row's normalisation computes them
hipError_t launch_row_stats(int64_t n, int d, float eps, const uint16_t *x, float *stats, hipStream_t st);
// out = bf16(h W^T) with h = bf16(AdaLN(x; shift, scale)) formed while the A tiles are loaded,
// from the row statistics above (x [n][d], W [c][d], out [n][c]; d % 64 == 0, c % 128 == 0)
hipError_t launch_head_gemm(int64_t n, int c, int d, const uint16_t *x, const float *stats, const uint16_t *shift,
                            const uint16_t *scale, const uint16_t *w, uint16_t *out, hipStream_t st);
hipError_t launch_quant_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v, int hm_hd,
                             int8_t *q, float *s, hipStream_t st);
hipError_t launch_gelu(int64_t count, const uint16_t *u, uint16_t *gl, hipStream_t st);
hipError_t launch_velocity_step(int64_t count, float dt, const uint16_t *v, uint16_t *z, hipStream_t st);
hipError_t launch_rope_split(int64_t n, int heads, int hd, const uint16_t *t, const float *cos_t,
                             const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *vt, hipStream_t st);
hipError_t launch_token_pair(const h3dit_layout &L, int d, const uint16_t *x, uint16_t *r, uint16_t *r_in,
                             hipStream_t st);
hipError_t launch_token_restore(const h3dit_layout &L, int d, uint16_t *x, const uint16_t *y,
                                const uint16_t *r_in, hipStream_t st);
// Work plan of a projection: tile width, whole tiles, and the split-K of the last round.
struct LinearPlan {
  int bn;           // tile width (rows: 256)
  int n_dp;         // tiles computed whole
  int split;        // K segments per split tile
  int kt_seg;       // 128-byte K slices per segment
  int n_split;      // split tiles
  size_t part_bytes;  // workspace for their partial tiles
  int64_t n_big;    // int8 column split: columns [0, n_big) in the wide tiles (n_dp of them),
  int n_small;      // the rest in n_small 128 x 128 tiles (a second launch); otherwise N and 0
};
LinearPlan plan_linear(const h3dit_linear_args &a);
size_t linear_workspace(const h3dit_linear_args &a);
void linear_a_extent(const h3dit_linear_args &a, uint64_t *max_end, uint64_t *bad);
hipError_t launch_linear(const h3dit_linear_args &a, hipStream_t st);
hipError_t launch_attention(int heads, int64_t n, int hd, const uint16_t *q, const uint16_t *k,
                            const uint16_t *vt, uint16_t *o, float *row_max, float *row_sum, hipStream_t st);

}  // namespace h3
