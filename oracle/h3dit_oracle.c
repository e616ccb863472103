/*
 * CPU oracle for the MiniMax-H3 single-stream Omni DiT block — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp32 implementation of what one block (and a stack of blocks) computes,
 * written from the pages' prose description.  It is what the HIP library is checked
 * against; nothing in the product path may call it.  Source abbreviations ([RV], [DD],
 * [NS]) are expanded in h3dit_oracle.h.
 *
 * What the pages fix, and where:
 *  - one single-stream transformer block over a joint video + text + audio token
 *    sequence, with full (non-sparse) attention: [RV] "h3.c README" table of components;
 *    [DD] "MiniMax H3：原生音频视频一体化生成" (single dense Omni Transformer);
 *  - AdaLN modulation that can be precomputed per block: [DD] same section;
 *  - a gated attention residual followed by the MLP's AdaLN, and the MLP residual gate
 *    followed by the next block's attention AdaLN, the rounded bf16 residual being
 *    written exactly between them: [DD] "DiT 融合内核", 门控 AdaLN 融合;
 *  - QKV projection written head-major for attention, then the attention-output
 *    projection: [DD] "h3.c 的核心设计" (TensorOps paragraph);
 *  - the int8 scheme (dynamic per-token activations, per-output-channel weight scales,
 *    one scale per 1024 channels of the FC2 input): [DD] "int8 量化：从 36 秒到 19 秒";
 *  - token reduction (horizontal video pairs after block 3, full-resolution bypass,
 *    restore as original value plus the pair's update before block 40):
 *    [DD] "Token 缩减：28% 的去噪时间消减".
 * Readings where the pages are silent (each repeated at its use): pre-norm AdaLN of the
 * form LN(x)(1+scale)+shift without a learned affine, eps 1e-6; no biases; GELU with the
 * tanh approximation; 3-axis rotary embedding with interleaved pairs; every projection
 * output rounded to bf16 before any following elementwise step; int8 scale = absmax/127
 * with round-half-even of v/s.
 *
 * Every function is parity pinned by the CPU test suite (closed forms, invariants,
 * brute force and library routines) except where its comment says otherwise.
 */
#include "h3dit_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 */

static float bf2f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest with ties to even on the 16 dropped bits (finite inputs). */
static uint16_t f2bf(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OpenMP threads the oracle's parallel loops use (the host cores it runs on). */
int32_t orc_num_threads(void) {
  int32_t n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = (int32_t)omp_get_num_threads();
  }
  return n;
}

void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = f2bf(in[i]);
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

/* ---------------------------------------------------------------- token layout + rotary */

/* Tokens: video (t, h, w) row-major, then text, then audio.  In the reduced layout each
 * (t, h) video row holds floor(w/2) pair tokens followed by the unpaired last column when
 * w is odd ([DD] "Token 缩减": horizontal neighbours are paired; order is a reading). */
int32_t orc_layout_tokens(const orc_layout *L, int32_t reduced) {
  int32_t wr = reduced ? (L->video_w / 2 + L->video_w % 2) : L->video_w;
  return L->video_t * L->video_h * wr + L->n_text + L->n_audio;
}

/* cos/sin tables [n_tokens][head_dim/2], angles in double, stored as fp32.
 * Reading (the pages only say that spatial rotary positions exist and are rescaled for a
 * preview canvas, [NS] "极简主控逻辑"): video tokens rotate pair j of the head dim by
 * the position along one axis; the first split_t/2 pairs use t, the next split_h/2 use h,
 * the last split_w/2 use w, each section with frequencies theta^(-2j/section_dim).
 * Text and audio tokens use plain 1-D rotary over the whole head dim with their index
 * inside their own segment.  A reduced pair token sits at w = 2k + 0.5. */
int32_t orc_rope_tables(const orc_layout *L, int32_t hd, int32_t reduced, float *cosv, float *sinv) {
  if (L->split_t + L->split_h + L->split_w != hd || (L->split_t | L->split_h | L->split_w) & 1)
    return -1;
  int32_t half = hd / 2;
  int32_t W = L->video_w;
  int32_t wr = reduced ? (W / 2 + W % 2) : W;
  int64_t n = 0;
  for (int32_t t = 0; t < L->video_t; t++)
    for (int32_t h = 0; h < L->video_h; h++)
      for (int32_t c = 0; c < wr; c++, n++) {
        double wpos = c;
        if (reduced) wpos = (c < W / 2) ? 2.0 * c + 0.5 : (double)(W - 1);
        for (int32_t j = 0; j < half; j++) {
          double pos, sec;
          int32_t jj;
          if (j < L->split_t / 2) {
            pos = t; sec = L->split_t; jj = j;
          } else if (j < (L->split_t + L->split_h) / 2) {
            pos = h; sec = L->split_h; jj = j - L->split_t / 2;
          } else {
            pos = wpos; sec = L->split_w; jj = j - (L->split_t + L->split_h) / 2;
          }
          double ang = pos * pow((double)L->theta, -2.0 * jj / sec);
          cosv[n * half + j] = (float)cos(ang);
          sinv[n * half + j] = (float)sin(ang);
        }
      }
  for (int32_t seg = 0; seg < 2; seg++) {
    int32_t len = seg == 0 ? L->n_text : L->n_audio;
    for (int32_t p = 0; p < len; p++, n++)
      for (int32_t j = 0; j < half; j++) {
        double ang = (double)p * pow((double)L->theta, -2.0 * j / hd);
        cosv[n * half + j] = (float)cos(ang);
        sinv[n * half + j] = (float)sin(ang);
      }
  }
  return (int32_t)n;
}

/* ---------------------------------------------------------------- AdaLN */

/* h = bf16( LN(x) * (1 + scale) + shift ), LN without learned affine.
 * Reading: mean, then biased variance about it (two passes, /d), eps inside the sqrt;
 * (x - mean) * rstd, times (1 + scale), plus shift, each an fp32 rounding. */
void orc_adaln(int64_t n, int32_t d, float eps, const uint16_t *x, const uint16_t *shift,
               const uint16_t *scale, uint16_t *h, float *mean, float *rstd) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++) {
    const uint16_t *xr = x + r * d;
    float mu = 0.0f;
    for (int32_t i = 0; i < d; i++) mu += bf2f(xr[i]);
    mu = mu / (float)d;
    float var = 0.0f;
    for (int32_t i = 0; i < d; i++) {
      float c = bf2f(xr[i]) - mu;
      var += c * c;
    }
    var = var / (float)d;
    float rs = 1.0f / sqrtf(var + eps);
    if (mean) mean[r] = mu;
    if (rstd) rstd[r] = rs;
    for (int32_t i = 0; i < d; i++) {
      float v = (bf2f(xr[i]) - mu) * rs;
      v = v * (1.0f + bf2f(scale[i])) + bf2f(shift[i]);
      h[r * d + i] = f2bf(v);
    }
  }
}

/* Final head of one modality ([DD] "DiT 融合内核", 最终片层直接绑定: the audio and video AdaLN
 * read their rows of the residual stream in place, and the bf16 head applies AdaLN on the way
 * into its projection): for n residual rows x, out = bf16(h W^T) with h = AdaLN(x; shift,
 * scale) rounded to bf16 (the rounding point of every other AdaLN), W bf16 [c][d], no bias. */
void orc_final_head(int64_t n, int32_t d, int32_t c, float eps, const uint16_t *x, const uint16_t *shift,
                    const uint16_t *scale, const uint16_t *w, uint16_t *out) {
  uint16_t *h = xmalloc(2 * (size_t)n * d);
  float *acc = xmalloc(sizeof(float) * (size_t)n * c);
  orc_adaln(n, d, eps, x, shift, scale, h, NULL, NULL);
  orc_gemm_f32(n, c, d, h, w, acc);
  orc_f32_to_bf16(acc, out, n * c);
  free(h);
  free(acc);
}

/* ---------------------------------------------------------------- denoising loop */

/* One Euler transition of the latents with the velocity the head predicts: each element becomes
 * bf(z + dt*v), the product and the sum each rounded in fp32.  The pages ([DD] "速度/质量预设
 * 矩阵") speak of denoiser velocities and extrapolated transitions but give no sampler; this
 * plain step is the reading. */
void orc_velocity_step(int64_t n, float dt, const uint16_t *v, uint16_t *z) {
  for (int64_t i = 0; i < n; i++) {
    float prod = dt * bf2f(v[i]);
    z[i] = f2bf(bf2f(z[i]) + prod);
  }
}

/* Schedule of a denoising run ([DD] "速度/质量预设矩阵" and "Token 缩减").  For each step i of
 * `steps` it writes fresh[i] (the denoiser is evaluated), core[i] (the block stack runs),
 * eval[i] (which stack run the velocity comes from) and restore[i] (that run's token restore
 * block, -1 without reduction).  Readings: with whole-denoiser reuse r, the evaluated steps are
 * the multiples of r and the last step (20 steps give 20, 11 and 8 evaluations for r = 1, 2,
 * 3, the counts the pages print); skipped steps keep the last velocity.  With core reuse c the
 * head runs every step and the stack on the multiples of c and the last step.  The first
 * `early` stack runs restore before block `restore_early`, the rest before `restore_late`
 * (40, 30 and ten on the pages).  Returns the number of stack runs, or -1 for an invalid
 * request (reuse and core reuse together, counts below one, a restore not after the
 * reduction block). */
int32_t orc_denoise_plan(int32_t steps, int32_t reuse, int32_t core_reuse, int32_t reduce_after,
                         int32_t restore_early, int32_t restore_late, int32_t early, int32_t *fresh,
                         int32_t *core, int32_t *eval, int32_t *restore) {
  if (steps < 1 || reuse < 1 || core_reuse < 1) return -1;
  if (reuse > 1 && core_reuse > 1) return -1;
  if (reduce_after >= 0 && (restore_early <= reduce_after || restore_late <= reduce_after || early < 0)) return -1;
  int32_t runs = 0;
  for (int32_t i = 0; i < steps; i++) {
    int32_t is_last = (i == steps - 1);
    fresh[i] = (i % reuse == 0) || is_last;
    core[i] = fresh[i] && ((i % core_reuse == 0) || is_last);
    if (core[i]) runs += 1;
    eval[i] = runs - 1;
    if (reduce_after < 0) restore[i] = -1;
    else restore[i] = (eval[i] < early) ? restore_early : restore_late;
  }
  return runs;
}

/* ---------------------------------------------------------------- int8 */

/* Symmetric int8 code of a span of bf16 values ([DD] "int8 量化"): scale = absmax / 127 by
 * IEEE division, code = round-half-even(v / scale), clamped to +-127; an all-zero span has
 * scale 0 and codes 0.  One span per (row, group); group == cols gives per-row codes. */
static void q8_span(const uint16_t *v, int64_t len, int8_t *q, float *s) {
  float a = 0.0f;
  for (int64_t i = 0; i < len; i++) {
    float m = fabsf(bf2f(v[i]));
    if (m > a) a = m;
  }
  float sc = a / 127.0f;
  *s = sc;
  for (int64_t i = 0; i < len; i++) {
    float c = 0.0f;
    if (sc != 0.0f) c = rintf(bf2f(v[i]) / sc);
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    q[i] = (int8_t)c;
  }
}

void orc_q8_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v, int8_t *q, float *s) {
  int64_t ng = cols / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t g = 0; g < ng; g++)
      q8_span(v + r * cols + g * group, group, q + r * cols + g * group, s + r * ng + g);
}

/* Per-output-channel weight codes: one span per row of W[out][in]. */
void orc_quantize_weights(int64_t rows, int64_t cols, const uint16_t *w, int8_t *q, float *s) {
  orc_q8_rows(rows, cols, cols, w, q, s);
}

/* ---------------------------------------------------------------- projections */

/* acc[m][n] = sum_k A[m][k] * W[n][k] in fp32, k ascending (W is [out][in]).
 * W is first copied transposed so the inner loop runs over n; each acc[m][n] still adds
 * its terms one at a time in ascending k. */
void orc_gemm_f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *W, float *acc) {
  float *wt = xmalloc(sizeof(float) * (size_t)(K * N));
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; k++)
    for (int64_t n = 0; n < N; n++) wt[k * N + n] = bf2f(W[n * K + k]);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    float *c = acc + m * N;
    for (int64_t n = 0; n < N; n++) c[n] = 0.0f;
    for (int64_t k = 0; k < K; k++) {
      float a = bf2f(A[m * K + k]);
      const float *w = wt + k * N;
      for (int64_t n = 0; n < N; n++) c[n] += a * w[n];
    }
  }
  free(wt);
}

/* acc[m][n] = sum_k A[m][k] * W[n][k] exactly in int32. */
void orc_gemm_i32(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *W, int32_t *acc) {
  int32_t *wt = xmalloc(sizeof(int32_t) * (size_t)(K * N));
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; k++)
    for (int64_t n = 0; n < N; n++) wt[k * N + n] = W[n * K + k];
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    int32_t *c = acc + m * N;
    for (int64_t n = 0; n < N; n++) c[n] = 0;
    for (int64_t k = 0; k < K; k++) {
      int32_t a = A[m * K + k];
      const int32_t *w = wt + k * N;
      for (int64_t n = 0; n < N; n++) c[n] += a * w[n];
    }
  }
  free(wt);
}

/* int8 projection output: bf16( ((float)acc * s_act[m]) * s_w[n] ) (order is a reading). */
void orc_dequant_bf16(int64_t M, int64_t N, const int32_t *acc, const float *sa, const float *sw,
                      uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) out[m * N + n] = f2bf(((float)acc[m * N + n] * sa[m]) * sw[n]);
}

/* FC2 on the int8 path ([DD] "int8 量化": the FC2 input carries one scale per 1024 channels
 * and the kernel keeps scaled partial products): per contiguous input group g an exact int32
 * sum, then a32 += (float)acc_g * s_act[m][g] for g ascending, then y = bf16(a32 * s_w[n]). */
void orc_fc2_int8(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t *qa, const float *sa,
                  const int8_t *qw, const float *sw, uint16_t *y) {
  int64_t ng = K / group;
  int32_t *wt = xmalloc(sizeof(int32_t) * (size_t)(K * N));
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; k++)
    for (int64_t n = 0; n < N; n++) wt[k * N + n] = qw[n * K + k];
#pragma omp parallel
  {
    int32_t *iacc = xmalloc(sizeof(int32_t) * (size_t)N);
    float *a32 = xmalloc(sizeof(float) * (size_t)N);
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; m++) {
      for (int64_t n = 0; n < N; n++) a32[n] = 0.0f;
      for (int64_t g = 0; g < ng; g++) {
        for (int64_t n = 0; n < N; n++) iacc[n] = 0;
        for (int64_t k = g * group; k < (g + 1) * group; k++) {
          int32_t a = qa[m * K + k];
          const int32_t *w = wt + k * N;
          for (int64_t n = 0; n < N; n++) iacc[n] += a * w[n];
        }
        float s = sa[m * ng + g];
        for (int64_t n = 0; n < N; n++) a32[n] = a32[n] + (float)iacc[n] * s;
      }
      for (int64_t n = 0; n < N; n++) y[m * N + n] = f2bf(a32[n] * sw[n]);
    }
    free(iacc);
    free(a32);
  }
  free(wt);
}

/* ---------------------------------------------------------------- rotary + head split */

/* t[N][3d] = [q | k | v] with head h at columns h*hd .. h*hd+hd-1 of each third.
 * q and k pair (2j, 2j+1) is rotated by the token's angle j: (a c - b s, a s + b c),
 * from the bf16-rounded projection, rounded once; v is copied.  Outputs are head-major
 * [H][N][hd] ([DD] "h3.c 的核心设计": Q/K/V are routed straight into the head-major
 * attention input).  Interleaved pairs are a reading. */
void orc_rope_split(int64_t N, int32_t d, int32_t H, int32_t hd, const uint16_t *t,
                    const float *cosv, const float *sinv, uint16_t *q, uint16_t *k, uint16_t *v) {
  int32_t half = hd / 2;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++)
    for (int32_t h = 0; h < H; h++) {
      const uint16_t *tq = t + n * 3 * d + h * hd;
      const uint16_t *tk = tq + d;
      const uint16_t *tv = tq + 2 * d;
      int64_t o = ((int64_t)h * N + n) * hd;
      for (int32_t j = 0; j < half; j++) {
        float c = cosv[n * half + j], s = sinv[n * half + j];
        float a = bf2f(tq[2 * j]), b = bf2f(tq[2 * j + 1]);
        q[o + 2 * j] = f2bf(a * c - b * s);
        q[o + 2 * j + 1] = f2bf(a * s + b * c);
        a = bf2f(tk[2 * j]);
        b = bf2f(tk[2 * j + 1]);
        k[o + 2 * j] = f2bf(a * c - b * s);
        k[o + 2 * j + 1] = f2bf(a * s + b * c);
      }
      for (int32_t i = 0; i < hd; i++) v[o + i] = tv[i];
    }
}

/* ---------------------------------------------------------------- attention */

/* Full non-causal attention per head ([RV] README: the public release uses full attention):
 * s_m = (1/sqrt(hd)) * <q_n, k_m>, M = max s, e_m = exp(s_m - M), L = sum e,
 * o_n = bf16( (sum_m e_m v_m) / L ).  Sums ascend in m and i.  q / o hold Nq query rows
 * per head (all N tokens, or any subset of them), k / v hold all N key rows. */
void orc_attention(int32_t H, int64_t Nq, int64_t N, int32_t hd, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, uint16_t *o, float *row_max, float *row_sum) {
  float alpha = 1.0f / sqrtf((float)hd);
  float *kf = xmalloc(sizeof(float) * (size_t)(H * N * hd));
  float *vf = xmalloc(sizeof(float) * (size_t)(H * N * hd));
  for (int64_t i = 0; i < (int64_t)H * N * hd; i++) {
    kf[i] = bf2f(k[i]);
    vf[i] = bf2f(v[i]);
  }
#pragma omp parallel
  {
    float *e = xmalloc(sizeof(float) * (size_t)N);
    float *acc = xmalloc(sizeof(float) * (size_t)hd);
    float *qf = xmalloc(sizeof(float) * (size_t)hd);
#pragma omp for schedule(static)
    for (int64_t hn = 0; hn < (int64_t)H * Nq; hn++) {
      int64_t h = hn / Nq;
      for (int32_t i = 0; i < hd; i++) qf[i] = bf2f(q[hn * hd + i]);
      float mx = -INFINITY;
      for (int64_t m = 0; m < N; m++) {
        const float *km = kf + (h * N + m) * hd;
        float dot = 0.0f;
        for (int32_t i = 0; i < hd; i++) dot += qf[i] * km[i];
        e[m] = alpha * dot;
        if (e[m] > mx) mx = e[m];
      }
      float sum = 0.0f;
      for (int64_t m = 0; m < N; m++) {
        e[m] = expf(e[m] - mx);
        sum += e[m];
      }
      for (int32_t i = 0; i < hd; i++) acc[i] = 0.0f;
      for (int64_t m = 0; m < N; m++) {
        const float *vm = vf + (h * N + m) * hd;
        for (int32_t i = 0; i < hd; i++) acc[i] += e[m] * vm[i];
      }
      for (int32_t i = 0; i < hd; i++) o[hn * hd + i] = f2bf(acc[i] / sum);
      if (row_max) row_max[hn] = mx;
      if (row_sum) row_sum[hn] = sum;
    }
    free(e);
    free(acc);
    free(qf);
  }
  free(kf);
  free(vf);
}

/* ---------------------------------------------------------------- MLP activation + gate */

/* GELU, tanh form (the pages leave the activation unnamed; a reading):
 * gelu(u) = 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), evaluated in double and
 * rounded once to fp32.  0.5 (1 + tanh z) = 1 / (1 + e^(-2z)) exactly; that form is used
 * because 1 + tanh(z) cancels for z << 0 (in fp32 it loses every bit below u ~ -3). */
float orc_gelu_tanh_f32(float u) {
  double x = u;
  double z = 0.7978845608 * (x + 0.044715 * x * x * x);
  return (float)(x / (1.0 + exp(-2.0 * z)));
}

void orc_gelu_rows(int64_t n, const uint16_t *u, uint16_t *gl) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) gl[i] = f2bf(orc_gelu_tanh_f32(bf2f(u[i])));
}

/* Gated residual: out = bf16(x + gate * y), gate broadcast over tokens ([DD] "DiT 融合内核":
 * the rounded bf16 residual is written).  gate*y of two bf16 values is exact in fp32. */
void orc_gate(int64_t n, int32_t d, const uint16_t *x, const uint16_t *gate, const uint16_t *y,
              uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++)
    for (int32_t i = 0; i < d; i++)
      out[r * d + i] = f2bf(bf2f(x[r * d + i]) + bf2f(gate[i]) * bf2f(y[r * d + i]));
}

/* ---------------------------------------------------------------- token reduction */

/* Pair step ([DD] "Token 缩减"): adjacent horizontal video tokens (t,h,2k), (t,h,2k+1) are
 * averaged into one token, bf16((a + b) * 0.5); the odd last column, text and audio tokens are
 * copied.  Returns the reduced token count. */
int32_t orc_token_pair(const orc_layout *L, int32_t d, const uint16_t *x, uint16_t *r) {
  int32_t W = L->video_w, pairs = W / 2, wr = W / 2 + W % 2;
  int64_t rows = (int64_t)L->video_t * L->video_h;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < rows; row++) {
    for (int32_t c = 0; c < wr; c++) {
      uint16_t *dst = r + (row * wr + c) * d;
      if (c < pairs) {
        const uint16_t *a = x + (row * W + 2 * c) * d;
        const uint16_t *b = a + d;
        for (int32_t i = 0; i < d; i++) dst[i] = f2bf((bf2f(a[i]) + bf2f(b[i])) * 0.5f);
      } else {
        memcpy(dst, x + (row * W + W - 1) * d, sizeof(uint16_t) * (size_t)d);
      }
    }
  }
  int64_t rest = L->n_text + L->n_audio;
  memcpy(r + rows * wr * d, x + rows * W * d, sizeof(uint16_t) * (size_t)(rest * d));
  return (int32_t)(rows * wr + rest);
}

/* Restore step ([DD] "Token 缩减": each token returns as its original value plus its pair's
 * learned update): paired token i of pair p gets bf16(bypass_i + (y_p - r_in_p)); the
 * unpaired column, text and audio take y directly.  r_in is the reduced residual as it
 * entered the first reduced block. */
int32_t orc_token_restore(const orc_layout *L, int32_t d, const uint16_t *bypass, const uint16_t *y,
                          const uint16_t *r_in, uint16_t *x) {
  int32_t W = L->video_w, pairs = W / 2, wr = W / 2 + W % 2;
  int64_t rows = (int64_t)L->video_t * L->video_h;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < rows; row++) {
    for (int32_t c = 0; c < W; c++) {
      int64_t i = row * W + c;
      int64_t p = row * wr + (c / 2 < pairs ? c / 2 : wr - 1);
      if (c / 2 < pairs) {
        for (int32_t e = 0; e < d; e++) {
          float upd = bf2f(y[p * d + e]) - bf2f(r_in[p * d + e]);
          x[i * d + e] = f2bf(bf2f(bypass[i * d + e]) + upd);
        }
      } else {
        memcpy(x + i * d, y + p * d, sizeof(uint16_t) * (size_t)d);
      }
    }
  }
  int64_t rest = L->n_text + L->n_audio;
  memcpy(x + rows * W * d, y + rows * wr * d, sizeof(uint16_t) * (size_t)(rest * d));
  return (int32_t)(rows * W + rest);
}

/* ---------------------------------------------------------------- block */

/* Modulation vector i (0 shift1, 1 scale1, 2 gate1, 3 shift2, 4 scale2, 5 gate2) of the set
 * that segment s uses.  With one set every token uses it ([DD] "MiniMax H3": the AdaLN branches
 * are per block); with three sets the video, text and audio tokens each take their own (a
 * reading of the per-segment conditioning in [DD] "引用系统：Ref2VA 的多模态条件控制", where
 * audio references are held at a fixed conditioning timestep, and of the separate audio and
 * video AdaLN of [DD] "DiT 融合内核"). */
static const uint16_t *mod_vec(const orc_block *b, int32_t d, int32_t s, int32_t i) {
  const int32_t set = b->mod_sets > 1 ? s : 0;
  return b->mod + ((int64_t)set * 6 + i) * d;
}

/* rows [r0, r1) of segment s (0 video, 1 text, 2 audio) of the current sequence */
static void segment_rows(const orc_dims *D, int32_t s, int64_t *r0, int64_t *r1) {
  const int64_t b1 = D->n_video, b2 = (int64_t)D->n_video + D->n_text, N = D->n_tokens;
  *r0 = s == 0 ? 0 : s == 1 ? b1 : b2;
  *r1 = s == 0 ? b1 : s == 1 ? b2 : N;
}

/* One projection y = bf16(A W^T): bf16 weights, or int8 codes of A per row (span K) with
 * per-output-channel weight codes and the dequantisation of orc_dequant_bf16. */
static void project(int64_t M, int64_t N, int64_t K, const uint16_t *A, int32_t int8,
                    const uint16_t *W, const int8_t *qw, const float *sw, uint16_t *out) {
  if (!int8) {
    float *acc = xmalloc(sizeof(float) * (size_t)(M * N));
    orc_gemm_f32(M, N, K, A, W, acc);
    orc_f32_to_bf16(acc, out, M * N);
    free(acc);
  } else {
    int8_t *qa = xmalloc((size_t)(M * K));
    float *sa = xmalloc(sizeof(float) * (size_t)M);
    int32_t *acc = xmalloc(sizeof(int32_t) * (size_t)(M * N));
    orc_q8_rows(M, K, K, A, qa, sa);
    orc_gemm_i32(M, N, K, qa, qw, acc);
    orc_dequant_bf16(M, N, acc, sa, sw, out);
    free(qa);
    free(sa);
    free(acc);
  }
}

/* Gate then AdaLN of the gated residual.  fused = one pass per row; otherwise the whole gate
 * first, then the whole AdaLN.  Both read the rounded residual, so both give the same bytes. */
static void gate_then_adaln(int64_t n, int32_t d, float eps, const uint16_t *x, const uint16_t *gate,
                            const uint16_t *y, uint16_t *xout, const uint16_t *shift,
                            const uint16_t *scale, uint16_t *h, int32_t fused) {
  if (!fused) {
    orc_gate(n, d, x, gate, y, xout);
    if (h) orc_adaln(n, d, eps, xout, shift, scale, h, NULL, NULL);
    return;
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++) {
    orc_gate(1, d, x + r * d, gate, y + r * d, xout + r * d);
    if (h) orc_adaln(1, d, eps, xout + r * d, shift, scale, h + r * d, NULL, NULL);
  }
}

/* Block body.  h1_in: AdaLN1 output already produced by the previous block (or NULL);
 * next: the following block whose AdaLN1 the final gate also produces into h1_next (or NULL). */
static int32_t block_body(const orc_dims *D, const orc_block *B, const float *cosv, const float *sinv,
                          uint16_t *x, const uint16_t *h1_in, const orc_block *next,
                          uint16_t *h1_next, int32_t fused, orc_taps *T) {
  int64_t N = D->n_tokens;
  int32_t d = D->hidden, H = D->heads, hd = D->head_dim, f = D->mlp;
  /* which projections run on int8 codes: 1 all four, 2 the MLP pair, 3 the attention pair */
  const int32_t i8_attn = B->int8 == 1 || B->int8 == 3, i8_mlp = B->int8 == 1 || B->int8 == 2;
  if (d != H * hd || N <= 0 || f <= 0 || B->int8 < 0 || B->int8 > 3 ||
      (i8_mlp && (D->fc2_group <= 0 || f % D->fc2_group)))
    return -1;
  if (D->n_video < 0 || D->n_text < 0 || (int64_t)D->n_video + D->n_text > N || (B->mod_sets != 1 && B->mod_sets != 3))
    return -1;
  size_t Nd = (size_t)N * d, Nf = (size_t)N * f;
  uint16_t *h1 = xmalloc(2 * Nd), *t = xmalloc(6 * Nd), *q = xmalloc(2 * Nd), *k = xmalloc(2 * Nd),
           *v = xmalloc(2 * Nd), *o = xmalloc(2 * Nd), *ot = xmalloc(2 * Nd), *y1 = xmalloc(2 * Nd),
           *x1 = xmalloc(2 * Nd), *h2 = xmalloc(2 * Nd), *u = xmalloc(2 * Nf), *gl = xmalloc(2 * Nf),
           *y2 = xmalloc(2 * Nd);

  /* AdaLN1 (shift1, scale1), segment by segment */
  if (h1_in) {
    memcpy(h1, h1_in, 2 * Nd);
  } else {
    for (int32_t sg = 0; sg < 3; sg++) {
      int64_t r0, r1;
      segment_rows(D, sg, &r0, &r1);
      if (r1 > r0)
        orc_adaln(r1 - r0, d, D->ln_eps, x + r0 * d, mod_vec(B, d, sg, 0), mod_vec(B, d, sg, 1), h1 + r0 * d,
                  NULL, NULL);
    }
  }
  /* QKV projection, rotary, head split */
  project(N, 3 * d, d, h1, i8_attn, B->wqkv, B->qqkv, B->sqkv, t);
  orc_rope_split(N, d, H, hd, t, cosv, sinv, q, k, v);
  /* attention, then the head-major output read as [N][d] (column h*hd + i) */
  orc_attention(H, N, N, hd, q, k, v, o, T ? T->att_max : NULL, T ? T->att_sum : NULL);
  for (int64_t n = 0; n < N; n++)
    for (int32_t h = 0; h < H; h++)
      memcpy(ot + n * d + h * hd, o + ((int64_t)h * N + n) * hd, 2 * (size_t)hd);
  /* output projection */
  project(N, d, d, ot, i8_attn, B->wo, B->qo, B->so, y1);
  /* gate1 (x1 = x + g1 y1) then AdaLN2 (shift2, scale2) of the rounded x1 */
  for (int32_t sg = 0; sg < 3; sg++) {
    int64_t r0, r1;
    segment_rows(D, sg, &r0, &r1);
    if (r1 > r0)
      gate_then_adaln(r1 - r0, d, D->ln_eps, x + r0 * d, mod_vec(B, d, sg, 2), y1 + r0 * d, x1 + r0 * d,
                      mod_vec(B, d, sg, 3), mod_vec(B, d, sg, 4), h2 + r0 * d, fused);
  }
  /* FC1, GELU */
  project(N, f, d, h2, i8_mlp, B->w1, B->q1, B->s1, u);
  orc_gelu_rows((int64_t)Nf, u, gl);
  /* FC2 */
  if (!i8_mlp) {
    project(N, d, f, gl, 0, B->w2, NULL, NULL, y2);
  } else {
    int64_t ng = f / D->fc2_group;
    int8_t *qg = xmalloc(Nf);
    float *sg = xmalloc(sizeof(float) * (size_t)N * ng);
    orc_q8_rows(N, f, D->fc2_group, gl, qg, sg);
    orc_fc2_int8(N, d, f, D->fc2_group, qg, sg, B->q2, B->s2, y2);
    free(qg);
    free(sg);
  }
  /* gate2 (x2 = x1 + g2 y2), optionally followed by the next block's AdaLN1 */
  for (int32_t sg = 0; sg < 3; sg++) {
    int64_t r0, r1;
    segment_rows(D, sg, &r0, &r1);
    if (r1 > r0)
      gate_then_adaln(r1 - r0, d, D->ln_eps, x1 + r0 * d, mod_vec(B, d, sg, 5), y2 + r0 * d, x + r0 * d,
                      next ? mod_vec(next, d, sg, 0) : NULL, next ? mod_vec(next, d, sg, 1) : NULL,
                      next ? h1_next + r0 * d : NULL, fused);
  }

  if (T) {
    if (T->h1) memcpy(T->h1, h1, 2 * Nd);
    if (T->t) memcpy(T->t, t, 6 * Nd);
    if (T->q) memcpy(T->q, q, 2 * Nd);
    if (T->k) memcpy(T->k, k, 2 * Nd);
    if (T->v) memcpy(T->v, v, 2 * Nd);
    if (T->o) memcpy(T->o, o, 2 * Nd);
    if (T->y1) memcpy(T->y1, y1, 2 * Nd);
    if (T->x1) memcpy(T->x1, x1, 2 * Nd);
    if (T->h2) memcpy(T->h2, h2, 2 * Nd);
    if (T->u) memcpy(T->u, u, 2 * Nf);
    if (T->gl) memcpy(T->gl, gl, 2 * Nf);
    if (T->y2) memcpy(T->y2, y2, 2 * Nd);
  }
  free(h1); free(t); free(q); free(k); free(v); free(o); free(ot); free(y1); free(x1);
  free(h2); free(u); free(gl); free(y2);
  return 0;
}

int32_t orc_block_fwd(const orc_dims *dims, const orc_block *blk, const float *cosv, const float *sinv,
                      uint16_t *x, int32_t fused, orc_taps *taps) {
  return block_body(dims, blk, cosv, sinv, x, NULL, NULL, NULL, fused, taps);
}

/* Stack of blocks with optional token reduction ([DD] "Token 缩减"; block indices from 0):
 * after block reduce_after the residual is paired (the full residual is kept as the bypass
 * and the reduced residual as r_in); before block restore_before (or after the last block
 * if the stack ends first) every token is restored.  fused != 0 lets each block's final
 * gate also produce the next block's AdaLN1, except across a pair or restore step. */
int32_t orc_stack_fwd(const orc_dims *dims, const orc_layout *L, int32_t n_blocks, const orc_block *blocks,
                      int32_t reduce_after, int32_t restore_before, uint16_t *x, int32_t fused,
                      const float *cf_in, const float *sf_in, const float *cr_in, const float *sr_in) {
  int32_t reduce = reduce_after >= 0;
  int32_t hd = dims->head_dim, d = dims->hidden;
  int32_t Nf = orc_layout_tokens(L, 0), Nr = orc_layout_tokens(L, 1);
  if (Nf != dims->n_tokens || n_blocks <= 0) return -1;
  if (reduce && (restore_before <= reduce_after || reduce_after >= n_blocks)) return -1;
  /* rotary tables: the caller's, else the layout's own */
  float *cf = xmalloc(sizeof(float) * (size_t)Nf * hd / 2), *sf = xmalloc(sizeof(float) * (size_t)Nf * hd / 2);
  float *cr = xmalloc(sizeof(float) * (size_t)Nr * hd / 2), *sr = xmalloc(sizeof(float) * (size_t)Nr * hd / 2);
  if (orc_rope_tables(L, hd, 0, cf, sf) < 0 || orc_rope_tables(L, hd, 1, cr, sr) < 0) return -1;
  if (cf_in && sf_in) {
    memcpy(cf, cf_in, sizeof(float) * (size_t)Nf * hd / 2);
    memcpy(sf, sf_in, sizeof(float) * (size_t)Nf * hd / 2);
  }
  if (cr_in && sr_in) {
    memcpy(cr, cr_in, sizeof(float) * (size_t)Nr * hd / 2);
    memcpy(sr, sr_in, sizeof(float) * (size_t)Nr * hd / 2);
  }
  uint16_t *bypass = xmalloc(2 * (size_t)Nf * d), *red = xmalloc(2 * (size_t)Nr * d),
           *r_in = xmalloc(2 * (size_t)Nr * d), *h1a = xmalloc(2 * (size_t)Nf * d),
           *h1b = xmalloc(2 * (size_t)Nf * d);
  int32_t reduced = 0, have_h1 = 0, rc = 0;
  for (int32_t b = 0; b < n_blocks && rc == 0; b++) {
    if (reduced && b == restore_before) {
      orc_token_restore(L, d, bypass, red, r_in, x);
      reduced = 0;
      have_h1 = 0;
    }
    orc_dims D = *dims;
    D.n_tokens = reduced ? Nr : Nf;
    D.n_video = (reduced ? Nr : Nf) - L->n_text - L->n_audio;
    D.n_text = L->n_text;
    uint16_t *cur = reduced ? red : x;
    int32_t boundary = (reduce && (b == reduce_after || b + 1 == restore_before)) || b + 1 == n_blocks;
    const orc_block *next = (fused && !boundary) ? &blocks[b + 1] : NULL;
    rc = block_body(&D, &blocks[b], reduced ? cr : cf, reduced ? sr : sf, cur, have_h1 ? h1a : NULL, next,
                    h1b, fused, NULL);
    uint16_t *tmp = h1a;
    h1a = h1b;
    h1b = tmp;
    have_h1 = next != NULL;
    if (reduce && b == reduce_after) {
      memcpy(bypass, x, 2 * (size_t)Nf * d);
      orc_token_pair(L, d, x, red);
      memcpy(r_in, red, 2 * (size_t)Nr * d);
      reduced = 1;
      have_h1 = 0;
    }
  }
  if (reduced) orc_token_restore(L, d, bypass, red, r_in, x);
  free(cf); free(sf); free(cr); free(sr); free(bypass); free(red); free(r_in); free(h1a); free(h1b);
  return rc;
}

/* Patch-embedding stand-in of the denoising loop (a reading: the pages name the latents and the
 * velocity head, not the map from latents to the residual): the embedding of a latent row is
 * its product with E rounded to bf16, added to the conditioning residual and rounded again. */
void orc_patch_embed(int64_t n, int32_t d, int32_t c, const uint16_t *x_in, const uint16_t *z, const uint16_t *E,
                     uint16_t *x_out) {
  float *acc = xmalloc(sizeof(float) * (size_t)(n * d));
  uint16_t *e = xmalloc(2 * (size_t)(n * d));
  orc_gemm_f32(n, d, c, z, E, acc);
  orc_f32_to_bf16(acc, e, n * d);
  for (int64_t i = 0; i < n * d; i++) acc[i] = bf2f(x_in[i]) + bf2f(e[i]);
  orc_f32_to_bf16(acc, x_out, n * d);
  free(acc);
  free(e);
}
