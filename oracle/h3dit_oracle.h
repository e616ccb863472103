/*
 * CPU oracle for the MiniMax-H3 single-stream Omni DiT block — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * call this library.  It shares no code, header, table or helper with the HIP path.
 *
 * Sources (web pages about antirez's h3.c / h3-metal engine):
 *   [RV]  alphalab.site, "h3-metal 把 MiniMax-H3 搬上 Apple Silicon：突破與代價（2026）"
 *   [DD]  linlog.top article 1265 (h3.c deep dive), sections
 *         "MiniMax H3：原生音频视频一体化生成", "h3.c 的核心设计", "int8 量化：从 36 秒到 19 秒",
 *         "DiT 融合内核：减少全局内存往返", "Token 缩减：28% 的去噪时间消减", "速度/质量预设矩阵"
 *   [NS]  daily.steinslab.io, "零 Python 依赖：Redis 作者的 3.5 秒端侧实验"
 * The pages describe the block in words only; widths, the activation, eps, the
 * rotary split and every rounding point are readings, each stated where it is used.
 *
 * Conventions: bf16 values travel as uint16_t bit patterns; every matrix is row-major;
 * weights are [out][in]; all arithmetic is IEEE fp32 (the library is built with
 * -ffp-contract=off, so a*b+c is two roundings), sums run in ascending index order.
 */
#ifndef H3DIT_ORACLE_H
#define H3DIT_ORACLE_H
#include <stdint.h>

typedef struct {
  int32_t n_tokens, hidden, heads, head_dim, mlp, fc2_group;
  float ln_eps;
  int32_t n_video, n_text;           /* segments of the current sequence: video rows, then text,
                                        then audio (the rest); they select the modulation set */
} orc_dims;

typedef struct {
  int32_t video_t, video_h, video_w; /* video tokens first, (t, h, w) row-major */
  int32_t n_text, n_audio;           /* then text, then audio */
  int32_t split_t, split_h, split_w; /* head-dim share of each video axis (sum = head_dim) */
  float theta;
} orc_layout;

typedef struct {
  int32_t int8;                         /* int8 projections ([DD] "int8 量化" table rows): 0 none
                                           (bf16); 1 all four; 2 FC1 and FC2 only ("int8 MLP");
                                           3 QKV and the output projection only (the int8-QKV-only
                                           path compared with the full int8 path) */
  const uint16_t *wqkv, *wo, *w1, *w2;  /* bf16 [3d][d], [d][d], [f][d], [d][f] */
  const int8_t *qqkv, *qo, *q1, *q2;    /* int8, same shapes */
  const float *sqkv, *so, *s1, *s2;     /* fp32 per output row */
  const uint16_t *mod;                  /* bf16 [mod_sets][6][d]: shift1 scale1 gate1 shift2 scale2 gate2 */
  int32_t mod_sets;                     /* 1: one set for every token; 3: video, text, audio sets */
} orc_block;

typedef struct {                        /* optional stage outputs; any pointer may be NULL */
  uint16_t *h1;                         /* [N][d] AdaLN1 output */
  uint16_t *t;                          /* [N][3d] QKV projection before rotary */
  uint16_t *q, *k, *v;                  /* [H][N][hd] */
  uint16_t *o;                          /* [H][N][hd] attention output */
  uint16_t *y1, *x1, *h2, *u, *gl, *y2; /* [N][d] ... [N][f] ... [N][d] */
  float *att_max, *att_sum;             /* [H][N] softmax row max and row sum */
} orc_taps;

/* scalar helpers exposed for the pins */
int32_t orc_num_threads(void);
void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t n);
float orc_gelu_tanh_f32(float u);
int32_t orc_layout_tokens(const orc_layout *L, int32_t reduced);
int32_t orc_rope_tables(const orc_layout *L, int32_t head_dim, int32_t reduced, float *cosv, float *sinv);

/* stages */
void orc_adaln(int64_t n, int32_t d, float eps, const uint16_t *x, const uint16_t *shift,
               const uint16_t *scale, uint16_t *h, float *mean, float *rstd);
void orc_q8_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v, int8_t *q, float *s);
void orc_quantize_weights(int64_t rows, int64_t cols, const uint16_t *w, int8_t *q, float *s);
void orc_gemm_f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *W, float *acc);
void orc_gemm_i32(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *W, int32_t *acc);
void orc_rope_split(int64_t N, int32_t d, int32_t H, int32_t hd, const uint16_t *t,
                    const float *cosv, const float *sinv, uint16_t *q, uint16_t *k, uint16_t *v);
void orc_attention(int32_t H, int64_t Nq, int64_t N, int32_t hd, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, uint16_t *o, float *row_max, float *row_sum);
void orc_gelu_rows(int64_t n, const uint16_t *u, uint16_t *gl);
void orc_gate(int64_t n, int32_t d, const uint16_t *x, const uint16_t *gate, const uint16_t *y,
              uint16_t *out);
void orc_fc2_int8(int64_t M, int64_t N, int64_t K, int64_t group, const int8_t *qa,
                  const float *sa, const int8_t *qw, const float *sw, uint16_t *y);
void orc_dequant_bf16(int64_t M, int64_t N, const int32_t *acc, const float *sa, const float *sw,
                      uint16_t *out);
void orc_final_head(int64_t n, int32_t d, int32_t c, float eps, const uint16_t *x, const uint16_t *shift,
                    const uint16_t *scale, const uint16_t *w, uint16_t *out);
void orc_velocity_step(int64_t n, float dt, const uint16_t *v, uint16_t *z);
int32_t orc_denoise_plan(int32_t steps, int32_t reuse, int32_t core_reuse, int32_t reduce_after,
                         int32_t restore_early, int32_t restore_late, int32_t early, int32_t *fresh,
                         int32_t *core, int32_t *eval, int32_t *restore);
int32_t orc_token_pair(const orc_layout *L, int32_t d, const uint16_t *x, uint16_t *r);
int32_t orc_token_restore(const orc_layout *L, int32_t d, const uint16_t *bypass,
                          const uint16_t *y, const uint16_t *r_in, uint16_t *x);

/* whole block and stack */
int32_t orc_block_fwd(const orc_dims *dims, const orc_block *blk, const float *cosv,
                      const float *sinv, uint16_t *x, int32_t fused, orc_taps *taps);
/* cf/sf: rotary tables of the full sequence, cr/sr of the paired one (fp32 [n][head_dim/2]);
 * NULL: the tables of orc_rope_tables for the layout. */
int32_t orc_stack_fwd(const orc_dims *dims, const orc_layout *L, int32_t n_blocks,
                      const orc_block *blocks, int32_t reduce_after, int32_t restore_before,
                      uint16_t *x, int32_t fused, const float *cf, const float *sf, const float *cr,
                      const float *sr);
/* patch-embedding stand-in of the denoising loop: x_out[r] = bf16(x_in[r] + bf16(z[r] . E[j]))
 * per row r < n and feature j < d; z bf16 [n][c], E bf16 [d][c] */
void orc_patch_embed(int64_t n, int32_t d, int32_t c, const uint16_t *x_in, const uint16_t *z,
                     const uint16_t *E, uint16_t *x_out);
#endif
