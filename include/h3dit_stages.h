/*
 * h3dit_stages.h — per-kernel entry points of the H3 DiT block library.
 *
 * These expose each kernel the block and stack calls are built from, so that every stage
 * can be checked on its own and timed on its own.  The rules of h3dit.h apply (device
 * pointers, 16-byte alignment, caller-owned memory, asynchronous on `stream`, validation
 * before launch, negative status on error).  A call with nothing to do (zero rows, tokens or
 * elements) checks its sizes, returns H3DIT_OK and does not examine its pointers.  Source
 * abbreviations [RV], [DD], [NS] as in h3dit.h.
 *
 * Layouts used below:
 *   token-major  [n][d]       row n holds the d features of token n
 *   head-major   [H][n][hd]   Q, K and the attention output O
 *   V^T          [H][hd][ldv] values, transposed so the attention kernel reads them along
 *                             tokens; row pitch ldv = n rounded up to a multiple of 16, and
 *                             token t at column (t & ~15) | (t & 3) | (t & 4) << 1 | (t & 8) >> 1
 *                             (bits 2 and 3 swapped inside each group of 16), the order in
 *                             which one MFMA step of the value product consumes keys
 *                             ([DD] "h3.c 的核心设计": the projection writes the attention
 *                             inputs directly in the layout attention wants)
 */
#ifndef H3DIT_STAGES_H
#define H3DIT_STAGES_H

#include "h3dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Rotary tables cos/sin fp32 [n][head_dim/2] (device) for the layout of h3dit.h; reduced != 0
 * gives the paired sequence, where pair token (t,h,k) sits at w = 2k + 0.5.  Returns the
 * token count (>= 0) or a negative status. */
H3DIT_API int h3dit_rope_tables(const h3dit_layout *layout, int32_t head_dim, int32_t reduced, float *cos_t,
                      float *sin_t, void *stream);

/* Row kernel ([DD] "DiT 融合内核", 门控 AdaLN 融合).  Per token row r of d features:
 *   if gate != NULL:  x_out[r] = bf16(x[r] + gate * y[r])     (the residual, written exactly)
 *                     else x_out is ignored and the row is x[r]
 *   if shift != NULL: LN over the (rounded) row: mean, biased variance, eps inside sqrt;
 *                     hv = bf16(((row - mean) * rstd) * (1 + scale) + shift)
 *                     h (bf16 [n][d]) receives hv if non-NULL;
 *                     q (int8 [n][d]) / s (fp32 [n]) receive the per-row int8 code of hv
 *                     ([DD] "int8 量化": absmax/127, round-half-even) if non-NULL.
 * gate/shift/scale: bf16 [d].  x_out may equal x (in place).  d % 8 == 0, d <= 8192. */
H3DIT_API int h3dit_row_gate_adaln(int64_t n, int32_t d, float eps, const uint16_t *x, const uint16_t *gate,
                         const uint16_t *y, uint16_t *x_out, const uint16_t *shift,
                         const uint16_t *scale, uint16_t *h, int8_t *q, float *s, void *stream);

/* int8 codes of bf16 values, one span per (row, group of `group` columns): s = absmax/127,
 * q = round-half-even(v/s) clamped to +-127 ([DD] "int8 量化").  v is token-major
 * [rows][cols], or, when headmajor_hd > 0, the head-major attention output [cols/hd][rows][hd]
 * read as token-major.  q: int8 [rows][cols]; s: fp32 [rows][cols/group].
 * cols % group == 0, group % 8 == 0; head-major input needs group <= 8192. */
H3DIT_API int h3dit_quantize_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v,
                        int32_t headmajor_hd, int8_t *q, float *s, void *stream);

/* Projection out = A W^T on MFMA ([DD] "h3.c 的核心设计", "int8 量化").
 *   precision H3DIT_BF16: A bf16 [M][K] (or, with a_headmajor_hd = 64 or 128, the head-major
 *     attention output [K/hd][M][hd]; out_kind BF16 or F32 only), W bf16 [N][K],
 *     fp32 accumulation; acc value = the fp32 sum.
 *   precision H3DIT_INT8: A int8 [M][K] with a_scale fp32 [M] (a_group == 0), W int8 [N][K]
 *     with w_scale fp32 [N]; int32 accumulation; value = ((float)acc * a_scale) * w_scale.
 *     With a_group > 0 (the FC2 input), a_scale is fp32 [M][K/a_group] and
 *     value = (sum over groups g ascending of (float)acc_g * a_scale[m][g]) * w_scale[n].
 * Epilogues (out_kind):
 *   H3DIT_OUT_BF16  out bf16 [M][N] = bf16(value)
 *   H3DIT_OUT_F32   out fp32 [M][N] = value before rounding (bf16 path only)
 *   H3DIT_OUT_I32   out int32 [M][N] = raw accumulator (int8 path, a_group == 0 only)
 *   H3DIT_OUT_GELU  out bf16 [M][N] = bf16(GELU_tanh(bf16(value)))
 *   H3DIT_OUT_QKV   N = 3*heads*head_dim; t = bf16(value) split into q | k | v; q and k rotated
 *                   pairwise by cos/sin (fp32 [M][head_dim/2]) and rounded once, written
 *                   head-major to out_q, out_k; v written as V^T to out_v.
 * M >= 1; N % 128 == 0; K % 128 == 0 (int8: K % 128 == 0 and K % a_group == 0).
 * Work plan: when the output tiles do not fill whole rounds of the chip, the last columns may
 * be computed in smaller tiles by a second launch (int8 path), or the tiles of the last
 * round are computed as K segments whose fp32 (int32 on the int8 path) partial tiles go to
 * `workspace` (device, 256-byte aligned, workspace_bytes long) and are summed in segment
 * order by a second launch.  h3dit_linear_workspace gives the bytes a call needs (0 when it
 * splits nothing); a call that needs more than workspace_bytes returns H3DIT_EWORKSPACE.  The
 * plan depends on M, N, K, precision, a_group and out_kind only, so equal shapes accumulate in
 * the same order; int8 results do not depend on it at all. */
#define H3DIT_OUT_BF16 0
#define H3DIT_OUT_F32 1
#define H3DIT_OUT_I32 2
#define H3DIT_OUT_GELU 3
#define H3DIT_OUT_QKV 4
typedef struct {
  int64_t M, N, K;
  int32_t precision;
  const void *a;
  int32_t a_headmajor_hd;
  const float *a_scale;
  int32_t a_group;
  const void *w;
  const float *w_scale;
  int32_t out_kind;
  void *out;
  const float *cos_t, *sin_t;
  int32_t heads, head_dim;
  uint16_t *out_q, *out_k, *out_v;
  void *workspace;
  uint64_t workspace_bytes;
} h3dit_linear_args;
H3DIT_API int h3dit_linear(const h3dit_linear_args *args, void *stream);
/* Workspace bytes h3dit_linear needs for these arguments, written to *bytes. */
H3DIT_API int h3dit_linear_workspace(const h3dit_linear_args *args, uint64_t *bytes);
/* Host only (no device work, pointers not dereferenced): walks every A-operand load of the
 * launch h3dit_linear would make for these arguments, with the kernel's own addressing, and
 * writes the largest byte offset past `a` that any load not masked by the buffer range check
 * reads (*max_end, at most M*K*element size when the addressing is right) and the number of
 * loads whose masking is wrong (*bad: a row < M masked, a row >= M not masked, or a load
 * straddling the end of its buffer resource).  Validation as h3dit_linear. */
H3DIT_API int h3dit_linear_a_extent(const h3dit_linear_args *args, uint64_t *max_end, uint64_t *bad);

/* Rotary + head split of a token-major projection t bf16 [n][3*heads*head_dim] into q, k
 * head-major and v as V^T; the same arithmetic as H3DIT_OUT_QKV. */
H3DIT_API int h3dit_rope_split(int64_t n, int32_t heads, int32_t head_dim, const uint16_t *t, const float *cos_t,
                     const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *vt, void *stream);

/* gl = bf16(GELU_tanh(u)) elementwise over count bf16 values (count % 8 == 0). */
H3DIT_API int h3dit_gelu(int64_t count, const uint16_t *u, uint16_t *gl, void *stream);

/* Full non-causal attention ([RV] README: full attention), per head h and query n:
 *   o[h][n] = bf16( sum_m softmax_m(q[h][n] . k[h][m] / sqrt(hd)) v[h][m] ),
 * computed with an online softmax (probabilities rounded to bf16 for the value product).
 * q, k: bf16 head-major [H][n][hd]; vt: bf16 V^T [H][hd][ldv]; o: bf16 [H][n][hd], may equal q
 * (each query tile reads its own rows before writing them); V^T columns past n may hold
 * anything.  row_max / row_sum (fp32
 * [H][n], optional) receive max_m(score) and sum_m exp(score - max) in natural-log units.
 * head_dim 64 or 128. */
H3DIT_API int h3dit_attention(int32_t heads, int64_t n, int32_t head_dim, const uint16_t *q, const uint16_t *k,
                    const uint16_t *vt, uint16_t *o, float *row_max, float *row_sum, void *stream);

/* Token pair step ([DD] "Token 缩减"): r = bf16((a + b) * 0.5) for each horizontal pair
 * (t,h,2k),(t,h,2k+1) of x (bf16 [n_full][d]), the odd last column, text and audio copied;
 * reduced order per (t,h) row: pairs, then the unpaired column; then text, audio.
 * r and r_in (bf16 [n_reduced][d]) both receive the result (r_in may be NULL). */
H3DIT_API int h3dit_token_pair(const h3dit_layout *layout, int32_t d, const uint16_t *x, uint16_t *r,
                     uint16_t *r_in, void *stream);

/* Token restore step ([DD] "Token 缩减"): for paired token i of pair p,
 * x[i] = bf16(x[i] + (y[p] - r_in[p])); every other token x[i] = y[p].  x (bf16 [n_full][d])
 * holds the bypass on entry and the restored residual on return. */
H3DIT_API int h3dit_token_restore(const h3dit_layout *layout, int32_t d, uint16_t *x, const uint16_t *y,
                        const uint16_t *r_in, void *stream);

#ifdef __cplusplus
}
#endif
#endif
