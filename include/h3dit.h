/*
 * h3dit.h — C ABI of the MI355X (gfx950) library for the MiniMax-H3 single-stream Omni DiT
 * block: the forward pass of one block, and of a stack of blocks for one denoising
 * evaluation, over a joint video + text + audio token sequence, in a bf16 path and an int8
 * path.  Every step runs in hand-written HIP kernels; the library never allocates device
 * memory.
 *
 * Sources (web pages about antirez's h3.c / h3-metal engine for MiniMax-H3):
 *   [RV] alphalab.site, "h3-metal 把 MiniMax-H3 搬上 Apple Silicon：突破與代價（2026）",
 *        sections "h3.c README" (components: 50-layer single-stream Omni Transformer, full
 *        attention in the first public release) and "h3-metal 的 SSD 串流：用速度換常駐記憶體"
 *        (two alternating weight slots, next block prefetched while the current one runs).
 *   [DD] linlog.top article 1265 (h3.c deep dive), sections "MiniMax H3：原生音频视频一体化
 *        生成" (dense Omni Transformer, precomputable AdaLN branches), "h3.c 的核心设计"
 *        (QKV and attention-output projections, Q/K/V routed head-major), "int8 量化：从 36
 *        秒到 19 秒" (int8 scheme and its table), "DiT 融合内核：减少全局内存往返" (gate +
 *        AdaLN fusion, cross-block AdaLN, activation aliasing, byte-identical fallbacks),
 *        "Token 缩减：28% 的去噪时间消减" (horizontal pairing after block 3, bypass,
 *        restore before block 40, before block 30 after the first ten noise evaluations),
 *        "速度/质量预设矩阵" (denoising steps, velocity reuse, active blocks, core reuse).
 *   [NS] daily.steinslab.io, "零 Python 依赖：Redis 作者的 3.5 秒端侧实验", sections "算力拆解：如何在
 *        M5 Max 上把 16.69 秒压到 12.60 秒" (row-level int8 FC2 option) and "极简主控逻辑"
 *        (spatial rotary positions).
 * The pages give the block in prose only; widths, activation, eps and rotary layout are
 * parameters here, and each reading of an unstated detail is named where it applies.
 *
 * Common rules for every entry point:
 *  - Pointers marked "device" must be device memory of the current HIP device; "host"
 *    pointers (the argument structs, the block array) are read during the call only, except
 *    the host weights of h3dit_stack_fwd_streamed, which its copies read later.
 *  - The caller owns every buffer.  Calls are asynchronous on `stream` (a hipStream_t;
 *    NULL means the default stream); no memory is allocated and the host never waits
 *    (h3dit_stack_fwd_streamed creates five HIP events per call, and its copies from
 *    pageable host memory may run synchronously).
 *  - bf16 is passed as uint16_t bit patterns.  Matrices are row-major; weights are
 *    [out][in].  Device pointers must be 16-byte aligned.
 *  - Return: H3DIT_OK, or a negative status.  Arguments are validated before any launch;
 *    on a validation error nothing is launched and no buffer is touched.
 *  - NaN/Inf in the inputs are not checked; they propagate.
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden default visibility). */
#define H3DIT_API __attribute__((visibility("default")))

#define H3DIT_OK 0
#define H3DIT_EINVAL (-1)       /* bad sizes, NULL or misaligned pointer, bad schedule */
#define H3DIT_EWORKSPACE (-2)   /* workspace too small; required size written back */
#define H3DIT_EUNSUPPORTED (-3) /* head_dim not 64/128, or device is not gfx950 */
#define H3DIT_EHIP (-4)         /* a HIP launch failed */

#define H3DIT_BF16 0
#define H3DIT_INT8 1
#define H3DIT_INT8_MLP 2   /* FC1 and FC2 in int8, QKV and output projection in bf16 */
#define H3DIT_INT8_ATTN 3  /* QKV and output projection in int8, FC1 and FC2 in bf16 */

/* Fusion switches ([DD] "DiT 融合内核": every fusion can be turned back into its step-wise
 * form for a byte-identical A/B).  Each flag selects the unfused sequence; the results are
 * byte-identical to the fused default. */
#define H3DIT_NOFUSE_GATE_ADALN 1u  /* gated residual and the following AdaLN as two kernels */
#define H3DIT_NOFUSE_ROPE 2u        /* QKV projection written token-major, then rotary + head split */
#define H3DIT_NOFUSE_GELU 4u        /* FC1 output written, then GELU as its own kernel */
#define H3DIT_NOFUSE_QUANT 8u       /* int8 path: AdaLN written in bf16, then quantised */
#define H3DIT_NOFUSE_CROSS_BLOCK 16u /* final gate does not produce the next block's AdaLN1 */
#define H3DIT_NO_ALIAS 32u          /* every activation in its own workspace region */

/* Widths.  hidden = heads * head_dim; head_dim 64 or 128; hidden % 256 == 0;
 * mlp % 256 == 0, and on the int8 path mlp % fc2_group == 0 with fc2_group % 128 == 0 and
 * fc2_group <= 8192 (1024 is the pages' group), or fc2_group == mlp: one code per token over
 * the whole FC2 input, the row-level int8 FC2 option of [NS] "算力拆解：如何在 M5 Max 上把
 * 16.69 秒压到 12.60 秒" (bit for bit the grouped formula with a single group).
 * ln_eps: LayerNorm epsilon (1e-6). */
typedef struct {
  int32_t n_tokens, hidden, heads, head_dim, mlp, fc2_group;
  float ln_eps;
} h3dit_dims;

/* Token layout: video tokens (t, h, w) row-major, then n_text text tokens, then n_audio
 * audio tokens; n_tokens must equal video_t*video_h*video_w + n_text + n_audio.
 * Rotary embedding (the pages only say spatial rotary positions exist, [DD] "h3.c 的核心
 * 设计" and the preview-mode note of the daily.steinslab.io article): video tokens rotate
 * head-dim pairs (2j, 2j+1) by their t, h and w position in three consecutive sections of
 * rope_t, rope_h, rope_w dims (even, summing to head_dim) with frequencies
 * theta^(-2j/section); text and audio use 1-D rotary over the whole head dim at their
 * index within their own segment.  These built-in tables are made on the device in double
 * precision whenever the caller passes no h3dit_rope tables of its own. */
typedef struct {
  int32_t video_t, video_h, video_w, n_text, n_audio;
  int32_t rope_t, rope_h, rope_w;
  float rope_theta;
  /* modulation sets in each block's `mod`: 0 or 1 = one set for every token; 3 = one set
   * each for the video, text and audio tokens (a reading of the per-segment conditioning of
   * [DD] "引用系统：Ref2VA 的多模态条件控制"; in the paired span the video segment is the
   * paired video tokens) */
  int32_t mod_sets;
} h3dit_layout;

/* One block's parameters (device pointers).
 * precision H3DIT_BF16: w_* are bf16 [3d][d] (rows q | k | v, head h = rows h*hd..),
 *   [d][d], [mlp][d], [d][mlp]; s_* unused.
 * precision H3DIT_INT8: w_* are int8 codes of the same shapes and s_* fp32 per-output-row
 *   scales, as written by h3dit_quantize_weights.
 * precision H3DIT_INT8_MLP ([DD] "int8 量化", the table's int8-MLP row): w_qkv, w_o bf16 as
 *   in H3DIT_BF16; w_fc1, w_fc2 int8 codes with s_fc1, s_fc2.
 * precision H3DIT_INT8_ATTN ([DD] "int8 量化", the int8-QKV-only path set against the full int8
 *   path after the table): w_qkv, w_o int8 codes with s_qkv, s_o (the output projection's
 *   input coded per token as in H3DIT_INT8); w_fc1, w_fc2 bf16 as in H3DIT_BF16.
 * Every block of a stack has the same precision.
 * mod: bf16 [mod_sets][6][d] modulation rows shift1, scale1, gate1, shift2, scale2, gate2 per
 *   set, each set broadcast over its tokens ([DD] AdaLN branches are precomputable per block). */
typedef struct {
  int32_t precision;
  const void *w_qkv, *w_o, *w_fc1, *w_fc2;
  const float *s_qkv, *s_o, *s_fc1, *s_fc2;
  const uint16_t *mod;
} h3dit_block_w;

/* Rotary tables ([DD] "h3.c 的核心设计": rotary positions applied to q and k before attention;
 * [DD] "引用系统：Ref2VA 的多模态条件控制" and the preview note of [NS] "极简主控逻辑" place tokens
 * on the rotary timeline in more than one way, so positions are data): cos, sin fp32
 * [n][head_dim/2] (device, 16-byte aligned), n the tokens of the sequence they serve.  Token t's
 * q and k pairs (2j, 2j+1) become (a cos[t][j] - b sin[t][j], a sin[t][j] + b cos[t][j]).
 * A NULL h3dit_rope pointer, or NULL cos and sin, selects the built-in tables of the layout
 * (h3dit_layout above; h3dit_rope_tables writes them out). */
typedef struct {
  const float *cos, *sin;
} h3dit_rope;

/* Token reduction ([DD] "Token 缩减"): after block index reduce_after (0-based) adjacent
 * horizontal video tokens (t,h,2k),(t,h,2k+1) are averaged into one token (the odd last
 * column, text and audio pass through); the full-resolution residual stays in x as the
 * bypass.  Before block index restore_before (or after the last block, whichever comes
 * first) each paired token becomes bypass + (reduced output - reduced input) and every
 * other token takes its reduced output.  Requires 0 <= reduce_after < restore_before and
 * reduce_after < n_blocks. */
typedef struct {
  int32_t reduce_after, restore_before;
  h3dit_rope rope_reduced;   /* rotary tables of the paired sequence; NULL pointers: built-in */
} h3dit_token_reduction;

/* Per-output-channel int8 weight codes ([DD] "int8 量化"): for each row r of w (bf16
 * [rows][cols], device), s[r] = max|w[r][:]| / 127 (IEEE division) and
 * q[r][c] = round-half-even(w[r][c] / s[r]) clamped to +-127 (0 when s[r] == 0).
 * q: int8 [rows][cols] device; s: fp32 [rows] device.  cols % 8 == 0, rows < 2^31. */
H3DIT_API int h3dit_quantize_weights(const uint16_t *w, int64_t rows, int64_t cols, int8_t *q, float *s,
                           void *stream);

/* One block, x <- block(x), with no cross-block fusion ([DD] "DiT 融合内核" for the order):
 *   h1 = AdaLN(x; shift1, scale1); [q|k|v] = h1 Wqkv^T; rotary on q, k; O = softmax(q k^T /
 *   sqrt(hd)) v per head (non-causal); y1 = O Wo^T; x1 = x + gate1*y1; h2 = AdaLN(x1; shift2,
 *   scale2); y2 = GELU_tanh(h2 W1^T) W2^T; x = x1 + gate2*y2,
 * with AdaLN(v; s, c) = LN(v)(1 + c) + s (no learned affine) and every intermediate rounded
 * to bf16.  int8 path: each projection input is quantised per token (FC2 input per
 * fc2_group channels), accumulated in int32 and dequantised as (acc * s_act) * s_w.
 * x: bf16 [n_tokens][hidden] device, in/out.  layout: token layout and rotary (host).
 * rope: rotary tables of the n_tokens tokens, or NULL for the built-in ones.
 * workspace: device scratch of *workspace_bytes bytes; with workspace == NULL the required
 * size is written to *workspace_bytes and H3DIT_OK returned without launching. */
H3DIT_API int h3dit_block_fwd(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_block_w *blk,
                              const h3dit_rope *rope, uint16_t *x, uint32_t flags, void *workspace,
                              size_t *workspace_bytes, void *stream);

/* A stack of n_blocks blocks for one denoising evaluation ([RV] README: 50-layer DiT;
 * [DD] fusion of each block's final gate with the next block's AdaLN1, and activation
 * arenas reused across lifetimes).  blocks: host array of n_blocks entries (device
 * pointers inside).  rope: tables of the full sequence (NULL: built-in).  tr: NULL for no
 * token reduction; its rope_reduced serves the blocks inside the paired span.  Other
 * arguments as h3dit_block_fwd. */
H3DIT_API int h3dit_stack_fwd(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks,
                              const h3dit_block_w *blocks, const h3dit_rope *rope, const h3dit_token_reduction *tr,
                              uint16_t *x, uint32_t flags, void *workspace, size_t *workspace_bytes, void *stream);

/* h3dit_stack_fwd with the block matrices left in host memory ([RV] section "h3-metal 的 SSD
 * 串流：用速度換常駐記憶體": the small per-block weights stay resident while two full matrix
 * slots alternate, the next block's matrices being fetched while the current block computes).
 * blocks: host array as in h3dit_stack_fwd, but w_qkv, w_o, w_fc1, w_fc2, s_* and mod are HOST
 * pointers (16-byte aligned; allocate them pinned, e.g. hipHostMalloc, or the copies run
 * synchronously and nothing overlaps).  Every block's mod rows are copied once into the
 * workspace; block b's matrices and scales are copied into slot b % 2 of the workspace on
 * copy_stream, after the block that last used that slot has finished on `stream` (for blocks 0
 * and 1: after all work enqueued on `stream` before the call, so back-to-back calls on one
 * workspace are safe), and block b waits for its copy.  Results are byte-identical to h3dit_stack_fwd with the same weights
 * resident.  copy_stream: a second stream for the copies (NULL or equal to `stream`: copies
 * on `stream`, no overlap).  workspace: as h3dit_stack_fwd plus the mod rows and two slots
 * (NULL queries the size).  The host weights must stay valid until `stream` has completed
 * the call's work.  Errors as h3dit_stack_fwd. */
H3DIT_API int h3dit_stack_fwd_streamed(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks,
                                       const h3dit_block_w *blocks, const h3dit_rope *rope,
                                       const h3dit_token_reduction *tr, uint16_t *x, uint32_t flags,
                                       void *workspace, size_t *workspace_bytes, void *stream, void *copy_stream);

/* One modality of the final head: mod bf16 [2][d] (shift, scale), w bf16 [channels][d],
 * channels % 128 == 0 (device pointers). */
typedef struct {
  const uint16_t *mod;
  const uint16_t *w;
  int32_t channels;
} h3dit_head_part;

/* Final head after the stack ([DD] "DiT 融合内核", final audio/video AdaLN bound to the residual
 * stream, the bf16 head applying AdaLN while it loads its projection tiles): for the video rows
 * [0, n_video) and the audio rows (the last n_audio) of x, out = bf16(h W^T) with
 * h = bf16(AdaLN(x_rows; shift, scale)) (as h3dit_block_fwd's AdaLN), no bias.  The rows are
 * read in place (no slice copies) and h is formed inside the GEMM's tile loads, never stored:
 * the workspace holds only each row's mean and 1/sqrt(var + eps) (8 bytes per row).  The head
 * sums K in one pass: its output equals h3dit_row_gate_adaln followed by h3dit_linear byte for
 * byte wherever that GEMM is not split along K (h3dit_linear_workspace 0), and differs from a
 * split one in fp32 summation order only.  video / audio: NULL to
 * skip that part; out_video bf16 [n_video][video->channels], out_audio bf16
 * [n_audio][audio->channels] (device).  workspace as in h3dit_block_fwd (NULL queries the
 * size).  x is not modified. */
H3DIT_API int h3dit_final_head(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_head_part *video,
                               const h3dit_head_part *audio, const uint16_t *x, uint16_t *out_video,
                               uint16_t *out_audio, void *workspace, size_t *workspace_bytes, void *stream);

/* h3dit_final_head without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the row
 * statistics go to a static device array of 512 KiB that the library holds on each device it
 * runs on until the process ends, so each part may have at most 65536 rows (n_video and
 * n_audio); larger parts return H3DIT_EWORKSPACE before any launch.  The caller still passes
 * x and the outputs.  Nothing in the array needs clearing (every row's statistics are written
 * before they are read).  All calls on one device share the array: calls that overlap on one
 * device (on different streams, or from different host threads without ordering) race and
 * must not be made.  Other arguments, results and errors as h3dit_final_head; the output is
 * byte-identical to it. */
H3DIT_API int h3dit_final_head_noalloc(const h3dit_dims *dims, const h3dit_layout *layout,
                                       const h3dit_head_part *video, const h3dit_head_part *audio, const uint16_t *x,
                                       uint16_t *out_video, uint16_t *out_audio, void *stream);

/* Denoising schedule ([DD] "速度/质量预设矩阵": denoising steps, whole-denoiser velocity reuse,
 * active blocks and core-residual reuse, with reuse and core reuse mutually exclusive;
 * [DD] "Token 缩减": the bypass comes back before block 40 in the first ten noise evaluations
 * and before block 30 in the later ones).  The pages give the controls and, for 20 steps,
 * 20 / 11 / 8 fresh evaluations at reuse 1 / 2 / 3; the rules below are readings:
 *  - reuse r: step i evaluates the denoiser when i % r == 0 or i is the last step; any other
 *    step repeats the most recent fresh velocity for its transition (this yields 20 / 11 / 8).
 *  - core_reuse c: the head is refreshed every step; the block stack runs when i % c == 0 or
 *    i is the last step, and in between its most recent output residual is reused.
 *  - layers L: the first L of the n_blocks blocks run.
 *  - token reduction (reduce_after >= 0): core evaluation e (counted from 0) restores before
 *    block restore_early when e < early_evals, else before block restore_late (40, 30, 10). */
typedef struct {
  int32_t steps, reuse, core_reuse, layers;
  int32_t reduce_after;                              /* -1: no token reduction */
  int32_t restore_early, restore_late, early_evals;
} h3dit_denoise_opts;

/* One step of a plan.  fresh: the velocity is evaluated (the head runs) at this step; core: the
 * block stack runs first; eval: index of the core evaluation whose residual the velocity
 * comes from; n_blocks: blocks that evaluation runs; restore_before: its token restore index
 * (-1 without token reduction). */
typedef struct {
  int32_t fresh, core, eval, n_blocks, restore_before;
} h3dit_denoise_step;

/* Fills plan[0 .. opts->steps-1] (host memory).  Returns the number of core evaluations
 * (>= 1), or H3DIT_EINVAL for: NULL pointers, steps < 1, reuse < 1, core_reuse < 1, reuse > 1
 * together with core_reuse > 1, layers outside [1, n_blocks], or, with token reduction,
 * reduce_after >= layers, a restore index <= reduce_after, or early_evals < 0.  Host only. */
H3DIT_API int h3dit_denoise_plan(const h3dit_denoise_opts *opts, int32_t n_blocks, h3dit_denoise_step *plan);

/* One transition of a velocity step: z[i] = bf16(z[i] + dt * v[i]) in fp32, product and sum
 * each rounded (an Euler step of the velocity the head predicts; the pages name velocities and
 * extrapolated transitions but no sampler, so this plain step is a reading).  z, v: bf16
 * [count] (device), count % 8 == 0. */
H3DIT_API int h3dit_velocity_step(int64_t count, float dt, const uint16_t *v, uint16_t *z, void *stream);

/* Stand-in for the patch embedding of the latents (the pages name latents and a velocity
 * head but not the embedding, so this linear map is a reading): w_video bf16 [hidden][c_v] and
 * w_audio bf16 [hidden][c_a] (device; c_v, c_a the head parts' channels).  A core evaluation
 * starts from x = x_in with video row r replaced by bf16(x_in[r] + bf16(z_video[r] w_video^T))
 * and audio row r by bf16(x_in[r] + bf16(z_audio[r] w_audio^T)) (text rows: x_in), so the
 * current latents feed the stack.  A NULL matrix leaves its rows at x_in. */
typedef struct {
  const uint16_t *w_video, *w_audio;
} h3dit_patch_embed;

/* A denoising loop over the plan of `opts`: for each step, a core step copies x_in into the
 * workspace residual, adds the patch embedding of the current latents (embed non-NULL), and
 * runs h3dit_stack_fwd over the first plan.n_blocks blocks (with the step's token reduction
 * and the rotary tables rope / rope_reduced, NULL for built-in); a fresh step runs
 * h3dit_final_head on that residual into velocity buffers; every step applies
 * h3dit_velocity_step with dt[step] to z_video and z_audio.  x_in (bf16 [n_tokens][hidden],
 * device) is the conditioning residual every core evaluation starts from; with embed == NULL
 * it is the whole stack input and the latents do not feed back.  dt: host fp32 [steps].
 * video / audio and z_video / z_audio as in h3dit_final_head (bf16 [n_video][channels],
 * [n_audio][channels], updated in place; at least one part).  workspace: NULL queries the
 * size.  Errors as h3dit_denoise_plan, h3dit_stack_fwd and h3dit_final_head. */
H3DIT_API int h3dit_denoise_fwd(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks,
                                const h3dit_block_w *blocks, const h3dit_rope *rope, const h3dit_rope *rope_reduced,
                                const h3dit_denoise_opts *opts, const float *dt, const uint16_t *x_in,
                                const h3dit_patch_embed *embed, const h3dit_head_part *video,
                                const h3dit_head_part *audio, uint16_t *z_video, uint16_t *z_audio, uint32_t flags,
                                void *workspace, size_t *workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif
