// C ABI of the H3 DiT block library: argument validation, the workspace (arena) plan, and
// the launch sequence of one block and of a stack of blocks.  Every arithmetic step runs in
// the kernels of rowops.hip, gemm.hip and attention.hip; this file only orders launches.
//
// Arena plan ([DD] "DiT 融合内核", 激活缓冲别名: activations follow their lifetime inside the
// block; the QKV arena is reused for the attention heads and then for the normalised MLP
// input, and the attention-output arena becomes the MLP output):
//   A  q | k | V^T  ->  attention output over q  ->  MLP input (h2 / int8 q2)  ->  int8 FC2 input
//   B  out-projection output y1  ->  FC2 output y2
//   C  AdaLN1 output (h1 / int8 q1)  ->  int8 attention output codes  ->  FC1+GELU output
// With H3DIT_NO_ALIAS each of these gets its own region.
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace {

using namespace h3;

constexpr size_t ALIGN = 256;
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t layout_tokens(const h3dit_layout &L, bool reduced) {
  const int64_t wr = reduced ? (L.video_w / 2 + L.video_w % 2) : L.video_w;
  return (int64_t)L.video_t * L.video_h * wr + L.n_text + L.n_audio;
}

int check_dims(const h3dit_dims *D, const h3dit_layout *L, int precision) {
  if (!D || !L) return H3DIT_EINVAL;
  if (D->n_tokens < 1 || D->heads < 1 || D->hidden != D->heads * D->head_dim) return H3DIT_EINVAL;
  if (D->head_dim != 64 && D->head_dim != 128) return H3DIT_EUNSUPPORTED;
  if (D->hidden % 256 || D->hidden > 8192 || D->mlp < 256 || D->mlp % 256) return H3DIT_EINVAL;
  if (!(D->ln_eps >= 0.0f)) return H3DIT_EINVAL;
  if (precision != H3DIT_BF16 && precision != H3DIT_INT8 && precision != H3DIT_INT8_MLP &&
      precision != H3DIT_INT8_ATTN)
    return H3DIT_EINVAL;
  if (precision == H3DIT_INT8 || precision == H3DIT_INT8_MLP) {
    // 1024-channel groups as on the pages, or one code per token over the whole FC2 input
    // (fc2_group == mlp, the row-level variant)
    if (D->fc2_group < 128 || D->fc2_group % 128 || (D->fc2_group > 8192 && D->fc2_group != D->mlp) ||
        D->mlp % D->fc2_group)
      return H3DIT_EINVAL;
  }
  if (L->video_t < 0 || L->video_h < 0 || L->video_w < 0 || L->n_text < 0 || L->n_audio < 0) return H3DIT_EINVAL;
  if (layout_tokens(*L, false) != D->n_tokens) return H3DIT_EINVAL;
  if (L->rope_t < 0 || L->rope_h < 0 || L->rope_w < 0 || (L->rope_t | L->rope_h | L->rope_w) & 1 ||
      L->rope_t + L->rope_h + L->rope_w != D->head_dim || !(L->rope_theta > 0.0f))
    return H3DIT_EINVAL;
  if (L->mod_sets != 0 && L->mod_sets != 1 && L->mod_sets != 3) return H3DIT_EINVAL;
  // 32-bit buffer offsets inside the kernels: the widest activation ([N][mlp] or the
  // token-major [N][3d] projection) and the largest weight ([mlp][d], [3d][d]) in bf16
  const int64_t widest = D->mlp > 3 * (int64_t)D->hidden ? D->mlp : 3 * (int64_t)D->hidden;
  if ((int64_t)D->n_tokens * widest * 2 >= ((int64_t)1 << 31)) return H3DIT_EINVAL;
  if (widest * D->hidden * 2 >= ((int64_t)1 << 31)) return H3DIT_EINVAL;
  return H3DIT_OK;
}

int check_block(const h3dit_block_w *b, int precision) {
  if (!b || b->precision != precision) return H3DIT_EINVAL;
  const void *w[4] = {b->w_qkv, b->w_o, b->w_fc1, b->w_fc2};
  for (const void *p : w)
    if (!p || !aligned(p, 16)) return H3DIT_EINVAL;
  if (!b->mod || !aligned(b->mod, 16)) return H3DIT_EINVAL;
  if (precision == H3DIT_INT8) {
    const float *s[4] = {b->s_qkv, b->s_o, b->s_fc1, b->s_fc2};
    for (const float *p : s)
      if (!p || !aligned(p, 4)) return H3DIT_EINVAL;
  } else if (precision == H3DIT_INT8_MLP) {
    const float *s[2] = {b->s_fc1, b->s_fc2};
    for (const float *p : s)
      if (!p || !aligned(p, 4)) return H3DIT_EINVAL;
  } else if (precision == H3DIT_INT8_ATTN) {
    const float *s[2] = {b->s_qkv, b->s_o};
    for (const float *p : s)
      if (!p || !aligned(p, 4)) return H3DIT_EINVAL;
  }
  return H3DIT_OK;
}

// Caller rotary tables: NULL (or both pointers NULL) selects the built-in ones; otherwise both
// must be given and 16-byte aligned (the QKV epilogue reads them four pairs at a time).
int check_rope(const h3dit_rope *r) {
  if (!r || (!r->cos && !r->sin)) return H3DIT_OK;
  if (!r->cos || !r->sin || !aligned(r->cos, 16) || !aligned(r->sin, 16)) return H3DIT_EINVAL;
  return H3DIT_OK;
}
bool has_rope(const h3dit_rope *r) { return r && r->cos && r->sin; }

// gfx950 check, once per device
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return H3DIT_EHIP;
  if (dev < 0 || dev >= 64) return H3DIT_EUNSUPPORTED;
  int v = g_arch_ok[dev].load();
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return H3DIT_EHIP;
    v = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(v);
  }
  return v == 1 ? H3DIT_OK : H3DIT_EUNSUPPORTED;
}

struct Plan {
  size_t total = 0;
  size_t cos_f = 0, sin_f = 0, cos_r = 0, sin_r = 0;
  size_t q = 0, k = 0, vt = 0, o = 0, h2 = 0, qg = 0;  // arena A roles
  size_t y1 = 0, y2 = 0;                              // arena B roles
  size_t h1 = 0, qo = 0, gl = 0;                      // arena C roles
  size_t t = 0, hb = 0;                               // unfused-only regions
  size_t sa = 0, sg = 0;                              // per-token / per-group scales
  size_t red = 0, r_in = 0;                           // token reduction
  size_t sk = 0, sk_bytes = 0;                        // split-K partial tiles of the projections
};

// Precision of the attention projections (QKV, output) and of the MLP projections.
int attn_prec(int precision) {
  return (precision == H3DIT_INT8 || precision == H3DIT_INT8_ATTN) ? H3DIT_INT8 : H3DIT_BF16;
}
int mlp_prec(int precision) {
  return (precision == H3DIT_INT8 || precision == H3DIT_INT8_MLP) ? H3DIT_INT8 : H3DIT_BF16;
}

// Largest split-K workspace of the block's four projections at n tokens.
size_t block_splitk_bytes(const h3dit_dims &D, int precision, int64_t n) {
  h3dit_linear_args la{};
  la.M = n;
  size_t m = 0;
  auto take = [&](int prec, int64_t N, int64_t K, int out_kind, int group) {
    la.precision = prec;
    la.N = N; la.K = K; la.out_kind = out_kind; la.a_group = group;
    la.heads = D.heads; la.head_dim = D.head_dim;
    const size_t b = linear_workspace(la);
    if (b > m) m = b;
  };
  const int pa = attn_prec(precision), pm = mlp_prec(precision);
  take(pa, 3 * (int64_t)D.hidden, D.hidden, H3DIT_OUT_QKV, 0);
  take(pa, 3 * (int64_t)D.hidden, D.hidden, H3DIT_OUT_BF16, 0);
  take(pa, D.hidden, D.hidden, H3DIT_OUT_BF16, 0);
  take(pm, D.mlp, D.hidden, H3DIT_OUT_GELU, 0);
  take(pm, D.hidden, D.mlp, H3DIT_OUT_BF16, (pm == H3DIT_INT8 && D.fc2_group != D.mlp) ? D.fc2_group : 0);
  return m;
}

Plan make_plan(const h3dit_dims &D, const h3dit_layout &L, int precision, uint32_t flags, bool reduction) {
  const size_t N = (size_t)D.n_tokens, d = (size_t)D.hidden, f = (size_t)D.mlp, hd = (size_t)D.head_dim;
  const size_t ldv = (size_t)vt_pitch((int64_t)N);
  const bool i8 = precision != H3DIT_BF16;   // the int8 buffers (a superset for the partly int8 blocks)
  const size_t Nd2 = N * d * 2;
  Plan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  p.cos_f = take(N * hd / 2 * 4);
  p.sin_f = take(N * hd / 2 * 4);
  if (reduction) {
    const size_t Nr = (size_t)layout_tokens(L, true);
    p.cos_r = take(Nr * hd / 2 * 4);
    p.sin_r = take(Nr * hd / 2 * 4);
    p.red = take(Nr * d * 2);
    p.r_in = take(Nr * d * 2);
  }
  p.sk_bytes = block_splitk_bytes(D, precision, (int64_t)N);
  if (reduction) {
    const size_t r = block_splitk_bytes(D, precision, layout_tokens(L, true));
    if (r > p.sk_bytes) p.sk_bytes = r;
  }
  if (p.sk_bytes) p.sk = take(p.sk_bytes);
  p.sa = take(N * 4);
  if (mlp_prec(precision) == H3DIT_INT8) p.sg = take(N * (f / (size_t)D.fc2_group) * 4);
  if (flags & H3DIT_NOFUSE_ROPE) p.t = take(3 * Nd2);
  if (flags & H3DIT_NOFUSE_QUANT) p.hb = take(Nd2);
  const size_t qkv = 2 * Nd2 + d * ldv * 2;
  if (!(flags & H3DIT_NO_ALIAS)) {
    const size_t A = take(i8 ? (qkv > N * f ? qkv : N * f) : qkv);
    const size_t B = take(Nd2);
    const size_t C = take(N * f * 2 > Nd2 ? N * f * 2 : Nd2);
    p.q = A; p.k = A + Nd2; p.vt = A + 2 * Nd2; p.o = A; p.h2 = A; p.qg = A;
    p.y1 = B; p.y2 = B;
    p.h1 = C; p.qo = C; p.gl = C;
  } else {
    p.q = take(Nd2); p.k = take(Nd2); p.vt = take(d * ldv * 2); p.o = take(Nd2);
    p.h2 = take(Nd2); p.y1 = take(Nd2); p.y2 = take(Nd2); p.h1 = take(Nd2); p.gl = take(N * f * 2);
    if (i8) { p.qo = take(N * d); p.qg = take(N * f); }
  }
  p.total = off;
  return p;
}

#define TRY(expr)                                   \
  do {                                              \
    if ((expr) != hipSuccess) return H3DIT_EHIP;    \
  } while (0)

struct Ctx {
  const h3dit_dims *D;
  const h3dit_layout *L;
  uint32_t flags;
  uint8_t *ws;
  Plan P;
  hipStream_t st;
  template <class T>
  T *at(size_t off) const { return reinterpret_cast<T *>(ws + off); }
  // row kernel on n rows (the full or the paired sequence), with the modulation set of each
  // row's segment: video rows first, then text, then audio
  hipError_t row(int64_t n, const uint16_t *x, const uint16_t *gate, const uint16_t *y, uint16_t *x_out,
                 const uint16_t *shift, const uint16_t *scale, uint16_t *h, int8_t *q, float *s) const {
    const int64_t seg1 = n - L->n_text - L->n_audio, seg2 = seg1 + L->n_text;
    const int64_t stride = L->mod_sets == 3 ? 6 * (int64_t)D->hidden : 0;
    return launch_row(n, D->hidden, D->ln_eps, x, gate, y, x_out, shift, scale, h, q, s, st, seg1, seg2, stride);
  }
};

// AdaLN (with optional gate) producing the projection input of the next GEMM: bf16 into
// dst_bf16, or int8 codes into dst_q plus per-token scales.
int adaln_into(const Ctx &c, int64_t n, const uint16_t *x, const uint16_t *gate, const uint16_t *y, uint16_t *x_out,
               const uint16_t *shift, const uint16_t *scale, bool i8, size_t dst) {
  const int d = c.D->hidden;
  if (!i8) {
    TRY(c.row(n, x, gate, y, x_out, shift, scale, c.at<uint16_t>(dst), nullptr, nullptr));
  } else if (!(c.flags & H3DIT_NOFUSE_QUANT)) {
    TRY(c.row(n, x, gate, y, x_out, shift, scale, nullptr, c.at<int8_t>(dst), c.at<float>(c.P.sa)));
  } else {
    TRY(c.row(n, x, gate, y, x_out, shift, scale, c.at<uint16_t>(c.P.hb), nullptr, nullptr));
    TRY(launch_quant_rows(n, d, d, c.at<uint16_t>(c.P.hb), 0, c.at<int8_t>(dst), c.at<float>(c.P.sa), c.st));
  }
  return H3DIT_OK;
}

// One block on x [n][d].  h1_ready: AdaLN1 output already in place (produced by the previous
// block's final gate).  next: block whose AdaLN1 the final gate also produces, or NULL.
int run_block(const Ctx &c, int64_t n, const float *cos_t, const float *sin_t, const h3dit_block_w &b, uint16_t *x,
              bool h1_ready, const h3dit_block_w *next) {
  const h3dit_dims &D = *c.D;
  const int d = D.hidden, H = D.heads, hd = D.head_dim, f = D.mlp;
  const int pa = attn_prec(b.precision), pm = mlp_prec(b.precision);
  const bool i8 = pa == H3DIT_INT8, i8m = pm == H3DIT_INT8;   // attention / MLP projections in int8
  const uint32_t F = c.flags;
  const uint16_t *mod = b.mod;
  const uint16_t *sh1 = mod, *sc1 = mod + d, *g1 = mod + 2 * d, *sh2 = mod + 3 * d, *sc2 = mod + 4 * d, *g2 = mod + 5 * d;
  const Plan &P = c.P;
  int rc;

  // AdaLN1
  if (!h1_ready && (rc = adaln_into(c, n, x, nullptr, nullptr, nullptr, sh1, sc1, i8, P.h1)) != H3DIT_OK) return rc;

  // QKV projection + rotary + head-major split
  h3dit_linear_args la{};
  la.M = n; la.N = 3 * d; la.K = d;
  la.precision = pa;
  la.a = c.at<void>(P.h1);
  la.a_scale = i8 ? c.at<float>(P.sa) : nullptr;
  la.w = b.w_qkv;
  la.w_scale = b.s_qkv;
  la.cos_t = cos_t; la.sin_t = sin_t; la.heads = H; la.head_dim = hd;
  la.workspace = c.at<void>(P.sk); la.workspace_bytes = P.sk_bytes;
  if (!(F & H3DIT_NOFUSE_ROPE)) {
    la.out_kind = H3DIT_OUT_QKV;
    la.out_q = c.at<uint16_t>(P.q); la.out_k = c.at<uint16_t>(P.k); la.out_v = c.at<uint16_t>(P.vt);
    TRY(launch_linear(la, c.st));
  } else {
    la.out_kind = H3DIT_OUT_BF16;
    la.out = c.at<void>(P.t);
    TRY(launch_linear(la, c.st));
    TRY(launch_rope_split(n, H, hd, c.at<uint16_t>(P.t), cos_t, sin_t, c.at<uint16_t>(P.q), c.at<uint16_t>(P.k),
                          c.at<uint16_t>(P.vt), c.st));
  }

  // attention (output over q in the aliased plan)
  TRY(launch_attention(H, n, hd, c.at<uint16_t>(P.q), c.at<uint16_t>(P.k), c.at<uint16_t>(P.vt), c.at<uint16_t>(P.o),
                       nullptr, nullptr, c.st));

  // output projection
  la = h3dit_linear_args{};
  la.M = n; la.N = d; la.K = d; la.precision = pa; la.w = b.w_o; la.w_scale = b.s_o;
  la.out_kind = H3DIT_OUT_BF16; la.out = c.at<void>(P.y1);
  la.workspace = c.at<void>(P.sk); la.workspace_bytes = P.sk_bytes;
  if (!i8) {
    la.a = c.at<void>(P.o);
    la.a_headmajor_hd = hd;
  } else {
    TRY(launch_quant_rows(n, d, d, c.at<uint16_t>(P.o), hd, c.at<int8_t>(P.qo), c.at<float>(P.sa), c.st));
    la.a = c.at<void>(P.qo);
    la.a_scale = c.at<float>(P.sa);
  }
  TRY(launch_linear(la, c.st));

  // gate1 + AdaLN2
  if (!(F & H3DIT_NOFUSE_GATE_ADALN)) {
    if ((rc = adaln_into(c, n, x, g1, c.at<uint16_t>(P.y1), x, sh2, sc2, i8m, P.h2)) != H3DIT_OK) return rc;
  } else {
    TRY(c.row(n, x, g1, c.at<uint16_t>(P.y1), x, nullptr, nullptr, nullptr, nullptr, nullptr));
    if ((rc = adaln_into(c, n, x, nullptr, nullptr, nullptr, sh2, sc2, i8m, P.h2)) != H3DIT_OK) return rc;
  }

  // FC1 + GELU
  la = h3dit_linear_args{};
  la.M = n; la.N = f; la.K = d; la.precision = pm; la.w = b.w_fc1; la.w_scale = b.s_fc1;
  la.a = c.at<void>(P.h2); la.a_scale = i8m ? c.at<float>(P.sa) : nullptr;
  la.out = c.at<void>(P.gl);
  la.out_kind = (F & H3DIT_NOFUSE_GELU) ? H3DIT_OUT_BF16 : H3DIT_OUT_GELU;
  la.workspace = c.at<void>(P.sk); la.workspace_bytes = P.sk_bytes;
  TRY(launch_linear(la, c.st));
  if (F & H3DIT_NOFUSE_GELU) TRY(launch_gelu((int64_t)n * f, c.at<uint16_t>(P.gl), c.at<uint16_t>(P.gl), c.st));

  // FC2
  la = h3dit_linear_args{};
  la.M = n; la.N = d; la.K = f; la.precision = pm; la.w = b.w_fc2; la.w_scale = b.s_fc2;
  la.out_kind = H3DIT_OUT_BF16; la.out = c.at<void>(P.y2);
  la.workspace = c.at<void>(P.sk); la.workspace_bytes = P.sk_bytes;
  if (!i8m) {
    la.a = c.at<void>(P.gl);
  } else {
    TRY(launch_quant_rows(n, f, D.fc2_group, c.at<uint16_t>(P.gl), 0, c.at<int8_t>(P.qg), c.at<float>(P.sg), c.st));
    la.a = c.at<void>(P.qg);
    la.a_scale = c.at<float>(P.sg);
    // one group per token is the per-token formula bit for bit ((0 + acc*s) * s_w): it runs on
    // the ungrouped kernels (256 x 256 tiles, split-K)
    la.a_group = D.fc2_group == D.mlp ? 0 : D.fc2_group;
  }
  TRY(launch_linear(la, c.st));

  // gate2, optionally with the next block's AdaLN1
  if (next) {
    const bool ni8 = attn_prec(next->precision) == H3DIT_INT8;
    if ((rc = adaln_into(c, n, x, g2, c.at<uint16_t>(P.y2), x, next->mod, next->mod + d, ni8, P.h1)) != H3DIT_OK)
      return rc;
  } else {
    TRY(c.row(n, x, g2, c.at<uint16_t>(P.y2), x, nullptr, nullptr, nullptr, nullptr, nullptr));
  }
  return H3DIT_OK;
}

// Validates the call, plans the workspace (plan.total bytes of activations, then `extra` bytes
// for the caller) and answers a size query (returns 1).
int prepare(const h3dit_dims *dims, const h3dit_layout *layout, int precision, uint32_t flags, bool reduction,
            uint16_t *x, void *workspace, size_t *workspace_bytes, Plan &plan, size_t extra = 0) {
  if (!workspace_bytes) return H3DIT_EINVAL;
  if (flags & ~(uint32_t)63) return H3DIT_EINVAL;
  int rc = check_dims(dims, layout, precision);
  if (rc) return rc;
  plan = make_plan(*dims, *layout, precision, flags, reduction);
  const size_t need = plan.total + extra;
  if (!workspace) {
    *workspace_bytes = need;
    return 1;  // size query answered
  }
  if (!x || !aligned(x, 16) || !aligned(workspace, ALIGN)) return H3DIT_EINVAL;
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return H3DIT_EWORKSPACE;
  }
  return H3DIT_OK;
}

// The stack loop: rotary tables, token pair / restore, cross-block fusion.  blocks[b] must
// hold device pointers by the time block b's kernels are enqueued; before(b) runs first and
// after(b) once they are enqueued (both may enqueue work).  The next block's AdaLN1, fused into
// block b's final gate, reads only blocks[b + 1].mod.
template <class Before, class After>
int run_stack(const Ctx &c, int32_t n_blocks, const h3dit_block_w *blocks, const h3dit_rope *rope,
              const h3dit_token_reduction *tr, uint16_t *x, Before before, After after) {
  const h3dit_dims *dims = c.D;
  const h3dit_layout *layout = c.L;
  const Plan &plan = c.P;
  // rotary tables: the caller's, or the built-in ones made in the workspace
  const float *cf = c.at<float>(plan.cos_f), *sf = c.at<float>(plan.sin_f);
  const float *cr = nullptr, *sr = nullptr;
  if (has_rope(rope)) {
    cf = rope->cos;
    sf = rope->sin;
  } else {
    TRY(launch_rope_tables(*layout, dims->head_dim, 0, c.at<float>(plan.cos_f), c.at<float>(plan.sin_f), c.st));
  }
  if (tr) {
    if (has_rope(&tr->rope_reduced)) {
      cr = tr->rope_reduced.cos;
      sr = tr->rope_reduced.sin;
    } else {
      cr = c.at<float>(plan.cos_r);
      sr = c.at<float>(plan.sin_r);
      TRY(launch_rope_tables(*layout, dims->head_dim, 1, c.at<float>(plan.cos_r), c.at<float>(plan.sin_r), c.st));
    }
  }
  const int64_t Nf = dims->n_tokens, Nr = layout_tokens(*layout, true);
  const int d = dims->hidden;
  uint16_t *red = tr ? c.at<uint16_t>(plan.red) : nullptr, *r_in = tr ? c.at<uint16_t>(plan.r_in) : nullptr;
  const bool cross = !(c.flags & (H3DIT_NOFUSE_CROSS_BLOCK | H3DIT_NOFUSE_GATE_ADALN));
  bool reduced = false, h1_ready = false;
  int rc;
  for (int32_t b = 0; b < n_blocks; b++) {
    if (reduced && b == tr->restore_before) {
      TRY(launch_token_restore(*layout, d, x, red, r_in, c.st));
      reduced = false;
      h1_ready = false;
    }
    if ((rc = before(b))) return rc;
    const bool boundary = (tr && (b == tr->reduce_after || b + 1 == tr->restore_before)) || b + 1 == n_blocks;
    const h3dit_block_w *next = (cross && !boundary) ? &blocks[b + 1] : nullptr;
    rc = run_block(c, reduced ? Nr : Nf, reduced ? cr : cf, reduced ? sr : sf, blocks[b], reduced ? red : x, h1_ready,
                   next);
    if (rc) return rc;
    if ((rc = after(b))) return rc;
    h1_ready = next != nullptr;
    if (tr && b == tr->reduce_after) {
      TRY(launch_token_pair(*layout, d, x, red, r_in, c.st));
      reduced = true;
      h1_ready = false;
    }
  }
  if (reduced) TRY(launch_token_restore(*layout, d, x, red, r_in, c.st));
  return H3DIT_OK;
}

// Device copy of one block's matrices and scales (a slot of the streamed stack): offsets of
// w_qkv, w_o, w_fc1, w_fc2, s_qkv, s_o, s_fc1, s_fc2 (0 bytes where a precision has no scale).
struct SlotLayout {
  size_t off[8] = {}, bytes[8] = {};
  size_t total = 0;
};

SlotLayout slot_layout(const h3dit_dims &D, int precision) {
  const size_t d = (size_t)D.hidden, f = (size_t)D.mlp;
  const size_t ea = attn_prec(precision) == H3DIT_INT8 ? 1 : 2, em = mlp_prec(precision) == H3DIT_INT8 ? 1 : 2;
  const size_t rows[4] = {3 * d, d, f, d};
  SlotLayout s;
  s.bytes[0] = 3 * d * d * ea;
  s.bytes[1] = d * d * ea;
  s.bytes[2] = f * d * em;
  s.bytes[3] = d * f * em;
  for (int i = 0; i < 4; i++) {
    const bool scaled = (i < 2 ? ea : em) == 1;
    s.bytes[4 + i] = scaled ? rows[i] * 4 : 0;
  }
  for (int i = 0; i < 8; i++) {
    s.off[i] = s.total;
    s.total += up(s.bytes[i]);
  }
  return s;
}

size_t mod_bytes(const h3dit_dims &D, const h3dit_layout &L) {
  return (size_t)(L.mod_sets == 3 ? 3 : 1) * 6 * (size_t)D.hidden * 2;
}

}  // namespace

extern "C" {

int h3dit_quantize_weights(const uint16_t *w, int64_t rows, int64_t cols, int8_t *q, float *s, void *stream) {
  if (!w || !q || !s || rows < 0 || cols < 8 || cols % 8 || rows > INT32_MAX) return H3DIT_EINVAL;
  if (!aligned(w, 16) || !aligned(q, 8) || !aligned(s, 4)) return H3DIT_EINVAL;
  if (rows == 0) return H3DIT_OK;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_quant_rows(rows, cols, cols, w, 0, q, s, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_block_fwd(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_block_w *blk,
                    const h3dit_rope *rope, uint16_t *x, uint32_t flags, void *workspace, size_t *workspace_bytes,
                    void *stream) {
  if (!blk) return H3DIT_EINVAL;
  Plan plan;
  int rc = prepare(dims, layout, blk->precision, flags, false, x, workspace, workspace_bytes, plan);
  if (rc == 1) return H3DIT_OK;
  if (rc) return rc;
  if ((rc = check_block(blk, blk->precision)) || (rc = check_rope(rope))) return rc;
  if ((rc = check_device())) return rc;
  Ctx c{dims, layout, flags, reinterpret_cast<uint8_t *>(workspace), plan, (hipStream_t)stream};
  const float *cf = c.at<float>(plan.cos_f), *sf = c.at<float>(plan.sin_f);
  if (has_rope(rope)) {
    cf = rope->cos;
    sf = rope->sin;
  } else {
    TRY(launch_rope_tables(*layout, dims->head_dim, 0, c.at<float>(plan.cos_f), c.at<float>(plan.sin_f), c.st));
  }
  return run_block(c, dims->n_tokens, cf, sf, *blk, x, false, nullptr);
}

int h3dit_stack_fwd(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks, const h3dit_block_w *blocks,
                    const h3dit_rope *rope, const h3dit_token_reduction *tr, uint16_t *x, uint32_t flags,
                    void *workspace, size_t *workspace_bytes, void *stream) {
  if (!blocks || n_blocks < 1) return H3DIT_EINVAL;
  const int precision = blocks[0].precision;
  if (tr && (tr->reduce_after < 0 || tr->restore_before <= tr->reduce_after || tr->reduce_after >= n_blocks))
    return H3DIT_EINVAL;
  Plan plan;
  int rc = prepare(dims, layout, precision, flags, tr != nullptr, x, workspace, workspace_bytes, plan);
  if (rc == 1) return H3DIT_OK;
  if (rc) return rc;
  for (int32_t b = 0; b < n_blocks; b++)
    if ((rc = check_block(&blocks[b], precision))) return rc;
  if ((rc = check_rope(rope)) || (tr && (rc = check_rope(&tr->rope_reduced)))) return rc;
  if ((rc = check_device())) return rc;
  Ctx c{dims, layout, flags, reinterpret_cast<uint8_t *>(workspace), plan, (hipStream_t)stream};
  auto none = [](int32_t) { return H3DIT_OK; };
  return run_stack(c, n_blocks, blocks, rope, tr, x, none, none);
}

int h3dit_stack_fwd_streamed(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks,
                             const h3dit_block_w *blocks, const h3dit_rope *rope, const h3dit_token_reduction *tr,
                             uint16_t *x, uint32_t flags, void *workspace, size_t *workspace_bytes, void *stream,
                             void *copy_stream) {
  if (!blocks || n_blocks < 1 || !dims || !layout) return H3DIT_EINVAL;
  const int precision = blocks[0].precision;
  if (tr && (tr->reduce_after < 0 || tr->restore_before <= tr->reduce_after || tr->reduce_after >= n_blocks))
    return H3DIT_EINVAL;
  int rc = check_dims(dims, layout, precision);   // the slot sizes below need valid widths
  if (rc) return rc;
  const SlotLayout sl = slot_layout(*dims, precision);
  const size_t mb = mod_bytes(*dims, *layout);
  const size_t mods_region = up(mb * (size_t)n_blocks);
  Plan plan;
  rc = prepare(dims, layout, precision, flags, tr != nullptr, x, workspace, workspace_bytes, plan,
               mods_region + 2 * sl.total);
  if (rc == 1) return H3DIT_OK;
  if (rc) return rc;
  for (int32_t b = 0; b < n_blocks; b++)
    if ((rc = check_block(&blocks[b], precision))) return rc;
  if ((rc = check_rope(rope)) || (tr && (rc = check_rope(&tr->rope_reduced)))) return rc;
  if ((rc = check_device())) return rc;
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  uint8_t *mods = ws + plan.total, *slot[2] = {mods + mods_region, mods + mods_region + sl.total};
  const hipStream_t st = (hipStream_t)stream;
  const hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : st;

  // device view of every block: matrices in slot b % 2, mod rows resident (host-side array; no
  // exception leaves the C ABI)
  std::vector<h3dit_block_w> dev;
  try {
    dev.resize((size_t)n_blocks);
  } catch (...) {
    return H3DIT_EINVAL;
  }
  for (int32_t b = 0; b < n_blocks; b++) {
    uint8_t *s = slot[b & 1];
    h3dit_block_w &v = dev[(size_t)b];
    v.precision = precision;
    v.w_qkv = s + sl.off[0]; v.w_o = s + sl.off[1]; v.w_fc1 = s + sl.off[2]; v.w_fc2 = s + sl.off[3];
    v.s_qkv = sl.bytes[4] ? reinterpret_cast<const float *>(s + sl.off[4]) : nullptr;
    v.s_o = sl.bytes[5] ? reinterpret_cast<const float *>(s + sl.off[5]) : nullptr;
    v.s_fc1 = sl.bytes[6] ? reinterpret_cast<const float *>(s + sl.off[6]) : nullptr;
    v.s_fc2 = sl.bytes[7] ? reinterpret_cast<const float *>(s + sl.off[7]) : nullptr;
    v.mod = reinterpret_cast<const uint16_t *>(mods + (size_t)b * mb);
    TRY(hipMemcpyAsync(mods + (size_t)b * mb, blocks[b].mod, mb, hipMemcpyHostToDevice, st));
  }
  // copied[s]: block weights in slot s are complete; freed[s]: the block that used slot s is
  // done; entry: everything enqueued on `stream` before this call (an earlier call's blocks
  // may still be reading the slots)
  struct Events {
    hipEvent_t e[5] = {};
    ~Events() {
      for (hipEvent_t x : e)
        if (x) (void)hipEventDestroy(x);
    }
  } ev;
  for (hipEvent_t &e : ev.e) TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  hipEvent_t *copied = ev.e, *freed = ev.e + 2, entry = ev.e[4];
  if (cs != st) {
    // the first two copies overwrite slots the previous call's last blocks may still read
    TRY(hipEventRecord(entry, st));
    TRY(hipStreamWaitEvent(cs, entry, 0));
  }
  auto copy_block = [&](int32_t b) -> int {
    const int s = b & 1;
    if (b >= 2) TRY(hipStreamWaitEvent(cs, freed[s], 0));
    const void *src[8] = {blocks[b].w_qkv, blocks[b].w_o, blocks[b].w_fc1, blocks[b].w_fc2,
                          blocks[b].s_qkv, blocks[b].s_o, blocks[b].s_fc1, blocks[b].s_fc2};
    for (int i = 0; i < 8; i++)
      if (sl.bytes[i]) TRY(hipMemcpyAsync(slot[s] + sl.off[i], src[i], sl.bytes[i], hipMemcpyHostToDevice, cs));
    TRY(hipEventRecord(copied[s], cs));
    return H3DIT_OK;
  };
  Ctx c{dims, layout, flags, ws, plan, st};
  if ((rc = copy_block(0))) return rc;
  auto before = [&](int32_t b) -> int {
    if (b + 1 < n_blocks && (rc = copy_block(b + 1))) return rc;
    TRY(hipStreamWaitEvent(st, copied[b & 1], 0));
    return H3DIT_OK;
  };
  auto after = [&](int32_t b) -> int {
    TRY(hipEventRecord(freed[b & 1], st));
    return H3DIT_OK;
  };
  return run_stack(c, n_blocks, dev.data(), rope, tr, x, before, after);
}

}  // extern "C"

namespace {

// The final head's checks, its statistics bytes (8 per row of the larger part), and, with
// stats != nullptr, its launches.  Returns H3DIT_OK, 1 for a size query answered, or an error.
int final_head_impl(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_head_part *video,
                    const h3dit_head_part *audio, const uint16_t *x, uint16_t *out_video, uint16_t *out_audio,
                    float *stats, size_t *stats_bytes, hipStream_t st) {
  int rc = check_dims(dims, layout, H3DIT_BF16);
  if (rc) return rc;
  const int64_t N = dims->n_tokens, d = dims->hidden;
  const int64_t n_video = N - layout->n_text - layout->n_audio, n_audio = layout->n_audio;
  struct Part {
    const h3dit_head_part *p;
    int64_t r0, n;
    uint16_t *out;
  } parts[2] = {{video, 0, n_video, out_video}, {audio, N - n_audio, n_audio, out_audio}};
  // per-row LayerNorm statistics (mean, 1/sqrt(var + eps)); the normalised rows themselves
  // are formed inside the head GEMM's tile loads and never stored
  size_t st_bytes = 0;
  for (const Part &q : parts) {
    if (!q.p) continue;
    if (!q.p->mod || !q.p->w || !aligned(q.p->mod, 16) || !aligned(q.p->w, 16)) return H3DIT_EINVAL;
    if (q.p->channels < 128 || q.p->channels % 128) return H3DIT_EINVAL;
    if ((size_t)q.n * 8 > st_bytes) st_bytes = (size_t)q.n * 8;
  }
  *stats_bytes = up(st_bytes);
  if (!stats) return 1;
  if (!x || !aligned(x, 16)) return H3DIT_EINVAL;
  for (const Part &q : parts)
    if (q.p && q.n > 0 && (!q.out || !aligned(q.out, 16))) return H3DIT_EINVAL;
  return H3DIT_OK;
}

int final_head_launch(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_head_part *video,
                      const h3dit_head_part *audio, const uint16_t *x, uint16_t *out_video, uint16_t *out_audio,
                      float *stats, hipStream_t st) {
  const int64_t N = dims->n_tokens, d = dims->hidden;
  const int64_t n_video = N - layout->n_text - layout->n_audio, n_audio = layout->n_audio;
  const struct {
    const h3dit_head_part *p;
    int64_t r0, n;
    uint16_t *out;
  } parts[2] = {{video, 0, n_video, out_video}, {audio, N - n_audio, n_audio, out_audio}};
  for (const auto &q : parts) {
    if (!q.p || q.n == 0) continue;
    // the modality's rows are read in place at their offset in the residual
    TRY(launch_row_stats(q.n, (int)d, dims->ln_eps, x + q.r0 * d, stats, st));
    TRY(launch_head_gemm(q.n, q.p->channels, (int)d, x + q.r0 * d, stats, q.p->mod, q.p->mod + d, q.p->w, q.out, st));
  }
  return H3DIT_OK;
}

// Scratch of the allocation-free final head: the row statistics of one part, in a file-scope
// device array (one copy per device, held until the process ends).  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address is taken once per
// device with hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kNoallocScratchBytes = (size_t)512 << 10;   // 65536 rows x 8 bytes
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch[64];

int scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return H3DIT_EHIP;
  if (dev < 0 || dev >= 64) return H3DIT_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return H3DIT_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return H3DIT_OK;
}

}  // namespace

extern "C" {

int h3dit_final_head(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_head_part *video,
                     const h3dit_head_part *audio, const uint16_t *x, uint16_t *out_video, uint16_t *out_audio,
                     void *workspace, size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes) return H3DIT_EINVAL;
  size_t total = 0;
  int rc = final_head_impl(dims, layout, video, audio, nullptr, nullptr, nullptr, nullptr, &total, nullptr);
  if (rc < 0) return rc;
  if (!workspace) {
    *workspace_bytes = total;
    return H3DIT_OK;
  }
  if (!aligned(workspace, ALIGN)) return H3DIT_EINVAL;
  rc = final_head_impl(dims, layout, video, audio, x, out_video, out_audio, reinterpret_cast<float *>(workspace),
                       &total, (hipStream_t)stream);
  if (rc) return rc;
  if (*workspace_bytes < total) {
    *workspace_bytes = total;
    return H3DIT_EWORKSPACE;
  }
  if ((rc = check_device())) return rc;
  return final_head_launch(dims, layout, video, audio, x, out_video, out_audio, reinterpret_cast<float *>(workspace),
                           (hipStream_t)stream);
}

int h3dit_final_head_noalloc(const h3dit_dims *dims, const h3dit_layout *layout, const h3dit_head_part *video,
                             const h3dit_head_part *audio, const uint16_t *x, uint16_t *out_video,
                             uint16_t *out_audio, void *stream) {
  size_t total = 0;
  int rc = final_head_impl(dims, layout, video, audio, nullptr, nullptr, nullptr, nullptr, &total, nullptr);
  if (rc < 0) return rc;
  if (total > kNoallocScratchBytes) return H3DIT_EWORKSPACE;
  if ((rc = check_device())) return rc;
  void *sp = nullptr;
  if ((rc = scratch_ptr(&sp))) return rc;
  rc = final_head_impl(dims, layout, video, audio, x, out_video, out_audio, reinterpret_cast<float *>(sp), &total,
                       (hipStream_t)stream);
  if (rc) return rc;
  return final_head_launch(dims, layout, video, audio, x, out_video, out_audio, reinterpret_cast<float *>(sp),
                           (hipStream_t)stream);
}

// ---------------------------------------------------------------- denoising loop

int h3dit_denoise_plan(const h3dit_denoise_opts *o, int32_t n_blocks, h3dit_denoise_step *plan) {
  if (!o || !plan) return H3DIT_EINVAL;
  if (o->steps < 1 || o->reuse < 1 || o->core_reuse < 1 || (o->reuse > 1 && o->core_reuse > 1)) return H3DIT_EINVAL;
  if (n_blocks < 1 || o->layers < 1 || o->layers > n_blocks) return H3DIT_EINVAL;
  const bool red = o->reduce_after >= 0;
  if (red && (o->reduce_after >= o->layers || o->restore_early <= o->reduce_after ||
              o->restore_late <= o->reduce_after || o->early_evals < 0))
    return H3DIT_EINVAL;
  int32_t evals = 0;
  for (int32_t i = 0; i < o->steps; i++) {
    const bool last = i + 1 == o->steps;
    const bool fresh = i % o->reuse == 0 || last;
    const bool core = fresh && (i % o->core_reuse == 0 || last);
    if (core) evals++;
    h3dit_denoise_step &st = plan[i];
    st.fresh = fresh;
    st.core = core;
    st.eval = evals - 1;
    st.n_blocks = o->layers;
    st.restore_before = red ? (st.eval < o->early_evals ? o->restore_early : o->restore_late) : -1;
  }
  return evals;
}

int h3dit_velocity_step(int64_t count, float dt, const uint16_t *v, uint16_t *z, void *stream) {
  if (count < 0 || count % 8 || !v || !z || !aligned(v, 16) || !aligned(z, 16)) return H3DIT_EINVAL;
  if (count == 0) return H3DIT_OK;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_velocity_step(count, dt, v, z, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_denoise_fwd(const h3dit_dims *dims, const h3dit_layout *layout, int32_t n_blocks,
                      const h3dit_block_w *blocks, const h3dit_rope *rope, const h3dit_rope *rope_reduced,
                      const h3dit_denoise_opts *opts, const float *dt, const uint16_t *x_in,
                      const h3dit_patch_embed *embed, const h3dit_head_part *video, const h3dit_head_part *audio,
                      uint16_t *z_video, uint16_t *z_audio, uint32_t flags, void *workspace, size_t *workspace_bytes,
                      void *stream) {
  if (!workspace_bytes || !dims || !layout || !blocks || !opts || n_blocks < 1 || (!video && !audio))
    return H3DIT_EINVAL;
  if (opts->steps < 1) return H3DIT_EINVAL;
  std::vector<h3dit_denoise_step> plan;
  try {
    plan.resize((size_t)opts->steps);
  } catch (...) {
    return H3DIT_EINVAL;
  }
  int rc = h3dit_denoise_plan(opts, n_blocks, plan.data());
  if (rc < 0) return rc;
  if ((rc = check_rope(rope)) || (rc = check_rope(rope_reduced))) return rc;
  const bool red = opts->reduce_after >= 0;
  // sizes: the working residual, the two velocity buffers, then the stack's, the head's or the
  // embedding's workspace (they run one after the other on the stream, so they share it)
  h3dit_token_reduction tr_q{opts->reduce_after,
                             opts->restore_early > opts->restore_late ? opts->restore_early : opts->restore_late,
                             {nullptr, nullptr}};
  size_t stack_bytes = 0, head_bytes = 0;
  if ((rc = h3dit_stack_fwd(dims, layout, opts->layers, blocks, nullptr, red ? &tr_q : nullptr, nullptr, flags,
                            nullptr, &stack_bytes, nullptr)))
    return rc;
  if ((rc = h3dit_final_head(dims, layout, video, audio, nullptr, nullptr, nullptr, nullptr, &head_bytes, nullptr)))
    return rc;
  const int64_t N = dims->n_tokens, d = dims->hidden;
  const int64_t n_audio = layout->n_audio, n_video = N - layout->n_text - n_audio;
  const int64_t cv = video ? (int64_t)video->channels * n_video : 0, ca = audio ? (int64_t)audio->channels * n_audio : 0;
  // patch embedding of each part: e = bf16(z W^T) into the shared region, then x_rows += e
  struct Embed {
    const uint16_t *w;
    const uint16_t *z;
    int64_t rows, r0, channels;
  } emb[2] = {{embed && video ? embed->w_video : nullptr, z_video, n_video, 0, video ? video->channels : 0},
              {embed && audio ? embed->w_audio : nullptr, z_audio, n_audio, N - n_audio, audio ? audio->channels : 0}};
  size_t emb_bytes = 0;
  h3dit_linear_args ela[2] = {};
  for (int i = 0; i < 2; i++) {
    Embed &e = emb[i];
    if (!e.w || e.rows == 0) {
      e.w = nullptr;
      continue;
    }
    if (!aligned(e.w, 16)) return H3DIT_EINVAL;
    h3dit_linear_args &la = ela[i];
    la.M = e.rows; la.N = d; la.K = e.channels; la.precision = H3DIT_BF16; la.out_kind = H3DIT_OUT_BF16;
    const size_t need = up((size_t)(e.rows * d * 2)) + linear_workspace(la);
    if (need > emb_bytes) emb_bytes = need;
  }
  const size_t x_off = 0, vv_off = up((size_t)(N * d * 2)), va_off = vv_off + up((size_t)cv * 2),
               rest_off = va_off + up((size_t)ca * 2);
  size_t rest = stack_bytes > head_bytes ? stack_bytes : head_bytes;
  if (emb_bytes > rest) rest = emb_bytes;
  const size_t total = rest_off + rest;
  if (!workspace) {
    *workspace_bytes = total;
    return H3DIT_OK;
  }
  if (!dt || !x_in || !aligned(x_in, 16) || !aligned(workspace, ALIGN)) return H3DIT_EINVAL;
  if ((video && cv > 0 && (!z_video || !aligned(z_video, 16))) || (audio && ca > 0 && (!z_audio || !aligned(z_audio, 16))))
    return H3DIT_EINVAL;
  if (*workspace_bytes < total) {
    *workspace_bytes = total;
    return H3DIT_EWORKSPACE;
  }
  for (int32_t b = 0; b < opts->layers; b++)
    if ((rc = check_block(&blocks[b], blocks[0].precision))) return rc;
  if ((rc = check_device())) return rc;
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  uint16_t *x = reinterpret_cast<uint16_t *>(ws + x_off);
  uint16_t *vv = reinterpret_cast<uint16_t *>(ws + vv_off), *va = reinterpret_cast<uint16_t *>(ws + va_off);
  const hipStream_t st = (hipStream_t)stream;
  for (const h3dit_denoise_step &s : plan) {
    if (s.core) {
      TRY(hipMemcpyAsync(x, x_in, (size_t)(N * d * 2), hipMemcpyDeviceToDevice, st));
      for (int i = 0; i < 2; i++) {
        const Embed &e = emb[i];
        if (!e.w) continue;
        uint16_t *eb = reinterpret_cast<uint16_t *>(ws + rest_off);
        h3dit_linear_args la = ela[i];
        la.a = e.z; la.w = e.w; la.out = eb;
        la.workspace = ws + rest_off + up((size_t)(e.rows * d * 2));
        la.workspace_bytes = rest - up((size_t)(e.rows * d * 2));
        TRY(launch_linear(la, st));
        // x_rows = bf16(x_rows + 1 * e): the velocity-step kernel with dt = 1 is exactly this sum
        TRY(launch_velocity_step(e.rows * d, 1.0f, eb, x + e.r0 * d, st));
      }
      h3dit_token_reduction tr{opts->reduce_after, s.restore_before,
                               {rope_reduced ? rope_reduced->cos : nullptr, rope_reduced ? rope_reduced->sin : nullptr}};
      size_t sb = rest;
      if ((rc = h3dit_stack_fwd(dims, layout, s.n_blocks, blocks, rope, red ? &tr : nullptr, x, flags, ws + rest_off,
                                &sb, stream)))
        return rc;
    }
    if (s.fresh) {
      size_t hb = rest;
      if ((rc = h3dit_final_head(dims, layout, video, audio, x, video ? vv : nullptr, audio ? va : nullptr,
                                 ws + rest_off, &hb, stream)))
        return rc;
    }
    const float step_dt = dt[&s - plan.data()];
    if (cv > 0) TRY(launch_velocity_step(cv, step_dt, vv, z_video, st));
    if (ca > 0) TRY(launch_velocity_step(ca, step_dt, va, z_audio, st));
  }
  return H3DIT_OK;
}

// ---------------------------------------------------------------- stage entry points

int h3dit_rope_tables(const h3dit_layout *L, int32_t head_dim, int32_t reduced, float *cos_t, float *sin_t,
                      void *stream) {
  if (!L || !cos_t || !sin_t || (head_dim != 64 && head_dim != 128)) return H3DIT_EINVAL;
  if (L->video_t < 0 || L->video_h < 0 || L->video_w < 0 || L->n_text < 0 || L->n_audio < 0) return H3DIT_EINVAL;
  if (L->rope_t < 0 || L->rope_h < 0 || L->rope_w < 0 || (L->rope_t | L->rope_h | L->rope_w) & 1 ||
      L->rope_t + L->rope_h + L->rope_w != head_dim || !(L->rope_theta > 0.0f))
    return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_rope_tables(*L, head_dim, reduced ? 1 : 0, cos_t, sin_t, (hipStream_t)stream));
  return (int)layout_tokens(*L, reduced != 0);
}

int h3dit_row_gate_adaln(int64_t n, int32_t d, float eps, const uint16_t *x, const uint16_t *gate, const uint16_t *y,
                         uint16_t *x_out, const uint16_t *shift, const uint16_t *scale, uint16_t *h, int8_t *q,
                         float *s, void *stream) {
  if (n < 0 || d < 8 || d % 8 || d > 8192) return H3DIT_EINVAL;
  if (!gate && !shift) return H3DIT_EINVAL;
  if (n == 0) return H3DIT_OK;   // nothing to do: pointers are not examined
  if (!x || !aligned(x, 16)) return H3DIT_EINVAL;
  if (gate && (!y || !x_out || !aligned(gate, 16) || !aligned(y, 16) || !aligned(x_out, 16))) return H3DIT_EINVAL;
  if (shift && (!scale || !aligned(shift, 16) || !aligned(scale, 16))) return H3DIT_EINVAL;
  if (shift && !h && !q) return H3DIT_EINVAL;
  if (h && !aligned(h, 16)) return H3DIT_EINVAL;
  if (q && (!s || !aligned(q, 8) || !aligned(s, 4))) return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_row(n, d, eps, x, gate, y, x_out, shift, scale, h, q, s, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_quantize_rows(int64_t rows, int64_t cols, int64_t group, const uint16_t *v, int32_t headmajor_hd, int8_t *q,
                        float *s, void *stream) {
  if (rows < 0 || cols < 8 || group < 8 || group % 8 || cols % group || rows > INT32_MAX) return H3DIT_EINVAL;
  if (headmajor_hd < 0 || (headmajor_hd > 0 && (headmajor_hd % 8 || cols % headmajor_hd || group > 8192)))
    return H3DIT_EINVAL;
  if (rows == 0) return H3DIT_OK;
  if (!v || !q || !s || !aligned(v, 16) || !aligned(q, 8) || !aligned(s, 4)) return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_quant_rows(rows, cols, group, v, headmajor_hd, q, s, (hipStream_t)stream));
  return H3DIT_OK;
}

static int check_linear(const h3dit_linear_args *a) {
  if (!a || a->M < 0 || a->N < 128 || a->N % 128 || a->K < 128 || a->K % 128) return H3DIT_EINVAL;
  if (a->M == 0) return H3DIT_OK;   // nothing to do: pointers are not examined
  if (!a->a || !a->w || !aligned(a->a, 16) || !aligned(a->w, 16)) return H3DIT_EINVAL;
  const bool i8 = a->precision == H3DIT_INT8;
  if (!i8 && a->precision != H3DIT_BF16) return H3DIT_EINVAL;
  const int esz = i8 ? 1 : 2;
  if ((a->M + 255) * a->K * esz >= ((int64_t)1 << 32) || a->N * a->K * esz >= ((int64_t)1 << 32)) return H3DIT_EINVAL;
  if (a->a_headmajor_hd && (i8 || (a->a_headmajor_hd != 64 && a->a_headmajor_hd != 128) || a->K % a->a_headmajor_hd ||
                            (a->out_kind != H3DIT_OUT_BF16 && a->out_kind != H3DIT_OUT_F32)))
    return H3DIT_EINVAL;
  if (i8) {
    if (!a->a_scale || !a->w_scale) return H3DIT_EINVAL;
    if (a->a_group && (a->a_group % 128 || a->K % a->a_group || a->out_kind != H3DIT_OUT_BF16)) return H3DIT_EINVAL;
    if (a->out_kind == H3DIT_OUT_F32) return H3DIT_EINVAL;
  } else if (a->out_kind == H3DIT_OUT_I32 || a->a_group) {
    return H3DIT_EINVAL;
  }
  if (a->out_kind == H3DIT_OUT_QKV) {
    if (a->head_dim != 64 && a->head_dim != 128) return H3DIT_EINVAL;
    const int64_t d = (int64_t)a->heads * a->head_dim;
    if (a->N != 3 * d || d % 128 || !a->cos_t || !a->sin_t || !a->out_q || !a->out_k || !a->out_v) return H3DIT_EINVAL;
    if (!aligned(a->cos_t, 16) || !aligned(a->sin_t, 16) || !aligned(a->out_q, 16) || !aligned(a->out_k, 16) ||
        !aligned(a->out_v, 16))
      return H3DIT_EINVAL;
  } else if (a->out_kind < 0 || a->out_kind > H3DIT_OUT_QKV || !a->out || !aligned(a->out, 16)) {
    return H3DIT_EINVAL;
  }
  if (a->workspace && !aligned(a->workspace, ALIGN)) return H3DIT_EINVAL;
  return H3DIT_OK;
}

int h3dit_linear_workspace(const h3dit_linear_args *a, uint64_t *bytes) {
  if (!bytes) return H3DIT_EINVAL;
  int rc = check_linear(a);
  if (rc) return rc;
  *bytes = linear_workspace(*a);
  return H3DIT_OK;
}

int h3dit_linear_a_extent(const h3dit_linear_args *a, uint64_t *max_end, uint64_t *bad) {
  if (!max_end || !bad) return H3DIT_EINVAL;
  int rc = check_linear(a);
  if (rc) return rc;
  *max_end = 0;
  *bad = 0;
  if (a->M > 0) linear_a_extent(*a, max_end, bad);
  return H3DIT_OK;
}

int h3dit_linear(const h3dit_linear_args *a, void *stream) {
  int rc = check_linear(a);
  if (rc) return rc;
  if (a->M == 0) return H3DIT_OK;
  const size_t need = linear_workspace(*a);
  if (need && (!a->workspace || a->workspace_bytes < need)) return H3DIT_EWORKSPACE;
  if ((rc = check_device())) return rc;
  TRY(launch_linear(*a, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_rope_split(int64_t n, int32_t heads, int32_t head_dim, const uint16_t *t, const float *cos_t,
                     const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *vt, void *stream) {
  if (n < 0 || heads < 1 || (head_dim != 64 && head_dim != 128)) return H3DIT_EINVAL;
  if (n == 0) return H3DIT_OK;
  if (!t || !cos_t || !sin_t || !q || !k || !vt || !aligned(t, 16) || !aligned(q, 16) || !aligned(k, 16))
    return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_rope_split(n, heads, head_dim, t, cos_t, sin_t, q, k, vt, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_gelu(int64_t count, const uint16_t *u, uint16_t *gl, void *stream) {
  if (count < 0 || count % 8) return H3DIT_EINVAL;
  if (count == 0) return H3DIT_OK;
  if (!u || !gl || !aligned(u, 16) || !aligned(gl, 16)) return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_gelu(count, u, gl, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_attention(int32_t heads, int64_t n, int32_t head_dim, const uint16_t *q, const uint16_t *k,
                    const uint16_t *vt, uint16_t *o, float *row_max, float *row_sum, void *stream) {
  if (heads < 1 || n < 0 || (head_dim != 64 && head_dim != 128)) return H3DIT_EINVAL;
  if (n == 0) return H3DIT_OK;
  if (!q || !k || !vt || !o || !aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(o, 16))
    return H3DIT_EINVAL;
  if ((row_max == nullptr) != (row_sum == nullptr)) return H3DIT_EINVAL;
  const int64_t ldv = vt_pitch(n);
  if ((int64_t)heads * (n + 64) * head_dim * 2 >= ((int64_t)1 << 32) ||
      (int64_t)heads * head_dim * (ldv + 64) * 2 >= ((int64_t)1 << 32))
    return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_attention(heads, n, head_dim, q, k, vt, o, row_max, row_sum, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_token_pair(const h3dit_layout *L, int32_t d, const uint16_t *x, uint16_t *r, uint16_t *r_in, void *stream) {
  if (!L || d < 8 || d % 8 || !x || !r || !aligned(x, 16) || !aligned(r, 16) || (r_in && !aligned(r_in, 16)))
    return H3DIT_EINVAL;
  if (L->video_t < 0 || L->video_h < 0 || L->video_w < 0 || L->n_text < 0 || L->n_audio < 0) return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_token_pair(*L, d, x, r, r_in, (hipStream_t)stream));
  return H3DIT_OK;
}

int h3dit_token_restore(const h3dit_layout *L, int32_t d, uint16_t *x, const uint16_t *y, const uint16_t *r_in,
                        void *stream) {
  if (!L || d < 8 || d % 8 || !x || !y || !r_in || !aligned(x, 16) || !aligned(y, 16) || !aligned(r_in, 16))
    return H3DIT_EINVAL;
  if (L->video_t < 0 || L->video_h < 0 || L->video_w < 0 || L->n_text < 0 || L->n_audio < 0) return H3DIT_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  TRY(launch_token_restore(*L, d, x, y, r_in, (hipStream_t)stream));
  return H3DIT_OK;
}

}  // extern "C"
