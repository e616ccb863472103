"""ctypes wrapper of the CPU oracle — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this package.
It wraps oracle/liboracle.so (plain C, fp32, OpenMP over rows), which shares no code
with the HIP library.  Tensors are torch CPU tensors; bf16 travels as its bit pattern.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# H3DIT_ORACLE_LIB names another build of the same source (the sanitizer build of the tests)
_LIB_PATH = os.environ.get("H3DIT_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
_lib = None


class Dims(C.Structure):
    _fields_ = [("n_tokens", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("mlp", C.c_int32), ("fc2_group", C.c_int32),
                ("ln_eps", C.c_float), ("n_video", C.c_int32), ("n_text", C.c_int32)]


class Layout(C.Structure):
    _fields_ = [("video_t", C.c_int32), ("video_h", C.c_int32), ("video_w", C.c_int32),
                ("n_text", C.c_int32), ("n_audio", C.c_int32), ("split_t", C.c_int32),
                ("split_h", C.c_int32), ("split_w", C.c_int32), ("theta", C.c_float)]


class Block(C.Structure):
    _fields_ = [("int8", C.c_int32)] + \
        [(n, C.c_void_p) for n in ("wqkv", "wo", "w1", "w2", "qqkv", "qo", "q1", "q2",
                                   "sqkv", "so", "s1", "s2", "mod")] + [("mod_sets", C.c_int32)]


class Taps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("h1", "t", "q", "k", "v", "o", "y1", "x1", "h2", "u",
                                          "gl", "y2", "att_max", "att_sum")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(_LIB_PATH)
        _lib.orc_gelu_tanh_f32.restype = C.c_float
        _lib.orc_gelu_tanh_f32.argtypes = [C.c_float]
        _lib.orc_num_threads.restype = C.c_int32
        for name in ("orc_layout_tokens", "orc_rope_tables", "orc_token_pair", "orc_token_restore",
                     "orc_block_fwd", "orc_stack_fwd", "orc_denoise_plan"):
            getattr(_lib, name).restype = C.c_int32
    return _lib


def _p(t):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return C.c_void_p(t.data_ptr())


def _i64(v):
    return C.c_int64(int(v))


def bf16(shape):
    return torch.empty(shape, dtype=torch.bfloat16)


def dims_of(w, n_tokens=None) -> Dims:
    """Widths and the segments of an n_tokens sequence: the workload's own, or its paired
    (reduced) sequence, whose video part is shorter by the number of pairs."""
    N = int(n_tokens if n_tokens is not None else w.n_tokens)
    n_video = N - w.n_text - w.n_audio
    if n_video < 0:
        raise ValueError("sequence shorter than the text and audio segments")
    return Dims(N, w.hidden, w.heads, w.head_dim, w.mlp, w.fc2_group, w.ln_eps, n_video, w.n_text)


def layout_of(w) -> Layout:
    st, sh, sw = w.split
    return Layout(w.video_t, w.video_h, w.video_w, w.n_text, w.n_audio, st, sh, sw, w.rope_theta)


# ------------------------------------------------------------------ helpers

def f32_to_bf16(x: torch.Tensor) -> torch.Tensor:
    x = x.contiguous().to(torch.float32)
    out = bf16(x.shape)
    lib().orc_f32_to_bf16(_p(x), _p(out), _i64(x.numel()))
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def gelu_tanh(u: float) -> float:
    return float(lib().orc_gelu_tanh_f32(C.c_float(u)))


def layout_tokens(w, reduced: bool) -> int:
    return int(lib().orc_layout_tokens(C.byref(layout_of(w)), int(reduced)))


def rope_tables(w, reduced: bool = False):
    n = layout_tokens(w, reduced)
    cos = torch.empty((n, w.head_dim // 2), dtype=torch.float32)
    sin = torch.empty_like(cos)
    rc = lib().orc_rope_tables(C.byref(layout_of(w)), w.head_dim, int(reduced), _p(cos), _p(sin))
    if rc != n:
        raise ValueError("bad rotary layout")
    return cos, sin


# ------------------------------------------------------------------ stages

def adaln(x, shift, scale, eps=1e-6, stats=False):
    n, d = x.shape
    h = bf16((n, d))
    mean = torch.empty(n, dtype=torch.float32)
    rstd = torch.empty(n, dtype=torch.float32)
    lib().orc_adaln(_i64(n), C.c_int32(d), C.c_float(eps), _p(x.contiguous()), _p(shift.contiguous()),
                    _p(scale.contiguous()), _p(h), _p(mean), _p(rstd))
    return (h, mean, rstd) if stats else h


def q8_rows(v, group=None):
    rows, cols = v.shape
    group = cols if group is None else group
    q = torch.empty((rows, cols), dtype=torch.int8)
    s = torch.empty((rows, cols // group), dtype=torch.float32)
    lib().orc_q8_rows(_i64(rows), _i64(cols), _i64(group), _p(v.contiguous()), _p(q), _p(s))
    return q, s


def quantize_weights(w):
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8)
    s = torch.empty(rows, dtype=torch.float32)
    lib().orc_quantize_weights(_i64(rows), _i64(cols), _p(w.contiguous()), _p(q), _p(s))
    return q, s


def gemm_f32(a, w):
    M, K = a.shape
    N = w.shape[0]
    acc = torch.empty((M, N), dtype=torch.float32)
    lib().orc_gemm_f32(_i64(M), _i64(N), _i64(K), _p(a.contiguous()), _p(w.contiguous()), _p(acc))
    return acc


def gemm_i32(qa, qw):
    M, K = qa.shape
    N = qw.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32)
    lib().orc_gemm_i32(_i64(M), _i64(N), _i64(K), _p(qa.contiguous()), _p(qw.contiguous()), _p(acc))
    return acc


def dequant_bf16(acc, sa, sw):
    M, N = acc.shape
    out = bf16((M, N))
    lib().orc_dequant_bf16(_i64(M), _i64(N), _p(acc.contiguous()), _p(sa.contiguous()),
                           _p(sw.contiguous()), _p(out))
    return out


def fc2_int8(qa, sa, qw, sw, group):
    M, K = qa.shape
    N = qw.shape[0]
    y = bf16((M, N))
    lib().orc_fc2_int8(_i64(M), _i64(N), _i64(K), _i64(group), _p(qa.contiguous()), _p(sa.contiguous()),
                       _p(qw.contiguous()), _p(sw.contiguous()), _p(y))
    return y


def rope_split(t, cos, sin, heads, head_dim):
    N = t.shape[0]
    d = heads * head_dim
    q, k, v = (bf16((heads, N, head_dim)) for _ in range(3))
    lib().orc_rope_split(_i64(N), C.c_int32(d), C.c_int32(heads), C.c_int32(head_dim), _p(t.contiguous()),
                         _p(cos.contiguous()), _p(sin.contiguous()), _p(q), _p(k), _p(v))
    return q, k, v


def attention(q, k, v, stats=False):
    """q: [H][Nq][hd] query rows (all tokens or a subset), k, v: [H][N][hd]."""
    H, Nq, hd = q.shape
    N = k.shape[1]
    o = bf16((H, Nq, hd))
    mx = torch.empty((H, Nq), dtype=torch.float32)
    sm = torch.empty((H, Nq), dtype=torch.float32)
    lib().orc_attention(C.c_int32(H), _i64(Nq), _i64(N), C.c_int32(hd), _p(q.contiguous()), _p(k.contiguous()),
                        _p(v.contiguous()), _p(o), _p(mx), _p(sm))
    return (o, mx, sm) if stats else o


def gelu_rows(u):
    gl = bf16(u.shape)
    lib().orc_gelu_rows(_i64(u.numel()), _p(u.contiguous()), _p(gl))
    return gl


def gate(x, g, y):
    n, d = x.shape
    out = bf16((n, d))
    lib().orc_gate(_i64(n), C.c_int32(d), _p(x.contiguous()), _p(g.contiguous()), _p(y.contiguous()), _p(out))
    return out


def token_pair(w, x):
    r = bf16((layout_tokens(w, True), x.shape[1]))
    lib().orc_token_pair(C.byref(layout_of(w)), C.c_int32(x.shape[1]), _p(x.contiguous()), _p(r))
    return r


def token_restore(w, bypass, y, r_in):
    x = bf16(bypass.shape)
    lib().orc_token_restore(C.byref(layout_of(w)), C.c_int32(bypass.shape[1]), _p(bypass.contiguous()),
                            _p(y.contiguous()), _p(r_in.contiguous()), _p(x))
    return x


def final_head(w, x, video=None, audio=None):
    """The final head on the video rows [0, n_video) and the audio rows (the last n_audio) of
    the residual x: each part is (mod bf16 [2][d] = shift, scale; W bf16 [c][d]); returns
    (out_video [n_video][c_v] or None, out_audio [n_audio][c_a] or None)."""
    n_video = x.shape[0] - w.n_text - w.n_audio
    outs = []
    for part, r0, n in ((video, 0, n_video), (audio, x.shape[0] - w.n_audio, w.n_audio)):
        if part is None:
            outs.append(None)
            continue
        mod, wt = part
        c = wt.shape[0]
        out = bf16((n, c))
        xs = x[r0:r0 + n].contiguous()
        lib().orc_final_head(_i64(n), C.c_int32(w.hidden), C.c_int32(c), C.c_float(w.ln_eps), _p(xs),
                             _p(mod[0].contiguous()), _p(mod[1].contiguous()), _p(wt.contiguous()), _p(out))
        outs.append(out)
    return tuple(outs)


# ------------------------------------------------------------------ block and stack

def _block_struct(p: dict, keep: list) -> Block:
    """p: bf16 weights {wqkv, wo, w1, w2, mod} and, for int8, {qqkv, sqkv, qo, so, q1, s1, q2, s2}."""
    b = Block()
    has_attn, has_mlp = "qqkv" in p, "q1" in p
    b.int8 = 1 if (has_attn and has_mlp) else 3 if has_attn else 2 if has_mlp else 0
    b.mod_sets = p["mod"].shape[0] // 6
    for name in ("wqkv", "wo", "w1", "w2", "qqkv", "qo", "q1", "q2", "sqkv", "so", "s1", "s2", "mod"):
        t = p.get(name)
        if t is not None:
            t = t.contiguous()
            keep.append(t)
            setattr(b, name, t.data_ptr())
    return b


def quantize_block(p: dict, mlp_only: bool = False, attn_only: bool = False) -> dict:
    """Adds the int8 codes and scales of the four weight matrices to a bf16 block dict; or of
    FC1 and FC2 only (mlp_only: the "int8 MLP" row of the pages' table); or of QKV and the
    output projection only (attn_only: the int8-QKV-only path the pages set against it)."""
    assert not (mlp_only and attn_only)
    out = dict(p)
    pairs = (("wqkv", "qqkv", "sqkv"), ("wo", "qo", "so"), ("w1", "q1", "s1"), ("w2", "q2", "s2"))
    sel = pairs[2:] if mlp_only else pairs[:2] if attn_only else pairs
    for w, q, s in sel:
        out[q], out[s] = quantize_weights(p[w])
    return out


TAP_NAMES = ("h1", "t", "q", "k", "v", "o", "y1", "x1", "h2", "u", "gl", "y2", "att_max", "att_sum")


def block_fwd(w, p: dict, x, cos=None, sin=None, fused=False, taps=False, n_tokens=None):
    """One block on x (bf16 [N][d]); returns the new residual (and a dict of stage tensors)."""
    N = x.shape[0] if n_tokens is None else n_tokens
    d, H, hd, f = w.hidden, w.heads, w.head_dim, w.mlp
    if cos is None:
        cos, sin = rope_tables(w)
    keep = []
    b = _block_struct(p, keep)
    xo = x.contiguous().clone()
    tp = None
    tapd = {}
    if taps:
        shapes = {"h1": (N, d), "t": (N, 3 * d), "q": (H, N, hd), "k": (H, N, hd), "v": (H, N, hd),
                  "o": (H, N, hd), "y1": (N, d), "x1": (N, d), "h2": (N, d), "u": (N, f), "gl": (N, f),
                  "y2": (N, d)}
        for k_, s_ in shapes.items():
            tapd[k_] = bf16(s_)
        tapd["att_max"] = torch.empty((H, N), dtype=torch.float32)
        tapd["att_sum"] = torch.empty((H, N), dtype=torch.float32)
        tp = Taps(*[tapd[n].data_ptr() for n in TAP_NAMES])
    rc = lib().orc_block_fwd(C.byref(dims_of(w, N)), C.byref(b), _p(cos.contiguous()), _p(sin.contiguous()),
                             _p(xo), int(fused), C.byref(tp) if tp is not None else None)
    if rc != 0:
        raise ValueError(f"orc_block_fwd failed: {rc}")
    return (xo, tapd) if taps else xo


def stack_fwd(w, blocks: list, x, reduce_after=-1, restore_before=-1, fused=False, rope=None, rope_reduced=None):
    """rope / rope_reduced: (cos, sin) fp32 tables of the full / paired sequence, or None for
    the layout's own (orc_rope_tables)."""
    keep = []
    arr = (Block * len(blocks))(*[_block_struct(p, keep) for p in blocks])
    xo = x.contiguous().clone()
    tabs = []
    for r in (rope, rope_reduced):
        if r is None:
            tabs += [None, None]
        else:
            c_, s_ = r[0].contiguous().to(torch.float32), r[1].contiguous().to(torch.float32)
            keep += [c_, s_]
            tabs += [_p(c_), _p(s_)]
    rc = lib().orc_stack_fwd(C.byref(dims_of(w)), C.byref(layout_of(w)), C.c_int32(len(blocks)), arr,
                             C.c_int32(reduce_after), C.c_int32(restore_before), _p(xo), int(fused), *tabs)
    if rc != 0:
        raise ValueError(f"orc_stack_fwd failed: {rc}")
    return xo


# ------------------------------------------------------------------ denoising loop

def velocity_step(z, v, dt: float):
    """bf(z + dt*v) elementwise (bf16 tensors of one shape); returns a new tensor."""
    zo = z.contiguous().clone()
    vc = v.contiguous()
    assert zo.numel() == vc.numel()
    lib().orc_velocity_step(_i64(zo.numel()), C.c_float(dt), _p(vc), _p(zo))
    return zo


def denoise_plan(steps, reuse=1, core_reuse=1, reduce_after=-1, restore_early=40, restore_late=30, early=10):
    """Per-step schedule: a list of dicts {fresh, core, eval, restore}."""
    arrs = [(C.c_int32 * int(steps))() for _ in range(4)]
    rc = lib().orc_denoise_plan(C.c_int32(steps), C.c_int32(reuse), C.c_int32(core_reuse), C.c_int32(reduce_after),
                                C.c_int32(restore_early), C.c_int32(restore_late), C.c_int32(early), *arrs)
    if rc < 0:
        raise ValueError(f"orc_denoise_plan failed: {rc}")
    return [dict(fresh=arrs[0][i], core=arrs[1][i], eval=arrs[2][i], restore=arrs[3][i]) for i in range(steps)]


def patch_embed(x_in, z, E):
    """x_in rows (bf16 [n][d]) plus the patch-embedding stand-in of latents z (bf16 [n][c]) by
    E (bf16 [d][c]): bf16(x_in + bf16(z E^T)) (orc_patch_embed)."""
    n, d = x_in.shape
    c = z.shape[1]
    out = bf16((n, d))
    lib().orc_patch_embed(_i64(n), C.c_int32(d), C.c_int32(c), _p(x_in.contiguous()), _p(z.contiguous()),
                          _p(E.contiguous()), _p(out))
    return out


def denoise(w, blocks: list, x_in, opts: dict, dt, video=None, audio=None, z_video=None, z_audio=None, embed=None,
            plan=None, rope=None, rope_reduced=None):
    """The denoising loop of the plan: a core step starts from x_in (plus the patch embedding of
    the current latents when embed = (E_video or None, E_audio or None) is given) and runs the
    first `layers` blocks (with the step's token restore), a fresh step runs the final head on
    that residual, and every step moves the latents by dt[i] times the latest velocity.
    plan: a per-step list as denoise_plan returns, to replace the plan of opts (tests plant
    wrong schedules through it).  Returns (z_video, z_audio)."""
    if plan is None:
        plan = denoise_plan(opts["steps"], opts.get("reuse", 1), opts.get("core_reuse", 1),
                            opts.get("reduce_after", -1), opts.get("restore_early", 40), opts.get("restore_late", 30),
                            opts.get("early_evals", 10))
    layers = opts.get("layers", len(blocks))
    zv = None if z_video is None else z_video.clone()
    za = None if z_audio is None else z_audio.clone()
    x = vv = va = None
    n_video = x_in.shape[0] - w.n_text - w.n_audio
    for i, s in enumerate(plan):
        if s["core"]:
            red = opts.get("reduce_after", -1)
            xs = x_in
            if embed is not None:
                xs = x_in.clone()
                if embed[0] is not None and zv is not None and n_video > 0:
                    xs[:n_video] = patch_embed(x_in[:n_video], zv, embed[0])
                if embed[1] is not None and za is not None and w.n_audio > 0:
                    xs[-w.n_audio:] = patch_embed(x_in[-w.n_audio:], za, embed[1])
            x = stack_fwd(w, blocks[:layers], xs, reduce_after=red, restore_before=s["restore"] if red >= 0 else -1,
                          fused=True, rope=rope, rope_reduced=rope_reduced)
        if s["fresh"]:
            vv, va = final_head(w, x, video, audio)
        if zv is not None:
            zv = velocity_step(zv, vv, float(dt[i]))
        if za is not None:
            za = velocity_step(za, va, float(dt[i]))
    return zv, za
