"""Python binding of libh3dit.so, the MI355X (gfx950) MiniMax-H3 DiT block library.

Argument marshalling only: every step of the block runs in the library's HIP kernels.
torch supplies device memory and the current stream.  Importing this package without the
built library raises ImportError; there is no fallback path.

Entry points mirror include/h3dit.h (quantize_weights, block_fwd, stack_fwd) and
include/h3dit_stages.h (one call per kernel, used for stage-wise checks and timing).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# H3DIT_LIB names another build of the same sources (the host-sanitizer build of the host tests)
LIB_PATH = os.environ.get("H3DIT_LIB") or os.path.join(HERE, "libh3dit.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python audio_diffusion_transformer_dit_amd/build.py`")

_lib = C.CDLL(LIB_PATH)

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4
BF16, INT8, INT8_MLP, INT8_ATTN = 0, 1, 2, 3
NOFUSE_GATE_ADALN, NOFUSE_ROPE, NOFUSE_GELU, NOFUSE_QUANT, NOFUSE_CROSS_BLOCK, NO_ALIAS = 1, 2, 4, 8, 16, 32
OUT_BF16, OUT_F32, OUT_I32, OUT_GELU, OUT_QKV = 0, 1, 2, 3, 4

EXPORTS = ("h3dit_quantize_weights", "h3dit_block_fwd", "h3dit_stack_fwd", "h3dit_rope_tables",
           "h3dit_row_gate_adaln", "h3dit_quantize_rows", "h3dit_linear", "h3dit_rope_split", "h3dit_gelu",
           "h3dit_attention", "h3dit_token_pair", "h3dit_token_restore", "h3dit_linear_workspace",
           "h3dit_final_head", "h3dit_stack_fwd_streamed", "h3dit_denoise_plan", "h3dit_velocity_step",
           "h3dit_denoise_fwd", "h3dit_linear_a_extent", "h3dit_final_head_noalloc")


class H3Error(RuntimeError):
    def __init__(self, name, code):
        names = {EINVAL: "EINVAL", EWORKSPACE: "EWORKSPACE", EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP"}
        super().__init__(f"{name} failed: {names.get(code, code)}")
        self.code = code


class Dims(C.Structure):
    _fields_ = [("n_tokens", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("mlp", C.c_int32), ("fc2_group", C.c_int32), ("ln_eps", C.c_float)]


class Layout(C.Structure):
    _fields_ = [("video_t", C.c_int32), ("video_h", C.c_int32), ("video_w", C.c_int32), ("n_text", C.c_int32),
                ("n_audio", C.c_int32), ("rope_t", C.c_int32), ("rope_h", C.c_int32), ("rope_w", C.c_int32),
                ("rope_theta", C.c_float), ("mod_sets", C.c_int32)]


class BlockW(C.Structure):
    _fields_ = [("precision", C.c_int32), ("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_fc1", C.c_void_p),
                ("w_fc2", C.c_void_p), ("s_qkv", C.c_void_p), ("s_o", C.c_void_p), ("s_fc1", C.c_void_p),
                ("s_fc2", C.c_void_p), ("mod", C.c_void_p)]


class Rope(C.Structure):
    _fields_ = [("cos", C.c_void_p), ("sin", C.c_void_p)]


class TokenReduction(C.Structure):
    _fields_ = [("reduce_after", C.c_int32), ("restore_before", C.c_int32), ("rope_reduced", Rope)]


class PatchEmbed(C.Structure):
    _fields_ = [("w_video", C.c_void_p), ("w_audio", C.c_void_p)]


class HeadPart(C.Structure):
    _fields_ = [("mod", C.c_void_p), ("w", C.c_void_p), ("channels", C.c_int32)]


class DenoiseOpts(C.Structure):
    _fields_ = [("steps", C.c_int32), ("reuse", C.c_int32), ("core_reuse", C.c_int32), ("layers", C.c_int32),
                ("reduce_after", C.c_int32), ("restore_early", C.c_int32), ("restore_late", C.c_int32),
                ("early_evals", C.c_int32)]


class DenoiseStep(C.Structure):
    _fields_ = [("fresh", C.c_int32), ("core", C.c_int32), ("eval", C.c_int32), ("n_blocks", C.c_int32),
                ("restore_before", C.c_int32)]


class LinearArgs(C.Structure):
    _fields_ = [("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64), ("precision", C.c_int32),
                ("a", C.c_void_p), ("a_headmajor_hd", C.c_int32), ("a_scale", C.c_void_p), ("a_group", C.c_int32),
                ("w", C.c_void_p), ("w_scale", C.c_void_p), ("out_kind", C.c_int32), ("out", C.c_void_p),
                ("cos_t", C.c_void_p), ("sin_t", C.c_void_p), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("out_q", C.c_void_p), ("out_k", C.c_void_p), ("out_v", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_uint64)]


_P = C.c_void_p
_lib.h3dit_quantize_weights.argtypes = [_P, C.c_int64, C.c_int64, _P, _P, _P]
_lib.h3dit_block_fwd.argtypes = [_P, _P, _P, _P, _P, C.c_uint32, _P, _P, _P]
_lib.h3dit_stack_fwd.argtypes = [_P, _P, C.c_int32, _P, _P, _P, _P, C.c_uint32, _P, _P, _P]
_lib.h3dit_stack_fwd_streamed.argtypes = [_P, _P, C.c_int32, _P, _P, _P, _P, C.c_uint32, _P, _P, _P, _P]
_lib.h3dit_rope_tables.argtypes = [_P, C.c_int32, C.c_int32, _P, _P, _P]
_lib.h3dit_row_gate_adaln.argtypes = [C.c_int64, C.c_int32, C.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.h3dit_quantize_rows.argtypes = [C.c_int64, C.c_int64, C.c_int64, _P, C.c_int32, _P, _P, _P]
_lib.h3dit_linear.argtypes = [_P, _P]
_lib.h3dit_linear_workspace.argtypes = [_P, _P]
_lib.h3dit_linear_a_extent.argtypes = [_P, _P, _P]
_lib.h3dit_final_head.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.h3dit_final_head_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P]
_lib.h3dit_denoise_plan.argtypes = [_P, C.c_int32, _P]
_lib.h3dit_velocity_step.argtypes = [C.c_int64, C.c_float, _P, _P, _P]
_lib.h3dit_denoise_fwd.argtypes = [_P, _P, C.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_uint32, _P,
                                   _P, _P]
_lib.h3dit_rope_split.argtypes = [C.c_int64, C.c_int32, C.c_int32, _P, _P, _P, _P, _P, _P, _P]
_lib.h3dit_gelu.argtypes = [C.c_int64, _P, _P, _P]
_lib.h3dit_attention.argtypes = [C.c_int32, C.c_int64, C.c_int32, _P, _P, _P, _P, _P, _P, _P]
_lib.h3dit_token_pair.argtypes = [_P, C.c_int32, _P, _P, _P, _P]
_lib.h3dit_token_restore.argtypes = [_P, C.c_int32, _P, _P, _P, _P]
for _n in EXPORTS:
    getattr(_lib, _n).restype = C.c_int


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(name, rc):
    if rc < 0:
        raise H3Error(name, rc)
    return rc


def dims_of(w, n_tokens=None) -> Dims:
    return Dims(int(w.n_tokens if n_tokens is None else n_tokens), w.hidden, w.heads, w.head_dim, w.mlp,
                w.fc2_group, w.ln_eps)


def layout_of(w) -> Layout:
    st, sh, sw = w.split
    return Layout(w.video_t, w.video_h, w.video_w, w.n_text, w.n_audio, st, sh, sw, w.rope_theta,
                  getattr(w, "mod_sets", 1))


def ldv(n: int) -> int:
    """Row pitch of V^T [H][hd][ldv]: tokens rounded up to a multiple of 16."""
    return (int(n) + 15) // 16 * 16


def vt_positions(n: int) -> torch.Tensor:
    """Column of token t inside a V^T row: keys are permuted within groups of 16 (bits 2 and
    3 of the index swapped), the layout the attention kernel reads."""
    t = torch.arange(int(n), dtype=torch.int64)
    return (t & ~15) | (t & 3) | ((t & 4) << 1) | ((t & 8) >> 1)


def vt_from_v(v: torch.Tensor) -> torch.Tensor:
    """V^T [H][hd][ldv] (padding zero) from head-major values [H][n][hd]."""
    H, n, hd = v.shape
    out = torch.zeros((H, hd, ldv(n)), dtype=v.dtype, device=v.device)
    out[:, :, vt_positions(n).to(v.device)] = v.transpose(1, 2)
    return out


def v_from_vt(vt: torch.Tensor, n: int) -> torch.Tensor:
    """Head-major values [H][n][hd] read back from V^T."""
    return vt[:, :, vt_positions(n).to(vt.device)].transpose(1, 2)


# ------------------------------------------------------------------ h3dit.h

def quantize_weights(w: torch.Tensor, stream=None):
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    s = torch.empty(rows, dtype=torch.float32, device=w.device)
    _check("h3dit_quantize_weights", _lib.h3dit_quantize_weights(_ptr(w), rows, cols, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def block_struct(p: dict) -> BlockW:
    """p: {wqkv, wo, w1, w2, mod} bf16 device tensors; or int8 codes {qqkv, qo, q1, q2} with
    scales {sqkv, so, s1, s2} and mod; or bf16 {wqkv, wo} with int8 {q1, q2, s1, s2} (int8 MLP);
    or int8 {qqkv, qo, sqkv, so} with bf16 {w1, w2} (int8 attention projections only)."""
    if "qqkv" in p and "q1" in p:
        return BlockW(INT8, _ptr(p["qqkv"]), _ptr(p["qo"]), _ptr(p["q1"]), _ptr(p["q2"]), _ptr(p["sqkv"]),
                      _ptr(p["so"]), _ptr(p["s1"]), _ptr(p["s2"]), _ptr(p["mod"]))
    if "qqkv" in p:
        return BlockW(INT8_ATTN, _ptr(p["qqkv"]), _ptr(p["qo"]), _ptr(p["w1"]), _ptr(p["w2"]), _ptr(p["sqkv"]),
                      _ptr(p["so"]), None, None, _ptr(p["mod"]))
    if "q1" in p:
        return BlockW(INT8_MLP, _ptr(p["wqkv"]), _ptr(p["wo"]), _ptr(p["q1"]), _ptr(p["q2"]), None, None,
                      _ptr(p["s1"]), _ptr(p["s2"]), _ptr(p["mod"]))
    return BlockW(BF16, _ptr(p["wqkv"]), _ptr(p["wo"]), _ptr(p["w1"]), _ptr(p["w2"]), None, None, None, None,
                  _ptr(p["mod"]))


def quantize_block(p: dict, stream=None, mlp_only: bool = False, attn_only: bool = False) -> dict:
    """int8 codes of the four projections; or (mlp_only) of FC1 and FC2 with QKV and the
    output projection kept in bf16; or (attn_only) of QKV and the output projection with FC1
    and FC2 kept in bf16."""
    assert not (mlp_only and attn_only)
    out = {"mod": p["mod"]}
    pairs = (("wqkv", "qqkv", "sqkv"), ("wo", "qo", "so"), ("w1", "q1", "s1"), ("w2", "q2", "s2"))
    if mlp_only:
        out["wqkv"], out["wo"] = p["wqkv"], p["wo"]
        pairs = pairs[2:]
    elif attn_only:
        out["w1"], out["w2"] = p["w1"], p["w2"]
        pairs = pairs[:2]
    for w, q, s in pairs:
        out[q], out[s] = quantize_weights(p[w], stream)
    return out


def rope_struct(rope):
    """h3dit_rope of (cos, sin) fp32 device tensors [n][head_dim/2], or None (built-in tables)."""
    return None if rope is None else Rope(_ptr(rope[0]), _ptr(rope[1]))


def reduction_struct(reduction, rope_reduced=None):
    if not reduction:
        return None
    tr = TokenReduction(int(reduction[0]), int(reduction[1]))
    if rope_reduced is not None:
        tr.rope_reduced = rope_struct(rope_reduced)
    return tr


def _ref(s):
    return C.byref(s) if s is not None else None


def block_workspace(w, p: dict, flags: int = 0) -> int:
    size = C.c_size_t(0)
    b = block_struct(p)
    _check("h3dit_block_fwd", _lib.h3dit_block_fwd(C.byref(dims_of(w)), C.byref(layout_of(w)), C.byref(b), None,
                                                   None, flags, None, C.byref(size), None))
    return size.value


def stack_workspace(w, blocks: list, flags: int = 0, reduction=None) -> int:
    size = C.c_size_t(0)
    arr = (BlockW * len(blocks))(*[block_struct(p) for p in blocks])
    tr = reduction_struct(reduction)
    _check("h3dit_stack_fwd", _lib.h3dit_stack_fwd(C.byref(dims_of(w)), C.byref(layout_of(w)), len(blocks), arr,
                                                   None, _ref(tr), None, flags, None, C.byref(size), None))
    return size.value


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def block_fwd(w, p: dict, x: torch.Tensor, flags: int = 0, workspace: torch.Tensor = None, stream=None,
              rope=None):
    """x (bf16 [N][d], device) is updated in place and returned.  rope: (cos, sin) tables or
    None for the built-in ones."""
    b = block_struct(p)
    if workspace is None:
        workspace = alloc_workspace(block_workspace(w, p, flags), x.device)
    size = C.c_size_t(workspace.numel())
    r = rope_struct(rope)
    _check("h3dit_block_fwd", _lib.h3dit_block_fwd(C.byref(dims_of(w)), C.byref(layout_of(w)), C.byref(b), _ref(r),
                                                   _ptr(x), flags, _ptr(workspace), C.byref(size), _stream(stream)))
    return x


class Stack:
    """Holds the host-side block array of a stack so repeated calls marshal nothing new."""

    def __init__(self, w, blocks: list, flags: int = 0, reduction=None, rope=None, rope_reduced=None):
        self.w = w
        self.blocks = blocks
        self.flags = flags
        self.arr = (BlockW * len(blocks))(*[block_struct(p) for p in blocks])
        self.rope_tensors = (rope, rope_reduced)   # kept alive while the structs point at them
        self.rope = rope_struct(rope)
        self.tr = reduction_struct(reduction, rope_reduced)
        self.dims = dims_of(w)
        self.layout = layout_of(w)
        self.workspace_bytes = stack_workspace(w, blocks, flags, reduction)

    def __call__(self, x: torch.Tensor, workspace: torch.Tensor, stream=None):
        size = C.c_size_t(workspace.numel())
        _check("h3dit_stack_fwd", _lib.h3dit_stack_fwd(C.byref(self.dims), C.byref(self.layout), len(self.blocks),
                                                       self.arr, _ref(self.rope), _ref(self.tr), _ptr(x),
                                                       self.flags, _ptr(workspace), C.byref(size), _stream(stream)))
        return x


def stack_fwd(w, blocks: list, x: torch.Tensor, flags: int = 0, reduction=None, workspace=None, stream=None,
              rope=None, rope_reduced=None):
    s = Stack(w, blocks, flags, reduction, rope, rope_reduced)
    if workspace is None:
        workspace = alloc_workspace(s.workspace_bytes, x.device)
    return s(x, workspace, stream)


def host_block(p: dict) -> dict:
    """Copies of a block's tensors in newly allocated pinned host memory (the weights of a
    streamed stack)."""
    return {k: torch.empty(v.shape, dtype=v.dtype, pin_memory=True).copy_(v) for k, v in p.items()}


def stack_streamed_workspace(w, blocks: list, flags: int = 0, reduction=None) -> int:
    size = C.c_size_t(0)
    arr = (BlockW * len(blocks))(*[block_struct(p) for p in blocks])
    tr = reduction_struct(reduction)
    _check("h3dit_stack_fwd_streamed",
           _lib.h3dit_stack_fwd_streamed(C.byref(dims_of(w)), C.byref(layout_of(w)), len(blocks), arr, None,
                                         _ref(tr), None, flags, None, C.byref(size), None, None))
    return size.value


class StreamedStack:
    """A stack whose block weights stay in host memory (pinned host tensors, see host_block):
    each block's matrices are copied into one of two device slots on `copy_stream` while the
    previous block computes."""

    def __init__(self, w, host_blocks: list, flags: int = 0, reduction=None, rope=None, rope_reduced=None):
        self.blocks = host_blocks
        self.flags = flags
        self.arr = (BlockW * len(host_blocks))(*[block_struct(p) for p in host_blocks])
        self.rope_tensors = (rope, rope_reduced)
        self.rope = rope_struct(rope)
        self.tr = reduction_struct(reduction, rope_reduced)
        self.dims = dims_of(w)
        self.layout = layout_of(w)
        self.workspace_bytes = stack_streamed_workspace(w, host_blocks, flags, reduction)

    def __call__(self, x: torch.Tensor, workspace: torch.Tensor, stream=None, copy_stream=None):
        size = C.c_size_t(workspace.numel())
        _check("h3dit_stack_fwd_streamed",
               _lib.h3dit_stack_fwd_streamed(C.byref(self.dims), C.byref(self.layout), len(self.blocks), self.arr,
                                             _ref(self.rope), _ref(self.tr), _ptr(x), self.flags,
                                             _ptr(workspace), C.byref(size), _stream(stream), copy_stream))
        return x


def denoise_opts(steps, reuse=1, core_reuse=1, layers=50, reduce_after=-1, restore_early=40, restore_late=30,
                 early_evals=10) -> DenoiseOpts:
    return DenoiseOpts(steps, reuse, core_reuse, layers, reduce_after, restore_early, restore_late, early_evals)


def denoise_plan(opts: DenoiseOpts, n_blocks: int):
    """(number of stack runs, list of per-step dicts {fresh, core, eval, n_blocks, restore_before})."""
    arr = (DenoiseStep * max(int(opts.steps), 1))()
    runs = _check("h3dit_denoise_plan", _lib.h3dit_denoise_plan(C.byref(opts), n_blocks, arr))
    return runs, [{k: getattr(arr[i], k) for k, _ in DenoiseStep._fields_} for i in range(opts.steps)]


def velocity_step(z, v, dt: float, stream=None):
    """z = bf16(z + dt * v) in place (bf16 device tensors of one size, a multiple of 8)."""
    _check("h3dit_velocity_step", _lib.h3dit_velocity_step(z.numel(), dt, _ptr(v), _ptr(z), _stream(stream)))
    return z


class Denoise:
    """The denoising loop of h3dit_denoise_fwd with its host-side arguments marshalled once:
    blocks (device weights), the plan options, per-step dt, the head parts (video / audio:
    (mod bf16 [2][d], W bf16 [c][d]) device tensors or None), the patch-embedding stand-in
    (embed: (W_video bf16 [d][c_v] or None, W_audio bf16 [d][c_a] or None), or None), and
    optional rotary tables (cos, sin) of the full and the paired sequence."""

    def __init__(self, w, blocks: list, opts: DenoiseOpts, dt, video=None, audio=None, flags: int = 0, embed=None,
                 rope=None, rope_reduced=None):
        self.blocks = blocks
        self.arr = (BlockW * len(blocks))(*[block_struct(p) for p in blocks])
        self.opts = opts
        self.dt = (C.c_float * int(opts.steps))(*[float(t) for t in dt])
        self.part_tensors = (video, audio)   # kept alive while the structs point at them
        self.parts = [None if p is None else HeadPart(_ptr(p[0]), _ptr(p[1]), p[1].shape[0]) for p in (video, audio)]
        self.embed_tensors = embed
        self.embed = None if embed is None else PatchEmbed(_ptr(embed[0]), _ptr(embed[1]))
        self.rope_tensors = (rope, rope_reduced)
        self.rope, self.rope_reduced = rope_struct(rope), rope_struct(rope_reduced)
        self.flags = flags
        self.dims = dims_of(w)
        self.layout = layout_of(w)
        size = C.c_size_t(0)
        _check("h3dit_denoise_fwd", _lib.h3dit_denoise_fwd(C.byref(self.dims), C.byref(self.layout), len(blocks),
                                                           self.arr, _ref(self.rope), _ref(self.rope_reduced),
                                                           C.byref(opts), self.dt, None, _ref(self.embed),
                                                           *self._refs(), None, None, flags, None, C.byref(size),
                                                           None))
        self.workspace_bytes = size.value

    def _refs(self):
        return [C.byref(p) if p is not None else None for p in self.parts]

    def __call__(self, x_in, z_video, z_audio, workspace, stream=None):
        size = C.c_size_t(workspace.numel())
        _check("h3dit_denoise_fwd", _lib.h3dit_denoise_fwd(C.byref(self.dims), C.byref(self.layout), len(self.blocks),
                                                           self.arr, _ref(self.rope), _ref(self.rope_reduced),
                                                           C.byref(self.opts), self.dt, _ptr(x_in), _ref(self.embed),
                                                           *self._refs(), _ptr(z_video), _ptr(z_audio), self.flags,
                                                           _ptr(workspace), C.byref(size), _stream(stream)))
        return z_video, z_audio


# ------------------------------------------------------------------ h3dit_stages.h

def rope_tables(w, reduced=False, device="cuda", stream=None):
    n = w.n_tokens if not reduced else (w.video_t * w.video_h * (w.video_w // 2 + w.video_w % 2) + w.n_text + w.n_audio)
    cos = torch.empty((n, w.head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check("h3dit_rope_tables", _lib.h3dit_rope_tables(C.byref(layout_of(w)), w.head_dim, int(reduced), _ptr(cos),
                                                       _ptr(sin), _stream(stream)))
    return cos, sin


def row_gate_adaln(x, gate=None, y=None, x_out=None, shift=None, scale=None, h=None, q=None, s=None, eps=1e-6,
                   stream=None):
    n, d = x.shape
    _check("h3dit_row_gate_adaln", _lib.h3dit_row_gate_adaln(n, d, eps, _ptr(x), _ptr(gate), _ptr(y), _ptr(x_out),
                                                             _ptr(shift), _ptr(scale), _ptr(h), _ptr(q), _ptr(s),
                                                             _stream(stream)))


def quantize_rows(v, rows, cols, group, headmajor_hd=0, stream=None):
    q = torch.empty((rows, cols), dtype=torch.int8, device=v.device)
    s = torch.empty((rows, cols // group), dtype=torch.float32, device=v.device)
    _check("h3dit_quantize_rows", _lib.h3dit_quantize_rows(rows, cols, group, _ptr(v), headmajor_hd, _ptr(q), _ptr(s),
                                                           _stream(stream)))
    return q, s


def linear(M, N, K, a, w, out_kind=OUT_BF16, out=None, precision=BF16, a_headmajor_hd=0, a_scale=None, a_group=0,
           w_scale=None, cos=None, sin=None, heads=0, head_dim=0, out_q=None, out_k=None, out_v=None, stream=None,
           workspace=None):
    """out = a w^T through h3dit_linear.  The split-K workspace the call needs (if any) is taken
    from `workspace` (a uint8 device tensor) when it is large enough, else allocated.  The C ABI
    sees pointers only; where `out` is a tensor its size is checked against the output kind
    here (M x N elements of 4 bytes for fp32 / int32 accumulators, 2 bytes otherwise)."""
    if out is not None and not isinstance(out, int) and out_kind != OUT_QKV:
        need_out = M * N * (4 if out_kind in (OUT_F32, OUT_I32) else 2)
        have = out.numel() * out.element_size()
        if have < need_out or not out.is_contiguous():
            raise ValueError(f"linear: output tensor holds {have} bytes (contiguous: {out.is_contiguous()}), "
                             f"the {M} x {N} output of kind {out_kind} needs {need_out}")
    args = LinearArgs(M, N, K, precision, _ptr(a), a_headmajor_hd, _ptr(a_scale), a_group, _ptr(w), _ptr(w_scale),
                      out_kind, _ptr(out), _ptr(cos), _ptr(sin), heads, head_dim, _ptr(out_q), _ptr(out_k),
                      _ptr(out_v))
    need = C.c_uint64(0)
    _check("h3dit_linear_workspace", _lib.h3dit_linear_workspace(C.byref(args), C.byref(need)))
    if need.value:
        if workspace is None or workspace.numel() < need.value:
            import torch
            workspace = torch.empty(need.value, dtype=torch.uint8, device=a.device)
        args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel()
    _check("h3dit_linear", _lib.h3dit_linear(C.byref(args), _stream(stream)))


def linear_workspace(M, N, K, precision=BF16, a_group=0, out_kind=OUT_BF16, heads=0, head_dim=0):
    """Split-K workspace bytes h3dit_linear needs for this shape (0 when it splits nothing).
    Validation needs non-NULL operand pointers; the query only reads the shape fields."""
    dummy = 1 << 20
    args = LinearArgs(M=M, N=N, K=K, precision=precision, a=dummy, a_scale=dummy, a_group=a_group, w=dummy,
                      w_scale=dummy, out_kind=out_kind, out=dummy, cos_t=dummy, sin_t=dummy, heads=heads,
                      head_dim=head_dim, out_q=dummy, out_k=dummy, out_v=dummy)
    need = C.c_uint64(0)
    _check("h3dit_linear_workspace", _lib.h3dit_linear_workspace(C.byref(args), C.byref(need)))
    return need.value


def linear_a_extent(M, N, K, precision=BF16, a_group=0, out_kind=OUT_BF16, a_headmajor_hd=0, heads=0,
                    head_dim=0):
    """(largest byte end any unmasked A load of the planned launch reads, loads masked wrongly):
    a host-only walk over the kernel's A-operand addressing (no device work)."""
    dummy = 1 << 20
    args = LinearArgs(M=M, N=N, K=K, precision=precision, a=dummy, a_headmajor_hd=a_headmajor_hd, a_scale=dummy,
                      a_group=a_group, w=dummy, w_scale=dummy, out_kind=out_kind, out=dummy, cos_t=dummy,
                      sin_t=dummy, heads=heads, head_dim=head_dim, out_q=dummy, out_k=dummy, out_v=dummy)
    end, bad = C.c_uint64(0), C.c_uint64(0)
    _check("h3dit_linear_a_extent", _lib.h3dit_linear_a_extent(C.byref(args), C.byref(end), C.byref(bad)))
    return end.value, bad.value


def final_head(w, x, video=None, audio=None, stream=None):
    """Final AdaLN head: video / audio are (mod bf16 [2][d], W bf16 [c][d]) device tensors or None.
    Returns (out_video [n_video][c] or None, out_audio [n_audio][c] or None)."""
    import torch
    n_video = w.n_tokens - w.n_text - w.n_audio
    parts, outs = [], []
    for part, n in ((video, n_video), (audio, w.n_audio)):
        if part is None:
            parts.append(None)
            outs.append(None)
            continue
        mod, wt = part
        parts.append(HeadPart(_ptr(mod), _ptr(wt), wt.shape[0]))
        outs.append(torch.empty((n, wt.shape[0]), dtype=torch.bfloat16, device=x.device))
    refs = [C.byref(p) if p is not None else None for p in parts]
    d, l = C.byref(dims_of(w)), C.byref(layout_of(w))
    size = C.c_size_t(0)
    _check("h3dit_final_head", _lib.h3dit_final_head(d, l, refs[0], refs[1], None, None, None, None, C.byref(size),
                                                     None))
    ws = torch.empty(max(size.value, 256), dtype=torch.uint8, device=x.device)
    size = C.c_size_t(ws.numel())
    _check("h3dit_final_head", _lib.h3dit_final_head(d, l, refs[0], refs[1], _ptr(x), _ptr(outs[0]), _ptr(outs[1]),
                                                     _ptr(ws), C.byref(size), _stream(stream)))
    return tuple(outs)


def final_head_noalloc(w, x, video=None, audio=None, outs=None, stream=None):
    """h3dit_final_head_noalloc: as final_head, with the row statistics in the library's static
    device array instead of a workspace.  outs: (out_video, out_audio) to write into, or None
    to allocate them here."""
    import torch
    n_video = w.n_tokens - w.n_text - w.n_audio
    parts = []
    if outs is None:
        outs = tuple(None if p is None else torch.empty((n, p[1].shape[0]), dtype=torch.bfloat16, device=x.device)
                     for p, n in ((video, n_video), (audio, w.n_audio)))
    for part in (video, audio):
        parts.append(None if part is None else HeadPart(_ptr(part[0]), _ptr(part[1]), part[1].shape[0]))
    refs = [C.byref(p) if p is not None else None for p in parts]
    _check("h3dit_final_head_noalloc",
           _lib.h3dit_final_head_noalloc(C.byref(dims_of(w)), C.byref(layout_of(w)), refs[0], refs[1], _ptr(x),
                                         _ptr(outs[0]), _ptr(outs[1]), _stream(stream)))
    return tuple(outs)


def rope_split(n, heads, head_dim, t, cos, sin, q, k, vt, stream=None):
    _check("h3dit_rope_split", _lib.h3dit_rope_split(n, heads, head_dim, _ptr(t), _ptr(cos), _ptr(sin), _ptr(q),
                                                     _ptr(k), _ptr(vt), _stream(stream)))


def gelu(u, gl, stream=None):
    _check("h3dit_gelu", _lib.h3dit_gelu(u.numel(), _ptr(u), _ptr(gl), _stream(stream)))


def attention(heads, n, head_dim, q, k, vt, o, row_max=None, row_sum=None, stream=None):
    _check("h3dit_attention", _lib.h3dit_attention(heads, n, head_dim, _ptr(q), _ptr(k), _ptr(vt), _ptr(o),
                                                   _ptr(row_max), _ptr(row_sum), _stream(stream)))


def token_pair(w, x, r, r_in=None, stream=None):
    _check("h3dit_token_pair", _lib.h3dit_token_pair(C.byref(layout_of(w)), x.shape[1], _ptr(x), _ptr(r), _ptr(r_in),
                                                     _stream(stream)))


def token_restore(w, x, y, r_in, stream=None):
    _check("h3dit_token_restore", _lib.h3dit_token_restore(C.byref(layout_of(w)), x.shape[1], _ptr(x), _ptr(y),
                                                           _ptr(r_in), _stream(stream)))
