"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function
include/*.h declares, answers workspace-size queries, and rejects bad arguments before any
launch (a call that reached the device here would fail with EHIP, not the code asserted)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import synth
from synth import WORKLOADS

h3 = pytest.importorskip("audio_diffusion_transformer_dit_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in ("h3dit.h", "h3dit_stages.h"):
        with open(os.path.join(ROOT, "include", hdr)) as fh:
            names.update(re.findall(r"^H3DIT_API\s+int\s+(h3dit_\w+)\s*\(", fh.read(), flags=re.M))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 13
    assert set(names) == set(h3.EXPORTS)
    for n in names:
        assert getattr(h3.lib(), n) is not None
    # and nothing else of the C ABI: the library is built with hidden default visibility
    out = subprocess.run(["nm", "-D", "--defined-only", h3.LIB_PATH], capture_output=True, text=True).stdout
    c_funcs = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert c_funcs == set(names)


def test_struct_sizes_match_header_layout():
    assert C.sizeof(h3.Dims) == 28
    assert C.sizeof(h3.Layout) == 40
    assert C.sizeof(h3.BlockW) == 8 + 9 * 8
    assert C.sizeof(h3.TokenReduction) == 24   # two int32, then the two table pointers of rope_reduced
    assert C.sizeof(h3.Rope) == 16
    assert C.sizeof(h3.PatchEmbed) == 16
    assert C.sizeof(h3.LinearArgs) == 160   # 14 pointer-sized / int64 fields + 4 int32 pairs + 2 padded int32


def fake_block(precision=h3.BF16):
    # 16-byte aligned fake addresses: never dereferenced by a size query or a rejected call
    a = 1 << 20
    return h3.BlockW(precision, a, a, a, a, a if precision else None, a if precision else None,
                     a if precision else None, a if precision else None, a)


def query(w, blk, flags=0):
    size = C.c_size_t(0)
    rc = h3.lib().h3dit_block_fwd(C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w)), C.byref(blk), None, None, flags,
                                  None, C.byref(size), None)
    return rc, size.value


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_workspace_query_bf16(cfg):
    w = WORKLOADS[cfg]
    rc, size = query(w, fake_block())
    assert rc == 0
    N, d, f = w.n_tokens, w.hidden, w.mlp
    # arenas: A = q|k|V^T, B = [N][d], C = [N][f]; plus rotary tables, per-token scales and
    # the largest split-K workspace of the four projections
    arenas = (2 * N * d * 2 + d * h3.ldv(N) * 2) + N * d * 2 + N * f * 2
    sk = max(h3.linear_workspace(N, 3 * d, d, out_kind=h3.OUT_QKV, heads=w.heads, head_dim=w.head_dim),
             h3.linear_workspace(N, 3 * d, d), h3.linear_workspace(N, d, d), h3.linear_workspace(N, f, d),
             h3.linear_workspace(N, d, f))
    assert arenas + sk <= size <= arenas + sk + N * w.head_dim * 4 + N * 4 + 16 * 256
    rc2, size2 = query(w, fake_block(), h3.NO_ALIAS)
    assert rc2 == 0 and size2 > size


def test_workspace_query_int8_and_unfused():
    w = WORKLOADS[2]
    rc, base = query(w, fake_block(h3.INT8))
    assert rc == 0
    for flag in (h3.NOFUSE_ROPE, h3.NOFUSE_QUANT):
        rc, s = query(w, fake_block(h3.INT8), flag)
        assert rc == 0 and s > base


def test_stack_workspace_with_reduction_is_larger():
    w = WORKLOADS[4]
    blocks = [fake_block(h3.INT8)] * 50
    arr = (h3.BlockW * 50)(*blocks)
    s0, s1 = C.c_size_t(0), C.c_size_t(0)
    tr = h3.TokenReduction(3, 40)
    lib = h3.lib()
    assert lib.h3dit_stack_fwd(C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w)), 50, arr, None, None, None, 0, None,
                               C.byref(s0), None) == 0
    assert lib.h3dit_stack_fwd(C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w)), 50, arr, None, C.byref(tr), None, 0, None,
                               C.byref(s1), None) == 0
    nr = w.video_t * w.video_h * (w.video_w // 2 + 1) + w.n_text + w.n_audio
    assert s1.value - s0.value >= 2 * nr * w.hidden * 2


@pytest.mark.parametrize("change,code", [
    (dict(hidden=5000), h3.EINVAL),                 # hidden != heads * head_dim
    (dict(head_dim=96, hidden=40 * 96), h3.EUNSUPPORTED),
    (dict(mlp=20000), h3.EINVAL),                   # mlp % 256
    (dict(n_text=255), h3.EINVAL),                  # n_tokens disagrees with the layout
    (dict(rope_split=(32, 48, 46)), h3.EINVAL),     # rotary sections do not cover head_dim
    (dict(rope_split=(31, 49, 48)), h3.EINVAL),     # odd section
])
def test_bad_dims_rejected(change, code):
    base = WORKLOADS[1]
    dims = h3.dims_of(base)
    w = base.replace(**{k: v for k, v in change.items() if k in ("rope_split",)})
    layout = h3.layout_of(w)
    if "hidden" in change:
        dims.hidden = change["hidden"]
    if "head_dim" in change:
        dims.head_dim = change["head_dim"]
    if "mlp" in change:
        dims.mlp = change["mlp"]
    if "n_text" in change:
        layout.n_text = change["n_text"]
    size = C.c_size_t(0)
    blk = fake_block()
    rc = h3.lib().h3dit_block_fwd(C.byref(dims), C.byref(layout), C.byref(blk), None, None, 0, None, C.byref(size), None)
    assert rc == code


def test_int8_group_rules():
    w = WORKLOADS[2]
    dims = h3.dims_of(w)
    size = C.c_size_t(0)
    blk = fake_block(h3.INT8)
    for g in (1000, 64, 3 * 1024):  # not a multiple of 128 / too small / does not divide mlp
        dims.fc2_group = g
        rc = h3.lib().h3dit_block_fwd(C.byref(dims), C.byref(h3.layout_of(w)), C.byref(blk), None, None, 0, None,
                                      C.byref(size), None)
        assert rc == h3.EINVAL, g


def test_call_argument_errors_before_launch():
    w = WORKLOADS[0]
    lib = h3.lib()
    blk = fake_block()
    size = C.c_size_t(1 << 30)
    ws = 1 << 24
    x = 1 << 22
    d, l = C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w))
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), None, None, 0, ws, C.byref(size), None) == h3.EINVAL     # x NULL
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), None, x + 2, 0, ws, C.byref(size), None) == h3.EINVAL   # misaligned x
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), None, x, 0, ws + 16, C.byref(size), None) == h3.EINVAL  # workspace align
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), None, x, 1 << 9, ws, C.byref(size), None) == h3.EINVAL  # unknown flag
    small = C.c_size_t(1024)
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), None, x, 0, ws, C.byref(small), None) == h3.EWORKSPACE
    assert small.value > 1024                                                                          # size written back
    bad = fake_block()
    bad.w_fc1 = None
    assert lib.h3dit_block_fwd(d, l, C.byref(bad), None, x, 0, ws, C.byref(size), None) == h3.EINVAL
    mixed = fake_block(h3.INT8)
    mixed.s_o = None
    assert lib.h3dit_block_fwd(d, l, C.byref(mixed), None, x, 0, ws, C.byref(size), None) == h3.EINVAL
    # int8 attention projections only: their two scale arrays are required, the MLP's are not
    attn = fake_block(h3.INT8_ATTN)
    attn.s_fc1 = attn.s_fc2 = None
    assert lib.h3dit_block_fwd(d, l, C.byref(attn), None, x, 0, ws, C.byref(size), None) not in (h3.EINVAL, h3.OK)
    attn.s_qkv = None
    assert lib.h3dit_block_fwd(d, l, C.byref(attn), None, x, 0, ws, C.byref(size), None) == h3.EINVAL
    # caller rotary tables: both or neither, 16-byte aligned
    for rope in (h3.Rope(x, None), h3.Rope(None, x), h3.Rope(x + 4, x), h3.Rope(x, x + 8)):
        assert lib.h3dit_block_fwd(d, l, C.byref(blk), C.byref(rope), x, 0, ws, C.byref(size), None) == h3.EINVAL
    ok = h3.Rope(x, x + 256)
    assert lib.h3dit_block_fwd(d, l, C.byref(blk), C.byref(ok), x, 0, ws, C.byref(size), None) not in (h3.EINVAL, h3.OK)
    arr = (h3.BlockW * 2)(fake_block(), fake_block())
    tr = h3.TokenReduction(0, 1, h3.Rope(x + 4, x))
    assert lib.h3dit_stack_fwd(d, l, 2, arr, None, C.byref(tr), x, 0, ws, C.byref(size), None) == h3.EINVAL
    for tr in (h3.TokenReduction(3, 3), h3.TokenReduction(-1, 4), h3.TokenReduction(2, 5)):
        assert lib.h3dit_stack_fwd(d, l, 2, arr, None, C.byref(tr), x, 0, ws, C.byref(size), None) == h3.EINVAL
    assert lib.h3dit_quantize_weights(x, 4, 12, x, x, None) == h3.EINVAL      # cols % 8
    assert lib.h3dit_attention(4, 100, 96, x, x, x, x, None, None, None) == h3.EINVAL
    args = h3.LinearArgs(M=10, N=100, K=128, precision=h3.BF16, a=x, w=x, out=x, out_kind=h3.OUT_BF16)
    assert lib.h3dit_linear(C.byref(args), None) == h3.EINVAL                 # N % 128
    args = h3.LinearArgs(M=10, N=128, K=128, precision=h3.BF16, a=x, w=x, out=x, out_kind=h3.OUT_I32)
    assert lib.h3dit_linear(C.byref(args), None) == h3.EINVAL                 # int32 output on the bf16 path
    args = h3.LinearArgs(M=10, N=128, K=128, precision=h3.BF16, a=x, a_headmajor_hd=64, w=x, out=x,
                         out_kind=h3.OUT_GELU)
    assert lib.h3dit_linear(C.byref(args), None) == h3.EINVAL                 # head-major A feeds BF16/F32 only
    args.a_headmajor_hd, args.out_kind = 96, h3.OUT_BF16
    assert lib.h3dit_linear(C.byref(args), None) == h3.EINVAL                 # head dim 96


def test_linear_workspace_plan():
    """Split-K only where the last round of 256 x 256 tiles is partial and K is long enough to
    pay for the partial tiles; the grouped int8 FC2 never splits."""
    ws = h3.linear_workspace
    assert ws(4096, 5120, 20480) == 64 * 256 * 256 * 4 * 4        # FC2: 64 leftover tiles x 4 segments
    assert ws(4096, 20480, 5120) == 0                              # FC1: 1280 tiles, whole rounds
    assert ws(4096, 5120, 20480, h3.INT8, 1024) == 0               # grouped FC2
    assert ws(4096, 5120, 5120) == 64 * 256 * 256 * 4 * 4         # out-projection: same split, summed chip-wide
    for kind in (h3.OUT_F32, h3.OUT_GELU):                         # the plan depends on shape and precision only
        assert ws(4096, 5120, 5120, h3.BF16, 0, kind) == ws(4096, 5120, 5120)
    assert ws(4096, 5120, 5120, h3.INT8) == 0                      # int8: half the K bytes, split does not pay
    assert ws(64, 256, 2048) == 8 * 256 * 256 * 4                  # one tile: 8 segments
    assert ws(64, 256, 256) == 0                                   # 4 K slices: too short to split
    args = h3.LinearArgs(M=4096, N=5120, K=20480, precision=h3.BF16, a=1 << 20, w=1 << 20, out=1 << 20,
                         out_kind=h3.OUT_BF16)
    assert h3.lib().h3dit_linear(C.byref(args), None) == h3.EWORKSPACE   # no workspace given
    args.workspace, args.workspace_bytes = 1 << 20, 1 << 20
    assert h3.lib().h3dit_linear(C.byref(args), None) == h3.EWORKSPACE   # too small
    args.workspace = (1 << 20) + 16
    assert h3.lib().h3dit_linear(C.byref(args), None) == h3.EINVAL       # misaligned


def test_linear_binding_checks_the_output_tensor():
    """The C ABI takes an output pointer only; the binding checks a tensor's bytes against the
    output kind before the call (fp32 / int32 accumulators need 4 bytes per element)."""
    import torch
    M, N, K = 4, 256, 128
    a = torch.zeros(M, K, dtype=torch.bfloat16)
    w = torch.zeros(N, K, dtype=torch.bfloat16)
    for kind, out in ((h3.OUT_F32, torch.zeros(M, N, dtype=torch.bfloat16)),
                      (h3.OUT_BF16, torch.zeros(M, N - 1, dtype=torch.bfloat16)),
                      (h3.OUT_BF16, torch.zeros(M, 2 * N, dtype=torch.bfloat16)[:, :N])):
        with pytest.raises(ValueError):
            h3.linear(M, N, K, a, w, kind, out)


@pytest.mark.parametrize("M", [1, 7, 64, 129, 255, 256, 257, 300, 513, 2048, 4097, 4480])
def test_linear_a_loads_stay_inside_a(M):
    """Walks every A-operand load (and, for the grouped FC2, every group-scale load) of the
    launch h3dit_linear plans, with the kernel's own addressing: a ragged last tile reads
    nothing past the M rows of A (largest byte end == M*K*element size), rows past M are the
    ones masked by the range check, and no load straddles its resource end."""
    for N, K, prec, group, hm in ((256, 256, h3.BF16, 0, 0),          # small: 256 x 128 tiles
                                  (5120, 5120, h3.BF16, 0, 0),        # 256 x 256 bf16, split-K tail
                                  (15360, 5120, h3.INT8, 0, 0),       # 256 x 256 int8 (8 waves)
                                  (5120, 5120, h3.INT8, 0, 0),        # int8: 256 x 256 and 128 x 128 tiles
                                  (5120, 5120, h3.BF16, 0, 128),      # head-major attention output
                                  (768, 256, h3.BF16, 0, 64),         # head-major, head_dim 64
                                  (1024, 4096, h3.INT8, 1024, 0),     # grouped FC2 (128 x 128)
                                  (5120, 2048, h3.INT8, 512, 0),      # grouped, 256 x 128 and 128 x 128 tiles
                                  (256, 8192, h3.INT8, 128, 0)):      # grouped, many groups
        end, bad = h3.linear_a_extent(M, N, K, prec, group, a_headmajor_hd=hm)
        esz = 1 if prec == h3.INT8 else 2
        assert bad == 0, (M, N, K, prec, group, hm, bad)
        assert end == M * K * esz, (M, N, K, prec, group, hm, end)


def test_linear_plan_depends_on_shape_and_precision_only():
    """A fused epilogue and its unfused sequence (bf16 output, then the GELU or rotary kernel)
    must split K alike for the fusion switches to stay byte-identical: the split-K workspace,
    which encodes the plan's split tiles and segments, is the same for every output form."""
    ws = h3.linear_workspace
    heads, hd = 40, 128
    for M in (1, 64, 256, 300, 1024, 2048, 2688, 4096, 4480, 8192):
        for N, K in ((5120, 5120), (5120, 20480), (20480, 5120), (15360, 5120), (512, 5120), (256, 2048)):
            for prec in (h3.BF16, h3.INT8):
                base = ws(M, N, K, prec)
                kinds = [h3.OUT_F32 if prec == h3.BF16 else h3.OUT_I32, h3.OUT_GELU]
                for kind in kinds:
                    assert ws(M, N, K, prec, 0, kind) == base, (M, N, K, prec, kind)
                if N == 3 * heads * hd:
                    assert ws(M, N, K, prec, 0, h3.OUT_QKV, heads, hd) == base, (M, N, K, prec, "qkv")


def test_stack_streamed_workspace_and_validation():
    """The streamed stack's workspace is the resident stack's plus every block's mod rows and
    two slots of one block's matrices (each region 256-byte aligned); bad arguments are
    rejected before anything runs."""
    up = lambda v: (v + 255) // 256 * 256
    w = WORKLOADS[1]
    d, f = w.hidden, w.mlp
    n = 3
    for prec, ea, em in ((h3.BF16, 2, 2), (h3.INT8, 1, 1), (h3.INT8_MLP, 2, 1)):
        arr = (h3.BlockW * n)(*[fake_block(prec) for _ in range(n)])
        dims, lay = h3.dims_of(w), h3.layout_of(w)
        res, stm = C.c_size_t(0), C.c_size_t(0)
        assert h3.lib().h3dit_stack_fwd(C.byref(dims), C.byref(lay), n, arr, None, None, None, 0, None, C.byref(res),
                                        None) == 0
        assert h3.lib().h3dit_stack_fwd_streamed(C.byref(dims), C.byref(lay), n, arr, None, None, None, 0, None,
                                                 C.byref(stm), None, None) == 0
        mats = [3 * d * d * ea, d * d * ea, f * d * em, d * f * em]
        scales = [3 * d * 4 if ea == 1 else 0, d * 4 if ea == 1 else 0, f * 4 if em == 1 else 0,
                  d * 4 if em == 1 else 0]
        slot = sum(up(b) for b in mats + scales)
        assert stm.value == res.value + up(n * 6 * d * 2) + 2 * slot, prec
    arr = (h3.BlockW * 1)(fake_block(h3.BF16))
    size = C.c_size_t(0)
    dims, lay = h3.dims_of(w), h3.layout_of(w)
    lib = h3.lib()
    assert lib.h3dit_stack_fwd_streamed(C.byref(dims), C.byref(lay), 0, arr, None, None, None, 0, None, C.byref(size),
                                        None, None) == h3.EINVAL                        # no blocks
    bad = h3.TokenReduction(1, 1)
    assert lib.h3dit_stack_fwd_streamed(C.byref(dims), C.byref(lay), 1, arr, None, C.byref(bad), None, 0, None,
                                        C.byref(size), None, None) == h3.EINVAL         # empty reduced span
    assert lib.h3dit_stack_fwd_streamed(C.byref(dims), C.byref(lay), 1, None, None, None, None, 0, None, C.byref(size),
                                        None, None) == h3.EINVAL                        # NULL block array
    arr2 = (h3.BlockW * 1)(fake_block(h3.BF16))
    arr2[0].w_o = (1 << 20) + 8
    x = 1 << 20
    size = C.c_size_t(1 << 40)
    assert lib.h3dit_stack_fwd_streamed(C.byref(dims), C.byref(lay), 1, arr2, None, None, x, 0, x, C.byref(size), None,
                                        None) == h3.EINVAL                              # misaligned host matrix


def test_int8_row_level_fc2_group_accepted():
    """fc2_group == mlp (one code per token over the FC2 input) is accepted above 8192;
    other groups above 8192 are not."""
    w = WORKLOADS[2]
    dims = h3.dims_of(w)
    size = C.c_size_t(0)
    blk = fake_block(h3.INT8)
    for g, ok in ((w.mlp, True), (10240, False), (4096, True)):
        dims.fc2_group = g
        rc = h3.lib().h3dit_block_fwd(C.byref(dims), C.byref(h3.layout_of(w)), C.byref(blk), None, None, 0, None,
                                      C.byref(size), None)
        assert (rc == 0) == ok, g


def test_mod_sets_validated():
    w = WORKLOADS[1]
    size = C.c_size_t(0)
    for m, ok in ((0, True), (1, True), (3, True), (2, False), (6, False)):
        lay = h3.layout_of(w)
        lay.mod_sets = m
        rc = h3.lib().h3dit_block_fwd(C.byref(h3.dims_of(w)), C.byref(lay), C.byref(fake_block()), None, None, 0, None,
                                      C.byref(size), None)
        assert (rc == 0) == ok, m


def test_zero_sized_stage_calls_return_ok_without_pointers():
    lib = h3.lib()
    assert lib.h3dit_row_gate_adaln(0, 256, 1e-6, None, None, None, None, 1 << 20, 1 << 20, None, None, None,
                                    None) == 0
    assert lib.h3dit_quantize_rows(0, 256, 256, None, 0, None, None, None) == 0
    assert lib.h3dit_attention(2, 0, 128, None, None, None, None, None, None, None) == 0
    assert lib.h3dit_gelu(0, None, None, None) == 0
    assert lib.h3dit_rope_split(0, 2, 64, None, None, None, None, None, None, None) == 0
    args = h3.LinearArgs(M=0, N=128, K=128, precision=h3.BF16, out_kind=h3.OUT_BF16)
    assert lib.h3dit_linear(C.byref(args), None) == 0
    # sizes are still checked
    assert lib.h3dit_row_gate_adaln(0, 100, 1e-6, None, None, None, None, 1 << 20, 1 << 20, None, None, None,
                                    None) == h3.EINVAL


def test_final_head_validation_and_workspace():
    w = WORKLOADS[3]
    lib = h3.lib()
    a = 1 << 20
    good = h3.HeadPart(a, a, 128)
    bad = h3.HeadPart(a, a, 100)
    size = C.c_size_t(0)
    d, l = C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w))
    assert lib.h3dit_final_head(d, l, C.byref(good), None, None, None, None, None, C.byref(size), None) == 0
    n_video = w.n_tokens - w.n_text - w.n_audio
    # only the row statistics: the normalised rows are formed in the GEMM's tile loads
    assert n_video * 8 <= size.value < n_video * w.hidden * 2
    assert lib.h3dit_final_head(d, l, C.byref(bad), None, None, None, None, None, C.byref(size), None) == h3.EINVAL
    assert lib.h3dit_final_head(d, l, None, None, None, None, None, None, C.byref(size), None) == 0
    small = C.c_size_t(16)
    assert lib.h3dit_final_head(d, l, C.byref(good), None, a, a, None, a, C.byref(small), None) == h3.EWORKSPACE


def test_denoise_plan_equals_oracle_and_validates():
    """h3dit_denoise_plan is host logic: bit for bit the oracle's schedule over a grid of
    options, with the pages' 20 / 11 / 8 fresh evaluations, and EINVAL for bad requests."""
    import oracle
    for steps in (1, 4, 5, 20, 33):
        for reuse, core in ((1, 1), (2, 1), (3, 1), (1, 4), (1, 6)):
            for red in ((-1, 40, 30, 10), (3, 40, 30, 10), (0, 2, 1, 1)):
                opts = h3.denoise_opts(steps, reuse, core, 45, *red)
                runs, plan = h3.denoise_plan(opts, 50)
                ref = oracle.denoise_plan(steps, reuse, core, *red)
                assert runs == sum(s["core"] for s in ref)
                for s, r in zip(plan, ref):
                    assert (s["fresh"], s["core"], s["eval"], s["restore_before"]) == \
                        (r["fresh"], r["core"], r["eval"], r["restore"])
                    assert s["n_blocks"] == 45
    assert [h3.denoise_plan(h3.denoise_opts(20, r), 50)[0] for r in (1, 2, 3)] == [20, 11, 8]
    lib = h3.lib()
    arr = (h3.DenoiseStep * 20)()
    for bad in (dict(reuse=2, core_reuse=4), dict(reuse=0), dict(core_reuse=0), dict(layers=0), dict(layers=51),
                dict(reduce_after=45), dict(reduce_after=3, restore_early=3), dict(reduce_after=3, early_evals=-1)):
        assert lib.h3dit_denoise_plan(C.byref(h3.denoise_opts(20, **bad)), 50, arr) == h3.EINVAL
    assert lib.h3dit_denoise_plan(C.byref(h3.denoise_opts(0)), 50, arr) == h3.EINVAL
    assert lib.h3dit_denoise_plan(None, 50, arr) == h3.EINVAL


def test_velocity_step_and_denoise_validation():
    lib = h3.lib()
    a = 1 << 20
    assert lib.h3dit_velocity_step(12, 0.5, a, a, None) == h3.EINVAL      # count % 8
    assert lib.h3dit_velocity_step(16, 0.5, None, a, None) == h3.EINVAL
    assert lib.h3dit_velocity_step(16, 0.5, a + 8, a, None) == h3.EINVAL  # alignment
    assert lib.h3dit_velocity_step(0, 0.5, None, None, None) == h3.EINVAL
    w = WORKLOADS[3]
    d, l = C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w))
    blocks = (h3.BlockW * 50)(*[h3.BlockW(h3.BF16, a, a, a, a, None, None, None, None, a)] * 50)
    head = h3.HeadPart(a, a, 128)
    dt = (C.c_float * 20)(*([-0.05] * 20))
    size = C.c_size_t(0)
    opts = h3.denoise_opts(20, reuse=2, layers=45)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(opts), dt, None, None, C.byref(head), None, None, None, 0, None,
                                 C.byref(size), None) == 0
    stack = h3.stack_workspace(w, [dict(wqkv=a, wo=a, w1=a, w2=a, mod=a)] * 45)
    n_video = w.n_tokens - w.n_text - w.n_audio
    assert size.value >= w.n_tokens * w.hidden * 2 + n_video * 128 * 2 + stack
    red = h3.denoise_opts(20, reuse=2, layers=45, reduce_after=3)
    rsize = C.c_size_t(0)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(red), dt, None, None, C.byref(head), None, None, None, 0, None,
                                 C.byref(rsize), None) == 0
    assert rsize.value > size.value
    # no head part, a bad plan, a short workspace: rejected before any launch
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(opts), dt, None, None, None, None, None, None, 0, None,
                                 C.byref(size), None) == h3.EINVAL
    bad = h3.denoise_opts(20, reuse=2, core_reuse=2, layers=45)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(bad), dt, None, None, C.byref(head), None, None, None, 0, None,
                                 C.byref(size), None) == h3.EINVAL
    small = C.c_size_t(256)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(opts), dt, a, None, C.byref(head), None, a, None, 0, a,
                                 C.byref(small), None) == h3.EWORKSPACE
    assert small.value == size.value
    # the patch-embedding stand-in: its product and row buffer fit the shared region (the size
    # does not grow at 4096 tokens, where the stack's arenas are larger), a misaligned matrix
    # is rejected, and so are misaligned caller tables
    emb = h3.PatchEmbed(a, None)
    esize = C.c_size_t(0)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(opts), dt, None, C.byref(emb), C.byref(head),
                                 None, None, None, 0, None, C.byref(esize), None) == 0
    assert esize.value == size.value
    emb = h3.PatchEmbed(a + 2, None)
    big = C.c_size_t(size.value)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, None, None, C.byref(opts), dt, a, C.byref(emb), C.byref(head),
                                 None, a, None, 0, a, C.byref(big), None) == h3.EINVAL
    rope = h3.Rope(a + 4, a)
    assert lib.h3dit_denoise_fwd(d, l, 50, blocks, C.byref(rope), None, C.byref(opts), dt, None, None, C.byref(head),
                                 None, None, None, 0, None, C.byref(esize), None) == h3.EINVAL


def test_sizes_beyond_32bit_offsets_rejected():
    """The kernels address buffers with 32-bit offsets: widths or token counts whose largest
    activation or weight reaches 2 GiB are refused before any launch; the largest accepted
    shapes still answer the size query."""
    lib = h3.lib()
    blk = fake_block()
    size = C.c_size_t(0)

    def query(n_video_w, mlp, hidden=5120, heads=40):
        w = WORKLOADS[1]
        layout = h3.layout_of(w)
        layout.video_t, layout.video_h, layout.video_w = 1, 1, n_video_w
        layout.n_text, layout.n_audio = 0, 0
        dims = h3.Dims(n_video_w, hidden, heads, 128, mlp, 1024, 1e-6)
        return lib.h3dit_block_fwd(C.byref(dims), C.byref(layout), C.byref(blk), None, None, 0, None, C.byref(size), None)

    assert query(52428, 20480) == 0                   # 52428 * 20480 * 2 < 2^31
    assert query(52429, 20480) == h3.EINVAL
    assert query(1024, 262144) == h3.EINVAL           # [mlp][d] weight: 262144 * 5120 * 2 B >= 2^31
    assert query(1024, 196608) == 0                   # 196608 * 5120 * 2 B < 2^31
    # a narrow MLP does not hide a wide [N][3d] projection
    assert query(45000, 256, hidden=8192, heads=64) == h3.EINVAL   # 45000 * 3 * 8192 * 2 B >= 2^31
    assert query(8192, 256, hidden=8192, heads=64) == 0


def test_denoise_plan_random_options_agree_with_oracle():
    """Random option sets: the library's plan and the oracle's agree step for step, and both
    reject the same invalid requests."""
    import random
    import oracle
    rng = random.Random(2026)
    for _ in range(400):
        steps = rng.randint(1, 60)
        reuse = rng.randint(0, 5)
        core = rng.randint(0, 6)
        red = rng.choice([-1, -1, 0, 1, 3, 5])
        early, late = rng.randint(0, 50), rng.randint(0, 50)
        n_early = rng.randint(-1, 20)
        layers = 50
        opts = h3.denoise_opts(steps, reuse, core, layers, red, early, late, n_early)
        arr = (h3.DenoiseStep * steps)()
        rc = h3.lib().h3dit_denoise_plan(C.byref(opts), 50, arr)
        try:
            ref = oracle.denoise_plan(steps, reuse, core, red, early, late, n_early)
        except ValueError:
            ref = None
        if ref is None:
            assert rc == h3.EINVAL, (steps, reuse, core, red, early, late, n_early)
            continue
        assert rc == sum(s["core"] for s in ref)
        for i, r in enumerate(ref):
            assert (arr[i].fresh, arr[i].core, arr[i].eval, arr[i].restore_before) == \
                (r["fresh"], r["core"], r["eval"], r["restore"])
