"""Block and stack parity of the HIP path (h3dit_block_fwd / h3dit_stack_fwd through the C ABI)
against the CPU oracle on the tiny workload and on ragged and token-reduction layouts; every
fusion switch and the unaliased workspace byte-identical to the default; gates of zero an
exact identity; run-to-run determinism."""
import pytest
import torch

import oracle
import synth
from synth import WORKLOADS
from parity import BF16_TOL, assert_bitexact, assert_close_bf16, assert_update_close, relerr

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("audio_diffusion_transformer_dit_amd")
DEV = "cuda"
W0 = WORKLOADS[0]


def cpu(t):
    torch.cuda.synchronize()
    return t.to("cpu")


def dev_block(p):
    return {k: v.to(DEV).contiguous() for k, v in p.items()}


def zero_gates(p):
    p = dict(p)
    mod = p["mod"].clone()
    mod[2] = 0
    mod[5] = 0
    p["mod"] = mod
    return p


def inputs(w, seed=1000, blocks=1):
    x = synth.make_x(w, seed)
    ps = [synth.make_block(w, seed, b) for b in range(blocks)]
    return x, ps


def gpu_params(ps, int8):
    out = []
    for p in ps:
        g = dev_block(p)
        out.append(h3.quantize_block(g) if int8 else g)
    return out


def cpu_params(ps, int8):
    return [oracle.quantize_block(p) if int8 else p for p in ps]


def check_residual(out, ref, x, what="", blocks=1):
    """Block or stack output at the bf16 bar, and its update out - x element by element and row
    by row (each row's mean update error within 10% of its mean update), so a wrong row or
    segment fails.  Element bar: 2e-2 of the update's max-norm plus 1 + blocks bf16 steps of
    the output: each block's final rounding may land one step away where its update differs
    by a rounding-sized amount, and a step taken in one block is carried by the residual
    into the next."""
    stats = assert_update_close(out, ref, x, what, ulps=1 + blocks)
    print(f"[update] {what}: residual {stats[0]:.2e}, element {stats[1]:.3f}, row {stats[2]:.3f}", flush=True)


RAGGED = W0.replace(video_t=3, video_h=5, video_w=7, n_text=11, n_audio=5)   # 121 tokens


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("w", [W0, RAGGED], ids=["tiny", "ragged121"])
def test_block_matches_oracle(w, int8):
    x, ps = inputs(w)
    pg = gpu_params(ps, int8)[0]
    pc = cpu_params(ps, int8)[0]
    if int8:  # the GPU's weight codes are the oracle's, bit for bit
        for k in ("qqkv", "sqkv", "qo", "so", "q1", "s1", "q2", "s2"):
            assert_bitexact(cpu(pg[k]), pc[k], k)
    xg = x.to(DEV)
    h3.block_fwd(w, pg, xg)
    ref = oracle.block_fwd(w, pc, x)
    check_residual(cpu(xg), ref, x)


@pytest.mark.parametrize("group", [1024, 4096], ids=["groups1024", "row"])
def test_block_int8_fc2_grouping(group):
    """FC2 input codes per 1024-channel group, or per token over the whole 4096-wide input (the
    row-level variant, run on the ungrouped kernels): each against the oracle's grouped FC2."""
    w = W0.replace(mlp=4096, fc2_group=group)
    x, ps = inputs(w)
    pg = gpu_params(ps, True)[0]
    pc = cpu_params(ps, True)[0]
    xg = x.to(DEV)
    h3.block_fwd(w, pg, xg)
    check_residual(cpu(xg), oracle.block_fwd(w, pc, x), x)


@pytest.mark.parametrize("int8", [False, True])
def test_block_zero_gates_is_identity(int8):
    x, ps = inputs(W0)
    pg = gpu_params([zero_gates(ps[0])], int8)[0]
    xg = x.to(DEV)
    h3.block_fwd(W0, pg, xg)
    assert_bitexact(cpu(xg), x)


@pytest.mark.parametrize("int8", [False, True])
def test_block_fusion_switches_byte_identical(int8):
    x, ps = inputs(RAGGED)
    pg = gpu_params(ps, int8)[0]
    base = x.to(DEV)
    h3.block_fwd(RAGGED, pg, base)
    flags = [h3.NOFUSE_GATE_ADALN, h3.NOFUSE_ROPE, h3.NOFUSE_GELU, h3.NO_ALIAS,
             h3.NOFUSE_GATE_ADALN | h3.NOFUSE_ROPE | h3.NOFUSE_GELU | h3.NO_ALIAS]
    if int8:
        flags += [h3.NOFUSE_QUANT, 63]
    for f in flags:
        xg = x.to(DEV)
        h3.block_fwd(RAGGED, pg, xg, flags=f)
        assert_bitexact(cpu(xg), cpu(base), f"flags {f}")


def test_block_deterministic_and_workspace_reuse():
    x, ps = inputs(W0)
    pg = gpu_params(ps, False)[0]
    ws = h3.alloc_workspace(h3.block_workspace(W0, pg))
    outs = []
    for fill in (0, 255, 0x7F):
        ws.fill_(fill)                 # whatever the workspace held before must not matter
        xg = x.to(DEV)
        h3.block_fwd(W0, pg, xg, workspace=ws)
        outs.append(cpu(xg))
    assert_bitexact(outs[1], outs[0])
    assert_bitexact(outs[2], outs[0])


SMALL_TR = WORKLOADS[4].replace(video_t=2, video_h=3, video_w=7, n_text=9, n_audio=5, hidden=256, heads=4,
                                head_dim=64, mlp=1024)


@pytest.mark.parametrize("int8", [False, True])
def test_stack_matches_oracle(int8):
    w = W0
    x, ps = inputs(w, blocks=3)
    pg = gpu_params(ps, int8)
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg)
    ref = oracle.stack_fwd(w, cpu_params(ps, int8), x, fused=True)
    check_residual(cpu(xg), ref, x, blocks=len(ps))


@pytest.mark.parametrize("int8", [False, True])
def test_stack_token_reduction_matches_oracle(int8):
    w = SMALL_TR
    x, ps = inputs(w, blocks=6)
    pg = gpu_params(ps, int8)
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg, reduction=(1, 4))
    ref = oracle.stack_fwd(w, cpu_params(ps, int8), x, reduce_after=1, restore_before=4, fused=True)
    check_residual(cpu(xg), ref, x, blocks=len(ps))


def test_stack_cross_block_fusion_byte_identical():
    x, ps = inputs(SMALL_TR, blocks=6)
    pg = gpu_params(ps, False)
    outs = []
    for f in (0, h3.NOFUSE_CROSS_BLOCK, h3.NOFUSE_GATE_ADALN, h3.NO_ALIAS):
        xg = x.to(DEV)
        h3.stack_fwd(SMALL_TR, pg, xg, flags=f, reduction=(1, 4))
        outs.append(cpu(xg))
    for o in outs[1:]:
        assert_bitexact(o, outs[0])


def test_stack_equals_block_sequence():
    x, ps = inputs(W0, blocks=3)
    pg = gpu_params(ps, False)
    xs = x.to(DEV)
    h3.stack_fwd(W0, pg, xs)
    xb = x.to(DEV)
    for p in pg:
        h3.block_fwd(W0, p, xb)
    assert_bitexact(cpu(xs), cpu(xb))


@pytest.mark.parametrize("int8", [False, True])
def test_stack_reduction_identity_middle(int8):
    # gates 0 in the reduced span: pair then restore is the identity on every token
    x, ps = inputs(SMALL_TR, blocks=5)
    for b in (2, 3):
        ps[b] = zero_gates(ps[b])
    pg = gpu_params(ps, int8)
    xr = x.to(DEV)
    h3.stack_fwd(SMALL_TR, pg, xr, reduction=(1, 4))
    xp = x.to(DEV)
    h3.stack_fwd(SMALL_TR, [pg[0], pg[1], pg[4]], xp)
    assert_bitexact(cpu(xr), cpu(xp))


def test_stack_reduction_restore_after_last_block():
    # the stack ends inside the reduced span: every token is restored at the end
    x, ps = inputs(SMALL_TR, blocks=3)
    pg = gpu_params(ps, False)
    xg = x.to(DEV)
    h3.stack_fwd(SMALL_TR, pg, xg, reduction=(0, 40))
    ref = oracle.stack_fwd(SMALL_TR, ps, x, reduce_after=0, restore_before=40, fused=True)
    check_residual(cpu(xg), ref, x, blocks=len(ps))


# ----------------------------------------------------------------------------- modulation sets

def _text_gates_zero(p, d):
    p = dict(p)
    mod = p["mod"].clone()
    mod[6 + 2] = 0
    mod[6 + 5] = 0
    p["mod"] = mod
    return p


@pytest.mark.parametrize("int8", [False, True])
def test_block_mod_sets_match_oracle(int8):
    """Three modulation sets (video, text, audio): against the oracle; three equal sets give
    the one-set bytes; zero gates in the text set leave exactly the text rows unchanged."""
    w = RAGGED.replace(mod_sets=3)
    x, ps = inputs(w)
    pg = gpu_params(ps, int8)[0]
    xg = x.to(DEV)
    h3.block_fwd(w, pg, xg)
    check_residual(cpu(xg), oracle.block_fwd(w, cpu_params(ps, int8)[0], x), x)
    # equal sets == one set
    one = dict(ps[0])
    one["mod"] = ps[0]["mod"][:6].contiguous()
    three = dict(ps[0])
    three["mod"] = one["mod"].repeat(3, 1).contiguous()
    a, b = x.to(DEV), x.to(DEV)
    h3.block_fwd(RAGGED, gpu_params([one], int8)[0], a)
    h3.block_fwd(w, gpu_params([three], int8)[0], b)
    assert_bitexact(cpu(b), cpu(a), "three equal sets")
    # text rows pass through with zero text gates
    z = x.to(DEV)
    h3.block_fwd(w, gpu_params([_text_gates_zero(ps[0], w.hidden)], int8)[0], z)
    nv, nt = w.n_video, w.n_text
    zc = cpu(z)
    assert_bitexact(zc[nv:nv + nt], x[nv:nv + nt], "text rows")
    assert not torch.equal(zc[:nv].view(torch.int16), x[:nv].view(torch.int16))


@pytest.mark.parametrize("int8", [False, True])
def test_stack_mod_sets_token_reduction_matches_oracle(int8):
    w = SMALL_TR.replace(mod_sets=3)
    x, ps = inputs(w, blocks=6)
    pg = gpu_params(ps, int8)
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg, reduction=(1, 4))
    ref = oracle.stack_fwd(w, cpu_params(ps, int8), x, reduce_after=1, restore_before=4, fused=True)
    check_residual(cpu(xg), ref, x, blocks=len(ps))


# ----------------------------------------------------------------------------- int8 MLP only

def test_block_int8_mlp_only_matches_oracle():
    """FC1 and FC2 in int8, QKV and output projection in bf16 (the pages' int8-MLP row)."""
    x, ps = inputs(RAGGED)
    pg = h3.quantize_block(dev_block(ps[0]), mlp_only=True)
    pc = oracle.quantize_block(ps[0], mlp_only=True)
    for k in ("q1", "s1", "q2", "s2"):
        assert_bitexact(cpu(pg[k]), pc[k], k)
    xg = x.to(DEV)
    h3.block_fwd(RAGGED, pg, xg)
    check_residual(cpu(xg), oracle.block_fwd(RAGGED, pc, x), x)
    # the fusion switches stay byte-identical on this path too
    for f in (h3.NOFUSE_GATE_ADALN, h3.NOFUSE_QUANT, h3.NO_ALIAS):
        y = x.to(DEV)
        h3.block_fwd(RAGGED, pg, y, flags=f)
        assert_bitexact(cpu(y), cpu(xg), f"flags {f}")


def test_stack_int8_mlp_only_token_reduction():
    w = SMALL_TR
    x, ps = inputs(w, blocks=5)
    pg = [h3.quantize_block(dev_block(p), mlp_only=True) for p in ps]
    pc = [oracle.quantize_block(p, mlp_only=True) for p in ps]
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg, reduction=(1, 3))
    ref = oracle.stack_fwd(w, pc, x, reduce_after=1, restore_before=3, fused=True)
    check_residual(cpu(xg), ref, x, blocks=len(ps))


# ----------------------------------------------------------------------------- streamed weights

def _streamed(w, pg, x, reduction=None, separate_copy_stream=True, pinned=True):
    """h3dit_stack_fwd_streamed with every block's tensors in host memory."""
    hb = [h3.host_block(p) if pinned else {k: v.to("cpu") for k, v in p.items()} for p in pg]
    s = h3.StreamedStack(w, hb, reduction=reduction)
    ws = h3.alloc_workspace(s.workspace_bytes, DEV)
    xg = x.to(DEV)
    cs = torch.cuda.Stream() if separate_copy_stream else None
    s(xg, ws, copy_stream=cs.cuda_stream if cs is not None else None)
    out = cpu(xg)
    del hb   # host weights stay alive until the stream is done (cpu() synchronised)
    return out


@pytest.mark.parametrize("prec", ["bf16", "int8", "int8_mlp", "int8_attn"])
def test_stack_streamed_equals_resident(prec):
    # matrices copied per block into two alternating device slots on a second stream: byte
    # for byte the resident stack, with token reduction, cross-block fusion and the slot reuse
    # of six blocks
    w = SMALL_TR
    x, ps = inputs(w, blocks=6)
    if prec == "int8_mlp":
        pg = [h3.quantize_block(dev_block(p), mlp_only=True) for p in ps]
    elif prec == "int8_attn":
        pg = [h3.quantize_block(dev_block(p), attn_only=True) for p in ps]
    else:
        pg = gpu_params(ps, prec == "int8")
    xr = x.to(DEV)
    h3.stack_fwd(w, pg, xr, reduction=(1, 4))
    assert_bitexact(_streamed(w, pg, x, reduction=(1, 4)), cpu(xr), "streamed vs resident stack")


def test_stack_streamed_single_stream_pageable_and_mod_sets():
    # copies on the compute stream, weights in ordinary (pageable) host memory, three
    # modulation sets: still the resident result
    w = SMALL_TR.replace(mod_sets=3)
    x, ps = inputs(w, blocks=3)
    pg = gpu_params(ps, False)
    xr = x.to(DEV)
    h3.stack_fwd(w, pg, xr)
    ref = cpu(xr)
    assert_bitexact(_streamed(w, pg, x, separate_copy_stream=False), ref, "single stream")
    assert_bitexact(_streamed(w, pg, x, pinned=False), ref, "pageable host weights")


# ----------------------------------------------------------------------------- limits

@pytest.mark.parametrize("int8", [False, True])
def test_block_maximum_hidden_width(int8):
    """hidden 8192 (64 heads x 128), the widest row the row kernels hold, against the oracle."""
    w = W0.replace(hidden=8192, heads=64, head_dim=128, mlp=8192, fc2_group=1024,
                   video_t=1, video_h=4, video_w=20, n_text=12, n_audio=4)
    assert w.n_tokens == 96
    x, ps = inputs(w)
    pg = gpu_params(ps, int8)[0]
    xg = x.to(DEV)
    h3.block_fwd(w, pg, xg)
    check_residual(cpu(xg), oracle.block_fwd(w, cpu_params(ps, int8)[0], x), x)


def test_zero_sized_stage_calls_touch_nothing():
    """n = 0 / M = 0 stage calls return OK and leave their outputs alone."""
    d = 256
    x = torch.randn((4, d), device=DEV).to(torch.bfloat16)
    sentinel = torch.full((4, d), 7.0, device=DEV, dtype=torch.bfloat16)
    mod = torch.zeros((6, d), device=DEV, dtype=torch.bfloat16)
    h3.row_gate_adaln(x[:0], gate=mod[2], y=x[:0], x_out=sentinel[:0], shift=mod[3], scale=mod[4], h=sentinel[:0])
    w = torch.randn((256, d), device=DEV).to(torch.bfloat16)
    h3.linear(0, 256, d, x, w, h3.OUT_BF16, sentinel)
    q = torch.zeros((2, 1, 128), device=DEV, dtype=torch.bfloat16)
    h3.attention(2, 0, 128, q, q, torch.zeros((2, 128, 16), device=DEV, dtype=torch.bfloat16), sentinel)
    torch.cuda.synchronize()
    assert bool((sentinel.float() == 7.0).all())


# ----------------------------------------------------------------------------- final head

@pytest.mark.parametrize("w", [W0, WORKLOADS[3].replace(blocks=1)], ids=["tiny", "4096tok"])
def test_final_head_matches_oracle(w):
    d = w.hidden
    x = synth.make_x(w, 1005)
    g = torch.Generator().manual_seed(3)
    mv = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    ma = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    wv = (torch.randn(128, d, generator=g) * 0.02).to(torch.bfloat16)
    wa = (torch.randn(256, d, generator=g) * 0.02).to(torch.bfloat16)
    xg = x.to(DEV)
    ov, oa = h3.final_head(w, xg, video=(mv.to(DEV), wv.to(DEV)), audio=(ma.to(DEV), wa.to(DEV)))
    rv, ra = oracle.final_head(w, x, video=(mv, wv), audio=(ma, wa))
    assert relerr(cpu(ov), rv) <= BF16_TOL
    assert relerr(cpu(oa), ra) <= BF16_TOL
    assert_bitexact(cpu(xg), x, "residual untouched")
    # one part alone gives the same bytes
    ov2, none = h3.final_head(w, xg, video=(mv.to(DEV), wv.to(DEV)))
    assert none is None
    assert_bitexact(cpu(ov2), cpu(ov), "video part alone")
    # AdaLN applied in the head GEMM's tile loads == the row kernel's stored AdaLN then the GEMM:
    # byte for byte where that GEMM sums K in one pass; where it is split along K (at 4096
    # tokens the audio part, 64 rows x 256 channels: one tile in 8 segments) only the order differs
    nv = w.n_tokens - w.n_text - w.n_audio
    for rows, (mod, wt), out in ((slice(0, nv), (mv, wv), ov), (slice(w.n_tokens - w.n_audio, w.n_tokens), (ma, wa), oa)):
        xs = xg[rows].contiguous()
        h = torch.empty_like(xs)
        h3.row_gate_adaln(xs, shift=mod[0].to(DEV).contiguous(), scale=mod[1].to(DEV).contiguous(), h=h, eps=w.ln_eps)
        ref = torch.empty((xs.shape[0], wt.shape[0]), dtype=torch.bfloat16, device=DEV)
        h3.linear(xs.shape[0], wt.shape[0], w.hidden, h, wt.to(DEV).contiguous(), h3.OUT_BF16, ref)
        if h3.linear_workspace(xs.shape[0], wt.shape[0], w.hidden) > 0:
            assert_close_bf16(cpu(out), cpu(ref), "fused head vs row kernel + split-K GEMM")
        else:
            assert_bitexact(cpu(out), cpu(ref), "fused head vs row kernel + GEMM")


# ----------------------------------------------------------------------------- int8 attention projections only

def test_block_int8_attn_only_matches_oracle():
    """QKV and the output projection in int8, FC1 and FC2 in bf16 (the int8-QKV-only path)."""
    x, ps = inputs(RAGGED)
    pg = h3.quantize_block(dev_block(ps[0]), attn_only=True)
    pc = oracle.quantize_block(ps[0], attn_only=True)
    for k in ("qqkv", "sqkv", "qo", "so"):
        assert_bitexact(cpu(pg[k]), pc[k], k)
    assert "q1" not in pg
    xg = x.to(DEV)
    h3.block_fwd(RAGGED, pg, xg)
    check_residual(cpu(xg), oracle.block_fwd(RAGGED, pc, x), x, "int8 attention only")
    for f in (h3.NOFUSE_GATE_ADALN, h3.NOFUSE_QUANT, h3.NOFUSE_ROPE, h3.NO_ALIAS):
        y = x.to(DEV)
        h3.block_fwd(RAGGED, pg, y, flags=f)
        assert_bitexact(cpu(y), cpu(xg), f"flags {f}")


def test_stack_int8_attn_only_token_reduction():
    w = SMALL_TR
    x, ps = inputs(w, blocks=5)
    pg = [h3.quantize_block(dev_block(p), attn_only=True) for p in ps]
    pc = [oracle.quantize_block(p, attn_only=True) for p in ps]
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg, reduction=(1, 3))
    ref = oracle.stack_fwd(w, pc, x, reduce_after=1, restore_before=3, fused=True)
    check_residual(cpu(xg), ref, x, "int8 attention only, token reduction", blocks=len(ps))
    xs = _streamed(w, pg, x, reduction=(1, 3))
    assert_bitexact(xs, cpu(xg), "streamed int8-attention stack")


# ----------------------------------------------------------------------------- caller rotary tables

def _angles_3axis(t, h, wpos, split, hd, theta):
    """Rotary angles [n][hd/2] of 3-axis positions (sections t | h | w of split dims)."""
    st, sh, sw = split
    cols = []
    for pos, sec in ((t, st), (h, sh), (wpos, sw)):
        j = torch.arange(sec // 2, dtype=torch.float64)
        cols.append(pos.to(torch.float64)[:, None] * theta ** (-2.0 * j / sec)[None, :])
    return torch.cat(cols, dim=1)


def audio_on_visual_timeline_tables(w):
    """Tables that are not the built-in ones: video and text as built in, but audio token a
    placed on the visual rotary timeline as if it were a row of width-32 visual tokens below the
    last video row (t = a // 32, h = video_h, w = a % 32), with the video's 3-axis sections."""
    cos, sin = oracle.rope_tables(w)
    a = torch.arange(w.n_audio)
    ang = _angles_3axis(a // 32, torch.full_like(a, w.video_h), a % 32, w.split, w.head_dim, w.rope_theta)
    cos, sin = cos.clone(), sin.clone()
    cos[-w.n_audio:] = torch.cos(ang).to(torch.float32)
    sin[-w.n_audio:] = torch.sin(ang).to(torch.float32)
    return cos, sin


@pytest.mark.parametrize("int8", [False, True])
def test_block_caller_rope_tables(int8):
    """The block with caller tables (audio on the visual timeline) against the oracle fed the
    same tables; the built-in tables passed explicitly give the default bytes; other tables give
    other bytes."""
    w = RAGGED
    x, ps = inputs(w)
    pg = gpu_params(ps, int8)[0]
    pc = cpu_params(ps, int8)[0]
    cos, sin = audio_on_visual_timeline_tables(w)
    xg = x.to(DEV)
    h3.block_fwd(w, pg, xg, rope=(cos.to(DEV), sin.to(DEV)))
    ref = oracle.block_fwd(w, pc, x, cos, sin)
    check_residual(cpu(xg), ref, x, "caller rope tables")
    base = x.to(DEV)
    h3.block_fwd(w, pg, base)
    own = h3.rope_tables(w, device=DEV)
    expl = x.to(DEV)
    h3.block_fwd(w, pg, expl, rope=own)
    assert_bitexact(cpu(expl), cpu(base), "built-in tables passed explicitly")
    assert not torch.equal(cpu(xg).view(torch.int16), cpu(base).view(torch.int16))


def test_stack_caller_rope_tables_with_reduction():
    """Full and paired-sequence tables both from the caller (audio on the visual timeline in
    both), through token reduction, against the oracle given the same tables."""
    w = SMALL_TR
    x, ps = inputs(w, blocks=5)
    pg = gpu_params(ps, False)
    cos, sin = audio_on_visual_timeline_tables(w)
    cr, sr = oracle.rope_tables(w, reduced=True)
    cr, sr = cr.clone(), sr.clone()
    cr[-w.n_audio:], sr[-w.n_audio:] = cos[-w.n_audio:], sin[-w.n_audio:]
    xg = x.to(DEV)
    h3.stack_fwd(w, pg, xg, reduction=(1, 4), rope=(cos.to(DEV), sin.to(DEV)), rope_reduced=(cr.to(DEV), sr.to(DEV)))
    ref = oracle.stack_fwd(w, ps, x, reduce_after=1, restore_before=4, fused=True, rope=(cos, sin),
                           rope_reduced=(cr, sr))
    check_residual(cpu(xg), ref, x, "stack, caller tables", blocks=len(ps))


# ----------------------------------------------------------------------------- streamed: back-to-back calls

def test_stack_streamed_back_to_back_calls():
    """Two streamed calls on one workspace, one after the other with no host synchronisation,
    copies on a second stream: the second call's first copies wait for the first call's last
    blocks, so both outputs equal the resident stack's."""
    w = SMALL_TR
    x, ps = inputs(w, blocks=5)
    pg = gpu_params(ps, False)
    xr = x.to(DEV)
    h3.stack_fwd(w, pg, xr, reduction=(1, 4))
    ref = cpu(xr)
    hb = [h3.host_block(p) for p in pg]
    s = h3.StreamedStack(w, hb, reduction=(1, 4))
    ws = h3.alloc_workspace(s.workspace_bytes, DEV)
    cs = torch.cuda.Stream()
    xa, xb = x.to(DEV), x.to(DEV)
    torch.cuda.synchronize()
    s(xa, ws, copy_stream=cs.cuda_stream)
    s(xb, ws, copy_stream=cs.cuda_stream)
    assert_bitexact(cpu(xa), ref, "first call")
    assert_bitexact(cpu(xb), ref, "second call")
    del hb


# ----------------------------------------------------------------------------- canaries

@pytest.mark.parametrize("int8", [False, True])
def test_stack_touches_only_x_and_its_workspace(int8):
    """Canary bytes around x and past the end of the planned workspace stay untouched by a
    token-reduction stack (the arenas, split-K partials and tables stay inside the plan)."""
    w = SMALL_TR
    x, ps = inputs(w, blocks=5)
    pg = gpu_params(ps, int8)
    stack = h3.Stack(w, pg, 0, (1, 4))
    pad = 4096
    n = stack.workspace_bytes
    ws_all = torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = ws_all[pad:pad + n]
    N, d = x.shape
    x_all = torch.full(((N + 2 * 16) * d,), 0x5A5A, dtype=torch.int16, device=DEV)
    xg = x_all[16 * d:(16 + N) * d].view(torch.bfloat16).view(N, d)
    xg.copy_(x.to(DEV))
    stack(xg, ws)
    ref = oracle.stack_fwd(w, cpu_params(ps, int8), x, reduce_after=1, restore_before=4, fused=True)
    check_residual(cpu(xg), ref, x, "canary run", blocks=len(ps))
    wc = cpu(ws_all)
    assert bool((wc[:pad] == 0xA5).all()) and bool((wc[pad + n:] == 0xA5).all()), "workspace canary"
    xc = cpu(x_all)
    assert bool((xc[:16 * d] == 0x5A5A).all()) and bool((xc[(16 + N) * d:] == 0x5A5A).all()), "x canary"
