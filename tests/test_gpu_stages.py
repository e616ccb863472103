"""Stage-wise parity of every HIP kernel against the CPU oracle, on seeded inputs that span
several tiles and a ragged tail.  Each kernel is fed the same bytes as the oracle; where the
kernel's arithmetic is fully ordered (gates, int8 codes, int32 sums, dequantisation, group
sums, rotary of a given projection, token pair/restore) the result must match bit for bit,
elsewhere to the tolerances of tests/parity.py."""
import pytest
import torch

import oracle
import synth
from synth import WORKLOADS
from parity import BF16_TOL, F32_TOL, assert_bitexact, assert_close_bf16, relerr

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("audio_diffusion_transformer_dit_amd")
DEV = "cuda"


def bf_randn(shape, seed, std=1.0, tid=9):
    return synth.normal_bf16(seed, 0, tid, shape, std)


def to_dev(t):
    return t.to(DEV).contiguous()


def cpu(t):
    torch.cuda.synchronize()
    return t.to("cpu")


# ----------------------------------------------------------------------------- rotary tables

@pytest.mark.parametrize("cfg,reduced", [(0, False), (1, False), (4, False), (4, True)])
def test_rope_tables(cfg, reduced):
    w = WORKLOADS[cfg]
    cg, sg = h3.rope_tables(w, reduced)
    co, so = oracle.rope_tables(w, reduced)
    assert cg.shape == co.shape
    # both round a double-precision cos/sin to fp32: equal up to the rare double-rounding case
    assert float((cpu(cg) - co).abs().max()) <= 1.2e-7
    assert float((cpu(sg) - so).abs().max()) <= 1.2e-7


# ----------------------------------------------------------------------------- row kernels

@pytest.mark.parametrize("n,d", [(300, 256), (129, 5120), (64, 1024)])
def test_gate_adaln_bf16(n, d):
    x = bf_randn((n, d), 1)
    y = bf_randn((n, d), 2)
    mod = bf_randn((6, d), 3, 0.1)
    xg, yg, modg = to_dev(x), to_dev(y), to_dev(mod)
    x1 = torch.empty_like(xg)
    h = torch.empty_like(xg)
    h3.row_gate_adaln(xg, gate=modg[2], y=yg, x_out=x1, shift=modg[3], scale=modg[4], h=h)
    x1_ref = oracle.gate(x, mod[2], y)
    assert_bitexact(cpu(x1), x1_ref, "gated residual")
    h_ref, _, _ = oracle.adaln(x1_ref, mod[3], mod[4], 1e-6, stats=True)
    hc = cpu(h)
    assert_close_bf16(hc, h_ref, "AdaLN (LN sums in another order)")
    # the two-kernel sequence (gate, then AdaLN of the written residual) gives the same bytes
    x1b = torch.empty_like(xg)
    hb = torch.empty_like(xg)
    h3.row_gate_adaln(xg, gate=modg[2], y=yg, x_out=x1b)
    h3.row_gate_adaln(x1b, shift=modg[3], scale=modg[4], h=hb)
    assert_bitexact(cpu(x1b), cpu(x1))
    assert_bitexact(cpu(hb), hc)
    # in place (x_out == x)
    xi = xg.clone()
    h3.row_gate_adaln(xi, gate=modg[2], y=yg, x_out=xi)
    assert_bitexact(cpu(xi), x1_ref)


@pytest.mark.parametrize("n,d", [(300, 256), (77, 5120)])
def test_adaln_int8_codes(n, d):
    x = bf_randn((n, d), 4)
    mod = bf_randn((6, d), 5, 0.1)
    xg, modg = to_dev(x), to_dev(mod)
    h = torch.empty_like(xg)
    q = torch.empty((n, d), dtype=torch.int8, device=DEV)
    s = torch.empty(n, dtype=torch.float32, device=DEV)
    h3.row_gate_adaln(xg, shift=modg[0], scale=modg[1], h=h, q=q, s=s)
    hc = cpu(h)
    assert_close_bf16(hc, oracle.adaln(x, mod[0], mod[1]), "AdaLN")
    q_ref, s_ref = oracle.q8_rows(hc)                     # the oracle's codes of the GPU's own bf16 row
    assert_bitexact(cpu(q), q_ref, "int8 codes")
    assert_bitexact(cpu(s), s_ref[:, 0], "scales")
    # codes only (no bf16 output) are the same bytes
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    h3.row_gate_adaln(xg, shift=modg[0], scale=modg[1], q=q2, s=s2)
    assert_bitexact(cpu(q2), q_ref)
    assert_bitexact(cpu(s2), s_ref[:, 0])


def test_gate_fused_int8_codes_of_gated_row():
    n, d = 200, 512
    x, y, mod = bf_randn((n, d), 6), bf_randn((n, d), 7), bf_randn((6, d), 8, 0.1)
    xg = to_dev(x)
    h = torch.empty_like(xg)
    q = torch.empty((n, d), dtype=torch.int8, device=DEV)
    s = torch.empty(n, dtype=torch.float32, device=DEV)
    h3.row_gate_adaln(xg, gate=to_dev(mod[2]), y=to_dev(y), x_out=xg, shift=to_dev(mod[3]), scale=to_dev(mod[4]),
                      h=h, q=q, s=s)
    assert_bitexact(cpu(xg), oracle.gate(x, mod[2], y))
    q_ref, s_ref = oracle.q8_rows(cpu(h))
    assert_bitexact(cpu(q), q_ref)
    assert_bitexact(cpu(s), s_ref[:, 0])


@pytest.mark.parametrize("rows,cols,group,hm", [(300, 2048, 1024, 0), (257, 5120, 5120, 0), (130, 512, 512, 128),
                                                (33, 256, 256, 64),
                                                # one wave per group: 20 groups; 6 groups (a half-idle
                                                # workgroup); one and four chunks per lane
                                                (300, 20480, 1024, 0), (129, 6144, 1024, 0), (64, 4096, 512, 0),
                                                (50, 8192, 2048, 0),
                                                # whole rows of 16384 / 20480 in registers; 40960 in two passes
                                                (30, 16384, 16384, 0), (64, 20480, 20480, 0), (8, 40960, 40960, 0)])
def test_quantize_rows(rows, cols, group, hm):
    v = bf_randn((rows, cols), 10)
    v[3] = 0                                               # an all-zero row
    if hm:
        vin = v.view(rows, cols // hm, hm).permute(1, 0, 2).contiguous()   # head-major
    else:
        vin = v
    q, s = h3.quantize_rows(to_dev(vin), rows, cols, group, hm)
    q_ref, s_ref = oracle.q8_rows(v, group)
    assert_bitexact(cpu(q), q_ref)
    assert_bitexact(cpu(s), s_ref)


def near_tie_rows(rows, cols, seed):
    """bf16 rows whose values sit on and next to the half-integer points of their own code
    scale: each row draws an absmax, and its values are bf16 roundings of (k + 1/2) * s nudged
    by -3..3 bf16 steps (k random), where a quotient approximated through 1/s and the correctly
    rounded quotient could round to different integers."""
    g = torch.Generator().manual_seed(seed)
    amax = torch.exp(torch.empty(rows, 1).uniform_(-6.0, 6.0, generator=g)).to(torch.bfloat16).to(torch.float64)
    # every fourth row: absmax 127 * 2^j, a scale of exactly 2^j, so (k + 1/2) * s is an exact tie
    amax[::4] = 127.0 * torch.exp2(torch.randint(-4, 5, (len(amax[::4]), 1), generator=g).to(torch.float64))
    s = (amax.to(torch.float32) / 127.0).to(torch.float64)
    k = torch.randint(-127, 127, (rows, cols), generator=g).to(torch.float64)
    v = ((k + 0.5) * s).to(torch.bfloat16)
    nudge = torch.randint(-3, 4, (rows, cols), generator=g, dtype=torch.int16)
    v = (v.view(torch.int16) + nudge).view(torch.bfloat16)
    v = torch.where(v.to(torch.float64).abs() > amax, amax.to(torch.bfloat16).expand(rows, cols), v)
    v[:, 0] = amax[:, 0].to(torch.bfloat16)                 # the absmax itself: code 127
    return v.contiguous()


@pytest.mark.parametrize("rows,cols,group", [(512, 1024, 1024), (64, 20480, 1024), (96, 5120, 5120), (8, 20480, 20480)])
def test_quantize_rows_near_ties_bitexact(rows, cols, group):
    """Codes of values on and next to half-integer quotients (ties go to even) equal the oracle's
    rintf(v / s) bit for bit, in every code kernel (1024 groups, whole 5120 and 20480 rows)."""
    v = near_tie_rows(rows, cols, rows + cols)
    q, s = h3.quantize_rows(to_dev(v), rows, cols, group)
    q_ref, s_ref = oracle.q8_rows(v, group)
    assert_bitexact(cpu(s), s_ref)
    assert_bitexact(cpu(q), q_ref)
    # and through the row kernel's fused codes (AdaLN with shift = value, scale = -1: h == shift)
    if cols == 5120:
        for r in range(0, rows, 32):
            zero = torch.zeros(cols, dtype=torch.bfloat16)
            minus = torch.full((cols,), -1.0, dtype=torch.bfloat16)
            x = bf_randn((1, cols), r + 1)
            qg = torch.empty((1, cols), dtype=torch.int8, device="cuda")
            sg = torch.empty(1, dtype=torch.float32, device="cuda")
            h3.row_gate_adaln(to_dev(x), shift=to_dev(v[r].contiguous()), scale=to_dev(minus), q=qg, s=sg)
            qr, sr = oracle.q8_rows(v[r:r + 1].contiguous())
            assert_bitexact(cpu(qg), qr, "row kernel codes")


def test_quantize_weights():
    w = bf_randn((384, 1024), 11, 0.02)
    q, s = h3.quantize_weights(to_dev(w))
    q_ref, s_ref = oracle.quantize_weights(w)
    assert_bitexact(cpu(q), q_ref)
    assert_bitexact(cpu(s), s_ref)


# ----------------------------------------------------------------------------- projections

@pytest.mark.parametrize("M,N,K", [(300, 768, 256), (513, 1024, 1024), (64, 256, 2048), (1, 128, 128),
                                   (512, 4096, 8192), (300, 2048, 4096)])
def test_linear_bf16(M, N, K):
    # shapes of under a round of 256 x 256 tiles with long K are computed as split-K segments
    # (512 x 4096 x 8192: 32 tiles; 64 x 256 x 2048: one tile; 300 x 2048 x 4096: 16 tiles)
    split = (M, N, K) in ((512, 4096, 8192), (64, 256, 2048), (300, 2048, 4096))
    assert (h3.linear_workspace(M, N, K) > 0) == split
    a = bf_randn((M, K), 12)
    wt = bf_randn((N, K), 13, 0.02)
    ag, wg = to_dev(a), to_dev(wt)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    h3.linear(M, N, K, ag, wg, h3.OUT_F32, acc)
    acc_ref = oracle.gemm_f32(a, wt)
    assert relerr(cpu(acc), acc_ref) <= F32_TOL
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, ag, wg, h3.OUT_BF16, out)
    assert_bitexact(cpu(out), cpu(acc).to(torch.bfloat16), "bf16 output = rounded fp32 accumulator")
    assert relerr(cpu(out), oracle.f32_to_bf16(acc_ref)) <= BF16_TOL
    gl = torch.empty_like(out)
    h3.linear(M, N, K, ag, wg, h3.OUT_GELU, gl)
    glc = cpu(gl)
    ref = oracle.gelu_rows(cpu(acc).to(torch.bfloat16))    # same plan (K order) as the fp32 output
    assert_close_bf16(glc, ref, "GELU epilogue")


@pytest.mark.parametrize("M,K,int8,N", [(4096, 128, False, 4096), (4000, 256, False, 4096), (4096, 384, False, 4096),
                                        (4096, 384, True, 4096), (3900, 640, True, 4096), (4096, 640, False, 20480)])
def test_linear_full_round_short_k(M, K, int8, N):
    # 16 x 16 tiles of 256 x 256 fill one round of the chip, so the plan takes whole 256 x 256
    # tiles (bf16: 4 waves of 128 x 128; int8: 8 waves of 128 x 64) with only a few K slices: the
    # paths where the steady loop runs zero or few times and the peeled tail does the work (int8
    # with 3 and 5 slices: odd counts); M = 4000 / 3900 leaves a ragged last tile row; N = 20480
    # gives five whole rounds of 10-slice tiles
    assert h3.linear_workspace(M, N, K, precision=h3.INT8 if int8 else h3.BF16) == 0
    a = bf_randn((M, K), 40 + K)
    wt = bf_randn((N, K), 41 + K, 0.02)
    if int8:
        qa, sa = oracle.q8_rows(a)
        qw, sw = oracle.quantize_weights(wt)
        sa = sa[:, 0].contiguous()
        acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
        h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_I32, acc, precision=h3.INT8, a_scale=to_dev(sa),
                  w_scale=to_dev(sw))
        assert_bitexact(cpu(acc), oracle.gemm_i32(qa, qw), "int32 accumulators")
        return
    ag, wg = to_dev(a), to_dev(wt)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    h3.linear(M, N, K, ag, wg, h3.OUT_F32, acc)
    assert relerr(cpu(acc), oracle.gemm_f32(a, wt)) <= F32_TOL
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, ag, wg, h3.OUT_BF16, out)
    assert_bitexact(cpu(out), cpu(acc).to(torch.bfloat16), "bf16 output = rounded fp32 accumulator")


@pytest.mark.parametrize("H,M,hd,N", [(4, 300, 64, 512), (40, 300, 128, 512)])
def test_linear_bf16_headmajor_input(H, M, hd, N):
    # the out-projection's form: A read head-major.  At K = 40 x 128 the 4 tiles are split into
    # K segments (fp32 output: the per-tile fixup; bf16 output: the chip-wide sum)
    K = H * hd
    assert (h3.linear_workspace(M, N, K) > 0) == (H == 40)
    assert h3.linear_workspace(M, N, K, out_kind=h3.OUT_F32) == h3.linear_workspace(M, N, K)
    o = bf_randn((H, M, hd), 14)
    wt = bf_randn((N, K), 15, 0.02)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    h3.linear(M, N, K, to_dev(o), to_dev(wt), h3.OUT_F32, acc, a_headmajor_hd=hd)
    tok = o.permute(1, 0, 2).reshape(M, K).contiguous()
    acc_ref = oracle.gemm_f32(tok, wt)
    assert relerr(cpu(acc), acc_ref) <= F32_TOL
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, to_dev(o), to_dev(wt), h3.OUT_BF16, out, a_headmajor_hd=hd)
    assert relerr(cpu(out), oracle.f32_to_bf16(acc_ref)) <= BF16_TOL
    assert_bitexact(cpu(out), cpu(acc).to(torch.bfloat16), "bf16 output = rounded fp32 accumulator")


@pytest.mark.parametrize("M,N,K", [(300, 768, 256), (257, 1024, 1024), (1, 256, 128), (512, 4096, 8192)])
def test_linear_int8(M, N, K):
    a = bf_randn((M, K), 16)
    wt = bf_randn((N, K), 17, 0.02)
    qa, sa = oracle.q8_rows(a)
    qw, sw = oracle.quantize_weights(wt)
    sa = sa[:, 0].contiguous()
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_I32, acc, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    acc_ref = oracle.gemm_i32(qa, qw)
    assert_bitexact(cpu(acc), acc_ref, "int32 accumulators")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_BF16, out, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    deq = oracle.dequant_bf16(acc_ref, sa, sw)
    assert_bitexact(cpu(out), deq, "dequantised output")
    gl = torch.empty_like(out)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_GELU, gl, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    assert relerr(cpu(gl), oracle.gelu_rows(deq)) <= BF16_TOL


@pytest.mark.parametrize("M,N,K", [(4096, 5120, 5120), (4000, 5120, 5120), (3500, 5120, 1024)])
def test_linear_int8_column_split_sampled_rows(M, N, K):
    """The int8 path's column split: at the out-projection's shape (M x 5120 x 5120) 256 x 256
    tiles over columns 0-4095 and a second launch of 128 x 128 tiles over 4096-5119 (one round
    each instead of 2.5 rounds of 256 x 128 tiles); M = 4000 leaves both launches a ragged last
    tile row; 3500 x 5120 x 1024 splits at column 4608.  Accumulators and dequantised output
    exact, GELU output at the bf16 bar, on sampled rows across both column ranges."""
    assert h3.linear_workspace(M, N, K, h3.INT8) == 0
    qa = torch.randint(-127, 128, (M, K), dtype=torch.int8, generator=torch.Generator().manual_seed(15))
    qw = torch.randint(-127, 128, (N, K), dtype=torch.int8, generator=torch.Generator().manual_seed(16))
    sa = torch.rand(M, generator=torch.Generator().manual_seed(17)) * 0.01 + 1e-3
    sw = torch.rand(N, generator=torch.Generator().manual_seed(18)) * 0.01 + 1e-3
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_I32, acc, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_BF16, out, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    rows = torch.tensor([0, 1, 127, 128, 255, 1029, 2048, 3071, 3333, 3456, M - 2, M - 1])
    ref = oracle.gemm_i32(qa[rows].contiguous(), qw)
    assert_bitexact(cpu(acc)[rows], ref, "int32 accumulators, both column ranges")
    deq = oracle.dequant_bf16(ref, sa[rows].contiguous(), sw)
    assert_bitexact(cpu(out)[rows], deq, "dequantised output")
    gl = torch.empty_like(out)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_GELU, gl, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    assert relerr(cpu(gl)[rows], oracle.gelu_rows(deq)) <= BF16_TOL


def test_linear_int8_splitk_sampled_rows():
    """4096 x 5120 x 20480 on the int8 path without groups: 64 of the 320 tiles are summed from
    4 K segments of int32 partials, which must give the exact accumulators."""
    M, N, K = 4096, 5120, 20480
    assert h3.linear_workspace(M, N, K, h3.INT8) > 0
    qa = torch.randint(-127, 128, (M, K), dtype=torch.int8, generator=torch.Generator().manual_seed(5))
    qw = torch.randint(-127, 128, (N, K), dtype=torch.int8, generator=torch.Generator().manual_seed(6))
    sa = torch.rand(M, generator=torch.Generator().manual_seed(7)) * 0.01 + 1e-3
    sw = torch.rand(N, generator=torch.Generator().manual_seed(8)) * 0.01 + 1e-3
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_I32, acc, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_BF16, out, precision=h3.INT8, a_scale=to_dev(sa),
              w_scale=to_dev(sw))
    # rows of whole tiles and of split tiles (tile rows 8..15 hold the split ones)
    rows = torch.tensor([0, 1, 255, 1029, 2048, 2049, 2560, 3071, 3333, 4094, 4095])
    ref = oracle.gemm_i32(qa[rows].contiguous(), qw)
    assert_bitexact(cpu(acc)[rows], ref, "int32 accumulators, split tiles included")
    assert_bitexact(cpu(out)[rows], oracle.dequant_bf16(ref, sa[rows].contiguous(), sw), "dequantised output")


@pytest.mark.parametrize("M,N,K,G", [(300, 256, 2048, 1024), (129, 512, 1024, 1024), (64, 256, 3072, 1024),
                                     (200, 256, 1024, 256),
                                     # 280 large tiles would take two rounds: 252 large tiles plus a
                                     # second launch of 128 x 128 tiles over the last 512 columns,
                                     # ragged in both
                                     (1700, 5120, 2048, 512)])
def test_fc2_grouped_int8(M, N, K, G):
    gl = bf_randn((M, K), 18)
    wt = bf_randn((N, K), 19, 0.02)
    qa, sa = oracle.q8_rows(gl, G)
    qw, sw = oracle.quantize_weights(wt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, to_dev(qa), to_dev(qw), h3.OUT_BF16, y, precision=h3.INT8, a_scale=to_dev(sa), a_group=G,
              w_scale=to_dev(sw))
    assert_bitexact(cpu(y), oracle.fc2_int8(qa, sa, qw, sw, G), "grouped FC2")


@pytest.mark.parametrize("M,N,K", [(300, 256, 4096), (257, 512, 20480)])
def test_fc2_row_codes_on_ungrouped_kernel(M, N, K):
    """Row-level FC2: one code per token over the whole input, multiplied on the ungrouped
    int8 kernel, equals the grouped formula with a single group bit for bit."""
    gl = bf_randn((M, K), 22)
    wt = bf_randn((N, K), 23, 0.02)
    qw, sw = oracle.quantize_weights(wt)
    qa, sa = h3.quantize_rows(to_dev(gl), M, K, K)
    qa_ref, sa_ref = oracle.q8_rows(gl, K)
    assert_bitexact(cpu(qa), qa_ref, "codes")
    assert_bitexact(cpu(sa), sa_ref, "scales")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, N, K, qa, to_dev(qw), h3.OUT_BF16, y, precision=h3.INT8, a_scale=sa[:, 0].contiguous(),
              w_scale=to_dev(sw))
    assert_bitexact(cpu(y), oracle.fc2_int8(qa_ref, sa_ref, qw, sw, K), "row-level FC2")


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("M,H,hd", [(300, 4, 64), (130, 2, 128), (4480, 40, 128)])
def test_linear_qkv_rope_headmajor(M, H, hd, int8):
    d = H * hd
    # 4480 tokens at d 5120 (the paired sequence of an 8192-token layout): on the bf16 path the
    # last round of tiles is split along K and the fixup launch runs the rotary epilogue
    assert (h3.linear_workspace(M, 3 * d, d, h3.INT8 if int8 else h3.BF16, 0, h3.OUT_QKV, H, hd) > 0) == \
        (M == 4480 and not int8)
    w = WORKLOADS[0].replace(hidden=d, heads=H, head_dim=hd, video_t=2, video_h=5, video_w=M // 10 - 3,
                             n_text=M - 10 * (M // 10 - 3) - 4, n_audio=4)
    assert w.n_tokens == M
    cos, sin = h3.rope_tables(w)
    a = bf_randn((M, d), 20)
    wt = bf_randn((3 * d, d), 21, 0.02)
    kw = {}
    if int8:
        qa, sa = oracle.q8_rows(a)
        qw, sw = oracle.quantize_weights(wt)
        ag, wg = to_dev(qa), to_dev(qw)
        kw = dict(precision=h3.INT8, a_scale=to_dev(sa[:, 0].contiguous()), w_scale=to_dev(sw))
    else:
        ag, wg = to_dev(a), to_dev(wt)
    t = torch.empty((M, 3 * d), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, 3 * d, d, ag, wg, h3.OUT_BF16, t, **kw)
    q = torch.empty((H, M, hd), dtype=torch.bfloat16, device=DEV)
    k = torch.empty_like(q)
    vt = torch.zeros((H, hd, h3.ldv(M)), dtype=torch.bfloat16, device=DEV)
    h3.linear(M, 3 * d, d, ag, wg, h3.OUT_QKV, None, cos=cos, sin=sin, heads=H, head_dim=hd, out_q=q, out_k=k,
              out_v=vt, **kw)
    qr, kr, vr = oracle.rope_split(cpu(t), cpu(cos), cpu(sin), H, hd)
    assert_bitexact(cpu(q), qr, "q")
    assert_bitexact(cpu(k), kr, "k")
    assert_bitexact(h3.v_from_vt(cpu(vt), M), vr, "V^T")
    # the unfused rotary + head split kernel gives the same bytes
    q2, k2, vt2 = torch.empty_like(q), torch.empty_like(k), torch.zeros_like(vt)
    h3.rope_split(M, H, hd, t, cos, sin, q2, k2, vt2)
    assert_bitexact(cpu(q2), cpu(q))
    assert_bitexact(cpu(k2), cpu(k))
    assert_bitexact(cpu(vt2), cpu(vt))


def test_gelu_kernel():
    u = bf_randn((4096,), 22, 3.0)
    gl = torch.empty((4096,), dtype=torch.bfloat16, device=DEV)
    h3.gelu(to_dev(u), gl)
    ref = oracle.gelu_rows(u)
    assert_close_bf16(cpu(gl), ref, "GELU")


# ----------------------------------------------------------------------------- attention

@pytest.mark.parametrize("H,N,hd", [(2, 1, 64), (3, 7, 64), (2, 64, 128), (4, 300, 64), (2, 257, 128),
                                    (1, 1000, 128), (64, 300, 64), (128, 257, 128)])
def test_attention(H, N, hd):
    # the last two: many heads, so query tiles of several heads share each XCD (head grouping)
    q = bf_randn((H, N, hd), 23, 2.0)
    k = bf_randn((H, N, hd), 24, 2.0)
    v = bf_randn((H, N, hd), 25)
    vt = h3.vt_from_v(v)
    qg = to_dev(q)
    o = torch.empty_like(qg)
    mx = torch.empty((H, N), dtype=torch.float32, device=DEV)
    sm = torch.empty_like(mx)
    h3.attention(H, N, hd, qg, to_dev(k), to_dev(vt), o, mx, sm)
    o_ref, mx_ref, sm_ref = oracle.attention(q, k, v, stats=True)
    assert relerr(cpu(o), o_ref) <= BF16_TOL
    assert relerr(cpu(mx), mx_ref) <= F32_TOL
    assert relerr(cpu(sm), sm_ref) <= F32_TOL
    # output written over q gives the same bytes
    qi = to_dev(q)
    h3.attention(H, N, hd, qi, to_dev(k), to_dev(vt), qi)
    assert_bitexact(cpu(qi), cpu(o))


def test_attention_garbage_padding_is_ignored():
    # values past the last key (the V^T pitch padding) may hold anything, even NaN
    H, N, hd = 2, 100, 64
    q, k, v = bf_randn((H, N, hd), 26), bf_randn((H, N, hd), 27), bf_randn((H, N, hd), 28)
    vt = torch.full((H, hd, h3.ldv(N)), float("nan"), dtype=torch.bfloat16)
    vt[:, :, h3.vt_positions(N)] = v.transpose(1, 2)
    o = torch.empty((H, N, hd), dtype=torch.bfloat16, device=DEV)
    h3.attention(H, N, hd, to_dev(q), to_dev(k), to_dev(vt), o)
    assert relerr(cpu(o), oracle.attention(q, k, v)) <= BF16_TOL


def test_attention_constant_values_and_single_key():
    H, N, hd = 2, 200, 128
    q, k = bf_randn((H, N, hd), 29, 3.0), bf_randn((H, N, hd), 30, 3.0)
    vt = torch.ones((H, hd, h3.ldv(N)), dtype=torch.bfloat16)
    o = torch.empty((H, N, hd), dtype=torch.bfloat16, device=DEV)
    h3.attention(H, N, hd, to_dev(q), to_dev(k), to_dev(vt), o)
    assert torch.all(cpu(o).float() == 1.0)     # rows of probabilities sum to 1


# ----------------------------------------------------------------------------- token reduction

@pytest.mark.parametrize("vw", [6, 7, 59])
def test_token_pair_restore(vw):
    w = WORKLOADS[4].replace(video_t=2, video_h=3, video_w=vw, n_text=9, n_audio=5, hidden=256, heads=4,
                             head_dim=64, mlp=1024)
    d = 256
    x = bf_randn((w.n_tokens, d), 31)
    nr = oracle.layout_tokens(w, True)
    r = torch.empty((nr, d), dtype=torch.bfloat16, device=DEV)
    r_in = torch.empty_like(r)
    xg = to_dev(x)
    h3.token_pair(w, xg, r, r_in)
    r_ref = oracle.token_pair(w, x)
    assert_bitexact(cpu(r), r_ref)
    assert_bitexact(cpu(r_in), r_ref)
    y = bf_randn((nr, d), 32)
    h3.token_restore(w, xg, to_dev(y), r_in)
    assert_bitexact(cpu(xg), oracle.token_restore(w, x, y, r_ref))
