"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, invariants, exact special cases, brute force in float64 and library
routines (torch's bf16 rounding, layer_norm, scaled_dot_product_attention, tanh-GELU,
int64 matmul, complex multiplication).  Each test names the property it pins.

The pages (web articles on antirez's h3.c engine for MiniMax-H3) print no worked example
or intermediate value, so no golden tensor from them exists; tests/golden/ holds the
small hand-derived cases used here, each with its derivation."""
import json
import math
import os

import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
W0 = WORKLOADS[0]


def bf(x):
    return x.to(torch.float32).to(torch.bfloat16)


def ulp_diff(a, b):
    """Distance in bf16 units of last place between two bf16 tensors of one sign pattern."""
    ai = a.view(torch.int16).to(torch.int32)
    bi = b.view(torch.int16).to(torch.int32)
    ai = torch.where(ai < 0, -(ai & 0x7FFF), ai)
    bi = torch.where(bi < 0, -(bi & 0x7FFF), bi)
    return (ai - bi).abs()


def relerr(g, r):
    g = g.to(torch.float64)
    r = r.to(torch.float64)
    return float((g - r).abs().max() / r.abs().max().clamp_min(1e-30))


# ----------------------------------------------------------------------------- generator

def test_philox_known_answer():
    # Philox-4x32-10, counter (0,0,0,0), key (0,0): Random123 known-answer vector.
    z = torch.zeros(1, dtype=torch.int64)
    out = synth.philox4x32_10(z, z, z, z, 0, 0)
    assert [int(o) for o in out] == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]


def test_generator_deterministic_and_normal():
    a = synth.normal_bf16(7, 3, 1, (300, 200), 0.02)
    b = synth.normal_bf16(7, 3, 1, (300, 200), 0.02)
    c = synth.normal_bf16(7, 4, 1, (300, 200), 0.02)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    x = a.to(torch.float64)
    assert abs(float(x.mean())) < 0.02 * 0.02
    assert abs(float(x.std()) - 0.02) < 0.02 * 0.02


# ----------------------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch_rne():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 4)
    ties = (torch.arange(4096, dtype=torch.int32) * 65536 + 0x3F800000 + 0x8000).view(torch.float32)
    x = torch.cat([x, ties, -ties, torch.tensor([0.0, -0.0, 1e-40, 3.0e38])])
    got = oracle.f32_to_bf16(x)
    assert torch.equal(got.view(torch.int16), x.to(torch.bfloat16).view(torch.int16))


# ----------------------------------------------------------------------------- GELU

def test_gelu_tanh_closed_forms_and_library():
    assert oracle.gelu_tanh(0.0) == 0.0
    xs = torch.linspace(-8, 8, 2001, dtype=torch.float64)
    ours = torch.tensor([oracle.gelu_tanh(float(v)) for v in xs], dtype=torch.float64)
    ref = F.gelu(xs, approximate="tanh")
    assert float((ours - ref).abs().max()) < 4e-6 * 8
    neg = torch.tensor([oracle.gelu_tanh(-float(v)) for v in xs], dtype=torch.float64)
    # gelu(x) - gelu(-x) = x
    assert float((ours - neg - xs).abs().max()) < 1e-5
    # large |x|: gelu -> x for x >> 0, -> 0 for x << 0
    assert oracle.gelu_tanh(10.0) == 10.0 and abs(oracle.gelu_tanh(-10.0)) < 1e-30
    # accurate in the negative tail too, where 1 + tanh(z) cancels: against the float64
    # library down to u = -4 (its 1 + tanh(z) keeps > 35 bits there) ...
    tail = torch.linspace(-4, -2, 401, dtype=torch.float32).to(torch.float64)
    ot = torch.tensor([oracle.gelu_tanh(float(v)) for v in tail], dtype=torch.float64)
    rt = F.gelu(tail, approximate="tanh")
    assert torch.all((ot - rt).abs() <= rt.abs() * 2.0 ** -22)
    # ... and below it against the series gelu(u) = u (e^(2z) - e^(4z) + O(e^(6z))), e^(4z) < 2^-30
    deep = torch.linspace(-12, -4, 801, dtype=torch.float32).to(torch.float64)
    od = torch.tensor([oracle.gelu_tanh(float(v)) for v in deep], dtype=torch.float64)
    z = math.sqrt(2 / math.pi) * (deep + 0.044715 * deep ** 3)
    ra = deep * (torch.exp(2 * z) - torch.exp(4 * z))
    keep = ra.abs() > 1e-37  # normal fp32 range
    assert torch.all((od - ra).abs()[keep] <= ra.abs()[keep] * 2.0 ** -22)


def test_gelu_rows_rounding():
    g = torch.Generator().manual_seed(11)
    u = bf(torch.randn(4096, generator=g, dtype=torch.float64) * 3)
    u = torch.cat([u, bf(torch.tensor([-9.5, -10.0, -11.0, -12.0], dtype=torch.float64))])
    got = oracle.gelu_rows(u)
    u64 = u.to(torch.float64)
    ref64 = F.gelu(u64, approximate="tanh")
    z = math.sqrt(2 / math.pi) * (u64 + 0.044715 * u64 ** 3)
    series = u64 * (torch.exp(2 * z) - torch.exp(4 * z))
    ref64 = torch.where(u64 < -4, series, ref64)  # the library's 1 + tanh(z) cancels below -4
    # fp64 evaluation rounded to fp32 then bf16: at most one bf16 step from the float64 value
    tiny = ref64.abs() < 1e-37
    assert int(ulp_diff(got[~tiny], bf(ref64)[~tiny]).max()) <= 1
    assert float(got[tiny].to(torch.float64).abs().max()) < 1e-37


# ----------------------------------------------------------------------------- AdaLN

def test_adaln_zero_modulation_is_layernorm():
    g = torch.Generator().manual_seed(1)
    x = bf(torch.randn(64, 256, generator=g) * 3 + 0.5)
    z = torch.zeros(256, dtype=torch.bfloat16)
    h, mean, rstd = oracle.adaln(x, z, z, 1e-6, stats=True)
    ref = F.layer_norm(x.to(torch.float64), (256,), eps=1e-6)
    assert int(ulp_diff(h, bf(ref)).max()) <= 1
    x64 = x.to(torch.float64)
    assert float((mean.to(torch.float64) - x64.mean(1)).abs().max()) < 1e-5
    var = x64.var(1, unbiased=False)
    assert float((rstd.to(torch.float64) - 1 / torch.sqrt(var + 1e-6)).abs().max() / rstd.max()) < 1e-5
    # normalised output: mean 0, variance v / (v + eps)
    hf = h.to(torch.float64)
    assert float(hf.mean(1).abs().max()) < 2e-2
    assert float((hf.var(1, unbiased=False) - var / (var + 1e-6)).abs().max()) < 2e-2


def test_adaln_modulation_form():
    g = torch.Generator().manual_seed(2)
    x = bf(torch.randn(32, 512, generator=g))
    sh = bf(torch.randn(512, generator=g) * 0.1)
    sc = bf(torch.randn(512, generator=g) * 0.1)
    h = oracle.adaln(x, sh, sc)
    ln = F.layer_norm(x.to(torch.float64), (512,), eps=1e-6)
    ref = bf(ln * (1 + sc.to(torch.float64)) + sh.to(torch.float64))
    assert int(ulp_diff(h, ref).max()) <= 1
    # scale = -1 cancels the normalised part: output is the shift
    h2 = oracle.adaln(x, sh, torch.full((512,), -1.0, dtype=torch.bfloat16))
    assert torch.equal(h2.view(torch.int16), sh.expand(32, 512).contiguous().view(torch.int16))


def test_adaln_constant_row_is_shift():
    x = torch.full((4, 5120), 1.375, dtype=torch.bfloat16)
    sh = bf(torch.linspace(-1, 1, 5120))
    h = oracle.adaln(x, sh, bf(torch.randn(5120)))
    assert torch.equal(h.view(torch.int16), sh.expand(4, 5120).contiguous().view(torch.int16))


# ----------------------------------------------------------------------------- int8 codes

def test_q8_worked_cases():
    with open(os.path.join(GOLDEN, "q8_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        v = torch.tensor([c["values"]], dtype=torch.float32).to(torch.bfloat16)
        q, s = oracle.q8_rows(v)
        assert q[0].tolist() == c["codes"], c["note"]
        assert float(s[0, 0]) == float(torch.tensor(c["scale"], dtype=torch.float32)), c["note"]


def test_q8_properties():
    g = torch.Generator().manual_seed(3)
    v = bf(torch.randn(200, 2048, generator=g) * torch.exp(torch.randn(200, 1, generator=g)))
    q, s = oracle.q8_rows(v, 1024)
    vf = v.to(torch.float64).view(200, 2, 1024)
    qf = q.to(torch.float64).view(200, 2, 1024)
    s64 = s.to(torch.float64).unsqueeze(-1)
    assert int(q.abs().max()) == 127
    assert torch.all(qf.abs().amax(-1) == 127)                      # absmax element maps to 127
    # rounding error <= s/2, up to the fp32 rounding of v/s (|v/s| <= 127)
    assert float(((vf - qf * s64).abs() - s64 * (0.5 + 127 * 2.0 ** -23)).max()) <= 0
    # scale is absmax / 127 in fp32
    am = v.to(torch.float32).view(200, 2, 1024).abs().amax(-1)
    assert torch.equal(s, am / 127.0)


def test_quantize_weights_is_per_row_q8():
    g = torch.Generator().manual_seed(4)
    w = bf(torch.randn(96, 320, generator=g) * 0.02)
    q, s = oracle.quantize_weights(w)
    q2, s2 = oracle.q8_rows(w)
    assert torch.equal(q, q2) and torch.equal(s, s2[:, 0])


# ----------------------------------------------------------------------------- projections

def test_gemm_i32_exact():
    g = torch.Generator().manual_seed(5)
    a = torch.randint(-127, 128, (33, 700), generator=g, dtype=torch.int8)
    w = torch.randint(-127, 128, (45, 700), generator=g, dtype=torch.int8)
    acc = oracle.gemm_i32(a, w)
    ref = a.to(torch.int64) @ w.to(torch.int64).T
    assert torch.equal(acc.to(torch.int64), ref)
    ones = torch.full((2, 20480), 127, dtype=torch.int8)
    assert int(oracle.gemm_i32(ones, ones)[0, 0]) == 20480 * 16129


def test_gemm_f32_against_float64():
    g = torch.Generator().manual_seed(6)
    a = bf(torch.randn(40, 1024, generator=g))
    w = bf(torch.randn(72, 1024, generator=g) * 0.02)
    acc = oracle.gemm_f32(a, w)
    ref = a.to(torch.float64) @ w.to(torch.float64).T
    bound = 1024 * 2.0 ** -24 * (a.to(torch.float64).abs() @ w.to(torch.float64).abs().T)
    assert torch.all((acc.to(torch.float64) - ref).abs() <= bound)
    # small integers: every partial sum exact
    ai = bf(torch.randint(-8, 9, (5, 64), generator=g).to(torch.float32))
    wi = bf(torch.randint(-8, 9, (7, 64), generator=g).to(torch.float32))
    assert torch.equal(oracle.gemm_f32(ai, wi), (ai.to(torch.float64) @ wi.to(torch.float64).T).to(torch.float32))
    # operand orientation: W is [out][in]
    e = torch.zeros(3, 64, dtype=torch.bfloat16)
    e[1, 5] = 1
    assert torch.equal(oracle.gemm_f32(ai, e)[:, 1], ai[:, 5].to(torch.float32))


def test_dequant_order():
    acc = torch.tensor([[123456789, -7]], dtype=torch.int32)
    sa = torch.tensor([0.01], dtype=torch.float32)
    sw = torch.tensor([0.003, 2.0], dtype=torch.float32)
    out = oracle.dequant_bf16(acc, sa, sw)
    ref = bf((acc.to(torch.float32) * sa[:, None]) * sw[None, :])
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_fc2_single_group_equals_per_token():
    g = torch.Generator().manual_seed(7)
    qa = torch.randint(-127, 128, (16, 1024), generator=g, dtype=torch.int8)
    sa = torch.rand(16, 1, generator=g) * 0.01
    qw = torch.randint(-127, 128, (40, 1024), generator=g, dtype=torch.int8)
    sw = torch.rand(40, generator=g) * 0.001
    y = oracle.fc2_int8(qa, sa, qw, sw, 1024)
    ref = oracle.dequant_bf16(oracle.gemm_i32(qa, qw), sa[:, 0], sw)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_fc2_groups_against_int64():
    g = torch.Generator().manual_seed(8)
    qa = torch.randint(-127, 128, (8, 4096), generator=g, dtype=torch.int8)
    sa = torch.rand(8, 4, generator=g) * 0.01
    qw = torch.randint(-127, 128, (24, 4096), generator=g, dtype=torch.int8)
    sw = torch.rand(24, generator=g) * 0.001
    y = oracle.fc2_int8(qa, sa, qw, sw, 1024)
    acc = torch.einsum("mgk,ngk->mng", qa.view(8, 4, 1024).to(torch.int64), qw.view(24, 4, 1024).to(torch.int64))
    ref = (acc.to(torch.float64) * sa.to(torch.float64)[:, None, :]).sum(-1) * sw.to(torch.float64)
    assert relerr(y, ref) < 8e-3
    # equal group scales: per-token result up to fp32 summation order
    sa_eq = sa[:, :1].expand(8, 4).contiguous()
    y_eq = oracle.fc2_int8(qa, sa_eq, qw, sw, 1024)
    ref_eq = oracle.dequant_bf16(oracle.gemm_i32(qa, qw), sa_eq[:, 0].contiguous(), sw)
    assert int(ulp_diff(y_eq, ref_eq).max()) <= 1


# ----------------------------------------------------------------------------- rotary

def test_rope_tables_closed_forms():
    w = W0
    cos, sin = oracle.rope_tables(w)
    N, half = cos.shape
    assert N == w.n_tokens and half == w.head_dim // 2
    # token (0,0,0) and the first text/audio tokens sit at position 0: identity rotation
    for n in (0, w.n_video, w.n_video + w.n_text):
        assert torch.all(cos[n] == 1) and torch.all(sin[n] == 0)
    assert torch.allclose(cos * cos + sin * sin, torch.ones_like(cos), atol=1e-6)
    st, sh, sw = w.split
    # video token (t,h,w): time pairs depend only on t, height pairs on h, width pairs on w
    def tok(t, h, x):
        return (t * w.video_h + h) * w.video_w + x
    a, b = tok(2, 5, 3), tok(2, 1, 7)
    assert torch.equal(cos[a, : st // 2], cos[b, : st // 2])
    assert not torch.equal(cos[a, st // 2:], cos[b, st // 2:])
    # the first pair of each section turns by exactly the position (frequency theta^0 = 1)
    assert abs(float(cos[a, 0]) - math.cos(2)) < 1e-7
    assert abs(float(cos[a, st // 2]) - math.cos(5)) < 1e-7
    assert abs(float(cos[a, (st + sh) // 2]) - math.cos(3)) < 1e-7
    # last pair of the width section: frequency theta^(-2(sw/2-1)/sw)
    f = 10000.0 ** (-2 * (sw // 2 - 1) / sw)
    assert abs(float(sin[a, half - 1]) - math.sin(3 * f)) < 1e-7
    # text token at index p: 1-D rotary over the whole head dim
    p = 7
    n = w.n_video + p
    j = torch.arange(half, dtype=torch.float64)
    assert torch.allclose(cos[n].to(torch.float64), torch.cos(p * 10000.0 ** (-2 * j / w.head_dim)), atol=1e-7)


def test_rope_relative_position_property():
    # <R(m) q, R(n) k> depends only on m - n, per axis (checked in float64 with the tables)
    w = W0.replace(video_w=16)
    cos, sin = oracle.rope_tables(w)
    g = torch.Generator().manual_seed(9)
    q = torch.randn(w.head_dim // 2, dtype=torch.complex128, generator=g)
    k = torch.randn(w.head_dim // 2, dtype=torch.complex128, generator=g)
    rot = torch.complex(cos.to(torch.float64), sin.to(torch.float64))

    def tok(t, h, x):
        return (t * w.video_h + h) * w.video_w + x

    def score(m, n):
        return float(((q * rot[m]) * torch.conj(k * rot[n])).real.sum())

    assert abs(score(tok(1, 2, 3), tok(0, 1, 1)) - score(tok(2, 3, 5), tok(1, 2, 3))) < 1e-5
    assert abs(score(tok(1, 2, 3), tok(0, 1, 1)) - score(tok(1, 2, 4), tok(0, 1, 1))) > 1e-3


def test_rope_reduced_positions_are_midpoints():
    w = WORKLOADS[4].replace(video_t=2, video_h=3, video_w=7, n_text=5, n_audio=3,
                             hidden=256, heads=4, head_dim=64, mlp=1024)
    cf, sf = oracle.rope_tables(w, reduced=False)
    cr, sr = oracle.rope_tables(w, reduced=True)
    assert cr.shape[0] == 2 * 3 * 4 + 8
    # pair token (t,h,k) lies between (t,h,2k) and (t,h,2k+1): rotations compose so that
    # R(mid)^2 = R(2k) R(2k+1) (angles add), per pair of the head dim
    full = torch.complex(cf.to(torch.float64), sf.to(torch.float64))
    red = torch.complex(cr.to(torch.float64), sr.to(torch.float64))
    for t in range(2):
        for h in range(3):
            for kk in range(3):
                a = full[(t * 3 + h) * 7 + 2 * kk]
                b = full[(t * 3 + h) * 7 + 2 * kk + 1]
                r = red[(t * 3 + h) * 4 + kk]
                assert torch.allclose(r * r, a * b, atol=1e-6)
            # unpaired last column keeps its rotation
            assert torch.allclose(red[(t * 3 + h) * 4 + 3], full[(t * 3 + h) * 7 + 6], atol=0)
    # text/audio unchanged
    assert torch.equal(cr[24:], cf[42:])


def test_rope_split_layout_and_sign():
    N, H, hd = 5, 3, 8
    d = H * hd
    g = torch.Generator().manual_seed(10)
    t = bf(torch.randn(N, 3 * d, generator=g))
    one = torch.ones(N, hd // 2)
    zero = torch.zeros(N, hd // 2)
    q, k, v = oracle.rope_split(t, one, zero, H, hd)
    tt = t.view(N, 3, H, hd).permute(1, 2, 0, 3)
    assert torch.equal(q.view(torch.int16), tt[0].contiguous().view(torch.int16))
    assert torch.equal(k.view(torch.int16), tt[1].contiguous().view(torch.int16))
    assert torch.equal(v.view(torch.int16), tt[2].contiguous().view(torch.int16))
    # quarter turn: (a, b) -> (-b, a), as multiplication by i of a + ib
    q, k, _ = oracle.rope_split(t, zero, one, H, hd)
    z = torch.view_as_complex(tt[0].to(torch.float32).reshape(H, N, hd // 2, 2).contiguous()) * 1j
    assert torch.equal(q.to(torch.float32), torch.view_as_real(z).reshape(H, N, hd))
    # general angle against complex multiplication in float64
    ang = torch.rand(N, hd // 2, generator=g) * 6.28
    c, s = torch.cos(ang), torch.sin(ang)
    q, k, _ = oracle.rope_split(t, c, s, H, hd)
    zq = torch.view_as_complex(tt[1].to(torch.float64).reshape(H, N, hd // 2, 2).contiguous())
    rk = torch.view_as_real(zq * torch.complex(c.to(torch.float64), s.to(torch.float64))).reshape(H, N, hd)
    assert int(ulp_diff(k, bf(rk)).max()) <= 1


# ----------------------------------------------------------------------------- attention

def test_attention_single_token_and_constant_values():
    g = torch.Generator().manual_seed(11)
    q = bf(torch.randn(2, 1, 64, generator=g))
    k = bf(torch.randn(2, 1, 64, generator=g))
    v = bf(torch.randn(2, 1, 64, generator=g))
    assert torch.equal(oracle.attention(q, k, v).view(torch.int16), v.view(torch.int16))  # N = 1
    q = bf(torch.randn(2, 50, 128, generator=g) * 3)
    k = bf(torch.randn(2, 50, 128, generator=g) * 3)
    ones = torch.ones(2, 50, 128, dtype=torch.bfloat16)
    assert torch.all(oracle.attention(q, k, ones).to(torch.float32) == 1.0)  # rows sum to 1
    # identical keys: uniform weights, output = mean of V
    kk = k[:, :1].expand(2, 50, 128).contiguous()
    v = bf(torch.randn(2, 50, 128, generator=g))
    o = oracle.attention(q, kk, v)
    assert int(ulp_diff(o, bf(v.to(torch.float64).mean(1, keepdim=True).expand_as(v))).max()) <= 1


@pytest.mark.parametrize("N,hd", [(7, 64), (64, 128), (33, 128)])
def test_attention_brute_force_float64(N, hd):
    g = torch.Generator().manual_seed(N + hd)
    q = bf(torch.randn(3, N, hd, generator=g) * 2)
    k = bf(torch.randn(3, N, hd, generator=g) * 2)
    v = bf(torch.randn(3, N, hd, generator=g))
    o, mx, sm = oracle.attention(q, k, v, stats=True)
    q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
    ref = F.scaled_dot_product_attention(q64, k64, v64)
    assert int(ulp_diff(o, bf(ref)).max()) <= 1
    s = (q64 @ k64.transpose(1, 2)) / math.sqrt(hd)
    assert torch.allclose(mx.to(torch.float64), s.amax(-1), rtol=1e-5, atol=1e-5)
    p = torch.exp(s - s.amax(-1, keepdim=True)).sum(-1)
    assert torch.allclose(sm.to(torch.float64), p, rtol=1e-5)
    # one-hot values read the probabilities out: column j of O is P[:, j]
    eye = torch.zeros(3, N, hd, dtype=torch.bfloat16)
    for j in range(min(N, hd)):
        eye[:, j, j] = 1
    P = torch.softmax(s, -1)
    o1 = oracle.attention(q, k, eye)
    assert int(ulp_diff(o1[:, :, : min(N, hd)], bf(P[:, :, : min(N, hd)])).max()) <= 1


# ----------------------------------------------------------------------------- gate

def test_gate_closed_forms():
    g = torch.Generator().manual_seed(12)
    x = bf(torch.randn(8, 256, generator=g))
    y = bf(torch.randn(8, 256, generator=g))
    zero = torch.zeros(256, dtype=torch.bfloat16)
    assert torch.equal(oracle.gate(x, zero, y).view(torch.int16), x.view(torch.int16))
    one = torch.ones(256, dtype=torch.bfloat16)
    assert torch.all(oracle.gate(x, one, bf(-x.to(torch.float32))).to(torch.float32) == 0)
    gg = bf(torch.randn(256, generator=g) * 0.1)
    ref = bf(x.to(torch.float64) + gg.to(torch.float64) * y.to(torch.float64))
    assert torch.equal(oracle.gate(x, gg, y).view(torch.int16), ref.view(torch.int16))


# ----------------------------------------------------------------------------- token reduction

def _small_tr(video_w):
    return WORKLOADS[4].replace(video_t=2, video_h=3, video_w=video_w, n_text=5, n_audio=3,
                                hidden=256, heads=4, head_dim=64, mlp=1024)


@pytest.mark.parametrize("video_w", [6, 7])
def test_token_pair_and_restore(video_w):
    w = _small_tr(video_w)
    g = torch.Generator().manual_seed(13)
    x = bf(torch.randn(w.n_tokens, 256, generator=g))
    r = oracle.token_pair(w, x)
    wr = video_w // 2 + video_w % 2
    assert r.shape[0] == 6 * wr + 8
    xv = x[: w.n_video].view(6, video_w, 256).to(torch.float64)
    rv = r[: 6 * wr].view(6, wr, 256)
    mean = bf((xv[:, 0: 2 * (video_w // 2): 2] + xv[:, 1: 2 * (video_w // 2): 2]) / 2)
    assert torch.equal(rv[:, : video_w // 2].contiguous().view(torch.int16), mean.view(torch.int16))
    if video_w % 2:
        assert torch.equal(rv[:, -1].view(torch.int16), x[: w.n_video].view(6, video_w, 256)[:, -1].view(torch.int16))
    assert torch.equal(r[6 * wr:].view(torch.int16), x[w.n_video:].view(torch.int16))
    # restore with an unchanged reduced residual is the identity on every token
    back = oracle.token_restore(w, x, r, r)
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))
    # restore = bypass + (pair update); unpaired, text and audio take the new value
    y = bf(r.to(torch.float32) + torch.randn(r.shape, generator=g) * 0.1)
    back = oracle.token_restore(w, x, y, r)
    upd = y.to(torch.float32) - r.to(torch.float32)
    for row in range(6):
        for c in range(video_w):
            i = row * video_w + c
            p = row * wr + min(c // 2, wr - 1)
            if c // 2 < video_w // 2:
                exp = bf(x[i].to(torch.float32) + upd[p])
            else:
                exp = y[p]
            assert torch.equal(back[i].view(torch.int16), exp.view(torch.int16))
    assert torch.equal(back[w.n_video:].view(torch.int16), y[6 * wr:].view(torch.int16))


# ----------------------------------------------------------------------------- whole block

def _tiny_inputs(seed=1000, w=W0):
    x = synth.make_x(w, seed)
    p = synth.make_block(w, seed, 0)
    return x, p


def _zero_gates(p):
    p = dict(p)
    mod = p["mod"].clone()
    mod[2] = 0
    mod[5] = 0
    p["mod"] = mod
    return p


@pytest.mark.parametrize("int8", [False, True])
def test_block_zero_gates_is_identity(int8):
    x, p = _tiny_inputs()
    p = _zero_gates(p)
    if int8:
        p = oracle.quantize_block(p)
    out = oracle.block_fwd(W0, p, x)
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("int8", [False, True])
def test_block_fused_equals_unfused(int8):
    x, p = _tiny_inputs()
    if int8:
        p = oracle.quantize_block(p)
    a = oracle.block_fwd(W0, p, x, fused=False)
    b = oracle.block_fwd(W0, p, x, fused=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), x.view(torch.int16))


def torch_block_float64(w, p, x, cos, sin):
    """The block from library routines in float64, rounded to bf16 at the same points:
    layer_norm, complex rotation, scaled_dot_product_attention, tanh-GELU, matmul."""
    N, d, H, hd = x.shape[0], w.hidden, w.heads, w.head_dim
    D = torch.float64
    mod = p["mod"].to(D)

    def adaln(v, sh, sc):
        return bf(F.layer_norm(v.to(D), (d,), eps=w.ln_eps) * (1 + sc) + sh)

    h1 = adaln(x, mod[0], mod[1])
    t = bf(h1.to(D) @ p["wqkv"].to(D).T)
    tq = t.view(N, 3, H, hd).permute(1, 2, 0, 3).to(D)
    rot = torch.complex(cos.to(D), sin.to(D))
    def rope(z):
        return bf(torch.view_as_real(torch.view_as_complex(z.reshape(H, N, hd // 2, 2).contiguous()) * rot).reshape(H, N, hd))
    q, k, v = rope(tq[0]), rope(tq[1]), bf(tq[2])
    o = bf(F.scaled_dot_product_attention(q.to(D), k.to(D), v.to(D)))
    ot = o.permute(1, 0, 2).reshape(N, d)
    y1 = bf(ot.to(D) @ p["wo"].to(D).T)
    x1 = bf(x.to(D) + mod[2] * y1.to(D))
    h2 = adaln(x1, mod[3], mod[4])
    u = bf(h2.to(D) @ p["w1"].to(D).T)
    gl = bf(F.gelu(u.to(D), approximate="tanh"))
    y2 = bf(gl.to(D) @ p["w2"].to(D).T)
    return bf(x1.to(D) + mod[5] * y2.to(D)), {"h1": h1, "q": q, "k": k, "v": v, "o": o, "y1": y1,
                                              "x1": x1, "h2": h2, "u": u, "gl": gl, "y2": y2}


def test_block_against_float64_library_composition():
    x, p = _tiny_inputs()
    cos, sin = oracle.rope_tables(W0)
    out, taps = oracle.block_fwd(W0, p, x, cos, sin, taps=True)
    ref, rt = torch_block_float64(W0, p, x, cos, sin)
    for name in ("h1", "q", "k", "v", "o", "y1", "x1", "h2", "u", "gl", "y2"):
        assert relerr(taps[name], rt[name]) < 2e-2, name
    assert relerr(out, ref) < 2e-2
    # the update itself (out - x) also agrees, not just the dominant residual
    assert relerr(out.to(torch.float64) - x.to(torch.float64), ref.to(torch.float64) - x.to(torch.float64)) < 3e-2


def test_int8_block_close_to_bf16_block():
    x, p = _tiny_inputs()
    # the int8 codes only perturb the projections: branch outputs stay within a few percent
    _, ta = oracle.block_fwd(W0, p, x, taps=True)
    _, tb = oracle.block_fwd(W0, oracle.quantize_block(p), x, taps=True)
    for name in ("t", "y1", "u", "y2"):
        assert relerr(tb[name], ta[name]) < 0.05, name


# ----------------------------------------------------------------------------- stack

def _stack_inputs(w, n_blocks, seed=1000):
    x = synth.make_x(w, seed)
    blocks = [synth.make_block(w, seed, b) for b in range(n_blocks)]
    return x, blocks


def test_stack_fused_equals_unfused_and_chains_blocks():
    w = W0
    x, blocks = _stack_inputs(w, 3)
    a = oracle.stack_fwd(w, blocks, x, fused=False)
    b = oracle.stack_fwd(w, blocks, x, fused=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    y = x
    for p in blocks:
        y = oracle.block_fwd(w, p, y)
    assert torch.equal(a.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("video_w", [6, 7])
def test_stack_reduction_with_identity_middle_is_identity(video_w):
    # gates 0 in the reduced span: pair then restore returns every token unchanged, so the
    # stack equals the unreduced stack whose middle blocks are skipped
    w = _small_tr(video_w)
    x, blocks = _stack_inputs(w, 5)
    for b in (2, 3):
        blocks[b] = _zero_gates(blocks[b])
    out = oracle.stack_fwd(w, blocks, x, reduce_after=1, restore_before=4, fused=True)
    ref = oracle.stack_fwd(w, [blocks[0], blocks[1], blocks[4]], x)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_stack_reduction_matches_stepwise():
    w = _small_tr(7)
    x, blocks = _stack_inputs(w, 4)
    out = oracle.stack_fwd(w, blocks, x, reduce_after=0, restore_before=3, fused=True)
    cr, sr = oracle.rope_tables(w, reduced=True)
    y = oracle.block_fwd(w, blocks[0], x)
    r = oracle.token_pair(w, y)
    z = oracle.block_fwd(w, blocks[1], r, cr, sr)
    z = oracle.block_fwd(w, blocks[2], z, cr, sr)
    y = oracle.token_restore(w, y, z, r)
    y = oracle.block_fwd(w, blocks[3], y)
    assert torch.equal(out.view(torch.int16), y.view(torch.int16))


# ----------------------------------------------------------------------------- modulation sets

def _three_sets(p, sets=None):
    """The block with modulation [3][6][d]: three copies of its one set, or the given sets."""
    q = dict(p)
    q["mod"] = p["mod"].repeat(3, 1).contiguous() if sets is None else sets
    return q


@pytest.mark.parametrize("int8", [False, True])
def test_three_equal_mod_sets_equal_one_set(int8):
    x, p = _tiny_inputs()
    q = _three_sets(p)
    if int8:
        p, q = oracle.quantize_block(p), oracle.quantize_block(q)
    w3 = W0.replace(mod_sets=3)
    for fused in (False, True):
        a = oracle.block_fwd(W0, p, x, fused=fused)
        b = oracle.block_fwd(w3, q, x, fused=fused)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mod_sets_select_token_segments():
    """Each segment takes its own set: gates of zero in the text set alone leave exactly the
    text rows unchanged; AdaLN1 of the audio rows uses the audio set's shift and scale."""
    w = W0.replace(mod_sets=3)
    x = synth.make_x(w, 1000)
    p = synth.make_block(w, 1000, 0)
    assert p["mod"].shape == (18, w.hidden)
    mod = p["mod"].clone()
    mod[6 + 2] = 0   # text gate1
    mod[6 + 5] = 0   # text gate2
    p["mod"] = mod
    out, taps = oracle.block_fwd(w, p, x, taps=True)
    nv, nt = w.n_video, w.n_text
    i16 = lambda t: t.view(torch.int16)
    assert torch.equal(i16(out[nv:nv + nt]), i16(x[nv:nv + nt]))
    assert not torch.equal(i16(out[:nv]), i16(x[:nv]))
    assert not torch.equal(i16(out[nv + nt:]), i16(x[nv + nt:]))
    ha = oracle.adaln(x[nv + nt:].contiguous(), mod[12], mod[13], w.ln_eps)
    hv = oracle.adaln(x[:nv].contiguous(), mod[0], mod[1], w.ln_eps)
    assert torch.equal(i16(taps["h1"][nv + nt:]), i16(ha))
    assert torch.equal(i16(taps["h1"][:nv]), i16(hv))


def test_mod_sets_in_a_reduced_stack():
    """Through pair and restore: three equal sets equal one set, and zero text gates in every
    block leave the text rows unchanged (the paired sequence keeps text and audio whole)."""
    w1 = _small_tr(7)
    w3 = w1.replace(mod_sets=3)
    x, blocks = _stack_inputs(w1, 4)
    b3 = [_three_sets(p) for p in blocks]
    a = oracle.stack_fwd(w1, blocks, x, reduce_after=0, restore_before=3, fused=True)
    b = oracle.stack_fwd(w3, b3, x, reduce_after=0, restore_before=3, fused=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for p in b3:
        mod = p["mod"].clone()
        mod[6 + 2] = 0
        mod[6 + 5] = 0
        p["mod"] = mod
    c = oracle.stack_fwd(w3, b3, x, reduce_after=0, restore_before=3, fused=True)
    nv, nt = w3.n_video, w3.n_text
    assert torch.equal(c[nv:nv + nt].view(torch.int16), x[nv:nv + nt].view(torch.int16))
    assert not torch.equal(c[:nv].view(torch.int16), x[:nv].view(torch.int16))


# ----------------------------------------------------------------------------- int8 MLP only

def test_int8_mlp_only_block():
    """FC1 and FC2 in int8, QKV and the output projection in bf16: every stage up to the MLP
    input is the bf16 block's, bytewise; FC1 is the int8 projection of that input."""
    x, p = _tiny_inputs()
    pm = oracle.quantize_block(p, mlp_only=True)
    assert "q1" in pm and "qqkv" not in pm
    _, ta = oracle.block_fwd(W0, p, x, taps=True)
    out, tm = oracle.block_fwd(W0, pm, x, taps=True)
    for name in ("h1", "t", "q", "k", "v", "o", "y1", "x1", "h2"):
        assert torch.equal(tm[name].view(torch.int16), ta[name].view(torch.int16)), name
    qa, sa = oracle.q8_rows(tm["h2"])
    u = oracle.dequant_bf16(oracle.gemm_i32(qa, pm["q1"]), sa[:, 0].contiguous(), pm["s1"])
    assert torch.equal(tm["u"].view(torch.int16), u.view(torch.int16))
    assert not torch.equal(tm["u"].view(torch.int16), ta["u"].view(torch.int16))
    # and the whole int8 block differs from it already in the attention branch
    _, t8 = oracle.block_fwd(W0, oracle.quantize_block(p), x, taps=True)
    assert not torch.equal(t8["t"].view(torch.int16), ta["t"].view(torch.int16))


# ----------------------------------------------------------------------------- final head

def test_final_head_identity_projection_is_layernorm():
    """shift = scale = 0 and W = I: the head returns the rows' LayerNorm (<= 1 bf16 step),
    the video rows from the front of the residual and the audio rows from its end."""
    w = W0
    d = w.hidden
    x = synth.make_x(w, 1000)
    zero = torch.zeros((2, d), dtype=torch.bfloat16)
    eye = torch.eye(d, dtype=torch.bfloat16)
    ov, oa = oracle.final_head(w, x, video=(zero, eye), audio=(zero, eye))
    nv = w.n_tokens - w.n_text - w.n_audio
    ref_v = bf(F.layer_norm(x[:nv].to(torch.float64), (d,), eps=w.ln_eps))
    ref_a = bf(F.layer_norm(x[-w.n_audio:].to(torch.float64), (d,), eps=w.ln_eps))
    assert int(ulp_diff(ov, ref_v).max()) <= 1
    assert int(ulp_diff(oa, ref_a).max()) <= 1


def test_final_head_orientation_and_modulation():
    """A one-hot W row picks one feature (W is [c][d]); a scale of -1 leaves only the shift;
    and the general case against a float64 composition of library routines."""
    w = W0
    d, c = w.hidden, 128
    x = synth.make_x(w, 1001)
    g = torch.Generator().manual_seed(7)
    mod = bf(torch.randn(2, d, generator=g, dtype=torch.float64) * 0.1)
    wt = torch.zeros((c, d), dtype=torch.bfloat16)
    wt[5, 17] = 1.0
    ov, _ = oracle.final_head(w, x, video=(mod, wt))
    nv = w.n_tokens - w.n_text - w.n_audio
    h = oracle.adaln(x[:nv].contiguous(), mod[0], mod[1], w.ln_eps)
    assert torch.equal(ov[:, 5].view(torch.int16), h[:, 17].view(torch.int16))
    assert float(ov[:, :5].abs().max()) == 0.0
    m2 = mod.clone()
    m2[1] = -1.0
    ov2, _ = oracle.final_head(w, x, video=(m2, wt))
    assert bool((ov2[:, 5] == m2[0, 17]).all())
    wt = bf(torch.randn(c, d, generator=g, dtype=torch.float64) * 0.02)
    _, oa = oracle.final_head(w, x, audio=(mod, wt))
    xa = x[-w.n_audio:].to(torch.float64)
    hh = bf(F.layer_norm(xa, (d,), eps=w.ln_eps) * (1 + mod[1].to(torch.float64)) + mod[0].to(torch.float64))
    ref = bf(hh.to(torch.float64) @ wt.to(torch.float64).T)
    assert relerr(oa, ref) < 2e-2


# ----------------------------------------------------------------------------- denoising loop

def test_denoise_plan_fresh_counts_are_the_pages():
    """20 steps at reuse 1 / 2 / 3 give 20 / 11 / 8 fresh denoiser evaluations, the counts the
    h3.c deep dive prints ("速度/质量预设矩阵"); the last step is always evaluated."""
    for r, n in ((1, 20), (2, 11), (3, 8)):
        plan = oracle.denoise_plan(20, reuse=r)
        assert sum(s["fresh"] for s in plan) == n
        assert sum(s["core"] for s in plan) == n
        assert plan[-1]["fresh"] == 1 and plan[0]["fresh"] == 1


def test_denoise_plan_token_restore_schedule():
    """Token reduction restores before block 40 in the first ten noise evaluations and before
    block 30 in the later ones ("Token 缩减"): at 20 fresh steps, ten of each."""
    plan = oracle.denoise_plan(20, reduce_after=3)
    assert [s["restore"] for s in plan] == [40] * 10 + [30] * 10
    # skipped steps use the latest evaluation; the schedule counts evaluations, not steps
    plan = oracle.denoise_plan(20, reuse=2, reduce_after=3)
    evals = [s["eval"] for s in plan]
    assert evals == [i // 2 for i in range(19)] + [10]
    assert [s["restore"] for s in plan] == [40] * 19 + [30]
    assert all(s["restore"] == -1 for s in oracle.denoise_plan(7))


def test_denoise_plan_rules_brute_force():
    """Against a direct enumeration: a step is evaluated iff it is a multiple of reuse or the
    last; with core reuse every step refreshes the head and the stack runs on multiples of
    core_reuse and the last step; reuse and core reuse together are rejected, as the pages
    state they are mutually exclusive; the 4-step budget at reuse 1 runs the model every step."""
    for steps in (1, 2, 3, 4, 7, 20, 50):
        for r in (1, 2, 3, 5):
            plan = oracle.denoise_plan(steps, reuse=r)
            fresh = [s["fresh"] for s in plan]
            assert fresh == [int(i % r == 0 or i == steps - 1) for i in range(steps)]
            last = -1
            for i, s in enumerate(plan):
                last += fresh[i]
                assert s["eval"] == last
        for c in (2, 4, 6):
            plan = oracle.denoise_plan(steps, core_reuse=c)
            assert all(s["fresh"] for s in plan)
            assert [s["core"] for s in plan] == [int(i % c == 0 or i == steps - 1) for i in range(steps)]
    assert all(s["core"] for s in oracle.denoise_plan(4, reuse=1))
    for bad in (dict(reuse=2, core_reuse=4), dict(reuse=0), dict(core_reuse=0), dict(reduce_after=3, restore_late=3)):
        with pytest.raises(ValueError):
            oracle.denoise_plan(20, **bad)


def test_velocity_step_rounding():
    """Hand-derived bf16 cases of z + dt*v: dt = 0 and v = 0 leave z; 1 + 2 * 0.5 = 2 exactly;
    1 + 2^-8 is a tie between 1 and 1 + 2^-7 and goes to the even 1; (1 + 2^-7) + 2^-8 is a
    tie that goes to the even 1 + 2^-6; and the general case against torch's float32
    arithmetic with its round-to-nearest-even bf16 conversion."""
    z = torch.tensor([1.0, 1.0, 1.0 + 2 ** -7, -3.0], dtype=torch.bfloat16)
    v = torch.tensor([2.0, 2 ** -8, 2 ** -8, 0.0], dtype=torch.bfloat16)
    out = oracle.velocity_step(z, v, 0.5)
    assert out.tolist() == [2.0, 1.0, 1.0 + 2 ** -7, -3.0]
    out = oracle.velocity_step(z, v, 1.0)
    assert out.tolist() == [3.0, 1.0, 1.0 + 2 ** -6, -3.0]
    g = torch.Generator().manual_seed(11)
    z = torch.randn(4096, generator=g).to(torch.bfloat16)
    v = torch.randn(4096, generator=g).to(torch.bfloat16)
    assert torch.equal(oracle.velocity_step(z, v, 0.0).view(torch.int16), z.view(torch.int16))
    for dt in (-0.05, 0.125, 1.0 / 3.0):
        prod = torch.tensor(dt, dtype=torch.float32) * v.to(torch.float32)
        ref = (z.to(torch.float32) + prod).to(torch.bfloat16)
        assert torch.equal(oracle.velocity_step(z, v, dt).view(torch.int16), ref.view(torch.int16))


def test_denoise_loop_is_euler_over_the_plan():
    """The oracle loop against its parts: with one fresh evaluation per step and a residual
    input that does not change, every evaluation gives the same velocity v, so the latents
    after the loop are the Euler steps of v; with reuse 3 over 4 steps the same holds (skipped
    steps repeat v); and with token reduction the early and late restore indices give
    velocities that differ."""
    w = W0
    d = w.hidden
    x = synth.make_x(w, 1007)
    blocks = [synth.make_block(w, 1007, b) for b in range(3)]
    g = torch.Generator().manual_seed(5)
    mv = bf(torch.randn(2, d, generator=g) * 0.1)
    wv = bf(torch.randn(128, d, generator=g) * 0.02)
    nv = w.n_tokens - w.n_text - w.n_audio
    z0 = bf(torch.randn(nv, 128, generator=g) * 0.01)
    dt = [-0.25] * 4
    zv, za = oracle.denoise(w, blocks, x, dict(steps=4, layers=2), dt, video=(mv, wv), z_video=z0)
    assert za is None
    v, _ = oracle.final_head(w, oracle.stack_fwd(w, blocks[:2], x, fused=True), video=(mv, wv))
    ref = z0
    for t in dt:
        ref = oracle.velocity_step(ref, v, t)
    assert torch.equal(zv.view(torch.int16), ref.view(torch.int16))
    zr, _ = oracle.denoise(w, blocks, x, dict(steps=4, reuse=3, layers=2), dt, video=(mv, wv), z_video=z0)
    assert torch.equal(zr.view(torch.int16), ref.view(torch.int16))
    opts = dict(steps=3, layers=3, reduce_after=0, restore_early=2, restore_late=1, early_evals=1)
    a, _ = oracle.denoise(w, blocks, x, opts, [-1.0, 0.0, 0.0], video=(mv, wv), z_video=z0)
    b, _ = oracle.denoise(w, blocks, x, opts, [0.0, 0.0, -1.0], video=(mv, wv), z_video=z0)
    assert not torch.equal(a.view(torch.int16), b.view(torch.int16))


# ----------------------------------------------------------------------------- int8 attention projections only

def _gate_zero(p, which):
    q = dict(p)
    mod = p["mod"].clone()
    mod[which] = 0
    q["mod"] = mod
    return q


def test_int8_attn_only_block():
    """QKV and the output projection in int8, FC1 and FC2 in bf16 (the int8-QKV-only path):
    its attention half is the full int8 block's, bytewise (both with gate2 = 0, whose output is
    x1 exactly, I1); its MLP half is the bf16 block's given the same x1 (a bf16 block with
    gate1 = 0 run from that x1), bytewise."""
    x, p = _tiny_inputs()
    pa = oracle.quantize_block(p, attn_only=True)
    assert "qqkv" in pa and "q1" not in pa
    out = oracle.block_fwd(W0, pa, x)
    x1_attn = oracle.block_fwd(W0, _gate_zero(pa, 5), x)
    x1_full = oracle.block_fwd(W0, _gate_zero(oracle.quantize_block(p), 5), x)
    assert torch.equal(x1_attn.view(torch.int16), x1_full.view(torch.int16))
    mlp_bf16 = oracle.block_fwd(W0, _gate_zero(p, 2), x1_attn)
    assert torch.equal(out.view(torch.int16), mlp_bf16.view(torch.int16))
    # and it is neither the bf16 block nor the full int8 block
    for other in (p, oracle.quantize_block(p)):
        assert not torch.equal(out.view(torch.int16), oracle.block_fwd(W0, other, x).view(torch.int16))


# ----------------------------------------------------------------------------- caller rotary tables

def _random_tables(n, hd, seed):
    g = torch.Generator().manual_seed(seed)
    ang = torch.rand(n, hd // 2, generator=g, dtype=torch.float64) * 2 * math.pi
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def test_stack_uses_caller_rotary_tables():
    """The stack with caller tables equals the blocks chained with those tables, bytewise (the
    block takes its tables as an input); the layout's own tables passed explicitly equal the
    default; other tables give another result; and the paired span uses the reduced tables
    (against the step-wise composition of block, pair, blocks, restore)."""
    w = _small_tr(7)
    x, blocks = _stack_inputs(w, 4)
    ct, st = _random_tables(w.n_tokens, w.head_dim, 1)
    a = oracle.stack_fwd(w, blocks[:2], x, fused=True, rope=(ct, st))
    y = x
    for p in blocks[:2]:
        y = oracle.block_fwd(w, p, y, ct, st)
    assert torch.equal(a.view(torch.int16), y.view(torch.int16))
    own = oracle.rope_tables(w)
    b = oracle.stack_fwd(w, blocks[:2], x, fused=True, rope=own)
    c = oracle.stack_fwd(w, blocks[:2], x, fused=True)
    assert torch.equal(b.view(torch.int16), c.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    cr, sr = _random_tables(oracle.layout_tokens(w, True), w.head_dim, 2)
    out = oracle.stack_fwd(w, blocks, x, reduce_after=0, restore_before=3, fused=True, rope=(ct, st),
                           rope_reduced=(cr, sr))
    y = oracle.block_fwd(w, blocks[0], x, ct, st)
    r = oracle.token_pair(w, y)
    z = oracle.block_fwd(w, blocks[1], r, cr, sr)
    z = oracle.block_fwd(w, blocks[2], z, cr, sr)
    y = oracle.token_restore(w, y, z, r)
    y = oracle.block_fwd(w, blocks[3], y, ct, st)
    assert torch.equal(out.view(torch.int16), y.view(torch.int16))


# ----------------------------------------------------------------------------- patch-embedding stand-in

def test_patch_embed_exact_cases():
    """bf16(x + bf16(z E^T)): with small-integer z and E every fp32 sum is exact, so the result
    equals the float64 composition bit for bit; E = 0 leaves x; a one-hot E row copies one
    latent channel into one feature (E is [d][c])."""
    g = torch.Generator().manual_seed(21)
    n, d, c = 37, 256, 128
    x = bf(torch.randn(n, d, generator=g, dtype=torch.float64))
    z = torch.randint(-4, 5, (n, c), generator=g).to(torch.bfloat16)
    E = torch.randint(-3, 4, (d, c), generator=g).to(torch.bfloat16)
    out = oracle.patch_embed(x, z, E)
    e = bf(z.to(torch.float64) @ E.to(torch.float64).T)
    ref = bf(x.to(torch.float64) + e.to(torch.float64))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    zero = torch.zeros((d, c), dtype=torch.bfloat16)
    assert torch.equal(oracle.patch_embed(x, z, zero).view(torch.int16), x.view(torch.int16))
    one = torch.zeros((d, c), dtype=torch.bfloat16)
    one[5, 3] = 1.0
    xz = torch.zeros((n, d), dtype=torch.bfloat16)
    got = oracle.patch_embed(xz, z, one)
    assert torch.equal(got[:, 5].view(torch.int16), z[:, 3].view(torch.int16))
    assert float(got[:, :5].abs().max()) == 0.0


def test_denoise_latents_feed_back_through_the_embedding():
    """With the embedding stand-in the loop is closed: E = 0 gives the loop without it, bytewise;
    otherwise each core evaluation starts from x_in plus the embedding of the latents of its own
    step (composition of the oracle's parts over a 3-step plan with reuse 2: steps 0 and 2
    evaluate, step 1 repeats the velocity of step 0)."""
    w = W0
    d = w.hidden
    x = synth.make_x(w, 1013)
    blocks = [synth.make_block(w, 1013, b) for b in range(2)]
    g = torch.Generator().manual_seed(6)
    mv = bf(torch.randn(2, d, generator=g) * 0.1)
    wv = bf(torch.randn(128, d, generator=g) * 0.02)
    ev = bf(torch.randn(d, 128, generator=g) * 0.2)
    nv = w.n_tokens - w.n_text - w.n_audio
    z0 = bf(torch.randn(nv, 128, generator=g))
    dt = [-0.3, -0.3, -0.4]
    opts = dict(steps=3, reuse=2, layers=2)
    plain, _ = oracle.denoise(w, blocks, x, opts, dt, video=(mv, wv), z_video=z0)
    zero, _ = oracle.denoise(w, blocks, x, opts, dt, video=(mv, wv), z_video=z0,
                             embed=(torch.zeros_like(ev), None))
    assert torch.equal(plain.view(torch.int16), zero.view(torch.int16))
    got, _ = oracle.denoise(w, blocks, x, opts, dt, video=(mv, wv), z_video=z0, embed=(ev, None))

    def velocity(z):
        xs = x.clone()
        xs[:nv] = oracle.patch_embed(x[:nv], z, ev)
        v, _ = oracle.final_head(w, oracle.stack_fwd(w, blocks, xs, fused=True), video=(mv, wv))
        return v

    v0 = velocity(z0)
    z1 = oracle.velocity_step(z0, v0, dt[0])
    z2 = oracle.velocity_step(z1, v0, dt[1])
    z3 = oracle.velocity_step(z2, velocity(z2), dt[2])
    assert torch.equal(got.view(torch.int16), z3.view(torch.int16))
    assert not torch.equal(got.view(torch.int16), plain.view(torch.int16))


# ----------------------------------------------------------------------------- the update check itself

def test_update_check_rejects_one_wrong_row():
    """The GPU tests judge a block's update (out - x) per element and per row: the oracle's own
    output passes, a one-step change of scattered elements passes, and one token row whose update
    is dropped, doubled or taken from another row fails (the residual max-norm alone accepts all
    of them, the update being small next to x)."""
    from parity import assert_update_close, update_stats
    x, p = _tiny_inputs()
    ref = oracle.block_fwd(W0, p, x)
    assert_update_close(ref, ref, x)
    nudged = ref.clone().view(torch.int16)
    nudged.view(-1)[::97] += 1                       # one bf16 step on 1% of the elements
    assert_update_close(nudged.view(torch.bfloat16), ref, x)
    for name, row_fn in (("dropped", lambda r: x[r]), ("doubled", lambda r: bf(2 * ref[r].double() - x[r].double())),
                         ("swapped", lambda r: bf(x[r].double() + ref[r + 1].double() - x[r + 1].double()))):
        bad = ref.clone()
        bad[200] = row_fn(200)
        res, elem, row = update_stats(bad, ref, x)
        assert res <= 2e-2, name                     # invisible on the residual
        with pytest.raises(AssertionError):
            assert_update_close(bad, ref, x, name)
