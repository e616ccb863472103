"""Comparison helpers shared by the GPU parity tests (no arithmetic of the block itself).

Tolerances (stated once, used everywhere): tensors rounded to bf16 are compared by the
relative max-norm error ||gpu - ref||_inf / ||ref||_inf <= 2e-2; fp32 accumulators and
softmax statistics by the same norm <= 1e-3; int8 codes, int32 accumulators and every
stage whose arithmetic is fully ordered are compared bit for bit."""
import torch

BF16_TOL = 2e-2
F32_TOL = 1e-3


def relerr(g, r) -> float:
    g = g.detach().to("cpu", torch.float64)
    r = r.detach().to("cpu", torch.float64)
    den = float(r.abs().max())
    return float((g - r).abs().max()) / (den if den > 0 else 1.0)


def bits(t):
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def assert_bitexact(g, r, what=""):
    gb, rb = bits(g), bits(r)
    assert gb.shape == rb.shape, (what, gb.shape, rb.shape)
    ne = (gb != rb)
    n = int(ne.sum())
    assert n == 0, f"{what}: {n} of {gb.numel()} elements differ; first at {ne.nonzero()[:4].tolist()}"


def ulp_max(g, r) -> int:
    a = bits(g).to(torch.int32)
    b = bits(r).to(torch.int32)
    a = torch.where(a < 0, -(a & 0x7FFF), a)
    b = torch.where(b < 0, -(b & 0x7FFF), b)
    return int((a - b).abs().max()) if a.numel() else 0


def sample_rows(n: int, k: int, seed: int = 0):
    """k distinct row indices of [0, n), always including the first and the last."""
    g = torch.Generator().manual_seed(seed)
    idx = torch.randperm(n, generator=g)[: max(0, k - 2)]
    idx = torch.unique(torch.cat([idx, torch.tensor([0, n - 1])]))
    return idx.sort().values


def assert_close_bf16(g, r, what="", max_frac_diff=0.02):
    """bf16 tensors from fp32 work done in another order: the spec bar (max-norm
    relative error <= 2e-2), at most `max_frac_diff` of the elements not bit-identical, and
    away from zero (|ref| above 1% of the max) at most one bf16 step apart."""
    assert relerr(g, r) <= BF16_TOL, (what, relerr(g, r))
    gb, rb = bits(g), bits(r)
    frac = float((gb != rb).double().mean()) if gb.numel() else 0.0
    assert frac <= max_frac_diff, (what, frac)
    rf = r.detach().to("cpu", torch.float64)
    big = rf.abs() > 0.01 * float(rf.abs().max())
    assert ulp_max(g.detach().to("cpu")[big], r.detach().to("cpu")[big]) <= 1, what


def bf16_ulp(r):
    """Spacing of bf16 numbers at |r| (float64 tensor): 2^(e - 7) for |r| in [2^e, 2^(e+1))."""
    a = r.abs().clamp_min(2.0 ** -126)
    return torch.exp2(torch.floor(torch.log2(a)) - 7)


def update_stats(out, ref, x):
    """Errors of a block or stack output judged on its update out - x (x is the input residual):
    (residual max-norm relative error, largest per-element error in units of
    (one bf16 step of |ref| + 2e-2 * max|ref - x|), largest per-row ratio of the mean update
    error to the row's mean |ref - x|)."""
    o = out.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    x0 = x.detach().to("cpu", torch.float64)
    dr = r - x0
    err = (o - r).abs()
    scale = float(dr.abs().max())
    elem = float((err / (bf16_ulp(r) + BF16_TOL * scale)).max()) if err.numel() else 0.0
    row_err = err.mean(dim=1)
    row_upd = dr.abs().mean(dim=1)
    row = float((row_err / row_upd.clamp_min(1e-30)).max()) if err.numel() else 0.0
    if bool(((row_upd == 0) & (row_err > 0)).any()):
        row = float("inf")
    return relerr(out, ref), elem, row


def assert_update_close(out, ref, x, what="", ulps=2.0, row_frac=0.1):
    """The bf16 bar on the output, and its update out - x checked element by element and row by
    row, so that one wrong token row, a ragged tail or one modulation segment fails even where
    the update is small next to x:
      - every element within `ulps` bf16 steps of |ref| plus 2e-2 of the update's max-norm (the
        output is bf16(x + update): a rounding-sized change of the update moves it by a step);
      - every row's mean |update error| within `row_frac` of that row's mean |update|."""
    res, elem, row = update_stats(out, ref, x)
    assert res <= BF16_TOL, (what, "residual", res)
    assert elem <= ulps, (what, "element", elem)
    assert row <= row_frac, (what, "row", row)
    return res, elem, row
