"""Seeded synthetic inputs for the MiniMax-H3 single-stream DiT block.

This module only draws random tensors and describes workload geometries; it holds
none of the block's arithmetic (no normalisation, projection, rotary, attention,
quantisation or token-reduction code).  Both the CPU oracle and the HIP path are
fed the very same bytes produced here.

Generator: Philox-4x32-10, the counter-based generator of Salmon, Moraes, Dror and
Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11), written out from its
published definition, followed by the Box-Muller transform in float64 and
round-to-nearest-even to float32 then bfloat16.  Every tensor is keyed by
(seed, block, tensor_id), so any block of a 50-block stack can be regenerated on
its own and on any device: the integer part is exact, so CPU and GPU agree on the
uniforms bit for bit.

Tensor ids: 0 residual x, 1 W_qkv, 2 W_o, 3 W_fc1, 4 W_fc2, 5 modulation vectors.
Distributions: weights N(0, 0.02^2), residual N(0, 1), modulation N(0, 0.1^2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

T_X, T_WQKV, T_WO, T_W1, T_W2, T_MOD = 0, 1, 2, 3, 4, 5
STD_W, STD_X, STD_MOD = 0.02, 1.0, 0.1


def _mulhilo32(m: int, c: torch.Tensor):
    """(hi, lo) 32-bit halves of m*c for a 32-bit constant m and int64 tensor c < 2^32.

    The product can exceed 2^63, so it is formed from 16-bit halves of c:
    m*c = X*2^16 + Y with X = m*(c>>16) and Y = m*(c & 0xFFFF), both < 2^48.
    """
    x = m * (c >> 16)
    y = m * (c & 0xFFFF)
    hi = (x + (y >> 16)) >> 16
    lo = (((x & 0xFFFF) << 16) + y) & MASK32
    return hi & MASK32, lo


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Ten Philox-4x32 rounds on int64 tensors holding 32-bit words."""
    for r in range(10):
        hi0, lo0 = _mulhilo32(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo32(PHILOX_M1, c2)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK32, lo1, (hi0 ^ c3 ^ k1) & MASK32, lo0
        if r < 9:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
    return c0, c1, c2, c3


def normal_bf16(seed: int, block: int, tensor_id: int, shape, std: float,
                device="cpu", chunk: int = 1 << 22) -> torch.Tensor:
    """bf16 tensor of the given shape, entries ~ N(0, std^2), keyed by (seed, block, tensor_id).

    Element e comes from counter (e//4 low word, e//4 high word, block, tensor_id),
    output word e%4; words (0,1) and (2,3) each feed one Box-Muller pair.
    """
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=torch.bfloat16, device=device)
    n_ctr = (numel + 3) // 4
    k0, k1 = seed & MASK32, (seed >> 32) & MASK32
    two_pi = 2.0 * math.pi
    for start in range(0, n_ctr, chunk):
        stop = min(n_ctr, start + chunk)
        i = torch.arange(start, stop, dtype=torch.int64, device=device)
        c0 = i & MASK32
        c1 = (i >> 32) & MASK32
        c2 = torch.full_like(i, block & MASK32)
        c3 = torch.full_like(i, tensor_id & MASK32)
        x0, x1, x2, x3 = philox4x32_10(c0, c1, c2, c3, k0, k1)
        scale = 2.0 ** -32
        zs = []
        for a, b in ((x0, x1), (x2, x3)):
            u1 = (a.to(torch.float64) + 1.0) * scale      # (0, 1]
            u2 = b.to(torch.float64) * scale              # [0, 1)
            rad = torch.sqrt(-2.0 * torch.log(u1))
            zs.append(rad * torch.cos(two_pi * u2))
            zs.append(rad * torch.sin(two_pi * u2))
        z = torch.stack(zs, dim=1).reshape(-1) * std
        e0 = start * 4
        e1 = min(numel, stop * 4)
        out[e0:e1] = z[: e1 - e0].to(torch.float32).to(torch.bfloat16)
    return out.reshape(tuple(int(s) for s in shape))


@dataclass(frozen=True)
class Workload:
    """Geometry of one workload: widths, token layout and optional token-reduction schedule."""
    name: str
    hidden: int
    heads: int
    head_dim: int
    mlp: int
    video_t: int
    video_h: int
    video_w: int
    n_text: int
    n_audio: int
    blocks: int = 1
    precision: str = "bf16"
    reduce_after: int = -1
    restore_before: int = -1
    fc2_group: int = 1024
    mod_sets: int = 1          # modulation sets: 1 for all tokens, or 3 (video, text, audio)
    ln_eps: float = 1e-6
    rope_theta: float = 10000.0
    rope_split: tuple = field(default=None)

    @property
    def n_video(self) -> int:
        return self.video_t * self.video_h * self.video_w

    @property
    def n_tokens(self) -> int:
        return self.n_video + self.n_text + self.n_audio

    @property
    def split(self) -> tuple:
        if self.rope_split is not None:
            return tuple(self.rope_split)
        # head dim shared by the time/height/width axes as 1/4, 3/8, 3/8 (16/24/24 at 64)
        q = self.head_dim // 8
        return (2 * q, 3 * q, 3 * q)

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads: a tiny CPU-checkable block, one production-width block in
# bf16 and in int8, the 50-block bf16 stack at 4096 tokens, and the 50-block int8
# stack at 8192 tokens with horizontal token pairing after block 3 / restore before 40.
WORKLOADS = {
    0: Workload("tiny-block", 256, 4, 64, 1024, 3, 8, 8, 48, 16),
    1: Workload("block-2048-bf16", 5120, 40, 128, 20480, 5, 16, 22, 256, 32),
    2: Workload("block-2048-int8", 5120, 40, 128, 20480, 5, 16, 22, 256, 32, precision="int8"),
    3: Workload("stack50-4096-bf16", 5120, 40, 128, 20480, 5, 22, 32, 512, 64, blocks=50),
    4: Workload("stack50-8192-int8-tokred", 5120, 40, 128, 20480, 8, 16, 59, 576, 64, blocks=50,
                precision="int8", reduce_after=3, restore_before=40),
}


def seed_for(config: int) -> int:
    return 1000 + int(config)


def make_x(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    """Residual stream [n_tokens][hidden] bf16, N(0, 1)."""
    return normal_bf16(seed, 0, T_X, (w.n_tokens, w.hidden), STD_X, device)


def make_block(w: Workload, seed: int, block: int, device="cpu") -> dict:
    """bf16 weights of one block, [out][in] row-major, plus the 6 modulation rows
    (shift1, scale1, gate1, shift2, scale2, gate2) per modulation set."""
    d, f = w.hidden, w.mlp
    return {
        "wqkv": normal_bf16(seed, block, T_WQKV, (3 * d, d), STD_W, device),
        "wo": normal_bf16(seed, block, T_WO, (d, d), STD_W, device),
        "w1": normal_bf16(seed, block, T_W1, (f, d), STD_W, device),
        "w2": normal_bf16(seed, block, T_W2, (d, f), STD_W, device),
        "mod": normal_bf16(seed, block, T_MOD, (6 * w.mod_sets, d), STD_MOD, device),
    }
