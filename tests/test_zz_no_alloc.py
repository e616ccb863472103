"""The allocation-free final head (h3dit_final_head_noalloc, row statistics in the library's
static device array) against h3dit_final_head with a caller workspace, through the C ABI: two
calls in a row, the second on a smaller input, each byte-identical to the workspace form;
and a part larger than the array's 65536 rows rejected before any launch."""
import ctypes as C

import pytest
import torch

import synth
from synth import WORKLOADS
from parity import assert_bitexact

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("audio_diffusion_transformer_dit_amd")
DEV = "cuda"


def _parts(w, seed, cv=128, ca=256):
    g = torch.Generator().manual_seed(seed)
    d = w.hidden
    mv = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    ma = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    wv = (torch.randn(cv, d, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    wa = (torch.randn(ca, d, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    return (mv, wv), (ma, wa)


def test_final_head_noalloc_equals_workspace_form_twice():
    big = WORKLOADS[3].replace(blocks=1)                     # 3520 video + 64 audio rows, d 5120
    small = WORKLOADS[0]                                     # 192 video + 16 audio rows, d 256
    for w, seed in ((big, 1), (small, 2)):
        x = synth.make_x(w, 1030 + seed, DEV)
        video, audio = _parts(w, seed)
        ref_v, ref_a = h3.final_head(w, x, video=video, audio=audio)
        got_v, got_a = h3.final_head_noalloc(w, x, video=video, audio=audio)
        torch.cuda.synchronize()
        assert_bitexact(got_v.cpu(), ref_v.cpu(), f"video rows, d={w.hidden}")
        assert_bitexact(got_a.cpu(), ref_a.cpu(), f"audio rows, d={w.hidden}")
        # one part alone
        only_a, = h3.final_head_noalloc(w, x, audio=audio)[1:]
        torch.cuda.synchronize()
        assert_bitexact(only_a.cpu(), ref_a.cpu(), "audio part alone")


def test_final_head_noalloc_rejects_parts_past_the_array():
    w = WORKLOADS[0].replace(video_t=1, video_h=257, video_w=256, n_text=0, n_audio=0)   # 65792 video rows
    assert w.n_tokens > 65536
    video, _ = _parts(w, 3)
    size = C.c_size_t(0)
    part = h3.HeadPart(video[0].data_ptr(), video[1].data_ptr(), 128)
    rc = h3.lib().h3dit_final_head_noalloc(C.byref(h3.dims_of(w)), C.byref(h3.layout_of(w)), C.byref(part), None,
                                           1 << 20, 1 << 20, None, None)
    assert rc == h3.EWORKSPACE
