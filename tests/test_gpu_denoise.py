"""The denoising loop through the C ABI (h3dit_velocity_step, h3dit_denoise_fwd) against the
CPU oracle: the velocity step bit for bit; the loop over a plan with velocity reuse, core
reuse, layer skipping and the early / late token-restore schedule at the bf16 bar."""
import pytest
import torch

import oracle
import synth
from synth import WORKLOADS
from parity import BF16_TOL, assert_bitexact, relerr

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("audio_diffusion_transformer_dit_amd")
DEV = "cuda"

SMALL_TR = WORKLOADS[4].replace(video_t=2, video_h=3, video_w=7, n_text=9, n_audio=5, hidden=256, heads=4,
                                head_dim=64, mlp=1024)


def cpu(t):
    torch.cuda.synchronize()
    return t.to("cpu")


@pytest.mark.parametrize("count", [8, 8 * 257, 4096 * 128])
def test_velocity_step_bitexact(count):
    g = torch.Generator().manual_seed(count)
    z = torch.randn(count, generator=g).to(torch.bfloat16)
    v = torch.randn(count, generator=g).to(torch.bfloat16)
    for dt in (-0.05, 1.0 / 3.0):
        zg = z.to(DEV)
        h3.velocity_step(zg, v.to(DEV), dt)
        assert_bitexact(cpu(zg), oracle.velocity_step(z, v, dt), f"dt={dt}")


def heads(w, seed):
    g = torch.Generator().manual_seed(seed)
    d = w.hidden
    mv = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    ma = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    wv = (torch.randn(128, d, generator=g) * 0.02).to(torch.bfloat16)
    wa = (torch.randn(256, d, generator=g) * 0.02).to(torch.bfloat16)
    nv = w.n_tokens - w.n_text - w.n_audio
    zv = (torch.randn(nv, 128, generator=g) * 0.01).to(torch.bfloat16)
    za = (torch.randn(w.n_audio, 256, generator=g) * 0.01).to(torch.bfloat16)
    return (mv, wv), (ma, wa), zv, za


CASES = {
    "reuse2_restore_schedule": dict(steps=5, reuse=2, layers=5, reduce_after=1, restore_early=4, restore_late=3,
                                    early_evals=2),
    "core_reuse2": dict(steps=5, core_reuse=2, layers=4, reduce_after=0, restore_early=3, restore_late=2,
                        early_evals=1),
    "plain_layers": dict(steps=3, layers=3),
}


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("case", list(CASES))
def test_denoise_matches_oracle(case, int8):
    w = SMALL_TR
    o = CASES[case]
    x = synth.make_x(w, 1011)
    ps = [synth.make_block(w, 1011, b) for b in range(6)]
    pg = [h3.quantize_block({k: v.to(DEV) for k, v in p.items()}) if int8 else {k: v.to(DEV) for k, v in p.items()}
          for p in ps]
    pc = [oracle.quantize_block(p) if int8 else p for p in ps]
    video, audio, zv, za = heads(w, 3)
    dt = [-1.0 / o["steps"]] * o["steps"]
    opts = h3.denoise_opts(o["steps"], o.get("reuse", 1), o.get("core_reuse", 1), o["layers"],
                           o.get("reduce_after", -1), o.get("restore_early", 40), o.get("restore_late", 30),
                           o.get("early_evals", 10))
    gv = tuple(t.to(DEV) for t in video)
    ga = tuple(t.to(DEV) for t in audio)
    run = h3.Denoise(w, pg, opts, dt, video=gv, audio=ga)
    ws = h3.alloc_workspace(run.workspace_bytes)
    zvg, zag = zv.to(DEV), za.to(DEV)
    xg = x.to(DEV)
    run(xg, zvg, zag, ws)
    rv, ra = oracle.denoise(w, pc, x, o, dt, video=video, audio=audio, z_video=zv, z_audio=za)
    # the velocity part of the latents is what the loop computes: compare it at the bf16 bar
    assert relerr(cpu(zvg).double() - zv.double(), rv.double() - zv.double()) <= BF16_TOL
    assert relerr(cpu(zag).double() - za.double(), ra.double() - za.double()) <= BF16_TOL
    assert_bitexact(cpu(xg), x, "x_in untouched")
    # a second call on the same workspace repeats the result
    zvg2, zag2 = zv.to(DEV), za.to(DEV)
    run(xg, zvg2, zag2, ws)
    assert_bitexact(cpu(zvg2), cpu(zvg), "repeat video")
    assert_bitexact(cpu(zag2), cpu(zag), "repeat audio")


def test_denoise_restore_schedule_is_applied():
    """Only the restore schedule differs between the two runs (every evaluation early versus
    the early / late split), and the latents differ accordingly, as in the oracle."""
    w = SMALL_TR
    x = synth.make_x(w, 1012)
    ps = [{k: v.to(DEV) for k, v in synth.make_block(w, 1012, b).items()} for b in range(5)]
    video, audio, zv, za = heads(w, 4)
    gv = tuple(t.to(DEV) for t in video)
    dt = [-0.25] * 4
    outs = []
    for early in (4, 2):
        opts = h3.denoise_opts(4, layers=5, reduce_after=1, restore_early=4, restore_late=3, early_evals=early)
        run = h3.Denoise(w, ps, opts, dt, video=gv)
        zg = zv.to(DEV)
        run(x.to(DEV), zg, None, h3.alloc_workspace(run.workspace_bytes))
        outs.append(cpu(zg))
    assert not torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def _planted_plans(plan, reuse):
    """Wrong schedules for the same options, planted on the oracle side: evaluations one step
    late (fresh at step 0, then at steps i with i % reuse == 1, and the last), and a fresh
    velocity at every step instead of the latest fresh one (the restore split kept per
    evaluation count as in the plan)."""
    early = {s["eval"]: s["restore"] for s in plan}
    def make(fresh):
        out, e = [], -1
        for i, f in enumerate(fresh):
            e += f
            out.append(dict(fresh=f, core=f, eval=e, restore=early.get(min(e, max(early)), plan[-1]["restore"])
                            if plan[0]["restore"] >= 0 else -1))
        return out
    n = len(plan)
    shifted = make([int(i == 0 or i % reuse == 1 or i == n - 1) for i in range(n)])
    current = make([1] * n)
    return {"shifted": shifted, "current": current}


@pytest.mark.parametrize("int8", [False, True])
def test_denoise_with_patch_embedding_matches_oracle_and_rejects_wrong_plans(int8):
    """The closed loop: each core evaluation starts from x_in plus the patch embedding of the
    current latents (the stand-in reading of h3dit_patch_embed), so every fresh evaluation sees
    other latents and gives another velocity.  The GPU loop matches the oracle's at the bf16
    bar on the latents' total update, and is far (more than 2.5x the bar) from the oracle run
    with a wrong schedule planted in it: evaluations shifted by one step, or a fresh velocity
    at every step instead of the latest fresh one."""
    w = SMALL_TR
    x = synth.make_x(w, 1021)
    ps = [synth.make_block(w, 1021, b) for b in range(5)]
    pg = [h3.quantize_block({k: v.to(DEV) for k, v in p.items()}) if int8 else {k: v.to(DEV) for k, v in p.items()}
          for p in ps]
    pc = [oracle.quantize_block(p) if int8 else p for p in ps]
    g = torch.Generator().manual_seed(8)
    d = w.hidden
    mv = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    ma = (torch.randn(2, d, generator=g) * 0.1).to(torch.bfloat16)
    wv = (torch.randn(128, d, generator=g) * 0.2).to(torch.bfloat16)
    wa = (torch.randn(256, d, generator=g) * 0.2).to(torch.bfloat16)
    ev = (torch.randn(d, 128, generator=g) * 0.1).to(torch.bfloat16)
    ea = (torch.randn(d, 256, generator=g) * 0.1).to(torch.bfloat16)
    nv = w.n_tokens - w.n_text - w.n_audio
    zv = torch.randn(nv, 128, generator=g).to(torch.bfloat16)
    za = torch.randn(w.n_audio, 256, generator=g).to(torch.bfloat16)
    o = dict(steps=5, reuse=2, layers=5, reduce_after=1, restore_early=4, restore_late=3, early_evals=2)
    dt = [-1.0 / 5] * 5
    opts = h3.denoise_opts(5, 2, 1, 5, 1, 4, 3, 2)
    run = h3.Denoise(w, pg, opts, dt, video=(mv.to(DEV), wv.to(DEV)), audio=(ma.to(DEV), wa.to(DEV)),
                     embed=(ev.to(DEV), ea.to(DEV)))
    ws = h3.alloc_workspace(run.workspace_bytes)
    zvg, zag = zv.to(DEV), za.to(DEV)
    run(x.to(DEV), zvg, zag, ws)
    gv, ga = cpu(zvg).double() - zv.double(), cpu(zag).double() - za.double()

    def oracle_run(plan=None):
        rv, ra = oracle.denoise(w, pc, x, o, dt, video=(mv, wv), audio=(ma, wa), z_video=zv, z_audio=za,
                                embed=(ev, ea), plan=plan)
        return rv.double() - zv.double(), ra.double() - za.double()

    rv, ra = oracle_run()
    ev_err, ea_err = relerr(gv, rv), relerr(ga, ra)
    print(f"[denoise+embed] update error video {ev_err:.3e} audio {ea_err:.3e}", flush=True)
    assert ev_err <= BF16_TOL and ea_err <= BF16_TOL
    plan = oracle.denoise_plan(5, 2, 1, 1, 4, 3, 2)
    for name, wrong in _planted_plans(plan, 2).items():
        wv_, wa_ = oracle_run(wrong)
        dv, da = relerr(gv, wv_), relerr(ga, wa_)
        print(f"[denoise+embed] planted {name}: distance video {dv:.3e} audio {da:.3e}", flush=True)
        assert max(dv, da) > 2.5 * BF16_TOL, name
