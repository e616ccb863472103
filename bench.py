"""Benchmark of the MiniMax-H3 DiT hot path on one MI355X.

A step is one denoising evaluation: the whole stack of DiT blocks (AdaLN, QKV with rotary,
full attention, output projection, gate + AdaLN, FC1 + GELU, FC2, gate) over one batch of
synthetic tokens.  Default workload: 50 blocks, 4096 tokens (3520 video 5x22x32 + 512 text +
64 audio), hidden 5120, 40 heads x 128, MLP 20480, bf16, independent seeded weights per block
resident in HBM.  `value` is the algorithmic TFLOP/s of the timed steps:
FLOP per block = 2 N (4 d^2 + 2 d f) + 4 N^2 d.

Besides the JSON line's required fields it reports: the same stack on the int8 path; a
per-kernel breakdown of one block measured with HIP events on the launch stream (the
dominant kernel gives `roofline`); and the CPU oracle timed on a bounded sample of the same
workload (`cpu_baseline`).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "int8": 5000.0}     # dense MFMA, TFLOP/s or TOP/s
HBM_PEAK = 8000.0                           # GB/s


def block_flops(N, d, f):
    return 2.0 * N * (4 * d * d + 2 * d * f) + 4.0 * N * N * d


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="workload index in synth.WORKLOADS (3 or 4)")
    ap.add_argument("--blocks", type=int, default=None, help="override the block count")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8 legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--only-kernels", action="store_true", help="per-kernel timing only (profiling runs)")
    ap.add_argument("--fc2-group", type=int, default=None,
                    help="int8 FC2-input group (1024 as on the pages; the MLP width gives one code per token, "
                         "the row-level variant)")
    ap.add_argument("--streamed", action="store_true",
                    help="also time the stack with every block's weights in pinned host memory "
                         "(h3dit_stack_fwd_streamed: two device slots filled over the host link)")
    ap.add_argument("--denoise", action="store_true",
                    help="also time 20-step denoising runs (h3dit_denoise_fwd) at the pages' slow, default and "
                         "token-reduction presets (kept out of the default run: its reduced-sequence launches share "
                         "kernel names with the full-size ones and would mix into the profiled per-kernel averages)")
    ap.add_argument("--precision", choices=["bf16", "int8", "int8_mlp", "int8_attn"], default=None,
                    help="precision of the main leg (default: the workload's)")
    ap.add_argument("--stack-only", action="store_true",
                    help="time the main stack leg only (no per-kernel loops, no other legs, no CPU leg): a "
                         "profiled run of it traces the kernels as they run inside the stack")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --only-kernels: also run one plain device copy of this many bytes, the reference "
                         "that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def make_blocks(w, n_blocks, seed, device, int8, mlp_only=False, attn_only=False):
    import synth
    import audio_diffusion_transformer_dit_amd as h3
    blocks = []
    for b in range(n_blocks):
        p = synth.make_block(w, seed, b, device)
        if int8:
            q = h3.quantize_block(p, mlp_only=mlp_only, attn_only=attn_only)
            del p
            p = q
        blocks.append(p)
        print(f"[bench] block {b + 1}/{n_blocks} generated", file=sys.stderr, flush=True) if (b + 1) % 10 == 0 else None
    return blocks


def time_stack(w, blocks, x, steps, warmup, reduction=None, per_step=None):
    """Mean ms per step over `steps` stack calls between two events on the launch stream (and,
    from events recorded between the calls, the median and minimum single step into per_step).
    Every step starts from the same seeded residual: x is restored from a saved copy (one
    device-to-device copy of [N][d] bf16, inside the timed step; its own time is reported) so
    the timed operands do not drift with the steps."""
    import torch
    import audio_diffusion_transformer_dit_amd as h3
    stack = h3.Stack(w, blocks, 0, reduction)
    ws = h3.alloc_workspace(stack.workspace_bytes, x.device)
    x0 = x.clone()
    for _ in range(warmup):
        x.copy_(x0)
        stack(x, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        x.copy_(x0)
        stack(x, ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if per_step is not None and steps > 0:
        one = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        per_step["step_ms_median"] = round(one[steps // 2] if steps % 2 else 0.5 * (one[steps // 2 - 1] + one[steps // 2]), 3)
        per_step["step_ms_min"] = round(one[0], 3)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            x.copy_(x0)
        e.record()
        torch.cuda.synchronize()
        per_step["input_restore_ms"] = round(s.elapsed_time(e) / 10, 4)
    x.copy_(x0)
    return ev[0].elapsed_time(ev[steps]) / steps, wall, stack.workspace_bytes


def time_streamed(w, blocks, x, steps, warmup, reduction=None):
    """The stack with the block matrices streamed from pinned host memory; also the
    host-to-device rate of one block's matrices copied alone."""
    import torch
    import audio_diffusion_transformer_dit_amd as h3
    hb = [h3.host_block(p) for p in blocks]
    torch.cuda.synchronize()
    stack = h3.StreamedStack(w, hb, 0, reduction)
    ws = h3.alloc_workspace(stack.workspace_bytes, x.device)
    cs = torch.cuda.Stream()
    for _ in range(warmup):
        stack(x, ws, copy_stream=cs.cuda_stream)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        stack(x, ws, copy_stream=cs.cuda_stream)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    mats = {k: t for k, t in hb[0].items() if k != "mod"}
    dst = {k: torch.empty_like(t, device=x.device) for k, t in mats.items()}
    nbytes = sum(t.numel() * t.element_size() for t in mats.values())
    for _ in range(2):
        for k, t in mats.items():
            dst[k].copy_(t, non_blocking=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(5):
        for k, t in mats.items():
            dst[k].copy_(t, non_blocking=True)
    e.record()
    torch.cuda.synchronize()
    copy_ms = s.elapsed_time(e) / 5
    del hb, dst
    return {"ms_per_step": round(ms, 3), "ms_per_block": round(ms / w.blocks, 3), "block_bytes": nbytes,
            "h2d_gbps": round(nbytes / (copy_ms / 1e3) / 1e9, 1),
            "copy_bound_ms_per_step": round(copy_ms * w.blocks, 3),
            "workspace_bytes": stack.workspace_bytes}


def kernel_breakdown(w, p, x, iters, int8, progress=False):
    """Times each kernel of one block where it runs in the block: `iters` passes over the
    block's launches in order, every launch bracketed by HIP events on the current stream (the
    stream the library launches on), so each kernel reads what the kernel before it just wrote,
    as in the stack; a stage's time is the mean of its launches' event intervals."""
    import torch
    import audio_diffusion_transformer_dit_amd as h3
    dev = x.device
    N, d, f, H, hd = w.n_tokens, w.hidden, w.mlp, w.heads, w.head_dim
    mod = p["mod"]
    cos, sin = h3.rope_tables(w, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    h1 = torch.empty((N, d), **bf)
    q = torch.empty((H, N, hd), **bf)
    k = torch.empty_like(q)
    vt = torch.empty((H, hd, h3.ldv(N)), **bf)
    o = torch.empty_like(q)
    y1 = torch.empty((N, d), **bf)
    x1 = torch.empty((N, d), **bf)
    h2 = torch.empty((N, d), **bf)
    gl = torch.empty((N, f), **bf)
    y2 = torch.empty((N, d), **bf)
    x2 = torch.empty((N, d), **bf)
    i8 = dict(dtype=torch.int8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    q1, s1 = torch.empty((N, d), **i8), torch.empty(N, **f32)
    qo, so = torch.empty((N, d), **i8), torch.empty(N, **f32)
    q2, s2 = torch.empty((N, d), **i8), torch.empty(N, **f32)
    qg, sg = torch.empty((N, f), **i8), torch.empty((N, f // w.fc2_group), **f32)

    if not int8:
        ops = {
            "adaln": (lambda: h3.row_gate_adaln(x, shift=mod[0], scale=mod[1], h=h1), 0, 4.0 * N * d),
            "qkv_rope_gemm": (lambda: h3.linear(N, 3 * d, d, h1, p["wqkv"], h3.OUT_QKV, None, cos=cos, sin=sin,
                                                heads=H, head_dim=hd, out_q=q, out_k=k, out_v=vt),
                              2.0 * N * d * 3 * d, 0),
            "attention": (lambda: h3.attention(H, N, hd, q, k, vt, o), 4.0 * N * N * d, 0),
            "out_proj_gemm": (lambda: h3.linear(N, d, d, o, p["wo"], h3.OUT_BF16, y1, a_headmajor_hd=hd),
                              2.0 * N * d * d, 0),
            "gate_adaln": (lambda: h3.row_gate_adaln(x, gate=mod[2], y=y1, x_out=x1, shift=mod[3], scale=mod[4], h=h2),
                           0, 8.0 * N * d),
            "fc1_gelu_gemm": (lambda: h3.linear(N, f, d, h2, p["w1"], h3.OUT_GELU, gl), 2.0 * N * d * f, 0),
            "fc2_gemm": (lambda: h3.linear(N, d, f, gl, p["w2"], h3.OUT_BF16, y2), 2.0 * N * f * d, 0),
            "gate": (lambda: h3.row_gate_adaln(x1, gate=mod[5], y=y2, x_out=x2), 0, 6.0 * N * d),
        }
    else:
        ops = {
            "adaln_q8": (lambda: h3.row_gate_adaln(x, shift=mod[0], scale=mod[1], q=q1, s=s1), 0, 3.0 * N * d + 4 * N),
            "qkv_rope_gemm_i8": (lambda: h3.linear(N, 3 * d, d, q1, p["qqkv"], h3.OUT_QKV, None, precision=h3.INT8,
                                                   a_scale=s1, w_scale=p["sqkv"], cos=cos, sin=sin, heads=H,
                                                   head_dim=hd, out_q=q, out_k=k, out_v=vt),
                                 2.0 * N * d * 3 * d, 0),
            "attention": (lambda: h3.attention(H, N, hd, q, k, vt, o), 4.0 * N * N * d, 0),
            "quant_o": (lambda: h3.lib().h3dit_quantize_rows(N, d, d, o.data_ptr(), hd, qo.data_ptr(), so.data_ptr(),
                                                             torch.cuda.current_stream().cuda_stream),
                        0, 3.0 * N * d + 4 * N),
            "out_proj_gemm_i8": (lambda: h3.linear(N, d, d, qo, p["qo"], h3.OUT_BF16, y1, precision=h3.INT8,
                                                   a_scale=so, w_scale=p["so"]), 2.0 * N * d * d, 0),
            "gate_adaln_q8": (lambda: h3.row_gate_adaln(x, gate=mod[2], y=y1, x_out=x1, shift=mod[3], scale=mod[4],
                                                        q=q2, s=s2), 0, 7.0 * N * d + 4 * N),
            "fc1_gelu_gemm_i8": (lambda: h3.linear(N, f, d, q2, p["q1"], h3.OUT_GELU, gl, precision=h3.INT8,
                                                   a_scale=s2, w_scale=p["s1"]), 2.0 * N * d * f, 0),
            "quant_fc2_in": (lambda: h3.lib().h3dit_quantize_rows(N, f, w.fc2_group, gl.data_ptr(), 0, qg.data_ptr(),
                                                                  sg.data_ptr(),
                                                                  torch.cuda.current_stream().cuda_stream),
                             0, 3.0 * N * f + 4.0 * N * f / w.fc2_group),
            "fc2_gemm_i8": (lambda: h3.linear(N, d, f, qg, p["q2"], h3.OUT_BF16, y2, precision=h3.INT8,
                                              a_scale=sg if w.fc2_group < f else sg[:, 0].contiguous(),
                                              a_group=w.fc2_group if w.fc2_group < f else 0, w_scale=p["s2"]),
                            2.0 * N * f * d, 0),
            "gate": (lambda: h3.row_gate_adaln(x1, gate=mod[5], y=y2, x_out=x2), 0, 6.0 * N * d),
        }
    if w.reduce_after >= 0:
        # token pair / restore ([DD] "Token 缩减"): unique bytes moved
        rows, W = w.video_t * w.video_h, w.video_w
        rest = w.n_text + w.n_audio
        n_full = rows * W + rest
        n_red = rows * (W // 2 + W % 2) + rest
        paired = rows * (W // 2) * 2
        xr = x[:n_full].clone()
        red = torch.empty((n_red, d), **bf)
        r_in = torch.zeros((n_red, d), **bf)
        yred = torch.zeros((n_red, d), **bf)
        ops["token_pair"] = (lambda: h3.token_pair(w, xr, red, r_in), 0, 2.0 * d * (n_full + 2 * n_red))
        ops["token_restore"] = (lambda: h3.token_restore(w, xr, yred, r_in), 0,
                                2.0 * d * (paired + n_full + n_red + paired // 2))
    # one pass in order so that every kernel reads realistic data
    for fn, _, _ in ops.values():
        fn()
    torch.cuda.synchronize()
    if progress:
        print(f"[bench] {'int8' if int8 else 'bf16'} block launches: first pass done", file=sys.stderr, flush=True)
    evs = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
           for name in ops}
    for it in range(iters):
        for name, (fn, _, _) in ops.items():
            s, e = evs[name][it]
            s.record()
            fn()
            e.record()
        if progress:   # profiled runs: the profiler serialises the launches, so this tracks the GPU
            print(f"[bench] {'int8' if int8 else 'bf16'} block launches: pass {it + 1}/{iters} issued", file=sys.stderr,
                  flush=True)
    torch.cuda.synchronize()
    res = {}
    for name, (fn, flop, nbytes) in ops.items():
        ms = sum(s.elapsed_time(e) for s, e in evs[name]) / iters
        r = {"ms": round(ms, 4)}
        if flop:
            r["tflops"] = round(flop / ms / 1e9, 1)
            r["flop"] = flop
        if nbytes:
            r["gbps"] = round(nbytes / ms / 1e6, 1)
            r["bytes"] = nbytes
        res[name] = r
    return res


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    ent = t.get(kernel)
    if not ent:
        return None
    h = hashlib.sha256()
    for src in sorted(ent.get("sources", [])):
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    return ent["bytes_per_launch"] if h.hexdigest() == ent.get("sha256") else None


def cpu_baseline(w):
    """The oracle on a bounded sample: one block at full width over 2688 tokens (the workload's
    22 x 32 spatial grid with 3 frames, its 512 text and 64 audio tokens)."""
    import oracle
    import synth
    sample = w.replace(video_t=3, video_h=22, video_w=32, n_text=512, n_audio=64, blocks=1)
    assert sample.n_tokens == 2688
    seed = synth.seed_for(3)
    x = synth.make_x(sample, seed)
    p = synth.make_block(sample, seed, 0)
    cos, sin = oracle.rope_tables(sample)
    t0 = time.perf_counter()
    oracle.block_fwd(sample, p, x, cos, sin)
    dt = time.perf_counter() - t0
    fl = block_flops(sample.n_tokens, sample.hidden, sample.mlp)
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one bf16 block at full width (d={sample.hidden}, H={sample.heads}x{sample.head_dim}, "
                      f"f={sample.mlp}) over {sample.n_tokens} tokens (3x22x32 video + 512 text + 64 audio): "
                      f"{fl / 1e9:.1f} GFLOP in {dt:.2f} s; extrapolated 50-block step at 4096 tokens "
                      f"{50 * block_flops(4096, 5120, 20480) / (fl / dt) :.0f} s"}


DENOISE_PRESETS = {
    # the pages' control matrix: slow reference, the verified --layers 45 --reuse 2 setting, and
    # that setting with token reduction (bypass restored before block 40, then 30)
    "slow_reference": dict(steps=20, reuse=1, layers=50),
    "layers45_reuse2": dict(steps=20, reuse=2, layers=45),
    "layers45_reuse2_token_reduction": dict(steps=20, reuse=2, layers=45, reduce_after=3),
}


def time_denoise(w, blocks, x, seed, channels=128):
    """Each preset once after one untimed run: the stack runs of its plan plus the head and
    the velocity steps (synthetic head weights; latents of `channels` per video / audio row)."""
    import torch
    import audio_diffusion_transformer_dit_amd as h3
    g = torch.Generator(device=x.device).manual_seed(seed + 77)
    d = w.hidden
    nv = w.n_tokens - w.n_text - w.n_audio

    def rnd(*shape, std):
        return (torch.randn(*shape, generator=g, device=x.device) * std).to(torch.bfloat16)

    video = (rnd(2, d, std=0.1), rnd(channels, d, std=0.02))
    audio = (rnd(2, d, std=0.1), rnd(channels, d, std=0.02))
    out = {}
    for name, o in DENOISE_PRESETS.items():
        layers = min(o["layers"], len(blocks))
        opts = h3.denoise_opts(o["steps"], o.get("reuse", 1), 1, layers, o.get("reduce_after", -1), 40, 30, 10)
        runs, plan = h3.denoise_plan(opts, len(blocks))
        run = h3.Denoise(w, blocks, opts, [-1.0 / o["steps"]] * o["steps"], video=video, audio=audio)
        ws = h3.alloc_workspace(run.workspace_bytes, x.device)
        zv, za = rnd(nv, channels, std=1.0), rnd(w.n_audio, channels, std=1.0)
        run(x, zv, za, ws)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        run(x, zv, za, ws)
        e.record()
        torch.cuda.synchronize()
        out[name] = {"ms": round(s.elapsed_time(e), 2), "stack_runs": runs, "blocks_per_run": layers,
                     "steps": o["steps"], "reuse": o.get("reuse", 1),
                     "token_reduction": [o["reduce_after"], 40, 30] if "reduce_after" in o else None}
        print(f"[bench] denoise {name}: {out[name]['ms']:.1f} ms ({runs} stack runs)", file=sys.stderr, flush=True)
        del ws
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this path runs on a single "
              "MI355X (sharding tokens by video rows with a K/V all-gather per block is the multi-GPU design, "
              "not built here).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import audio_diffusion_transformer_dit_amd as h3

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    if args.blocks:
        w = w.replace(blocks=args.blocks)
    if args.fc2_group:
        w = w.replace(fc2_group=args.fc2_group)
    seed = synth.seed_for(args.workload)
    main_prec = args.precision or w.precision
    int8_main = main_prec != "bf16"
    if main_prec in ("int8_mlp", "int8_attn") and not args.stack_only:
        print("--precision int8_mlp / int8_attn time the stack only: add --stack-only (the default run times "
              "those paths as extra legs)", file=sys.stderr)
        sys.exit(2)
    red = (w.reduce_after, w.restore_before) if w.reduce_after >= 0 else None
    N, d, f = w.n_tokens, w.hidden, w.mlp
    print(f"[bench] workload {w.name}: {w.blocks} blocks, N={N}, d={d}, f={f}, {w.precision}", file=sys.stderr,
          flush=True)

    x = synth.make_x(w, seed, dev)
    torch.cuda.synchronize()
    print("[bench] input residual ready", file=sys.stderr, flush=True)
    out = {}
    if args.only_kernels:
        p = make_blocks(w, 1, seed, dev, int8_main)[0]
        torch.cuda.synchronize()
        print("[bench] block weights ready", file=sys.stderr, flush=True)
        out["kernels"] = kernel_breakdown(w, p, x, args.kernel_iters, int8_main, progress=True)
        if not int8_main and not args.no_int8:
            import audio_diffusion_transformer_dit_amd as h3
            out["kernels_int8"] = kernel_breakdown(w, h3.quantize_block(p), x, args.kernel_iters, True, progress=True)
        if args.copy_bytes:
            src = torch.ones(args.copy_bytes // 2, dtype=torch.bfloat16, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            out["copy_bytes"] = args.copy_bytes
        print(json.dumps(out))
        return

    blocks = make_blocks(w, w.blocks, seed, dev, int8_main, mlp_only=main_prec == "int8_mlp",
                         attn_only=main_prec == "int8_attn")
    torch.cuda.synchronize()
    print("[bench] weights resident; timing the stack", file=sys.stderr, flush=True)
    step_stats = {}
    ms, wall, ws_bytes = time_stack(w, blocks, x, args.steps, args.warmup, red, step_stats)
    if args.stack_only:
        print(json.dumps({"workload": w.name, "precision": main_prec, "ms_per_step": round(ms, 3), **step_stats}),
              flush=True)
        return
    if red:
        nr = w.video_t * w.video_h * (w.video_w // 2 + w.video_w % 2) + w.n_text + w.n_audio
        full = red[0] + 1 + max(0, w.blocks - red[1])
        step_flop = full * block_flops(N, d, f) + (w.blocks - full) * block_flops(nr, d, f)
    else:
        step_flop = w.blocks * block_flops(N, d, f)
    value = step_flop / (ms / 1e3) / 1e12
    print(f"[bench] {ms:.2f} ms/step, {value:.1f} TFLOP/s", file=sys.stderr, flush=True)

    kern = kernel_breakdown(w, blocks[0], x, args.kernel_iters, int8_main)
    mm = {k: v for k, v in kern.items() if "flop" in v}
    dom = max(mm, key=lambda k: mm[k]["ms"])
    prec = main_prec
    # attention multiplies bf16 on both paths; the int8 path's projections use the int8 peak
    kprec = "int8" if (int8_main and dom != "attention") else "bf16"
    roof = {"bound": "mfma", "kernel": dom, "achieved": mm[dom]["tflops"], "peak": PEAK[kprec],
            "unit": "TFLOP/s" if kprec == "bf16" else "TOP/s", "frac": round(mm[dom]["tflops"] / PEAK[kprec], 4),
            "traffic": traffic_for(dom)}
    extra = {"ms_per_block": round(ms / w.blocks, 3), **step_stats, "tflop_per_step": round(step_flop / 1e12, 2),
             "workspace_bytes": ws_bytes, "kernels": kern,
             "kernels_note": "per-launch HIP event intervals over repeated passes of one block's launch sequence",
             "wall_s_timed": round(wall, 3)}
    if args.streamed:
        print("[bench] timing the stack with weights streamed from host memory", file=sys.stderr, flush=True)
        extra["streamed"] = time_streamed(w, blocks, x, args.steps, args.warmup, red)

    if args.denoise:
        extra["denoise"] = time_denoise(w, blocks, x, seed)

    if not args.no_int8 and not int8_main:
        del blocks
        torch.cuda.empty_cache()
        blocks8 = make_blocks(w, w.blocks, seed, dev, True)
        step8 = {}
        ms8, _, _ = time_stack(w, blocks8, x, args.steps, args.warmup, red, step8)
        extra["int8"] = {"ms_per_step": round(ms8, 3), **step8, "ms_per_block": round(ms8 / w.blocks, 3),
                         "fc2_group": w.fc2_group,
                         "tops": round(step_flop / (ms8 / 1e3) / 1e12, 1),
                         "kernels": kernel_breakdown(w, blocks8[0], x, args.kernel_iters, True)}
        if args.streamed:
            extra["int8"]["streamed"] = time_streamed(w, blocks8, x, args.steps, args.warmup, red)
        if args.denoise:
            extra["int8"]["denoise"] = time_denoise(w, blocks8, x, seed)
        del blocks8
        torch.cuda.empty_cache()
        # the middle row of the pages' int8 table: FC1 and FC2 in int8, attention projections bf16
        blocks8m = make_blocks(w, w.blocks, seed, dev, True, mlp_only=True)
        ms8m, _, _ = time_stack(w, blocks8m, x, args.steps, args.warmup, red)
        extra["int8_mlp_only"] = {"ms_per_step": round(ms8m, 3), "ms_per_block": round(ms8m / w.blocks, 3),
                                  "tflops_equiv": round(step_flop / (ms8m / 1e3) / 1e12, 1)}
        del blocks8m
        torch.cuda.empty_cache()
        # the int8-QKV-only path the pages set against the full int8 path: QKV and the output
        # projection in int8, the MLP in bf16
        blocks8a = make_blocks(w, w.blocks, seed, dev, True, attn_only=True)
        ms8a, _, _ = time_stack(w, blocks8a, x, args.steps, args.warmup, red)
        extra["int8_attn_only"] = {"ms_per_step": round(ms8a, 3), "ms_per_block": round(ms8a / w.blocks, 3),
                                   "tflops_equiv": round(step_flop / (ms8a / 1e3) / 1e12, 1)}
        del blocks8a
        torch.cuda.empty_cache()

    line = {
        "metric": "DiT block TFLOP/s (bf16, int8) + ms per 50-block step, 4096 tokens",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": prec, "data": "synthetic (seeded Philox-4x32-10 normals; random-init weights per block)",
        "config": {"workload": w.name, "n_tokens": N, "video": [w.video_t, w.video_h, w.video_w],
                   "text": w.n_text, "audio": w.n_audio, "hidden": d, "heads": w.heads, "head_dim": w.head_dim,
                   "mlp": f, "blocks": w.blocks, "token_reduction": list(red) if red else None,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
