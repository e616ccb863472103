"""Whole-stack parity at the production sizes: the 50-block stack over 4096 tokens (d 5120,
40x128 heads, MLP 20480; or another workload, e.g. 8192 tokens with token reduction), GPU
against the CPU oracle.  Test infrastructure, run by hand in
two phases because the oracle needs about half an hour of 16 CPU cores for 146 TFLOP:

  python tests/full_stack_parity.py gpu OUT.pt [--int8] [--blocks B] [--workload W] [--half H]
  python tests/full_stack_parity.py join OUT.pt HALF0.pt HALF1.pt
                                                           # on an MI355X: the library's stack,
                                                           # launched as the benchmark launches it
  python tests/full_stack_parity.py oracle OUT.pt          # on any host: the oracle block by block
      [--from B --to E --state S.pt] [--gen-device cuda]   # (in sittings: blocks [B, E), residual in S.pt)

Both phases draw the same seeded inputs and weights (synth is bit-exact across devices).  The
oracle runs the blocks one at a time, which equals its fused stack bit for bit (pinned in
test_oracle_pins.py), printing progress after each block.  The comparison: the residual in the
max norm and the stack's total update on average, against the single-stage bars (2e-2, 5%)
raised, where it is larger, to 1.5x the divergence that a one-step change of a single input
element causes over the same blocks.  This is the chain argument of the collected six-block
production-width test (test_gpu_fullsize.test_stack_production_width_matches_oracle): GPU and
oracle add in different orders, every stage differs by rounding-sized amounts, and down a chain
such differences grow as the chain amplifies a rounding-sized change of its input.  That test
measures the amplification with the oracle itself; at 50 blocks a second oracle chain would
take another half hour, so this script measures it on the GPU (the GPU and the oracle compute
the same chain, so their amplification of a one-step input change is the same to within its
own rounding noise)."""
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import synth  # noqa: E402

WORKLOAD = 3


def gpu_phase(path, int8, n_blocks=None, workload=WORKLOAD, half=None):
    """The library's stack over the first n_blocks blocks (all by default), and the same stack
    from x with one element moved by one bf16 step: how far the two outputs end up apart is the
    sensitivity of the computation itself to one rounding-sized change, stored with the output."""
    import audio_diffusion_transformer_dit_amd as h3
    from parity import relerr
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[workload]
    if n_blocks is not None:
        w = w.replace(blocks=n_blocks)
    seed = synth.seed_for(workload)
    red = (w.reduce_after, w.restore_before) if w.reduce_after >= 0 else None
    x = synth.make_x(w, seed, dev)
    blocks = []
    for b in range(w.blocks):
        p = synth.make_block(w, seed, b, dev)
        blocks.append(h3.quantize_block(p) if int8 else p)
    stack = h3.Stack(w, blocks, reduction=red)
    ws = h3.alloc_workspace(stack.workspace_bytes, dev)
    x0 = x.clone()
    stack(x, ws)
    torch.cuda.synchronize()
    if True:
        xp = x0.clone()
        bits = xp.view(torch.int16)
        bits[w.n_tokens // 2, w.hidden // 2] += 1
        stack(xp, ws)
        torch.cuda.synchronize()
        du, dp = x.double() - x0.double(), xp.double() - x0.double()
        noise_rel, noise_upd = relerr(xp, x), float((dp - du).abs().mean() / du.abs().mean())
        print(f"one-step input perturbation after {w.blocks} blocks ({'int8' if int8 else 'bf16'}): residual rel err "
              f"{noise_rel:.3e}, mean rel err of the total update {noise_upd:.3e}", flush=True)
    out = x.cpu()
    if half is not None:   # one half of the rows (a result file must stay small enough to copy back)
        lo, hi = (0, w.n_tokens // 2) if half == 0 else (w.n_tokens // 2, w.n_tokens)
        out = out[lo:hi].clone()
    torch.save({"workload": workload, "int8": int8, "blocks": w.blocks, "x_out": out, "noise_rel": noise_rel,
                "noise_upd": noise_upd, "half": half}, path)
    print(f"gpu stack ({'int8' if int8 else 'bf16'}, {w.blocks} blocks, N={w.n_tokens}) written to {path}", flush=True)


def oracle_phase(path, first=0, last=None, state=None, gen_device="cpu"):
    """Blocks [first, last) of the oracle chain; with `state`, the residual is read from it
    (first > 0) and written back to it, so the chain can run in several sittings.  Inside the
    token-reduced span the state holds only the reduced residual: the bypass and the reduced
    input are derived again by rerunning the blocks up to the pairing.  gen_device: where
    synth draws the inputs (bit-identical on any device; the arithmetic stays in the oracle)."""
    import oracle
    from parity import BF16_TOL, relerr
    saved = torch.load(path, weights_only=True)
    w = synth.WORKLOADS[saved["workload"]]
    seed = synth.seed_for(saved["workload"])
    last = saved["blocks"] if last is None else last
    x0 = synth.make_x(w, seed)
    # token reduction as the stack runs it: pair after block reduce_after (x stays as the
    # bypass, r is the reduced input, z the reduced residual), restore before block
    # restore_before or after the last block
    ra, rb = (w.reduce_after, w.restore_before) if w.reduce_after >= 0 else (-1, -1)
    cr, sr = oracle.rope_tables(w, reduced=True) if ra >= 0 else (None, None)
    def block(b):
        p = {k: v.cpu() for k, v in synth.make_block(w, seed, b, gen_device).items()}
        return oracle.quantize_block(p) if saved["int8"] else p

    st = torch.load(state, weights_only=True) if first > 0 else {"x": x0, "z": None, "r": None}
    x, z, r = st["x"], st["z"], st["r"]
    t0 = time.time()
    if z is not None and x is None:
        # resume inside the reduced span: bypass = the residual after block reduce_after
        x = x0
        for b in range(ra + 1):
            x = oracle.block_fwd(w, block(b), x, fused=True)
            print(f"bypass: block {b + 1}/{ra + 1} again, {time.time() - t0:.0f} s", flush=True)
        r = oracle.token_pair(w, x)
        print(f"bypass and reduced input derived again ({ra + 1} blocks), {time.time() - t0:.0f} s", flush=True)
    for b in range(first, last):
        if z is not None and b == rb:
            x, z, r = oracle.token_restore(w, x, z, r), None, None
        p = block(b)
        if z is not None:
            z = oracle.block_fwd(w, p, z, cr, sr, fused=True)
        else:
            x = oracle.block_fwd(w, p, x, fused=True)
        if b == ra:
            r = oracle.token_pair(w, x)
            z = r
        print(f"oracle block {b + 1}/{saved['blocks']} done, {time.time() - t0:.0f} s", flush=True)
    if state is not None:
        inside = z is not None
        torch.save({"x": None if inside else x, "z": z, "r": None, "next_block": last}, state)
    if last < saved["blocks"]:
        return 0
    if z is not None:
        x = oracle.token_restore(w, x, z, r)
    g = saved["x_out"]
    err = relerr(g, x)
    du, dr = g.double() - x0.double(), x.double() - x0.double()
    upd = float((du - dr).abs().mean() / dr.abs().mean())
    # The GPU and the oracle add in different orders, i.e. they differ by rounding-sized amounts
    # at every stage; over many blocks such differences grow to what one rounding-sized change
    # of the input grows to.  The bar is the single-stage one, or 1.5x that measured growth.
    bar_rel = max(BF16_TOL, 1.5 * saved.get("noise_rel", 0.0))
    bar_upd = max(0.05, 1.5 * saved.get("noise_upd", 0.0))
    ok = err <= bar_rel and upd <= bar_upd
    print(f"{'int8' if saved['int8'] else 'bf16'} {saved['blocks']}-block stack: residual rel err {err:.3e} "
          f"(bar {bar_rel:.3e}), mean rel err of the total update {upd:.3e} (bar {bar_upd:.3e}); one-step input "
          f"perturbation on the GPU: {saved.get('noise_rel', float('nan')):.3e} / "
          f"{saved.get('noise_upd', float('nan')):.3e}: {'ok' if ok else 'FAIL'}", flush=True)
    if state is None:
        torch.save({"x": x, "z": None, "r": None, "next_block": last}, path + ".oracle")
    return 0 if ok else 1


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("gpu", "oracle", "join"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "gpu":
        nb = int(sys.argv[sys.argv.index("--blocks") + 1]) if "--blocks" in sys.argv else None
        wl = int(sys.argv[sys.argv.index("--workload") + 1]) if "--workload" in sys.argv else WORKLOAD
        hf = int(sys.argv[sys.argv.index("--half") + 1]) if "--half" in sys.argv else None
        gpu_phase(sys.argv[2], "--int8" in sys.argv, nb, wl, hf)
    elif sys.argv[1] == "join":
        # join the two halves written with --half 0 and --half 1 into one result file
        a, b = (torch.load(f, weights_only=True) for f in sys.argv[3:5])
        assert (a["half"], b["half"]) == (0, 1) and a["noise_rel"] == b["noise_rel"]
        a["x_out"], a["half"] = torch.cat([a["x_out"], b["x_out"]]), None
        torch.save(a, sys.argv[2])
    else:
        args = sys.argv[3:]
        first = int(args[args.index("--from") + 1]) if "--from" in args else 0
        last = int(args[args.index("--to") + 1]) if "--to" in args else None
        state = args[args.index("--state") + 1] if "--state" in args else None
        gen = args[args.index("--gen-device") + 1] if "--gen-device" in args else "cpu"
        sys.exit(oracle_phase(sys.argv[2], first, last, state, gen))
