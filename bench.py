#!/usr/bin/env python3
"""Benchmark of the denoising-transformer hot path on one MI355X.

One step = one dit_denoise call on the named workload: seeded noise (Philox, in the library),
then n Euler steps, each a full transformer forward (every block: LayerNorm + adaLN, fused
QKV + SwiGLU projection, QK RMSNorm + RoPE, attention, gated output projection) and the
output head.  Inputs (weights, text embeddings) are resident in HBM before timing starts.
Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--compute f16|bf16]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (AMD spec)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, cfg):
    """The oracle, as it stands, on a bounded sample: block 0 of the workload at its full token
    count, every row (float64 NumPy; BLAS threads = host cores)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from latent_flow_matching_amd import synth as S
    from oracle import dit_oracle as O

    segs = (wl.n_txt, wl.n_img, wl.n_ref)
    n = sum(segs)
    w = S.gen_block_weights(cfg, 0)
    w.update(S.gen_weights(cfg, names={f"mod.0.s{s}" for s in range(cfg.n_mod_sets(0))}))
    f64 = lambda a: np.asarray(a, np.float64)
    sets = [O.WeightSet(*(f64(w[f"blk0.s{s}.{t}"]) for t in ("w1", "w2", "qn", "kn")))
            for s in range(cfg.sets_of_block(0))]
    kind, sos, mask = O.block_plan(cfg.arch, 0, cfg.n_stream_blocks)
    cond = f64(S.gen_cond(3, cfg.hidden))
    mods = O.segment_mods([f64(w[f"mod.0.s{s}"]) for s in range(cfg.n_mod_sets(0))], sos, cond)
    x = f64(S.gen_tokens(n, cfg.hidden))
    pos = O.positions(wl.n_txt, wl.grid, (wl.ref_grid,) if wl.ref_grid else ())
    dims = O.Dims(hidden=cfg.hidden, heads=cfg.heads, mlp_hidden=cfg.mlp_hidden,
                  in_channels=cfg.in_channels, time_dim=cfg.time_dim)
    t0 = time.perf_counter()
    O.block_forward(x, segs, sets, sos, mods, pos, mask, dims)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": n / dt, "unit": "block tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one {'double' if cfg.arch == 0 else 'per-mode'}-stream block (block 0) "
                      f"at {'+'.join(str(s) for s in segs if s)} tokens, all rows, float64 "
                      f"NumPy/OpenBLAS, {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="flux2_stack_512txt_4096img_4step")
    ap.add_argument("--compute", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    from dataclasses import replace

    import numpy as np
    import torch

    from latent_flow_matching_amd import dit, synth as S

    wl = S.WORKLOADS[args.workload]
    if wl.blocks != "stack":
        raise SystemExit(f"{args.workload} is a parity configuration, not a bench workload")
    cfg = replace(wl.model, compute=args.compute)
    n = wl.n_tokens
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    weights = S.gen_weights(cfg, bits=True)
    log(f"weights generated in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    ctx = dit.DiT(cfg, weights, max_tokens=n)
    del weights
    log(f"context created in {time.perf_counter() - t0:.1f} s")
    txt = torch.tensor(S.gen_text(wl.n_txt, cfg.hidden), device="cuda")
    ref = (torch.tensor(S.gen_latents(wl.n_ref, cfg.in_channels, key=(1,)), device="cuda")
           if wl.n_ref else None)
    lat = torch.empty((wl.n_img, cfg.in_channels), device="cuda")
    ref_grid = wl.ref_grid or (0, 0)

    def step(i):
        ctx.denoise(lat, txt, wl.grid, wl.steps, seed=1000 + i, ref_lat=ref, ref_grid=ref_grid)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ctx.profile_start(args.steps * wl.steps * (cfg.n_blocks * 5 + 8) + 64)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    prof = ctx.profile_stop()
    ms = start.elapsed_time(end)
    assert torch.isfinite(lat).all(), "non-finite latents"

    per_step_ms = ms / args.steps
    blocks = cfg.n_blocks
    block_tokens = n * blocks * wl.steps * args.steps
    total_flops = sum(v[2] for v in prof.values())
    tflops = total_flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.compute]
    kernels = {}
    for k, (kms, cnt, fl, by) in prof.items():
        if cnt == 0:
            continue
        e = {"avg_us": round(kms / cnt * 1e3, 2), "launches": cnt,
             "share": round(kms / ms, 4)}
        if fl:
            e["tflops"] = round(fl / (kms * 1e-3) / 1e12, 1)
        if by:
            e["gbs"] = round(by / (kms * 1e-3) / 1e9, 1)
        kernels[k] = e
        log(f"  {k:14s} {e}")
    dom = max((k for k in prof if prof[k][2] > 0), key=lambda k: prof[k][0])
    dms, dcnt, dfl, _ = prof[dom]
    achieved = dfl / dcnt / (dms / dcnt * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "flops_per_launch": dfl / dcnt}

    result = {
        "metric": "DiT block tokens/sec and attention+GEMM TFLOP/s (% bf16 MFMA peak)",
        "value": round(block_tokens / (ms * 1e-3), 1),
        "unit": "block tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(per_step_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.compute, "data": "synthetic",
        "config": {"workload": wl.name, "tokens": n, "n_txt": wl.n_txt, "n_img": wl.n_img,
                   "n_ref": wl.n_ref, "blocks": blocks, "euler_steps": wl.steps,
                   "weights": "bf16", "accumulate": "f32", "parallelism": "none"},
        "tflops": round(tflops, 1),
        "pct_peak": round(100 * tflops / peak, 2),
        "kernels": kernels,
        "roofline": roofline,
    }
    if args.cpu_baseline == "on":
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(wl, cfg)
    ctx.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
