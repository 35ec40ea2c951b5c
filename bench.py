#!/usr/bin/env python3
"""Benchmark of the denoising-transformer hot path on one MI355X.

One step = one dit_denoise call on the named workload: seeded noise (Philox, in the library),
then n Euler steps, each a full transformer forward (every block: LayerNorm + adaLN, fused
QKV + SwiGLU projection, QK RMSNorm + RoPE, attention, gated output projection) and the
output head.  Inputs (weights, text embeddings) are resident in HBM before timing starts.
Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--compute f16|bf16|fp8]
    (fp8: the block projections in row-wise E4M3 on the FP8 MFMA, everything else f16)
    python bench.py --mode copy-calibration      # elementwise copy of 1 GiB, for PMC scaling
    python bench.py --mode attention-balance     # attention, split last round vs whole units
    python bench.py --summarize-rocprof DIR ...  # rocprofv3 CSVs -> profiles/*.md (CPU only)
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3,    # MI355X dense MFMA (AMD spec)
               "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SOURCES = {"f16": ("gemm_mfma.hip", "gemm_common.h"), "bf16": ("gemm_mfma.hip", "gemm_common.h"),
                "fp8": ("gemm_fp8.hip", "gemm_common.h")}
COPY_BYTES = 1 << 30          # copy-calibration: 1 GiB read + 1 GiB written per launch
# rocprofv3 kernel names of the library's launches, by the classes the library's profiler uses
# (patterns match the mangled or demangled names rocprofv3 prints: the epilogue is the template
# argument after the operand type, followed by the token-tile height)
KERNEL_CLASSES = [("linear1", r"k_gemm(?:_v3|_mfma|8|_f32m)?I.*Li1E(?:Li\d+E)?EEv|k_gemm8<1(?:, \d+)?>"),
                  ("linear2", r"k_gemm(?:_v3|_mfma|8|_f32m)?I.*Li2E(?:Li\d+E)?EEv|k_gemm8<2(?:, \d+)?>"
                              r"|k_gemm_reduceILi2E|k_gemm_reduce<2(?:, \d+)?>"),
                  ("fp8_quant", r"k_quant_rows"),
                  ("attention", r"k_attn_"), ("qk_norm_rope", r"k_qk_norm_rope"),
                  ("ln_modulate", r"k_ln_modulate"),
                  ("final/embed", r"k_gemm_simple|k_gemm(?:_v3|_mfma|8|_f32m)?I.*Li0E(?:Li\d+E)?EEv"
                                  r"|k_gemm8<0(?:, \d+)?>|k_gemm_reduceILi0E|k_gemm_reduce<0(?:, \d+)?>|k_to_half"),
                  ("conditioning", r"k_gemv|k_timestep_embed"), ("euler noise", r"k_philox")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, cfg):
    """The oracle, as it stands, on a bounded sample of the workload: blocks 0 and 1 (double /
    per-mode stream blocks) and the first two shared blocks, each at the full token count with
    every row (float64 NumPy; BLAS threads = host cores)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from latent_flow_matching_amd import synth as S
    from oracle import dit_oracle as O

    segs = (wl.n_txt, wl.n_img, wl.n_ref)
    n = sum(segs)
    fp8 = cfg.compute == "fp8"
    f64 = lambda a: np.asarray(a, np.float64)
    dims = O.Dims(hidden=cfg.hidden, heads=cfg.heads, mlp_hidden=cfg.mlp_hidden,
                  in_channels=cfg.in_channels, time_dim=cfg.time_dim)
    pos = O.positions(wl.n_txt, wl.grid, (wl.ref_grid,) if wl.ref_grid else ())
    cond = f64(S.gen_cond(3, cfg.hidden))
    x = f64(S.gen_tokens(n, cfg.hidden))
    first_shared = cfg.n_stream_blocks
    blocks = sorted({0, min(1, cfg.n_blocks - 1), first_shared % cfg.n_blocks,
                     min(first_shared + 1, cfg.n_blocks - 1)})
    dt = 0.0
    for b in blocks:
        kind, sos, mask = O.block_plan(cfg.arch, b, cfg.n_stream_blocks)
        w = S.gen_block_weights(cfg, b)
        w.update(S.gen_weights(cfg, names={f"mod.{kind}.s{s}" for s in range(cfg.n_mod_sets(kind))}))
        sets = [O.WeightSet(*(f64(w[f"blk{b}.s{s}.{t}"]) for t in ("w1", "w2", "qn", "kn")))
                for s in range(cfg.sets_of_block(b))]
        if fp8:  # the weights' E4M3 values (a load-time step, not timed)
            sets = O.quantize_weights_fp8(sets)
        mods = O.segment_mods([f64(w[f"mod.{kind}.s{s}"]) for s in range(cfg.n_mod_sets(kind))],
                              sos, cond)
        t0 = time.perf_counter()
        x = O.block_forward(x, segs, sets, sos, mods, pos, mask, dims, act_fp8=fp8)
        dt += time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model, nproc = host_cpu()
    return {"value": len(blocks) * n / dt, "unit": "block tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "nproc": nproc,
            "sample": f"blocks {', '.join(map(str, blocks))} of the stack in sequence at "
                      f"{'+'.join(str(s) for s in segs if s)} tokens, all rows, float64 "
                      f"NumPy with {threads} BLAS threads, {dt:.1f} s of oracle time"
                      + ("; row-wise E4M3 projections" if fp8 else "")
                      + ("; with guidance the oracle runs each branch as such a sequence"
                         if wl.guidance is not None else "")}


def source_sha256(compute="f16"):
    """Hash of the GEMM's sources (kernel file and the shared epilogue header)."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES[compute]:
        with open(os.path.join(ROOT, "latent_flow_matching_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_name(kernel, workload, compute):
    return f"traffic_{kernel}_{workload}" + ("_fp8" if compute == "fp8" else "") + ".md"


def load_traffic(kernel, workload, compute="f16"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary, or None when
    there is none or the kernel source has changed since the counters were taken."""
    path = os.path.join(PROFILES, traffic_name(kernel, workload, compute))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^traffic_json: (\{.*\})$", f.read(), re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha256") != source_sha256(compute):
        return None
    return d


def copy_calibration():
    """One elementwise kernel that reads COPY_BYTES and writes COPY_BYTES, three launches; its
    FETCH_SIZE / WRITE_SIZE readings scale the counters to bytes."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": 3}), flush=True)


def _csv_rows(d, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _kernel_class(name):
    for cls, pat in KERNEL_CLASSES:
        if re.search(pat, name):
            return cls
    return None


def summarize_rocprof(args):
    """Write profiles/*.md from rocprofv3 output folders (runs on the CPU, reads CSV only)."""
    os.makedirs(PROFILES, exist_ok=True)
    wl = args.workload
    sfx = "_fp8" if args.compute == "fp8" else ""
    if args.trace_dir:
        rows = _csv_rows(args.trace_dir, "kernel_stats.csv")
        if not rows:
            raise SystemExit(f"no kernel_stats.csv under {args.trace_dir}")
        total = sum(float(r["TotalDurationNs"]) for r in rows)
        lines = [f"# Kernel trace: {wl}, {args.compute}", "",
                 "Command (from the repository root on an MI355X, after `cd /tmp && export "
                 "TMPDIR=/tmp`):", "", "```", args.trace_cmd, "```", "",
                 "| kernel class | kernel | calls | avg us | total ms | share |",
                 "|---|---|---|---|---|---|"]
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"]
            cls = _kernel_class(name) or "other"
            short = name.replace("_ZN3dit12_GLOBAL__N_1", "")
            lines.append(f"| {cls} | `{short[:70]}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                         f"{float(r['TotalDurationNs']) / total:.3f} |")
        per_class = {}
        for r in rows:
            cls = _kernel_class(r["Name"])
            if cls is None:
                continue
            c = per_class.setdefault(cls, [0.0, 0])
            c[0] += float(r["TotalDurationNs"])
            c[1] += int(r["Calls"])
        tj = {"workload": wl, "compute": args.compute, "sources_sha256": all_sources_sha256(),
              "avg_us": {k: round(v[0] / v[1] / 1e3, 2) for k, v in sorted(per_class.items())}}
        lines += ["", "Average launch duration per kernel class, read by bench.py for "
                  "`roofline.trace_avg_launch_us` while the library's sources hash to the same "
                  "value:", "", "trace_json: " + json.dumps(tj)]
        out = os.path.join(PROFILES, f"kernel_trace_{wl}{sfx}.md")
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {out}")
    if args.mfma_dir:
        acc = {}
        for r in _csv_rows(args.mfma_dir, "counter_collection.csv"):
            cls = _kernel_class(r["Kernel_Name"])
            if cls is None:
                continue
            c = acc.setdefault(cls, {})
            c.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if not acc:
            raise SystemExit(f"no counter_collection.csv rows under {args.mfma_dir}")
        lines = [f"# MFMA utilisation per kernel: {wl}, {args.compute}", "",
                 "rocprofv3 derived counters: MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / "
                 "(max(GRBM_GUI_ACTIVE) x SIMD count) x 100, the share of SIMD-cycles the matrix "
                 "cores were busy while the kernel ran; MfmaFlopsF16 = MFMA f16 MOPS x 512, the "
                 "executed matrix flops.", "", "Command (from /tmp, TMPDIR=/tmp):", "", "```",
                 args.mfma_cmd, "```", "",
                 "| kernel class | launches | MFMA busy % (mean) | executed MFMA TFLOP per launch |",
                 "|---|---|---|---|"]
        for cls, c in sorted(acc.items()):
            util = c.get("MfmaUtil", [])
            fl = c.get("MfmaFlopsF16", []) or c.get("MfmaFlopsBF16", [])
            n = max(len(util), len(fl))
            flc = f"{sum(fl) / len(fl) / 1e12:.3f}" if fl else "- (not collected)"
            lines.append(f"| {cls} | {n} | {sum(util) / len(util):.1f} | {flc} |" if util else
                         f"| {cls} | {n} | - | {flc} |")
        out = os.path.join(PROFILES, f"mfma_util_{wl}{sfx}.md")
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {out}")
    if args.fetch_dir and args.write_dir and args.copy_fetch_dir and args.copy_write_dir:
        def per_kernel(d, counter):
            acc = {}
            for r in _csv_rows(d, "counter_collection.csv"):
                if r.get("Counter_Name") != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            return acc

        def copy_kib(d, counter):
            vals = [v for k, vs in per_kernel(d, counter).items() if "mul" in k.lower()
                    for v in vs]
            if not vals:
                raise SystemExit(f"no multiply kernel with {counter} in {d}")
            return sorted(vals)[len(vals) // 2]

        f_scale = COPY_BYTES / copy_kib(args.copy_fetch_dir, "FETCH_SIZE")
        w_scale = COPY_BYTES / copy_kib(args.copy_write_dir, "WRITE_SIZE")
        fetch = per_kernel(args.fetch_dir, "FETCH_SIZE")
        write = per_kernel(args.write_dir, "WRITE_SIZE")
        lines = [f"# HBM traffic per launch: {wl}, {args.compute}", "",
                 "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one rocprofv3 pass each, "
                 "scaled by what the same counter reads for an elementwise kernel that reads and "
                 f"writes exactly {COPY_BYTES} bytes (bytes per counter unit: fetch "
                 f"{f_scale:.1f}, write {w_scale:.1f}).", "", "Commands (from /tmp, "
                 "TMPDIR=/tmp):", "", "```", *args.pmc_cmd, "```", "",
                 "| kernel class | launches | fetch MB / launch | write MB / launch |",
                 "|---|---|---|---|"]
        per_class = {}
        for k, vs in fetch.items():
            cls = _kernel_class(k)
            if cls is None:
                continue
            ws = write.get(k, [])
            c = per_class.setdefault(cls, [0, 0.0, 0.0, 0])
            c[0] += len(vs)
            c[1] += sum(vs) * f_scale
            c[2] += sum(ws) * w_scale
            c[3] += len(ws)
        out_json = None
        for cls, (n, fb, wb, nw) in sorted(per_class.items()):
            lines.append(f"| {cls} | {n} | {fb / n / 1e6:.1f} | {wb / max(nw, 1) / 1e6:.1f} |")
            if cls == args.traffic_kernel:
                out_json = {"kernel": cls, "workload": wl, "compute": args.compute,
                            "fetch_bytes_per_launch": fb / n,
                            "write_bytes_per_launch": wb / max(nw, 1),
                            "bytes_per_launch": fb / n + wb / max(nw, 1),
                            "source_sha256": source_sha256(args.compute)}
        if out_json:
            lines += ["", "Used by bench.py for `roofline.traffic` while the GEMM source hash "
                      "matches:", "", "traffic_json: " + json.dumps(out_json)]
        out = os.path.join(PROFILES, traffic_name(args.traffic_kernel, wl, args.compute))
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {out}")


def all_sources_sha256():
    """Hash of every kernel and runtime source of the library (what a kernel trace measured)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latent_flow_matching_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def load_trace_avg(kernel, workload, compute):
    """Average duration (us) of `kernel` in the committed rocprofv3 trace of this workload, or
    None when there is none or the library's sources have changed since it was taken."""
    path = os.path.join(PROFILES, f"kernel_trace_{workload}" + ("_fp8" if compute == "fp8" else "") + ".md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^trace_json: (\{.*\})$", f.read(), re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("sources_sha256") != all_sources_sha256():
        return None
    return d.get("avg_us", {}).get(kernel), path


def host_cpu():
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return model, nproc


def make_context(cfg, max_tokens):
    from latent_flow_matching_amd import dit, synth as S
    t0 = time.perf_counter()
    weights = S.gen_weights(cfg, bits=True)
    ctx = dit.DiT(cfg, weights, max_tokens=max_tokens)
    del weights
    log(f"context for {cfg.arch=} {cfg.compute=} {cfg.n_blocks} blocks created in {time.perf_counter() - t0:.1f} s")
    return ctx


def time_stack(ctx, wl, cfg, steps, warmup, profile=True):
    """Time `steps` full denoise calls of a stack workload on ctx (inputs resident in HBM).
    With profile: one more untimed step with events around every launch (the per-kernel
    breakdown), and events around the dominant kernel class during the timed steps."""
    import torch

    from latent_flow_matching_amd import synth as S
    nseq = 1 if wl.guidance is None else 2
    txt = torch.tensor(S.gen_text(wl.n_txt, cfg.hidden), device="cuda")
    txt_u = torch.tensor(S.gen_text(wl.n_txt, cfg.hidden, seed=S.SEED_T + 7), device="cuda")
    ref = (torch.tensor(S.gen_latents(wl.n_ref, cfg.in_channels, key=(1,)), device="cuda")
           if wl.n_ref else None)
    lat = torch.empty((wl.n_img, cfg.in_channels), device="cuda")
    ref_grid = wl.ref_grid or (0, 0)
    feat = (torch.tensor(S.gen_normal((wl.n_txt, cfg.txt_feat_dim), S.SEED_T, (5,)), device="cuda")
            if cfg.txt_feat_dim else None)

    def step(i):
        if feat is not None:  # the text projection runs once per image, inside the step
            ctx.text_features(feat, txt)
        if nseq == 2:
            ctx.denoise_cfg(lat, txt, txt_u, wl.grid, wl.steps, wl.guidance, seed=1000 + i,
                            ref_lat=ref, ref_grid=ref_grid)
        else:
            ctx.denoise(lat, txt, wl.grid, wl.steps, seed=1000 + i, ref_lat=ref, ref_grid=ref_grid)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    launches = wl.steps * (cfg.n_blocks * 7 + 8 + 4 * nseq) + 64  # room for fp8 and sequential blocks
    prof, dom = None, None
    if profile:
        ctx.profile_start(launches)
        step(warmup)
        torch.cuda.synchronize()
        prof = ctx.profile_stop()
        dom = max((k for k in prof if prof[k][2] > 0), key=lambda k: prof[k][0])
        ctx.profile_start(steps * launches, kernels=dom)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # an event between consecutive steps as well, for the per-step median (the total is the
    # span of the first and last events, as before)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)]
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(warmup + 1 + i)
        if i + 1 < steps:
            marks[i].record()
    end.record()
    torch.cuda.synchronize()
    timed = ctx.profile_stop() if profile else None
    ms = start.elapsed_time(end)
    evs = [start, *marks, end]
    each = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    assert torch.isfinite(lat).all(), "non-finite latents"
    return {"ms": ms, "steps": steps, "prof": prof, "timed": timed, "dom": dom, "nseq": nseq,
            "each_ms": each}


def stack_flops(wl, cfg):
    """GEMM + attention flops of one denoise call (all steps, both branches with guidance)."""
    from latent_flow_matching_amd import synth as S
    segs = (wl.n_txt, wl.n_img, wl.n_ref)
    segs = tuple(x for x in segs if x)
    per_mode = cfg.arch == S.ARCH_FLUX3
    fl = (cfg.n_stream_blocks * S.flops_per_block(segs, cfg.hidden, cfg.mlp_hidden, per_mode) +
          cfg.n_shared_blocks * S.flops_per_block(segs, cfg.hidden, cfg.mlp_hidden, False))
    return fl * wl.steps * (1 if wl.guidance is None else 2)


def stack_summary(wl, cfg, r, mfma_peak):
    ms_step = r["ms"] / r["steps"]
    tf = stack_flops(wl, cfg) / (ms_step * 1e-3) / 1e12
    toks = wl.n_tokens * r["nseq"] * cfg.n_blocks * wl.steps / (ms_step * 1e-3)
    each = sorted(r["each_ms"])
    out = {"ms_per_step": round(ms_step, 3), "ms_per_step_median": round(each[len(each) // 2], 3),
           "block_tokens_per_s": round(toks, 1),
           "tflops": round(tf, 1), "pct_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 2)}
    if mfma_peak:
        out["pct_measured_peak"] = round(100 * tf / mfma_peak, 2)
    return out


def attention_balance(reps=20):
    """Attention of a FLUX.2 double and single block at 512 text + 1024 / 4096 image tokens
    and of a FLUX.3 joint block at 512 + 4096 + 4096 tokens, with the launcher's default
    (whole units, the last round split when it is under 40% full) and with one workgroup per
    unit (DIT_ATTN_GRID=0): the measurements behind that rule."""
    from dataclasses import replace

    import torch

    from latent_flow_matching_amd import dit, synth as S
    out = {}
    for name, base, segs in (("512txt_1024img", S.FLUX2_KLEIN, (512, 1024, 0)),
                             ("512txt_4096img", S.FLUX2_KLEIN, (512, 4096, 0)),
                             ("512txt_4096img_4096ref_joint", S.FLUX3_KLEIN, (512, 4096, 4096))):
        blocks = (0,) if base is S.FLUX3_KLEIN else (0, 1)
        cfg = replace(base, n_stream_blocks=0 if base is S.FLUX3_KLEIN else 1, n_shared_blocks=1)
        n = sum(segs)
        w = S.gen_weights(cfg, bits=True)
        row = {}
        for mode, grid in (("default", None), ("whole_units", "0")):
            if grid is None:
                os.environ.pop("DIT_ATTN_GRID", None)
            else:
                os.environ["DIT_ATTN_GRID"] = grid
            ctx = dit.DiT(cfg, w, max_tokens=n)
            x = torch.tensor(S.gen_tokens(n, cfg.hidden), device="cuda")
            pos = torch.zeros((n, 4), device="cuda")
            cond = torch.tensor(S.gen_cond(sum(1 for v in segs if v), cfg.hidden), device="cuda")
            for _ in range(3):
                for b in blocks:
                    ctx.block_forward(b, x, *segs, pos, cond)
            torch.cuda.synchronize()
            ctx.profile_start(4000, kernels="attention")
            for _ in range(reps):
                for b in blocks:
                    ctx.block_forward(b, x, *segs, pos, cond)
            torch.cuda.synchronize()
            ms, cnt, _, _ = ctx.profile_stop()["attention"]
            row[mode + "_us"] = round(ms / cnt * 1e3, 1)
            ctx.close()
        os.environ.pop("DIT_ATTN_GRID", None)
        out[name] = row
        log(f"  attention {name}: {row}")
    print(json.dumps({"mode": "attention-balance", "attention": out}), flush=True)


def time_block_workload(wl, steps=20, warmup=3):
    """One block of a single-block configuration through dit_block_forward (its modulation
    GEMVs included): us per call, and the bytes it must stream, W1 and W2 of its weight sets
    and their modulation projections, over that time (these configurations are bound by that
    weight stream).  The RoPE coordinates are zeros: their values do not change the work."""
    import torch

    from latent_flow_matching_amd import synth as S
    cfg = wl.model
    n = wl.n_tokens
    ctx = make_context(cfg, n)
    d, f = cfg.hidden, cfg.mlp_hidden
    kind = 0 if cfg.n_stream_blocks else 1
    sets = cfg.sets_of_block(0)
    es = 4 if cfg.compute == "f32" else 2
    wbytes = es * (sets * ((3 * d + 2 * f) * d + d * (d + f)) + cfg.n_mod_sets(kind) * 3 * d * d)
    x = torch.tensor(S.gen_tokens(n, d), device="cuda")
    pos = torch.zeros((n, 4), device="cuda")
    segs = (wl.n_txt, wl.n_img, wl.n_ref)
    cond = torch.tensor(S.gen_cond(sum(1 for v in segs if v), d), device="cuda")
    for _ in range(warmup):
        ctx.block_forward(0, x, *segs, pos, cond)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        ctx.block_forward(0, x, *segs, pos, cond)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ctx.close()
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / steps
    each = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
    fl = S.flops_per_block(tuple(v for v in segs if v), d, f, False)
    return {"us_per_block": round(us, 1), "us_per_block_median": round(each[steps // 2], 1),
            "bound": "hbm", "weight_bytes": wbytes,
            "gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "tflops": round(fl / (us * 1e-6) / 1e12, 2), "operands": cfg.compute,
            "block": "double" if kind == 0 else "single"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="flux2_stack_512txt_4096img_4step")
    ap.add_argument("--compute", default="f16", choices=["f16", "bf16", "fp8"])
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--extras", default="on", choices=["on", "off"],
                    help="also time the other configurations (bf16 operands, 512x512, FLUX.3 "
                         "with a reference, the single double and single blocks)")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy-calibration", "attention-balance"])
    ap.add_argument("--summarize-rocprof", action="store_true")
    ap.add_argument("--trace-dir")
    ap.add_argument("--trace-cmd", default="")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--pmc-cmd", action="append", default=[])
    ap.add_argument("--traffic-kernel", default="linear1")
    ap.add_argument("--mfma-dir")
    ap.add_argument("--mfma-cmd", default="")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    from dataclasses import replace

    import torch

    if args.mode == "copy-calibration":
        torch.cuda.set_device(0)
        copy_calibration()
        return
    if args.mode == "attention-balance":
        torch.cuda.set_device(0)
        attention_balance()
        return

    from latent_flow_matching_amd import dit, synth as S

    wl = S.WORKLOADS[args.workload]
    if wl.blocks != "stack":
        raise SystemExit(f"{args.workload} is a single-block configuration; it is timed with the "
                         "extras of a stack workload")
    cfg = replace(wl.model, compute=args.compute)
    torch.cuda.set_device(0)
    mfma = {}
    for c in ("f16", "bf16"):
        tf, ghz = dit.mfma_rate(c)
        mfma[c] = {"tflops": round(tf, 1), "implied_clock_ghz": round(ghz, 3)}
        log(f"sustained 16x16x32 MFMA rate, {c}: {tf:.1f} TFLOP/s (implies {ghz:.2f} GHz at one "
            f"MFMA per 16 cycles per SIMD)")
    mpeak = mfma["bf16" if args.compute == "bf16" else "f16"]["tflops"] if args.compute != "fp8" else None

    nseq = 1 if wl.guidance is None else 2
    ctx = make_context(cfg, wl.n_tokens * nseq)
    r = time_stack(ctx, wl, cfg, args.steps, args.warmup)
    prof, dom, ms = r["prof"], r["dom"], r["ms"]
    n = wl.n_tokens
    per_step_ms = ms / args.steps
    blocks = cfg.n_blocks
    block_tokens = n * nseq * blocks * wl.steps * args.steps
    # headline: GEMM + attention flops of the timed steps over their whole wall time (norms,
    # RoPE, conditioning, output head and Euler update included in the time)
    total_flops = sum(prof[k][2] for k in ("linear1", "linear2", "attention")) * args.steps
    tflops = total_flops / (ms * 1e-3) / 1e12
    # the metric is a share of the bf16 MFMA peak whatever the operand type
    peak = PEAK_TFLOPS["bf16"]
    kernels = {}
    step_ms = sum(v[0] for v in prof.values())
    for k, (kms, cnt, fl, by) in prof.items():
        if cnt == 0:
            continue
        e = {"avg_us": round(kms / cnt * 1e3, 2), "launches": cnt,
             "share": round(kms / step_ms, 4)}
        if fl:
            e["tflops"] = round(fl / (kms * 1e-3) / 1e12, 1)
        if by:
            e["gbs"] = round(by / (kms * 1e-3) / 1e9, 1)
        kernels[k] = e
        log(f"  {k:14s} {e}")
    dms, dcnt, dfl, _ = r["timed"][dom]  # live, over the timed steps
    achieved = dfl / dcnt / (dms / dcnt * 1e-3) / 1e12
    tr = load_traffic(dom, wl.name, args.compute)
    # a contraction is priced at the peak of its own operand type
    dpeak = PEAK_TFLOPS["fp8" if args.compute == "fp8" and dom in ("linear1", "linear2") else
                        ("f32" if args.compute == "f32" else "bf16")]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": dpeak,
                "unit": "TFLOP/s", "frac": round(achieved / dpeak, 4),
                "traffic": round(tr["bytes_per_launch"]) if tr else None,
                "flops_per_launch": dfl / dcnt, "avg_launch_us": round(dms / dcnt * 1e3, 2),
                "avg_launch_source": "hipEvents around every launch of this kernel in the timed steps"}
    if dom == "linear1" and args.compute != "f32":
        # the launch also runs QK-RMSNorm, RoPE and the V transpose in its epilogue; the flops
        # counted are the projection's only
        roofline["epilogue_includes"] = "SwiGLU, QK-RMSNorm + RoPE, V transpose (not in flops_per_launch)"
    if tr:
        roofline["traffic_source"] = "profiles/" + traffic_name(dom, wl.name, args.compute)
    trace = load_trace_avg(dom, wl.name, args.compute)
    if trace and trace[0]:
        t_us = trace[0]
        roofline["trace_avg_launch_us"] = round(t_us, 2)
        roofline["trace_frac"] = round(dfl / dcnt / (t_us * 1e-6) / 1e12 / dpeak, 4)
        roofline["trace_source"] = os.path.relpath(trace[1], ROOT)
    if mpeak and dom != "fp8_quant":
        roofline["frac_of_measured_peak"] = round(achieved / mpeak, 4)

    result = {
        "metric": "DiT block tokens/sec and attention+GEMM TFLOP/s (% bf16 MFMA peak)",
        "value": round(block_tokens / (ms * 1e-3), 1),
        "unit": "block tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(per_step_ms, 3),
        "ms_per_step_median": round(sorted(r["each_ms"])[args.steps // 2], 3),
        "ms_each_step": [round(v, 3) for v in r["each_ms"]],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.compute, "data": "synthetic",
        "config": {"workload": wl.name, "tokens": n * nseq, "sequences": nseq,
                   "guidance": wl.guidance, "n_txt": wl.n_txt, "n_img": wl.n_img,
                   "n_ref": wl.n_ref, "blocks": blocks, "euler_steps": wl.steps,
                   "operands": {"f16": "fp16 activations, bf16 weights held exactly in fp16",
                                "bf16": "bf16 activations and weights",
                                "fp8": "E4M3 row-wise block projections, the rest fp16"}[args.compute],
                   "weights": "e4m3 row-wise (from bf16)" if args.compute == "fp8" else "bf16",
                   "accumulate": "f32", "parallelism": "none"},
        "tflops": round(tflops, 1),
        "pct_peak": round(100 * tflops / peak, 2),
        "mfma_measured": mfma,
        "kernels": kernels,
        "roofline": roofline,
    }
    if mpeak:
        result["pct_measured_peak"] = round(100 * tflops / mpeak, 2)
    extras = {}
    if args.extras == "on" and args.workload == "flux2_stack_512txt_4096img_4step" and args.compute == "f16":
        # 512x512 px on the same model (the context's workspace covers it)
        c3 = S.WORKLOADS["flux2_stack_512txt_1024img_4step"]
        r3 = time_stack(ctx, c3, cfg, max(3, args.steps // 2), 2, profile=False)
        extras[c3.name] = stack_summary(c3, cfg, r3, mpeak)
    ctx.close()
    if args.extras == "on" and args.workload == "flux2_stack_512txt_4096img_4step" and args.compute == "f16":
        # the same workload with bf16 MFMA operands
        cb = replace(cfg, compute="bf16")
        ctx = make_context(cb, wl.n_tokens)
        rb = time_stack(ctx, wl, cb, max(3, args.steps // 2), 2, profile=False)
        ctx.close()
        extras[wl.name + "_bf16_operands"] = stack_summary(wl, cb, rb, mfma["bf16"]["tflops"])
        # FLUX.3 with one 1024x1024 reference, one step
        c5 = S.WORKLOADS["flux3_stack_512txt_4096img_4096ref_1step"]
        ctx = make_context(c5.model, c5.n_tokens)
        r5 = time_stack(ctx, c5, c5.model, max(3, args.steps // 2), 2, profile=False)
        ctx.close()
        extras[c5.name] = stack_summary(c5, c5.model, r5, mpeak)
        for name in ("double_block_bf16_128txt_256img", "single_block_fp32_32txt_16img"):
            extras[name] = time_block_workload(S.WORKLOADS[name])
    if extras:
        result["other_workloads"] = extras
        for k, v in extras.items():
            log(f"  {k}: {v}")
    if args.cpu_baseline == "on":
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(wl, cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
