"""Error model of the row-wise E4M3 ("fp8r") blocks, and the parity bars derived from it.

    python tests/golden/fp8_error_model.py        (writes tests/golden/fp8_error_model.json)

The oracle's E4M3 block is exact float64 arithmetic on E4M3 codes.  The GPU path differs from
it in two ways:
  1. its own 16-bit roundings before the quantizers: q, k, v are stored as fp16 (before and
     after the QK RMSNorm + RoPE), the softmax numerators P are fp16 operands while the row
     sums stay fp32, the attention output and the SwiGLU output are stored as fp16, and the
     LayerNorm runs in fp32;
  2. as a consequence, E4M3 code flips: a quantizer input that differs from the oracle's by d
     crosses a rounding boundary with probability about |d| / step and then moves by one whole
     E4M3 step (up to 2^-3 of the value); every other code is identical to the oracle's.
This script applies exactly those rounding points around the oracle's own functions (nothing
of the GPU path is run or imported), measures the update error of each block test case, and
sets the bars at twice the emulated RMS and max errors.  The bars are fixed here, before and
independently of any GPU run; the GPU tests read them from the JSON.

Block cases: update error = |out - oracle| over the block update u = oracle - x, as RMS and as
max, both divided by RMS(u).  Whole calls (a forward, sampling loops with guidance or a flow
map) run the oracle's own loop with the emulated blocks, fp16 latents into the input
projection and an fp16 operand into the output head; their metric is max |error| / RMS of the
velocity or of the accumulated latent update.
"""
from __future__ import annotations

import json
import math
import os
import sys
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from latent_flow_matching_amd import synth as S  # noqa: E402  (seeded inputs only)
from oracle import dit_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_error_model.json")
MARGIN = 2.0


def r16(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def r32(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def emulated_block(x, segs, sets, sos, mods, pos, mask, dims, rows=None):
    """O.block_forward with act_fp8, plus the 16-bit path's rounding points listed above."""
    n, d = x.shape
    nh, hd, f = dims.heads, dims.head_dim, dims.mlp_hidden
    seg = O.segment_ids(*segs)
    y = O.layer_norm(x, dims.ln_eps)
    xm = np.empty_like(y)
    for s in range(3):
        sel = seg == s
        if sel.any():
            shift, scale, _ = O.split_modulation(mods[s], d)
            xm[sel] = y[sel] * (1.0 + scale) + shift
    xm = O.fp8_round_rows(r32(xm))
    h = np.empty((n, 3 * d + 2 * f))
    for s in range(3):
        sel = seg == s
        if sel.any():
            h[sel] = xm[sel] @ sets[sos[s]].w1.T
    q = r16(h[:, 0:d]).reshape(n, nh, hd)
    k = r16(h[:, d:2 * d]).reshape(n, nh, hd)
    v = r16(h[:, 2 * d:3 * d]).reshape(n, nh, hd)
    qn, kn = np.empty_like(q), np.empty_like(k)
    for s in range(3):
        sel = seg == s
        if sel.any():
            qn[sel] = O.rms_norm(q[sel], sets[sos[s]].qn, dims.rms_eps)
            kn[sel] = O.rms_norm(k[sel], sets[sos[s]].kn, dims.rms_eps)
    ang = O.rope_angles(pos, dims.rope_theta)
    qn = r16(O.apply_rope(qn, ang))
    kn = r16(O.apply_rope(kn, ang))
    rows = np.arange(n) if rows is None else np.asarray(rows)
    o = np.empty((rows.shape[0], nh, hd))
    for hh in range(nh):
        sc = (qn[rows, hh, :] @ kn[:, hh, :].T) / math.sqrt(hd)
        if mask != O.MASK_FULL:
            sc = np.where(seg[rows][:, None] == seg[None, :], sc, -np.inf)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        o[:, hh, :] = (r16(p) @ v[:, hh, :]) / p.sum(axis=1, keepdims=True)
    m = r16(O.silu(h[rows, 3 * d:3 * d + f]) * h[rows, 3 * d + f:])
    cat = O.fp8_round_rows(np.concatenate([r16(o.reshape(rows.shape[0], d)), m], axis=1))
    out = x[rows].copy()
    for s in range(3):
        sel = seg[rows] == s
        if sel.any():
            _, _, gate = O.split_modulation(mods[s], d)
            out[sel] = out[sel] + gate * (cat[sel] @ sets[sos[s]].w2.T)
    return out


def emulated_sequential(x, segs, sets, sos, mods6, pos, mask, dims, rows=None):
    """The sequentially wired double block, built like O.block_forward_sequential from two
    emulated halves (the attention half on all rows: the MLP half needs every row's update
    only when rows is None)."""
    d, f = dims.hidden, dims.mlp_hidden
    seg = O.segment_ids(*segs)
    attn = [O.WeightSet(np.concatenate([ws.w1[:3 * d], np.zeros((2 * f, d))]),
                        np.concatenate([ws.w2[:, :d], np.zeros((d, f))], axis=1), ws.qn, ws.kn)
            for ws in sets]
    mlp = [O.WeightSet(np.concatenate([np.zeros((3 * d, d)), ws.w1[3 * d:]]),
                       np.concatenate([np.zeros((d, d)), ws.w2[:, d:]], axis=1), ws.qn, ws.kn)
           for ws in sets]
    x1 = emulated_block(x, segs, attn, sos, [m[:3 * d] for m in mods6], pos, mask, dims, rows)
    if rows is None:
        return emulated_block(x1, segs, mlp, sos, [m[3 * d:] for m in mods6], pos, mask, dims)
    rows = np.asarray(rows)
    sub = tuple(int(np.sum(seg[rows] == s)) for s in range(3))
    return emulated_block(x1, sub, mlp, sos, [m[3 * d:] for m in mods6], pos[rows], mask, dims)


class emulation:
    """Within this context the oracle's forward and sampling loops run the emulated blocks,
    round the latents to fp16 before the input projection and the output head's modulated
    LayerNorm to fp16 before its projection (the 16-bit operands of those GEMMs)."""

    def __enter__(self):
        self.saved = (O.forward, O.block_forward, O.block_forward_sequential, O.final_layer)
        fwd, blk, seq, fin = self.saved

        def forward(model, lat, txt, grid, t, ref_lat=None, ref_grid=None, **kw):
            return fwd(model, r16(lat), txt, grid, t, None if ref_lat is None else r16(ref_lat),
                       ref_grid, **kw)

        def block_forward(x, segs, sets, sos, mods, pos, mask, dims, rows=None, act_fp8=False):
            if not act_fp8:
                return blk(x, segs, sets, sos, mods, pos, mask, dims, rows=rows)
            return emulated_block(x, segs, sets, sos, mods, pos, mask, dims, rows)

        def block_forward_sequential(x, segs, sets, sos, mods6, pos, mask, dims, rows=None,
                                     act_fp8=False):
            if not act_fp8:
                return seq(x, segs, sets, sos, mods6, pos, mask, dims, rows=rows)
            return emulated_sequential(x, segs, sets, sos, mods6, pos, mask, dims, rows)

        def final_layer(x_img, cond_img, w_fmod, w_out, eps):
            d = x_img.shape[1]
            fm = w_fmod @ O.silu(cond_img)
            y = O.layer_norm(x_img, eps) * (1.0 + fm[d:2 * d]) + fm[0:d]
            return r16(y) @ w_out.T

        O.forward, O.block_forward = forward, block_forward
        O.block_forward_sequential, O.final_layer = block_forward_sequential, final_layer
        return self

    def __exit__(self, *exc):
        O.forward, O.block_forward, O.block_forward_sequential, O.final_layer = self.saved
        return False


def sample_rows(n, k=24, seed=0):
    """The rows the full-width GPU tests compare (both ends and k random rows)."""
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], r.choice(n, k, replace=False)]))


TINY2 = replace(S.FLUX2_KLEIN, hidden=256, heads=2, mlp_hidden=256, in_channels=64, time_dim=64,
                n_stream_blocks=1, n_shared_blocks=1, compute="fp8")
TINY3 = replace(TINY2, arch=S.ARCH_FLUX3)
TINY3_FM = replace(TINY3, flow_map=True, txt_feat_dim=20480)
FULL2 = replace(S.FLUX2_KLEIN, n_stream_blocks=1, n_shared_blocks=1, compute="fp8")
FULL3 = replace(S.FLUX3_KLEIN, n_stream_blocks=1, n_shared_blocks=1, compute="fp8")

# name -> (model, block, n_txt, image grid, reference grid, sampled rows?)
CASES = {
    "tiny_flux2_stream": (TINY2, 0, 77, (13, 11), None, False),
    "tiny_flux2_shared": (TINY2, 1, 77, (13, 11), None, False),
    "tiny_flux3_stream": (TINY3, 0, 77, (13, 11), (9, 10), False),
    "tiny_flux3_shared": (TINY3, 1, 77, (13, 11), (9, 10), False),
    "tiny_sequential_double": (replace(TINY2, double_wiring=True), 0, 37, (9, 11), (5, 6), False),
    "flux2_double_512txt_4096img": (FULL2, 0, 512, (64, 64), None, True),
    "flux2_single_512txt_4096img": (FULL2, 1, 512, (64, 64), None, True),
    "flux2_double_512txt_1024img": (FULL2, 0, 512, (32, 32), None, True),
    "flux2_single_512txt_1024img": (FULL2, 1, 512, (32, 32), None, True),
    "flux3_per_mode_512txt_4096img_4096ref": (FULL3, 0, 512, (64, 64), (64, 64), True),
    "flux3_joint_512txt_4096img_4096ref": (FULL3, 1, 512, (64, 64), (64, 64), True),
}


# whole calls: name -> (model, kind of call); their metric is max |error| / RMS(reference) of the
# velocity (forward) or of the accumulated latent update (sampling loops)
CALLS = {
    "tiny_forward_flux2": (TINY2, "forward"),
    "tiny_forward_flux3": (TINY3, "forward"),
    "tiny_denoise_cfg_flux3": (TINY3, "denoise_cfg"),
    "tiny_flow_map_denoise_flux3": (TINY3_FM, "denoise"),
}


def oracle_model(cfg):
    """The oracle's model of a configuration's seeded weights (E4M3 block projections)."""
    w = S.gen_weights(cfg)
    f64 = lambda a: np.asarray(a, np.float64)
    dims = O.Dims(hidden=cfg.hidden, heads=cfg.heads, head_dim=cfg.head_dim, mlp_hidden=cfg.mlp_hidden,
                  in_channels=cfg.in_channels, time_dim=cfg.time_dim)
    m = O.Model(arch=cfg.arch, dims=dims, n_stream=cfg.n_stream_blocks, n_shared=cfg.n_shared_blocks,
                img_in=f64(w["img_in"]), temb_l1=f64(w["temb.l1"]), temb_l2=f64(w["temb.l2"]),
                final_mod=f64(w["final.mod"]), final_out=f64(w["final.out"]))
    m.mods = [[f64(w[f"mod.{k}.s{s}"]) for s in range(cfg.n_mod_sets(k))] for k in (0, 1)]
    m.blocks = [O.quantize_weights_fp8([O.WeightSet(*(f64(w[f"blk{b}.s{s}.{t}"]) for t in ("w1", "w2", "qn", "kn")))
                                        for s in range(cfg.sets_of_block(b))]) for b in range(cfg.n_blocks)]
    if cfg.flow_map:
        m.temb_tgt_l1, m.temb_tgt_l2 = f64(w["temb_tgt.l1"]), f64(w["temb_tgt.l2"])
    m.fp8 = True
    return m


def call(name):
    """(reference, emulated, subtracted start) of a whole-call case, inputs as the GPU test
    draws them."""
    cfg, kind = CALLS[name]
    m = oracle_model(cfg)
    f64 = lambda a: np.asarray(a, np.float64)

    def run():
        if kind == "forward":
            lat = S.gen_latents(63, cfg.in_channels)
            ref = S.gen_latents(30, cfg.in_channels, key=(1,))
            txt = S.gen_text(50, cfg.hidden)
            return O.forward(m, f64(lat), f64(txt), (9, 7), float(np.float32(0.75)), f64(ref), (6, 5)), 0.0
        noise = f64(S.gen_latents(48, cfg.in_channels, key=(2,)))
        txt = f64(S.gen_text(20, cfg.hidden))
        if kind == "denoise_cfg":
            ref = f64(S.gen_latents(16, cfg.in_channels, key=(1,)))
            txt_u = f64(S.gen_text(20, cfg.hidden, seed=S.SEED_T + 7))
            return O.denoise_cfg(m, noise, txt, txt_u, (8, 6), 3, 2.5, ref, (4, 4)), noise
        ref = f64(S.gen_latents(16, cfg.in_channels, key=(3,)))
        return O.denoise(m, noise, txt, (8, 6), 4, ref, (4, 4)), noise

    want, start = run()
    with emulation():
        emu, _ = run()
    return want, emu, start


def evaluate_call(name):
    want, emu, start = call(name)
    ref = want - start
    rms = float(np.sqrt(np.mean(ref * ref)))
    return {"emulated_max": float(np.max(np.abs((emu - start) - ref))) / rms}


def case_inputs(name):
    """Seeded inputs of a case, exactly as the GPU test draws them."""
    cfg, b, n_txt, grid, ref_grid, sampled = CASES[name]
    segs = (n_txt, grid[0] * grid[1], 0 if ref_grid is None else ref_grid[0] * ref_grid[1])
    n = sum(segs)
    x = S.gen_tokens(n, cfg.hidden, key=(0,))
    cond = S.gen_cond(3, cfg.hidden)
    pos = O.positions(n_txt, grid, (ref_grid,) if ref_grid else ())
    rows = sample_rows(n) if sampled else None
    return cfg, b, segs, x, cond, pos, rows


def evaluate(name):
    cfg, b, segs, x, cond, pos, rows = case_inputs(name)
    kind, sos, mask = O.block_plan(cfg.arch, b, cfg.n_stream_blocks)
    names = {f"blk{b}.s{s}.{t}" for s in range(cfg.sets_of_block(b)) for t in ("w1", "w2", "qn", "kn")}
    names |= {f"mod.{kind}.s{s}" for s in range(cfg.n_mod_sets(kind))}
    w = S.gen_weights(cfg, names=names)
    f64 = lambda a: np.asarray(a, np.float64)
    sets = O.quantize_weights_fp8([O.WeightSet(*(f64(w[f"blk{b}.s{s}.{t}"]) for t in ("w1", "w2", "qn", "kn")))
                                   for s in range(cfg.sets_of_block(b))])
    mods = O.segment_mods([f64(w[f"mod.{kind}.s{s}"]) for s in range(cfg.n_mod_sets(kind))], sos,
                          [f64(c) for c in cond])
    dims = O.Dims(hidden=cfg.hidden, heads=cfg.heads, head_dim=cfg.head_dim, mlp_hidden=cfg.mlp_hidden,
                  in_channels=cfg.in_channels, time_dim=cfg.time_dim)
    x = f64(x)
    if cfg.double_wiring and kind == 0:
        ref = O.block_forward_sequential(x, segs, sets, sos, mods, pos, mask, dims, rows=rows, act_fp8=True)
        emu = emulated_sequential(x, segs, sets, sos, mods, pos, mask, dims, rows)
    else:
        ref = O.block_forward(x, segs, sets, sos, mods, pos, mask, dims, rows=rows, act_fp8=True)
        emu = emulated_block(x, segs, sets, sos, mods, pos, mask, dims, rows)
    xs = x if rows is None else x[rows]
    u = ref - xs
    rms_u = float(np.sqrt(np.mean(u * u)))
    e = emu - ref
    return {"emulated_rms": float(np.sqrt(np.mean(e * e))) / rms_u,
            "emulated_max": float(np.max(np.abs(e))) / rms_u}


def main(names=None):
    res = {}
    if os.path.exists(OUT):
        with open(OUT) as fh:
            res = json.load(fh).get("cases", {})
    for name in names or list(CASES) + list(CALLS):
        r = evaluate(name) if name in CASES else evaluate_call(name)
        if "emulated_rms" in r:
            r["bar_rms"] = MARGIN * r["emulated_rms"]
        r["bar_max"] = MARGIN * r["emulated_max"]
        res[name] = r
        print(name, {k: f"{v:.3e}" for k, v in r.items()}, flush=True)
    doc = {"description": "Row-wise E4M3 parity bars: twice the error of the oracle's E4M3 block "
                          "(or whole call) with the 16-bit path's rounding points applied, against "
                          "the oracle.  Blocks: RMS and max of the update error over RMS of the "
                          "update; whole calls: max error over RMS of the velocity or latent "
                          "update.  Written by tests/golden/fp8_error_model.py, which runs only "
                          "the oracle.",
           "margin": MARGIN, "cases": {k: res[k] for k in list(CASES) + list(CALLS) if k in res}}
    with open(OUT, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or None)
