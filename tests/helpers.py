"""Shared test plumbing: build oracle models from the seeded weights, compare with the
stated tolerances, locate the built library."""
from __future__ import annotations

import os
from dataclasses import replace

import numpy as np

from latent_flow_matching_amd import synth as S
from oracle import dit_oracle as O

BF16_TOL = 2e-2   # max|gpu - oracle| <= 2e-2 * RMS(oracle) for bf16 paths
F32_TOL = 1e-4    # ... <= 1e-4 * RMS(oracle) for the fp32 path

FP8_TOL = 2e-2           # row-wise E4M3 path: forward outputs against the E4M3 oracle
FP8_BARS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_error_model.json")
BF16_OPERAND_TOL = 5e-2   # bf16 MFMA operands: the rounding points alone give 2.5-3.8e-2 of the
                           # block update (CPU emulation), so the update is held to 5e-2 at every
                           # width and the output to 5e-2 at full width

TINY2 = replace(S.FLUX2_KLEIN, hidden=256, heads=2, mlp_hidden=256, in_channels=64, time_dim=64,
                n_stream_blocks=1, n_shared_blocks=1)
TINY3 = replace(TINY2, arch=S.ARCH_FLUX3)


def lib_built() -> bool:
    from latent_flow_matching_amd import dit
    return os.path.exists(dit.LIB_PATH)


def dims_of(cfg: S.ModelConfig) -> O.Dims:
    return O.Dims(hidden=cfg.hidden, heads=cfg.heads, head_dim=cfg.head_dim,
                  mlp_hidden=cfg.mlp_hidden, in_channels=cfg.in_channels, time_dim=cfg.time_dim,
                  ln_eps=cfg.ln_eps, rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta)


def f64(a):
    return np.asarray(a, dtype=np.float64)


_FP8_SETS = {}  # E4M3 weight sets of the last weight table (quantizing full width takes seconds)


def oracle_sets(cfg, w, b):
    sets = [O.WeightSet(w1=f64(w[f"blk{b}.s{s}.w1"]), w2=f64(w[f"blk{b}.s{s}.w2"]),
                        qn=f64(w[f"blk{b}.s{s}.qn"]), kn=f64(w[f"blk{b}.s{s}.kn"]))
            for s in range(cfg.sets_of_block(b))]
    if cfg.compute != "fp8":
        return sets
    key = (id(w), cfg, b)
    if key not in _FP8_SETS:
        if len(_FP8_SETS) > 4:
            _FP8_SETS.clear()
        _FP8_SETS[key] = O.quantize_weights_fp8(sets)
    return _FP8_SETS[key]


def oracle_mod_sets(cfg, w, kind):
    return [f64(w[f"mod.{kind}.s{s}"]) for s in range(cfg.n_mod_sets(kind))]


def oracle_block_mod_sets(cfg, w, b):
    """Modulation projections of block b's weight sets: its own, or its kind's shared ones."""
    kind = 0 if b < cfg.n_stream_blocks else 1
    if cfg.mod_per_block:
        return [f64(w[f"blk{b}.s{s}.mod"]) for s in range(cfg.sets_of_block(b))]
    return oracle_mod_sets(cfg, w, kind)


def mod_names(cfg, b):
    """Weight names of block b's modulation projections."""
    kind = 0 if b < cfg.n_stream_blocks else 1
    if cfg.mod_per_block:
        return {f"blk{b}.s{s}.mod" for s in range(cfg.sets_of_block(b))}
    return {f"mod.{kind}.s{s}" for s in range(cfg.n_mod_sets(kind))}


def oracle_model(cfg, w) -> O.Model:
    m = O.Model(arch=cfg.arch, dims=dims_of(cfg), n_stream=cfg.n_stream_blocks,
                n_shared=cfg.n_shared_blocks, img_in=f64(w["img_in"]), temb_l1=f64(w["temb.l1"]),
                temb_l2=f64(w["temb.l2"]), final_mod=f64(w["final.mod"]),
                final_out=f64(w["final.out"]))
    if cfg.mod_per_block:
        m.block_mods = [oracle_block_mod_sets(cfg, w, b) for b in range(cfg.n_blocks)]
    else:
        m.mods = [oracle_mod_sets(cfg, w, 0) if cfg.n_stream_blocks else [],
                  oracle_mod_sets(cfg, w, 1) if cfg.n_shared_blocks else []]
    m.blocks = [oracle_sets(cfg, w, b) for b in range(cfg.n_blocks)]
    if cfg.flow_map:
        m.temb_tgt_l1, m.temb_tgt_l2 = f64(w["temb_tgt.l1"]), f64(w["temb_tgt.l2"])
    if cfg.txt_feat_dim:
        m.txt_in = f64(w["txt_in"])
    m.double_wiring = int(cfg.double_wiring)
    m.fp8 = cfg.compute == "fp8"
    return m


def oracle_block(cfg, w, b, x, segs, pos, cond, mask=None, rows=None):
    """Oracle output of block b for residual x, conditioning rows cond[3], positions pos."""
    kind, sos, default_mask = O.block_plan(cfg.arch, b, cfg.n_stream_blocks)
    mods = O.segment_mods(oracle_block_mod_sets(cfg, w, b), sos, [f64(c) for c in cond])
    mask = default_mask if mask is None else mask
    fp8 = cfg.compute == "fp8"
    if cfg.double_wiring and kind == 0:
        return O.block_forward_sequential(f64(x), segs, oracle_sets(cfg, w, b), sos, mods,
                                          f64(pos), mask, dims_of(cfg), rows=rows, act_fp8=fp8)
    return O.block_forward(f64(x), segs, oracle_sets(cfg, w, b), sos, mods, f64(pos), mask,
                           dims_of(cfg), rows=rows, act_fp8=fp8)


def fp8_bars(case: str) -> dict:
    """Update-error bars of a row-wise E4M3 block case, from the error model's JSON."""
    import json
    with open(FP8_BARS) as f:
        return json.load(f)["cases"][case]


def seg_cond(cond, segs):
    """The conditioning rows a block call takes: one per non-empty segment, in order."""
    return cond[[s for s in range(3) if segs[s] > 0]]


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)."""
    ref = f64(ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(f64(got) - ref))) / rms


def tol(cfg, full_width=False) -> float:
    """Bar on max |gpu - oracle| / RMS(oracle) of a block output or a forward / loop output."""
    if cfg.compute == "fp8":
        return FP8_TOL
    if cfg.compute == "f32":
        return F32_TOL
    if cfg.compute == "bf16" and full_width:
        return BF16_OPERAND_TOL
    return BF16_TOL


def tol_update(cfg) -> float:
    """Bar on the block update: max |(gpu - x) - (oracle - x)| / RMS(oracle - x), after one fp32
    rounding of the output is allowed for (update_err)."""
    if cfg.compute == "f32":
        return F32_TOL
    if cfg.compute == "bf16":
        return BF16_OPERAND_TOL
    return BF16_TOL


def update_err(got, ref, x) -> float:
    """max |got - ref| / RMS(ref - x), each element's error first reduced by one fp32 rounding
    of the output (2^-24 |ref|, the last step of x + update in the fp32 residual)."""
    got, ref, x = f64(got), f64(ref), f64(x)
    u = ref - x
    e = np.maximum(np.abs(got - ref) - 2.0 ** -24 * np.abs(ref), 0.0)
    return float(np.max(e)) / float(np.sqrt(np.mean(u * u)))


def gpu_weights(cfg, w32):
    """Upload form of the float32 weights: bf16 bit patterns for bf16 runs."""
    if cfg.bf16:
        return {k: S.bf16_bits(v) for k, v in w32.items()}
    return w32
