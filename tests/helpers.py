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
# Row-wise E4M3 blocks, judged on the block update u = out - x.  The GPU's inputs to the E4M3
# quantizer differ from the oracle's by the fp16-level error of attention and linear1, and
# every difference that crosses a rounding boundary moves one value by a whole E4M3 step
# (up to 2^-3 of it).  A CPU emulation of just that (the oracle block with relative noise
# 1e-3 / 2e-4 on the attention / SwiGLU halves of linear2's input) gives RMS errors of
# 0.4-0.7% and max errors of 6-14% of RMS(u); the bars keep about 3x and 1.5x margin.
FP8_UPDATE_RMS_TOL = 2e-2
FP8_UPDATE_MAX_TOL = 2e-1
# Sequentially wired double blocks at full width compound those flips: the attention half's
# error reaches the second LayerNorm, whose E4M3 codes then flip as well, and so on through
# the MLP half.  The same emulation on that block (512 + 4096 tokens) gives 3.8% RMS and 38%
# max; the bars keep about 2x and 1.6x margin.
FP8_SEQ_UPDATE_RMS_TOL = 8e-2
FP8_SEQ_UPDATE_MAX_TOL = 6e-1
BF16_OPERAND_TOL = 5e-2   # bf16 MFMA operands at full width: rounding of xm and the SwiGLU
                           # output alone exceeds 2e-2 (CPU emulation of the rounding points)

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


def oracle_model(cfg, w) -> O.Model:
    m = O.Model(arch=cfg.arch, dims=dims_of(cfg), n_stream=cfg.n_stream_blocks,
                n_shared=cfg.n_shared_blocks, img_in=f64(w["img_in"]), temb_l1=f64(w["temb.l1"]),
                temb_l2=f64(w["temb.l2"]), final_mod=f64(w["final.mod"]),
                final_out=f64(w["final.out"]))
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
    mods = O.segment_mods(oracle_mod_sets(cfg, w, kind), sos, [f64(c) for c in cond])
    mask = default_mask if mask is None else mask
    fp8 = cfg.compute == "fp8"
    if cfg.double_wiring and kind == 0:
        return O.block_forward_sequential(f64(x), segs, oracle_sets(cfg, w, b), sos, mods,
                                          f64(pos), mask, dims_of(cfg), rows=rows, act_fp8=fp8)
    return O.block_forward(f64(x), segs, oracle_sets(cfg, w, b), sos, mods, f64(pos), mask,
                           dims_of(cfg), rows=rows, act_fp8=fp8)


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)."""
    ref = f64(ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(f64(got) - ref))) / rms


def tol(cfg, full_width=True) -> float:
    if cfg.compute == "fp8":
        return FP8_TOL
    if cfg.compute == "f32":
        return F32_TOL
    if cfg.compute == "bf16" and full_width:
        return BF16_OPERAND_TOL
    return BF16_TOL


def gpu_weights(cfg, w32):
    """Upload form of the float32 weights: bf16 bit patterns for bf16 runs."""
    if cfg.bf16:
        return {k: S.bf16_bits(v) for k, v in w32.items()}
    return w32
