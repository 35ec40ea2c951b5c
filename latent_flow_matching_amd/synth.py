"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU oracle harness.

This module only draws random numbers and lays them out under the weight names of the C ABI.
It holds none of the transformer's arithmetic.  Both the GPU path and the oracle receive the
identical values it produces (bf16-rounded with round-to-nearest-even when the run is bf16).

Recipe (per tensor, so one block can be regenerated on its own):
  * linear weights  N(0, 0.02^2)
  * RMSNorm scales  U(0.5, 1.5)   (N(0, 0.02^2) scales would flatten every attention row)
  * tokens, text embeddings, cond vectors, latents  N(0, 1)
  * generator: NumPy PCG64 seeded with SeedSequence([seed, group, block, set, tensor]).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

ARCH_FLUX2 = 0
ARCH_FLUX3 = 1

SEED_W, SEED_X, SEED_C, SEED_T = 0, 1, 2, 3

# tensor-group codes used in the seed sequence
_G_GLOBAL, _G_MOD, _G_BLOCK, _G_DATA = 11, 12, 13, 14
_T_W1, _T_W2, _T_QN, _T_KN = 0, 1, 2, 3


@dataclass(frozen=True)
class ModelConfig:
    arch: int = ARCH_FLUX2
    hidden: int = 3072
    heads: int = 24
    head_dim: int = 128
    mlp_hidden: int = 9216
    in_channels: int = 128
    time_dim: int = 256
    n_stream_blocks: int = 5
    n_shared_blocks: int = 20
    bf16: bool = True            # weights are bf16 values (the checkpoint format)
    compute: str = "f16"         # MFMA operand type of the library: "f16", "bf16", "f32", or "fp8"
                                 # (row-wise E4M3 block projections, the rest as "f16")
    rope_theta: float = 10000.0
    ln_eps: float = 1e-6
    rms_eps: float = 1e-6
    txt_feat_dim: int = 0        # > 0: text features of this width are projected by txt_in
    flow_map: bool = False       # timestep-distilled model with a target-time embedding
    double_wiring: bool = False  # FLUX.2 double blocks: attention, then MLP (own LN and gate)
    mod_per_block: bool = False  # every block has its own modulation projections (blk{b}.s{s}.mod)

    @property
    def n_blocks(self) -> int:
        return self.n_stream_blocks + self.n_shared_blocks

    def sets_of_block(self, b: int) -> int:
        if b < self.n_stream_blocks:
            return 2 if self.arch == ARCH_FLUX2 else 3
        return 1

    def n_mod_sets(self, kind: int) -> int:
        if kind == 0:
            return 2 if self.arch == ARCH_FLUX2 else 3
        return 1


FLUX2_KLEIN = ModelConfig()
FLUX3_KLEIN = ModelConfig(arch=ARCH_FLUX3, n_stream_blocks=5, n_shared_blocks=28)


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    n_txt: int
    grid: tuple
    ref_grid: tuple | None
    steps: int
    blocks: str          # "one" = a single block through dit_block_forward, "stack" = full denoise
    description: str
    guidance: float | None = None  # classifier-free guidance scale: both branches as a batch of 2

    @property
    def n_img(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def n_ref(self) -> int:
        return 0 if self.ref_grid is None else self.ref_grid[0] * self.ref_grid[1]

    @property
    def n_tokens(self) -> int:
        return self.n_txt + self.n_img + self.n_ref


WORKLOADS = {
    "single_block_fp32_32txt_16img": Workload(
        "single_block_fp32_32txt_16img",
        replace(FLUX2_KLEIN, n_stream_blocks=0, n_shared_blocks=1, bf16=False, compute="f32"),
        32, (4, 4), None, 0, "one",
        "one single-stream block, 32 text + 16 image tokens (64x64 px), fp32"),
    "double_block_bf16_128txt_256img": Workload(
        "double_block_bf16_128txt_256img",
        replace(FLUX2_KLEIN, n_stream_blocks=1, n_shared_blocks=0),
        128, (16, 16), None, 0, "one",
        "one double-stream block, 128 text + 256 image tokens (256x256 px), bf16"),
    "flux2_stack_512txt_1024img_4step": Workload(
        "flux2_stack_512txt_1024img_4step", FLUX2_KLEIN, 512, (32, 32), None, 4, "stack",
        "5 double + 20 single blocks, 512 text + 1024 image tokens (512x512 px), 4 Euler steps"),
    "flux2_stack_512txt_4096img_4step": Workload(
        "flux2_stack_512txt_4096img_4step", FLUX2_KLEIN, 512, (64, 64), None, 4, "stack",
        "5 double + 20 single blocks, 512 text + 4096 image tokens (1024x1024 px), 4 Euler steps"),
    "flux3_stack_512txt_4096img_4096ref_1step": Workload(
        "flux3_stack_512txt_4096img_4096ref_1step", FLUX3_KLEIN, 512, (64, 64), (64, 64), 1,
        "stack",
        "5 per-mode + 28 joint blocks, 512 text + 4096 image + 4096 reference tokens, 1 step"),
    "flux3_distilled_512txt_4096img_16step": Workload(
        "flux3_distilled_512txt_4096img_16step",
        replace(FLUX3_KLEIN, flow_map=True, txt_feat_dim=20480), 512, (64, 64), None, 16, "stack",
        "timestep-distilled FLUX.3 (flow map, the distilled checkpoint's 16 steps, no guidance): "
        "text-encoder features [512, 20480] projected once per image, then 5 per-mode + 28 joint "
        "blocks on 512 text + 4096 image tokens per step"),
    "flux3_cfg_512txt_4096img_50step": Workload(
        "flux3_cfg_512txt_4096img_50step", FLUX3_KLEIN, 512, (64, 64), None, 50, "stack",
        "5 per-mode + 28 joint blocks, 512 text + 4096 image tokens, 50 Euler steps with "
        "classifier-free guidance 3.5 (the base checkpoint's published setting): conditional and "
        "unconditional branch as one batch of 2 sequences", guidance=3.5),
}


# ----------------------------------------------------------------------------------------
# bf16 helpers (data format only)
# ----------------------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 values, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(a))


# ----------------------------------------------------------------------------------------
# Weight table schema
# ----------------------------------------------------------------------------------------

def weight_specs(cfg: ModelConfig):
    """[(name, shape, dist, seed_key)] for every tensor of the model, in a fixed order."""
    d, f, c, td, hd = cfg.hidden, cfg.mlp_hidden, cfg.in_channels, cfg.time_dim, cfg.head_dim
    specs = [
        ("img_in", (d, c), "linear", (_G_GLOBAL, 0)),
        ("temb.l1", (d, td), "linear", (_G_GLOBAL, 1)),
        ("temb.l2", (d, d), "linear", (_G_GLOBAL, 2)),
        ("final.mod", (2 * d, d), "linear", (_G_GLOBAL, 3)),
        ("final.out", (c, d), "linear", (_G_GLOBAL, 4)),
    ]
    if cfg.flow_map:
        specs.append(("temb_tgt.l1", (d, td), "linear", (_G_GLOBAL, 5)))
        specs.append(("temb_tgt.l2", (d, d), "linear", (_G_GLOBAL, 6)))
    if cfg.txt_feat_dim:
        specs.append(("txt_in", (d, cfg.txt_feat_dim), "linear", (_G_GLOBAL, 7)))
    for kind in (0, 1):
        if (kind == 0 and cfg.n_stream_blocks == 0) or (kind == 1 and cfg.n_shared_blocks == 0):
            continue
        if cfg.mod_per_block:
            continue
        for s in range(cfg.n_mod_sets(kind)):
            rows = 6 * d if (kind == 0 and cfg.double_wiring) else 3 * d
            specs.append((f"mod.{kind}.s{s}", (rows, d), "linear", (_G_MOD, kind, s)))
    if cfg.mod_per_block:
        for b in range(cfg.n_blocks):
            kind = 0 if b < cfg.n_stream_blocks else 1
            rows = 6 * d if (kind == 0 and cfg.double_wiring) else 3 * d
            for s in range(cfg.sets_of_block(b)):
                specs.append((f"blk{b}.s{s}.mod", (rows, d), "linear", (_G_MOD, kind, s, 1000 + b)))
    for b in range(cfg.n_blocks):
        for s in range(cfg.sets_of_block(b)):
            p = f"blk{b}.s{s}"
            specs.append((p + ".w1", (3 * d + 2 * f, d), "linear", (_G_BLOCK, b, s, _T_W1)))
            specs.append((p + ".w2", (d, d + f), "linear", (_G_BLOCK, b, s, _T_W2)))
            specs.append((p + ".qn", (hd,), "norm", (_G_BLOCK, b, s, _T_QN)))
            specs.append((p + ".kn", (hd,), "norm", (_G_BLOCK, b, s, _T_KN)))
    return specs


def _rng(seed: int, key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def gen_tensor(shape, dist: str, key, seed_w: int = SEED_W, bf16: bool = True,
               bits: bool = False) -> np.ndarray:
    """One weight tensor: float32 values (bf16-rounded if bf16), or uint16 bits if bits."""
    g = _rng(seed_w, key)
    if dist == "linear":
        a = g.standard_normal(shape, dtype=np.float32)
        a *= np.float32(0.02)
    elif dist == "norm":
        a = g.uniform(0.5, 1.5, size=shape).astype(np.float32)
    else:
        raise ValueError(dist)
    if bits:
        return bf16_bits(a)
    return bf16_round(a) if bf16 else a


def gen_weights(cfg: ModelConfig, seed_w: int = SEED_W, bits: bool | None = None,
                names=None, threads: int | None = None) -> dict:
    """All (or the named) weights.  bits=True -> uint16 bf16 patterns (for upload), else
    float32 values (bf16-rounded when cfg.bf16)."""
    if bits is None:
        bits = False
    specs = [s for s in weight_specs(cfg) if names is None or s[0] in names]
    threads = threads or min(16, os.cpu_count() or 1)

    def one(spec):
        name, shape, dist, key = spec
        return name, gen_tensor(shape, dist, key, seed_w, bf16=cfg.bf16, bits=bits)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(one, specs))


def gen_block_weights(cfg: ModelConfig, b: int, seed_w: int = SEED_W) -> dict:
    names = {f"blk{b}.s{s}.{t}" for s in range(cfg.sets_of_block(b))
             for t in ("w1", "w2", "qn", "kn")}
    return gen_weights(cfg, seed_w, names=names)


# ----------------------------------------------------------------------------------------
# Activations
# ----------------------------------------------------------------------------------------

def gen_normal(shape, seed: int, key=(0,), bf16: bool = False) -> np.ndarray:
    a = _rng(seed, (_G_DATA, *key)).standard_normal(shape, dtype=np.float32)
    return bf16_round(a) if bf16 else a


def gen_tokens(n: int, d: int, seed: int = SEED_X, key=(0,)) -> np.ndarray:
    """Residual-stream tokens N(0,1) (fp32, the residual is kept in fp32)."""
    return gen_normal((n, d), seed, (1, *key))


def gen_text(n_txt: int, d: int, seed: int = SEED_T, bf16: bool = False) -> np.ndarray:
    return gen_normal((n_txt, d), seed, (2,), bf16=bf16)


def gen_cond(n: int, d: int, seed: int = SEED_C) -> np.ndarray:
    return gen_normal((n, d), seed, (3,))


def gen_latents(n_img: int, c: int, seed: int = SEED_X, key=(0,)) -> np.ndarray:
    return gen_normal((n_img, c), seed, (4, *key))


def flops_per_block(n_tokens_by_seg, d: int, f: int, mask_segment: bool) -> float:
    """Algorithmic FLOPs of one block: the two fused projections plus 4*D per attended
    (query, key) pair.  A count, not part of the computed method."""
    n = sum(n_tokens_by_seg)
    gemm = 2.0 * n * d * (3 * d + 2 * f) + 2.0 * n * (d + f) * d
    pairs = sum(x * x for x in n_tokens_by_seg) if mask_segment else n * n
    return gemm + 4.0 * d * pairs


def tiles(n: int, t: int) -> int:
    return math.ceil(n / t)
