"""Plain CPU oracle for the FLUX.2-klein / FLUX.3-Klein denoising-transformer forward pass.

TEST INFRASTRUCTURE ONLY.  This module is the independent definition that the HIP path is
checked against.  Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the GPU library (``latent_flow_matching_amd``) never does, and this
module imports nothing from it.

Everything is NumPy float64: each step is the plain textbook definition (a matmul from the
BLAS library is the only library primitive), with no tiling, no fusion, no online softmax.
The N x N score matrix is materialised per head.

Sources (web pages; cited by title and section):
  [GN]  "Flux 2 Klein: Reine C-basierte Inferenz" (GeekNews), sections
        "Modellarchitektur und Leistung", "C-Bibliotheks-API".
  [HK]  hakusoku.com "FLUX.2-klein-4B Pure C" article, sections
        "技術詳細", "CライブラリAPI", "コマンドラインオプション".
  [KS]  "FLUX.3 Image Klein: offene Gewichte und Diffusers-Start mit Layout-Box-Steuerung",
        sections "Was sich geändert hat", "Grenzen und offene Fragen".
  [WE]  we0.ai "FLUX 3 Image Klein" specs article, checkpoint table.
  [MV]  "FLUX.3 Image Klein in Diffusers: Architektur, Layout-Steuerung und
        Systemanforderungen im Überblick" (mindverse), sections
        "Zweistufiger Transformer und Tokenisierung im Detail" (Tokens),
        "Entkoppelte Vorverarbeitung und gemeinsame Attention-Blöcke" (Blocks),
        "Modulation pro Token-Typ, Flow-Map-Destillation und 4D-RoPE" (Modulation/RoPE),
        "Einfluss von Referenzbildern auf die Sequenzlänge und Rechenzeit" (Refs),
        "Verarbeitung einzelner Prompts und Batching-Architektur in der Praxis" (Batching).

Where the pages leave a step open the plainest reading is taken; every such reading is
listed at the definition that uses it (tagged "reading:").

Parity pins (what ties each function to something other than itself) live in
tests/test_oracle_pins.py.  Functions without an independent pin say "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------------------
# Token accounting  ([MV] Tokens; [MV] Refs; [MV] Batching; [GN] "Build und Ausführung")
# ----------------------------------------------------------------------------------------

PIXELS_PER_TOKEN_SIDE = 16   # VAE /8 then 2x2 packing: one token covers 16x16 pixels ([MV] Tokens)
TEXT_PAD_MULTIPLE = 80       # prompts are padded to a multiple of 80 tokens ([MV] Batching)


def image_token_grid(height_px: int, width_px: int) -> tuple[int, int]:
    """Token grid (rows, cols) of an image: one token per 16x16 pixel patch ([MV] Tokens).

    Sides must be multiples of 16 (the FLUX.2 C tool's resolution rule, [HK] ベンチマーク
    "解像度制限"; [GN] "Build und Ausführung")."""
    if height_px <= 0 or width_px <= 0:
        raise ValueError("image sides must be positive")
    if height_px % PIXELS_PER_TOKEN_SIDE or width_px % PIXELS_PER_TOKEN_SIDE:
        raise ValueError("image sides must be multiples of 16 pixels")
    return height_px // PIXELS_PER_TOKEN_SIDE, width_px // PIXELS_PER_TOKEN_SIDE


def image_tokens(height_px: int, width_px: int) -> int:
    gh, gw = image_token_grid(height_px, width_px)
    return gh * gw


def padded_text_tokens(n_prompt_tokens: int) -> int:
    """Prompt length after padding to a multiple of 80 tokens ([MV] Batching)."""
    if n_prompt_tokens < 0:
        raise ValueError("negative prompt length")
    return TEXT_PAD_MULTIPLE * math.ceil(n_prompt_tokens / TEXT_PAD_MULTIPLE)


def tokens_per_call(n_prompt_tokens: int, out_hw: tuple[int, int],
                    ref_hws: tuple[tuple[int, int], ...] = ()) -> int:
    """Sequence length of one transformer call: padded text + output image + each reference,
    concatenated in the order text, image, reference ([MV] Blocks; [MV] Refs)."""
    n = padded_text_tokens(n_prompt_tokens) + image_tokens(*out_hw)
    for hw in ref_hws:
        n += image_tokens(*hw)
    return n


# ----------------------------------------------------------------------------------------
# 4D RoPE coordinates  ([MV] Modulation/RoPE, the three bullet points)
# ----------------------------------------------------------------------------------------

def positions(n_txt: int, grid: tuple[int, int], ref_grids: tuple[tuple[int, int], ...] = ()):
    """(t, h, w, l) coordinates for the sequence text || image || refs, float64 [N, 4].

    text token i          -> (0, 0, 0, i)
    image token (r, c)    -> (0, r, c, 0)
    ref k token (r, c)    -> (0, r, c, -(k+1))

    reading: the pages write h = row/2, w = col/2 with row/col counted in VAE-latent cells;
    two latent cells per token side (2x2 packing, [MV] Tokens) make that the integer token
    row/column r, c used here.  Tokens within an image are row-major."""
    rows = []
    for i in range(n_txt):
        rows.append((0.0, 0.0, 0.0, float(i)))
    gh, gw = grid
    for r in range(gh):
        for c in range(gw):
            rows.append((0.0, float(r), float(c), 0.0))
    for k, (rh, rw) in enumerate(ref_grids):
        for r in range(rh):
            for c in range(rw):
                rows.append((0.0, float(r), float(c), float(-(k + 1))))
    return np.array(rows, dtype=np.float64).reshape(-1, 4)


ROPE_AXES = 4          # t, h, w, l
ROPE_AXIS_DIM = 32     # 128 head dims / 4 axes ([MV] Modulation/RoPE)


def rope_angles(pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotation angles [N, 4, 16]: axis a, pair j -> pos[:, a] * theta^(-2j/32).

    reading: standard rotary frequencies within each 32-dim axis slice (RoFormer), base
    theta = 10000, axis slices in the order t, h, w, l as listed on the page."""
    j = np.arange(ROPE_AXIS_DIM // 2, dtype=np.float64)
    freqs = theta ** (-2.0 * j / ROPE_AXIS_DIM)                 # [16]
    return pos[:, :, None].astype(np.float64) * freqs[None, None, :]


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (x[2j], x[2j+1]) of every 32-dim axis slice of every head.

    x: [N, H, 128]; angles: [N, 4, 16].
    reading: adjacent-pair convention (RoFormer), rotation (a, b) -> (a cos - b sin,
    a sin + b cos)."""
    n, h, d = x.shape
    xr = x.reshape(n, h, ROPE_AXES, ROPE_AXIS_DIM // 2, 2)
    a = xr[..., 0]
    b = xr[..., 1]
    c = np.cos(angles)[:, None, :, :]
    s = np.sin(angles)[:, None, :, :]
    out = np.empty_like(xr)
    out[..., 0] = a * c - b * s
    out[..., 1] = a * s + b * c
    return out.reshape(n, h, d)


# ----------------------------------------------------------------------------------------
# Norms, activations, modulation  ([MV] Blocks; [MV] Modulation/RoPE)
# ----------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis without learned scale or shift ([MV] Modulation/RoPE:
    blocks start with a parameter-free LayerNorm).  Two-pass mean / biased variance.
    reading: eps = 1e-6 (not printed)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with a learned per-dim scale ([MV] Blocks: queries and keys
    are RMS-normalised before attention).  reading: learned [128] scale per weight set,
    eps = 1e-6."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * weight


def split_modulation(mod: np.ndarray, d: int):
    """Split a [3D] modulation vector into (shift, scale, gate).
    reading: chunk order shift || scale || gate (DiT adaLN convention; the page names the
    three but fixes no order)."""
    return mod[0:d], mod[d:2 * d], mod[2 * d:3 * d]


def modulation(w_mod: np.ndarray, cond: np.ndarray) -> np.ndarray:
    """mod = W_mod . SiLU(cond): scale, shift and gate come from the timestep embedding
    ([MV] Modulation/RoPE).  w_mod [3D, D], cond [D] -> [3D].
    reading: no bias; one projection per (block kind, weight set), shared by the blocks of
    that kind (the printed 5.6 B parameter count does not fit one projection per block)."""
    return w_mod @ silu(cond)


def timestep_embedding(t: float, dim: int = 256, max_period: float = 10000.0,
                       time_factor: float = 1000.0) -> np.ndarray:
    """Sinusoidal embedding of the scalar time t: [cos(1000 t f_k), sin(1000 t f_k)],
    f_k = 10000^(-k/(dim/2)).  Parity unpinned beyond its closed form (the pages only say
    modulation derives from a timestep embedding; reading: Transformer/DiT sinusoid)."""
    half = dim // 2
    k = np.arange(half, dtype=np.float64)
    f = max_period ** (-k / half)
    arg = time_factor * float(t) * f
    return np.concatenate([np.cos(arg), np.sin(arg)])


def cond_vector(t: float, w_l1: np.ndarray, w_l2: np.ndarray) -> np.ndarray:
    """cond(t) = W_l2 . SiLU(W_l1 . e(t)); reading: two-layer MLP without biases."""
    return w_l2 @ silu(w_l1 @ timestep_embedding(t, dim=w_l1.shape[1]))


# ----------------------------------------------------------------------------------------
# Attention ([MV] Blocks)
# ----------------------------------------------------------------------------------------

MASK_FULL = 0      # every token attends every token (double / single / joint blocks)
MASK_SEGMENT = 1   # tokens attend only their own stream (per-mode blocks)


def segment_ids(n_txt: int, n_img: int, n_ref: int) -> np.ndarray:
    return np.concatenate([np.zeros(n_txt, np.int64), np.ones(n_img, np.int64),
                           np.full(n_ref, 2, np.int64)])


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seg: np.ndarray, mask: int,
              check_rows: bool = True) -> np.ndarray:
    """Softmax self-attention per head, materialising the full score matrix.

    q, k, v: [N, H, d].  S = q k^T / sqrt(d); disallowed keys get -inf; P = softmax rows;
    o = P v.  mask FULL: all N keys ([MV] Blocks, joint blocks: every token attends every
    token).  mask SEGMENT: keys of the query's own stream only ([MV] Blocks, per-mode blocks).
    No padding mask: padded prompt tokens are attended ([MV] Batching)."""
    n, h, d = q.shape
    out = np.empty_like(q)
    allowed = np.ones((n, n), dtype=bool) if mask == MASK_FULL else (seg[:, None] == seg[None, :])
    for hh in range(h):
        s = (q[:, hh, :] @ k[:, hh, :].T) / math.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        if check_rows:
            assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
        out[:, hh, :] = p @ v[:, hh, :]
    return out


# ----------------------------------------------------------------------------------------
# One transformer block ([MV] Blocks; [MV] Modulation/RoPE)
# ----------------------------------------------------------------------------------------

@dataclass
class Dims:
    hidden: int = 3072
    heads: int = 24
    head_dim: int = 128
    mlp_hidden: int = 9216
    in_channels: int = 128
    time_dim: int = 256
    ln_eps: float = 1e-6
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0


@dataclass
class WeightSet:
    """One weight set of a block.  w1 [3D+2F, D] = rows Q | K | V | gate | up (head-major
    Q/K/V); w2 [D, D+F] acting on [attention output || SwiGLU output]; qn, kn [head_dim]."""
    w1: np.ndarray
    w2: np.ndarray
    qn: np.ndarray
    kn: np.ndarray


# ----------------------------------------------------------------------------------------
# Row-wise FP8 ("fp8r") projections.  The FLUX.3 transformer ships as single-file weights in
# row-wise FP8 ([KS] "Was sich geändert hat"); GPUs with fast FP8 kernels compute with them,
# others dequantize the weights at every step ([WE] "Hardwareanforderungen, Quantisierung und
# Inferenzlatenz").
# reading: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
# value 448; no infinities).  One scale per row: per output feature for a weight, per token
# for an activation.  scale = max|row| / 448 is the dequantization factor, and each code is
# the E4M3 value nearest to value / scale = value * 448 / max|row| (ties to even mantissa);
# a row of zeros has scale 0 and codes 0.  Everything here is float64: the quotient of a
# value with at most 24 significant bits is correctly rounded and never lands within one
# double rounding of an E4M3 tie unless it is the tie, so the codes are those of the exact
# quotient.  A projection y = x W^T then equals scale_x scale_w sum_k code_x code_w.  Only
# the two big projections of every block (W1, W2) and their inputs (the modulated LayerNorm
# output and [attention || SwiGLU]) use it.
# ----------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value of each element (float64 in, float64 out), ties to even mantissa,
    magnitudes beyond 448 saturate to 448.  Normal values have a quantum of 2^(e-3) in
    binade [2^e, 2^(e+1)), e >= -6; below 2^-6 the subnormal quantum is 2^-9."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                       # a = m 2^ex, m in [0.5, 1): binade e = ex - 1
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)
    quantum = np.exp2(e - 3.0)
    r = np.round(a / quantum) * quantum       # np.round: half to even; a / quantum is exact
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """uint8 codes of values already on the E4M3 grid (|v| <= 448)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** -6
    mant_n = np.where(normal, a / np.exp2(np.where(normal, e, 0)) * 8 - 8, 0)
    code_n = ((e + 7) << 3) + mant_n.astype(np.int64)
    code_s = (a / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s).astype(np.uint8)
    return code | sign


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of uint8 E4M3 codes; the two NaN codes (exponent and mantissa all ones)
    give NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def quantize_rows_fp8(x: np.ndarray):
    """(codes uint8 [rows, cols], scales float64 [rows]) of the row-wise E4M3 quantization of
    x: scale = max|row| / 448, code = nearest E4M3 value of x * 448 / max|row|."""
    x = np.asarray(x, np.float64)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    live = amax > 0
    q = np.zeros_like(x)
    q[live] = x[live] * E4M3_MAX / amax[live, None]
    return e4m3_encode(e4m3_round(q)), amax / E4M3_MAX


def fp8_round_rows(x: np.ndarray) -> np.ndarray:
    """The values a row-wise E4M3 operand stands for: code * scale, per row (float64)."""
    codes, scale = quantize_rows_fp8(x)
    return e4m3_decode(codes) * scale[:, None]


def quantize_weights_fp8(sets: list[WeightSet]) -> list[WeightSet]:
    """W1 and W2 of every weight set replaced by their row-wise E4M3 values (rows = output
    features); the RMSNorm scales stay as they are."""
    return [WeightSet(fp8_round_rows(ws.w1), fp8_round_rows(ws.w2), ws.qn, ws.kn) for ws in sets]


def block_forward(x: np.ndarray, segs: tuple[int, int, int], sets: list[WeightSet],
                  set_of_segment: tuple[int, int, int], mods: list[np.ndarray],
                  pos: np.ndarray, mask: int, dims: Dims, rows: np.ndarray | None = None,
                  act_fp8: bool = False):
    """One block: x + gate_s * ([attn || SwiGLU](adaLN(LN(x))) . W2^T).

    x: [N, D] residual; segs = (n_txt, n_img, n_ref), segments contiguous in the order text,
    image, reference ([MV] Blocks).  Row i of segment s uses weight set set_of_segment[s]
    and modulation mods[s] = [shift || scale || gate] ([3D]).

    Steps, in the order the page gives them:
      LayerNorm without affine, then y * (1 + scale) + shift ([MV] Modulation/RoPE);
      attention and SwiGLU MLP in parallel on the same normalised input, both added to the
      residual ([MV] Blocks); RMSNorm on queries and keys before attention ([MV] Blocks);
      4D RoPE on queries and keys ([MV] Modulation/RoPE).
    reading: one fused input projection W1 and one fused output projection W2 (single-stream
    block shapes), gated residual x + gate * out (DiT adaLN), no biases; SwiGLU = SiLU(first
    F columns) * (second F columns).

    rows: if given, only these output rows are computed (keys/values still use all rows);
    returns [len(rows), D].  Used to check sampled rows at full size.

    act_fp8: the inputs of the two projections (the modulated LayerNorm output, and
    [attention || SwiGLU]) go through the row-wise E4M3 quantization first (the fp8r path;
    the weights are expected in their E4M3 values already, quantize_weights_fp8)."""
    n, d = x.shape
    nh, hd, f = dims.heads, dims.head_dim, dims.mlp_hidden
    seg = segment_ids(*segs)
    assert seg.shape[0] == n
    # adaLN-modulated LayerNorm
    y = layer_norm(x, dims.ln_eps)
    xm = np.empty_like(y)
    for s in range(3):
        sel = seg == s
        if not sel.any():
            continue
        shift, scale, _ = split_modulation(mods[s], d)
        xm[sel] = y[sel] * (1.0 + scale) + shift
    if act_fp8:
        xm = fp8_round_rows(xm)
    # fused projection per weight set
    h = np.empty((n, 3 * d + 2 * f))
    for s in range(3):
        sel = seg == s
        if sel.any():
            h[sel] = xm[sel] @ sets[set_of_segment[s]].w1.T
    q = h[:, 0:d].reshape(n, nh, hd)
    k = h[:, d:2 * d].reshape(n, nh, hd)
    v = h[:, 2 * d:3 * d].reshape(n, nh, hd)
    g = h[:, 3 * d:3 * d + f]
    u = h[:, 3 * d + f:3 * d + 2 * f]
    # QK RMSNorm (per weight set) then RoPE
    qn = np.empty_like(q)
    kn = np.empty_like(k)
    for s in range(3):
        sel = seg == s
        if sel.any():
            ws = sets[set_of_segment[s]]
            qn[sel] = rms_norm(q[sel], ws.qn, dims.rms_eps)
            kn[sel] = rms_norm(k[sel], ws.kn, dims.rms_eps)
    ang = rope_angles(pos, dims.rope_theta)
    qn = apply_rope(qn, ang)
    kn = apply_rope(kn, ang)
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    # attention for the requested query rows over all allowed keys
    o = np.empty((rows.shape[0], nh, hd))
    allowed_all = mask == MASK_FULL
    for hh in range(nh):
        s_ = (qn[rows, hh, :] @ kn[:, hh, :].T) / math.sqrt(hd)
        if not allowed_all:
            s_ = np.where(seg[rows][:, None] == seg[None, :], s_, -np.inf)
        s_ = s_ - s_.max(axis=1, keepdims=True)
        p = np.exp(s_)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, hh, :] = p @ v[:, hh, :]
    m = silu(g[rows]) * u[rows]
    cat = np.concatenate([o.reshape(rows.shape[0], d), m], axis=1)
    if act_fp8:
        cat = fp8_round_rows(cat)
    out = x[rows].copy()
    for s in range(3):
        sel = seg[rows] == s
        if sel.any():
            _, _, gate = split_modulation(mods[s], d)
            out[sel] = out[sel] + gate * (cat[sel] @ sets[set_of_segment[s]].w2.T)
    return out


def block_forward_sequential(x: np.ndarray, segs: tuple[int, int, int], sets: list[WeightSet],
                             set_of_segment: tuple[int, int, int], mods6: list[np.ndarray],
                             pos: np.ndarray, mask: int, dims: Dims,
                             rows: np.ndarray | None = None, act_fp8: bool = False):
    """A double-stream block wired in sequence (the FLUX.1-style reading of the pages' double
    blocks, the alternative to the parallel wiring of block_forward): attention first, then
    the MLP on the updated residual, each after its own modulated LayerNorm and with its own
    gate; mods6[s] = [shift1 || scale1 || gate1 || shift2 || scale2 || gate2] ([6D]).

    reading: the same weight tensors as block_forward, used in two halves: W1's Q|K|V rows and
    W2's first D columns for attention, W1's gate/up rows and W2's last F columns for the
    SwiGLU MLP.

    rows: if given (sorted), only these output rows are computed ([len(rows), D]); the MLP
    half is row-local, so it runs on those rows alone.  act_fp8 as in block_forward: each
    half quantizes its own projection inputs (the zero columns of the other half change no
    row maximum)."""
    n, d = x.shape
    f = dims.mlp_hidden
    seg = segment_ids(*segs)
    half1 = [np.asarray(m[:3 * d]) for m in mods6]
    half2 = [np.asarray(m[3 * d:]) for m in mods6]
    attn_sets = [WeightSet(np.concatenate([ws.w1[:3 * d], np.zeros((2 * f, d))], axis=0),
                           np.concatenate([ws.w2[:, :d], np.zeros((d, f))], axis=1), ws.qn, ws.kn)
                 for ws in sets]
    mlp_sets = [WeightSet(np.concatenate([np.zeros((3 * d, d)), ws.w1[3 * d:]], axis=0),
                          np.concatenate([np.zeros((d, d)), ws.w2[:, d:]], axis=1), ws.qn, ws.kn)
                for ws in sets]
    # attention half: zero gate/up rows give SiLU(0) * 0 = 0 for the MLP columns
    x1 = block_forward(x, segs, attn_sets, set_of_segment, half1, pos, mask, dims, rows=rows,
                       act_fp8=act_fp8)
    # MLP half: zero Q|K|V rows give uniform attention over V = 0, which W2's zeroed attention
    # columns drop anyway
    if rows is None:
        return block_forward(x1, segs, mlp_sets, set_of_segment, half2, pos, mask, dims,
                             act_fp8=act_fp8)
    rows = np.asarray(rows)
    assert np.all(np.diff(rows) > 0)
    sub = tuple(int(np.sum(seg[rows] == s)) for s in range(3))
    return block_forward(x1, sub, mlp_sets, set_of_segment, half2, pos[rows], mask, dims,
                         act_fp8=act_fp8)


# ----------------------------------------------------------------------------------------
# Block schedule, output head, Euler loop ([GN] Architektur; [MV] Blocks/Modulation; [WE])
# ----------------------------------------------------------------------------------------

ARCH_FLUX2 = 0   # 5 double-stream blocks then 20 single-stream blocks ([GN], [HK] 技術詳細)
ARCH_FLUX3 = 1   # 5 per-mode blocks then 28 joint blocks ([MV] Blocks)


def block_plan(arch: int, b: int, n_stream: int):
    """(kind, set_of_segment, mask) of block b.

    FLUX.2 double: sets text=0, image=1, reference=1 (reference tokens travel with the image
      stream; reading), full attention from the first block ([MV] Blocks).
    FLUX.2 single: one set, full attention.
    FLUX.3 per-mode: sets text=0, image=1, reference=2, attention within the stream only.
    FLUX.3 joint: one set shared by all streams, full attention ([MV] Blocks).
    kind: 0 = stream (double / per-mode), 1 = shared (single / joint)."""
    if b < n_stream:
        if arch == ARCH_FLUX2:
            return 0, (0, 1, 1), MASK_FULL
        return 0, (0, 1, 2), MASK_SEGMENT
    return 1, (0, 0, 0), MASK_FULL


def cond_rows(arch: int, t: float, w_l1, w_l2):
    """Conditioning vector per segment (text, image, reference).
    FLUX.1/2: one timestep for all tokens.  FLUX.3: image tokens use t, text and reference
    tokens always use t = 0 ([MV] Modulation/RoPE)."""
    ct = cond_vector(t, w_l1, w_l2)
    if arch == ARCH_FLUX2:
        return [ct, ct, ct]
    c0 = cond_vector(0.0, w_l1, w_l2)
    return [c0, ct, c0]


def flow_map_cond_rows(arch: int, t: float, t_target: float, w_l1, w_l2, w_tl1, w_tl2):
    """Conditioning rows of a flow-map (timestep-distilled) model: besides its current time,
    the model is told the time its step jumps to, through an embedding of its own that is
    added to the modulation of every token ([MV] Modulation/RoPE, flow-map distillation).
    reading: the target time goes through the same sinusoid and a separate two-layer MLP
    (w_tl1, w_tl2), and the result is added to every segment's conditioning vector, the
    input of all modulation projections."""
    tgt = cond_vector(t_target, w_tl1, w_tl2)
    return [c + tgt for c in cond_rows(arch, t, w_l1, w_l2)]


def segment_mods(w_mod_sets: list[np.ndarray], set_of_segment, conds):
    """Per-segment [3D] modulation vectors for one block kind."""
    return [modulation(w_mod_sets[set_of_segment[s]], conds[s]) for s in range(3)]


def final_layer(x_img: np.ndarray, cond_img: np.ndarray, w_fmod: np.ndarray,
                w_out: np.ndarray, eps: float) -> np.ndarray:
    """Velocity for the image tokens: text and reference tokens are dropped, image tokens go
    through the output layers ([MV] Blocks).  reading: LN without affine, modulation
    (shift || scale) = W_fmod . SiLU(cond), projection W_out [C, D], no bias."""
    d = x_img.shape[1]
    fm = w_fmod @ silu(cond_img)
    shift, scale = fm[0:d], fm[d:2 * d]
    y = layer_norm(x_img, eps) * (1.0 + scale) + shift
    return y @ w_out.T


@dataclass
class Model:
    """All weights of one model, as float64 arrays (already bf16-rounded for bf16 runs).
    blocks[b] = list of WeightSet; mods[kind] = list of [3D, D] per set."""
    arch: int
    dims: Dims
    n_stream: int
    n_shared: int
    img_in: np.ndarray            # [D, C]
    temb_l1: np.ndarray           # [D, time_dim]
    temb_l2: np.ndarray           # [D, D]
    final_mod: np.ndarray         # [2D, D]
    final_out: np.ndarray         # [C, D]
    mods: list = field(default_factory=list)
    blocks: list = field(default_factory=list)
    temb_tgt_l1: np.ndarray | None = None   # [D, time_dim]  flow-map models only
    temb_tgt_l2: np.ndarray | None = None   # [D, D]
    txt_in: np.ndarray | None = None        # [D, 8 * 2560]  text-feature projection
    double_wiring: int = 0                  # FLUX.2 double blocks: 0 parallel, 1 sequential
    fp8: bool = False                       # row-wise E4M3 block projections (fp8r)
    block_mods: list | None = None          # [b][set]: each block's own modulation projections


# ----------------------------------------------------------------------------------------
# Text features ([MV] Tokens): the text encoder's hidden states of layers 4, 8, ..., 32 (of
# 36) are stacked per token to 8 x 2560 = 20480 values and projected by one linear layer to
# the transformer width 3072.
# ----------------------------------------------------------------------------------------

TEXT_ENCODER_DEPTH = 36
TEXT_FEATURE_LAYERS = (4, 8, 12, 16, 20, 24, 28, 32)
TEXT_HIDDEN = 2560


def stack_text_features(hidden_by_layer: dict) -> np.ndarray:
    """hidden_by_layer[l] = [n_txt, hidden] state after encoder layer l; the result is
    [n_txt, 8 * hidden] with the layers in the order listed.  reading: stacking is
    concatenation along the feature axis, shallowest layer first."""
    return np.concatenate([np.asarray(hidden_by_layer[l], np.float64)
                           for l in TEXT_FEATURE_LAYERS], axis=1)


def project_text(feat: np.ndarray, w_txt_in: np.ndarray) -> np.ndarray:
    """[n_txt, D] text rows of the transformer sequence.  reading: no bias (Q10)."""
    return feat @ w_txt_in.T


def forward(model: Model, lat: np.ndarray, txt: np.ndarray, grid, t: float,
            ref_lat: np.ndarray | None = None, ref_grid=None, block_hook=None,
            t_target: float | None = None):
    """One transformer call: velocity [n_img, C] for latents lat [n_img, C] at time t.

    Sequence = text || image || reference ([MV] Blocks).  Image and reference latents go
    through the same input projection (same VAE and packing, [MV] Tokens); text embeddings
    enter at width D (reading: precomputed embeddings, cf. the C tool's embeddings option,
    [HK] コマンドラインオプション).  ref_grid is one (rows, cols) grid, or a list of grids for
    several reference images whose latents follow one another in ref_lat (up to ten, [WE];
    each keeps its own size, [MV] Tokens)."""
    dims = model.dims
    n_txt = txt.shape[0]
    n_img = lat.shape[0]
    n_ref = 0 if ref_lat is None else ref_lat.shape[0]
    parts = [txt, lat @ model.img_in.T]
    ref_grids = ()
    if n_ref:
        parts.append(ref_lat @ model.img_in.T)
        ref_grids = tuple(ref_grid) if isinstance(ref_grid, list) else (ref_grid,)
        assert sum(h * w for h, w in ref_grids) == n_ref
    x = np.concatenate(parts, axis=0)
    pos = positions(n_txt, grid, ref_grids)
    if model.temb_tgt_l1 is not None:
        if t_target is None:
            raise ValueError("a flow-map model needs the target time of the step")
        conds = flow_map_cond_rows(model.arch, t, t_target, model.temb_l1, model.temb_l2,
                                   model.temb_tgt_l1, model.temb_tgt_l2)
    else:
        conds = cond_rows(model.arch, t, model.temb_l1, model.temb_l2)
    for b in range(model.n_stream + model.n_shared):
        kind, sos, mask = block_plan(model.arch, b, model.n_stream)
        # reading: one modulation projection per (block kind, weight set), shared by the blocks
        # of that kind, unless the model gives each block its own (block_mods); the pages tie
        # scale, shift and gate to the timestep embedding without fixing which
        mods = segment_mods(model.mods[kind] if model.block_mods is None else model.block_mods[b],
                            sos, conds)
        if block_hook is not None:
            block_hook(b, x)
        if model.arch == ARCH_FLUX2 and kind == 0 and model.double_wiring:
            x = block_forward_sequential(x, (n_txt, n_img, n_ref), model.blocks[b], sos, mods, pos,
                                         mask, dims, act_fp8=model.fp8)
        else:
            x = block_forward(x, (n_txt, n_img, n_ref), model.blocks[b], sos, mods, pos, mask, dims,
                              act_fp8=model.fp8)
    return final_layer(x[n_txt:n_txt + n_img], conds[1], model.final_mod, model.final_out,
                       dims.ln_eps)


def euler_schedule(n_steps: int) -> np.ndarray:
    """t_i = 1 - i/n, i = 0..n: t = 1 is pure noise, t = 0 the clean image ([MV]
    Modulation/RoPE: t = 0 marks clean context).  reading: uniform schedule (the shifted
    schedules of real checkpoints are not on the pages)."""
    return 1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps


def euler_step(lat: np.ndarray, v: np.ndarray, t_cur: float, t_next: float) -> np.ndarray:
    """lat <- lat + (t_cur - t_next) * v, with v pointing from noise toward the clean image
    ([MV] Blocks: the output layers predict the velocity from noise to the clean image)."""
    return lat + (t_cur - t_next) * v


def denoise(model: Model, noise: np.ndarray, txt: np.ndarray, grid, n_steps: int,
            ref_lat=None, ref_grid=None) -> np.ndarray:
    """Few-step sampling loop: n_steps Euler steps from t = 1 to t = 0 (FLUX.2-klein: 4
    steps, [GN] Architektur; FLUX.3 distilled: 16, base: 50, [WE] checkpoint table)."""
    ts = euler_schedule(n_steps)
    lat = noise.astype(np.float64).copy()
    for i in range(n_steps):
        v = forward(model, lat, txt, grid, ts[i], ref_lat, ref_grid, t_target=ts[i + 1])
        lat = euler_step(lat, v, ts[i], ts[i + 1])
    return lat


# ----------------------------------------------------------------------------------------
# Image-to-image.  The C tool transforms an input image with a strength in [0, 1], default
# 0.75 ([HK] コマンドラインオプション, -t/--strength; CライブラリAPI, strength).  reading: as
# in rectified-flow image-to-image, the clean latents are moved to the time t_s = strength
# along the straight path to the noise, x_t = t noise + (1 - t) x, and the Euler loop runs
# only the last floor(n strength) of its n steps (the schedule is cut, not re-spaced).
# ----------------------------------------------------------------------------------------

def img2img_first_step(n_steps: int, strength: float) -> int:
    """Index of the first Euler step that runs: n - floor(n strength)."""
    return n_steps - int(math.floor(n_steps * strength))


def noise_mix(x_clean: np.ndarray, noise: np.ndarray, t: float) -> np.ndarray:
    """The point at time t on the straight path from the clean latents (t = 0) to the noise
    (t = 1)."""
    return t * noise + (1.0 - t) * x_clean


def img2img(model: Model, x_clean: np.ndarray, noise: np.ndarray, txt: np.ndarray, grid,
            n_steps: int, strength: float, ref_lat=None, ref_grid=None, txt_uncond=None,
            guidance: float = 1.0) -> np.ndarray:
    """Image-to-image sampling; strength 1 starts from pure noise and is denoise()."""
    ts = euler_schedule(n_steps)
    i0 = img2img_first_step(n_steps, strength)
    if i0 >= n_steps:
        raise ValueError("strength too small for any step")
    lat = noise_mix(np.asarray(x_clean, np.float64), np.asarray(noise, np.float64), ts[i0])
    for i in range(i0, n_steps):
        if txt_uncond is None:
            v = forward(model, lat, txt, grid, ts[i], ref_lat, ref_grid, t_target=ts[i + 1])
        else:
            v = forward_cfg(model, lat, txt, txt_uncond, grid, ts[i], guidance, ref_lat,
                            ref_grid, t_target=ts[i + 1])
        lat = euler_step(lat, v, ts[i], ts[i + 1])
    return lat


# ----------------------------------------------------------------------------------------
# Classifier-free guidance.  The C tool's generation parameters carry a CFG scale ([HK]
# CライブラリAPI, guidance_scale); the non-distilled base checkpoint samples with guidance
# 3.5 over 50 steps and the distilled one without guidance ([WE] checkpoint table; [KS]
# "Was sich geändert hat").  reading: the pages print no formula; the standard combination of
# J. Ho and T. Salimans, "Classifier-Free Diffusion Guidance" (2022), in velocity form, with
# the unconditional branch being the same call on the unconditional text embeddings.
# ----------------------------------------------------------------------------------------

def guided_velocity(v_cond: np.ndarray, v_uncond: np.ndarray, guidance: float) -> np.ndarray:
    """v = v_u + g (v_c - v_u): g = 1 is the conditional prediction, g = 0 the unconditional
    one, g > 1 extrapolates away from the unconditional prediction."""
    return v_uncond + guidance * (v_cond - v_uncond)


def forward_cfg(model: Model, lat: np.ndarray, txt: np.ndarray, txt_uncond: np.ndarray, grid,
                t: float, guidance: float, ref_lat: np.ndarray | None = None, ref_grid=None,
                t_target: float | None = None):
    """Guided velocity of one Euler step: the transformer on the conditional and on the
    unconditional text, same latents, references and time, combined by guided_velocity."""
    v_c = forward(model, lat, txt, grid, t, ref_lat, ref_grid, t_target=t_target)
    v_u = forward(model, lat, txt_uncond, grid, t, ref_lat, ref_grid, t_target=t_target)
    return guided_velocity(v_c, v_u, guidance)


def denoise_cfg(model: Model, noise: np.ndarray, txt: np.ndarray, txt_uncond: np.ndarray, grid,
                n_steps: int, guidance: float, ref_lat=None, ref_grid=None) -> np.ndarray:
    """The Euler loop of denoise with the guided velocity at every step."""
    ts = euler_schedule(n_steps)
    lat = noise.astype(np.float64).copy()
    for i in range(n_steps):
        v = forward_cfg(model, lat, txt, txt_uncond, grid, ts[i], guidance, ref_lat, ref_grid,
                        t_target=ts[i + 1])
        lat = euler_step(lat, v, ts[i], ts[i + 1])
    return lat


# ----------------------------------------------------------------------------------------
# Seeded starting noise.  The C tool makes generation reproducible from a seed ([HK]
# 再現性・シード管理); the noise here is a counter-based generator written from its
# published definition: Philox-4x32 with 10 rounds (J. K. Salmon, M. A. Moraes, R. O. Dror,
# D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), then the Box-Muller
# transform (G. E. P. Box, M. E. Muller, 1958).
# ----------------------------------------------------------------------------------------

PHILOX_MUL = (0xD2511F53, 0xCD9E8D57)     # round multipliers of Philox-4x32
PHILOX_BUMP = (0x9E3779B9, 0xBB67AE85)    # Weyl key increments (golden ratio, sqrt(3) - 1)
_U32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10) -> np.ndarray:
    """Philox-4x32 bijection of 128-bit counters under a 64-bit key.

    counter: integer array [..., 4] of 32-bit words; key: (k0, k1).  One round multiplies
    words 0 and 2 by the two constants (64-bit products split into high and low halves) and
    forms (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key words
    advance by the Weyl increments between rounds."""
    c = np.asarray(counter, dtype=np.uint64)
    x0, x1, x2, x3 = (c[..., i] & _U32 for i in range(4))
    k0, k1 = int(key[0]) & _U32, int(key[1]) & _U32
    m0, m1 = np.uint64(PHILOX_MUL[0]), np.uint64(PHILOX_MUL[1])
    for _ in range(rounds):
        p0, p1 = x0 * m0, x2 * m1           # < 2^64: exact in uint64
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(k0), p1 & np.uint64(_U32),
                          (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(k1), p0 & np.uint64(_U32))
        k0, k1 = (k0 + PHILOX_BUMP[0]) & _U32, (k1 + PHILOX_BUMP[1]) & _U32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def box_muller(u0: np.ndarray, u1: np.ndarray):
    """Two independent N(0,1) values from two uniforms in (0, 1)."""
    r = np.sqrt(-2.0 * np.log(u0))
    return r * np.cos(2.0 * np.pi * u1), r * np.sin(2.0 * np.pi * u1)


def noise(n: int, seed: int) -> np.ndarray:
    """n values of N(0,1) noise for a seed (the library's seeded latents, row-major).

    Element e comes from the Philox block of counter (e // 4 as two 32-bit words, 0, 0) and
    key (seed low word, seed high word), output word e % 4; words 0,1 and 2,3 form two
    Box-Muller pairs with uniforms u = (word + 1/2) / 2^32 (never 0 or 1)."""
    if n < 0:
        raise ValueError("negative length")
    groups = (n + 3) // 4
    g = np.arange(groups, dtype=np.uint64)
    ctr = np.stack([g & np.uint64(_U32), g >> np.uint64(32), np.zeros_like(g), np.zeros_like(g)], -1)
    seed = int(seed)
    words = philox4x32(ctr, (seed & _U32, (seed >> 32) & _U32)).astype(np.float64)
    u = (words + 0.5) / 4294967296.0
    z0, z1 = box_muller(u[:, 0], u[:, 1])
    z2, z3 = box_muller(u[:, 2], u[:, 3])
    return np.stack([z0, z1, z2, z3], axis=-1).reshape(-1)[:n]
