"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to a value printed on the pages, a closed form, an
invariant the pages fix, or an independent library routine (torch float64 CPU ops), so that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand) fails here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dit_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_counts.json")
PHILOX_KAT = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")

TINY = O.Dims(hidden=256, heads=2, head_dim=128, mlp_hidden=192, in_channels=64,
              time_dim=32)


def rng(seed=0):
    return np.random.default_rng(seed)


def rand_set(r, dims, scale=0.05):
    d, f = dims.hidden, dims.mlp_hidden
    return O.WeightSet(w1=r.normal(0, scale, (3 * d + 2 * f, d)),
                       w2=r.normal(0, scale, (d, d + f)),
                       qn=r.uniform(0.5, 1.5, dims.head_dim),
                       kn=r.uniform(0.5, 1.5, dims.head_dim))


def rand_mods(r, dims, n=3, gate_zero=False):
    d = dims.hidden
    out = []
    for _ in range(n):
        m = r.normal(0, 0.5, 3 * d)
        if gate_zero:
            m[2 * d:] = 0.0
        out.append(m)
    return out


# ------------------------------------------------------------------ token accounting

def test_token_counts_match_printed_values():
    g = json.load(open(GOLDEN))
    for case in g["image_tokens"]:
        assert O.image_token_grid(*case["hw"]) == tuple(case["grid"])
        assert O.image_tokens(*case["hw"]) == case["tokens"]
    for case in g["tokens_per_call"]:
        img = O.image_tokens(*case["out_hw"]) + sum(O.image_tokens(*hw) for hw in case["ref_hws"])
        # the printed total must be reachable with a padded prompt: some prompt length
        # gives exactly the printed count, and the text part is a positive multiple of 80
        txt = case["tokens"] - img
        assert txt > 0 and txt % g["text_pad_multiple"]["value"] == 0, case
        ok = [L for L in range(1, 1000)
              if O.tokens_per_call(L, tuple(case["out_hw"]),
                                   tuple(tuple(h) for h in case["ref_hws"])) == case["tokens"]]
        assert ok and ok == list(range(txt - 79, txt + 1)), case


def test_config_token_counts():
    # the benchmark configurations: 64x64 px -> 16 tokens, 256^2 -> 256, 512^2 -> 1024
    assert O.image_tokens(64, 64) == 16
    assert O.image_token_grid(256, 256) == (16, 16)
    assert O.image_tokens(512, 512) == 1024
    assert O.padded_text_tokens(0) == 0 and O.padded_text_tokens(1) == 80
    assert O.padded_text_tokens(80) == 80 and O.padded_text_tokens(81) == 160
    with pytest.raises(ValueError):
        O.image_token_grid(100, 64)


# ------------------------------------------------------------------ positions and RoPE

def test_positions_structure():
    pos = O.positions(5, (3, 4), ((3, 4), (2, 2)))
    assert pos.shape == (5 + 12 + 12 + 4, 4)
    assert np.all(pos[:, 0] == 0)                             # t is 0 for every token
    assert np.all(pos[:5, 1:3] == 0) and np.all(pos[:5, 3] == np.arange(5))
    img = pos[5:17]
    ref0 = pos[17:29]
    ref1 = pos[29:]
    assert np.all(img[:, 3] == 0) and np.all(ref0[:, 3] == -1) and np.all(ref1[:, 3] == -2)
    # reference tokens share the image's (h, w) grid (same place -> same coordinates)
    assert np.array_equal(img[:, 1:3], ref0[:, 1:3])
    assert img[:, 1].max() == 2 and img[:, 2].max() == 3
    # row-major inside an image
    assert tuple(img[5, 1:3]) == (1, 1)


def rope_complex(x, pos, theta):
    """Independent formulation: each adjacent pair is a complex number multiplied by
    exp(i * pos_axis * theta^(-j/16))."""
    n, h, d = x.shape
    xc = torch.view_as_complex(torch.tensor(x).reshape(n, h, d // 2, 2).contiguous())
    p = torch.arange(d // 2, dtype=torch.float64)
    axis = (p // 16).long()
    j = p % 16
    ang = torch.tensor(pos)[:, axis] * theta ** (-j / 16.0)
    rot = torch.polar(torch.ones_like(ang), ang)
    return torch.view_as_real(xc * rot[:, None, :]).reshape(n, h, d).numpy()


def _parameter_count(arch, n_stream, n_shared, per_block_mod=False, tied_shared=False,
                     text_proj=0, target_time=False):
    """Generator parameters of a model built as the oracle reads the pages: each block's
    weight sets (block_plan) hold W1 [3D+2F, D], W2 [D, D+F] and two [128] norm scales; the
    modulation projections [3D, D] are one per (block kind, set), or one per (block, set) with
    per_block_mod; tied_shared makes all shared / joint blocks one set."""
    d, f, c, hd, td = 3072, 9216, 128, 128, 256
    per_set = (3 * d + 2 * f) * d + d * (d + f) + 2 * hd
    mod = 3 * d * d
    sets = [len(set(O.block_plan(arch, b, n_stream)[1])) for b in range(n_stream + n_shared)]
    blocks = sum(sets[:n_stream]) + (1 if tied_shared else sum(sets[n_stream:]))
    mods = sum(sets) if per_block_mod else len(set(O.block_plan(arch, 0, n_stream)[1])) + 1
    globals_ = d * c + d * td + d * d + 2 * d * d + c * d  # img_in, cond MLP, final layer
    globals_ += text_proj * d + (d * td + d * d if target_time else 0)
    return blocks * per_set + mods * mod + globals_


def test_parameter_count_fits_printed_total():
    """Readings Q2 (modulation projections shared per block kind and weight set) and Q16 (the
    28 joint blocks are distinct, each one set shared by the streams) against the printed
    generator size: 5.6 billion parameters without the text encoder, 11.2 GB of bf16 weights
    (we0.ai "FLUX 3 Image Klein" article: introduction; "Hardwareanforderungen, Quantisierung
    und Inferenzlatenz").  Per-block projections or tied joint blocks miss it by far."""
    kw = dict(arch=O.ARCH_FLUX3, n_stream=5, n_shared=28, text_proj=20480, target_time=True)
    shared = _parameter_count(**kw)
    per_block = _parameter_count(per_block_mod=True, **kw)
    tied = _parameter_count(tied_shared=True, **kw)
    printed = 5.6e9
    assert abs(shared / printed - 1) < 0.05, shared
    assert abs(2 * shared / 11.2e9 - 1) < 0.05
    assert per_block / printed - 1 > 0.15, per_block
    assert 1 - tied / printed > 0.5, tied
    # FLUX.2-klein "4B" (the model name, "Flux 2 Klein: Reine C-basierte Inferenz"): the same
    # structure with 5 double and 20 single blocks comes to about 3.8 billion
    flux2 = _parameter_count(O.ARCH_FLUX2, 5, 20)
    assert abs(flux2 / 4e9 - 1) < 0.1, flux2


def test_rope_matches_complex_rotation():
    r = rng(1)
    pos = O.positions(7, (3, 3), ((2, 3),))
    x = r.normal(size=(pos.shape[0], 2, 128))
    got = O.apply_rope(x, O.rope_angles(pos, 10000.0))
    np.testing.assert_allclose(got, rope_complex(x, pos, 10000.0), rtol=0, atol=1e-12)


def test_rope_invariants():
    r = rng(2)
    pos = O.positions(6, (4, 5), ((4, 5),))
    n = pos.shape[0]
    x = r.normal(size=(n, 3, 128))
    y = O.apply_rope(x, O.rope_angles(pos))
    # rotations preserve norms (per pair, hence per head)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # t slice untouched for all tokens; l slice untouched for image tokens;
    # h and w slices untouched for text tokens
    np.testing.assert_array_equal(y[:, :, 0:32], x[:, :, 0:32])
    np.testing.assert_array_equal(y[6:26, :, 96:128], x[6:26, :, 96:128])
    np.testing.assert_array_equal(y[:6, :, 32:96], x[:6, :, 32:96])
    # pos = 0 is the identity
    np.testing.assert_array_equal(O.apply_rope(x, O.rope_angles(np.zeros((n, 4)))), x)
    # the first pair of each axis turns by exactly pos radians (frequency theta^0 = 1)
    e = np.zeros((1, 1, 128))
    e[0, 0, 96] = 1.0
    out = O.apply_rope(e, O.rope_angles(np.array([[0.0, 0.0, 0.0, 1.0]])))
    assert abs(out[0, 0, 96] - math.cos(1.0)) < 1e-15 and abs(out[0, 0, 97] - math.sin(1.0)) < 1e-15


def test_rope_relative_position():
    # scores between rotated q and k depend only on the position difference
    r = rng(3)
    q = r.normal(size=(1, 1, 128))
    k = r.normal(size=(1, 1, 128))
    p1 = np.array([[0.0, 3.0, 5.0, 7.0]])
    k1 = np.array([[0.0, 1.0, 2.0, 4.0]])
    shift = np.array([[0.0, 11.0, -4.0, 9.0]])

    def score(pq, pk):
        return float((O.apply_rope(q, O.rope_angles(pq)) * O.apply_rope(k, O.rope_angles(pk))).sum())

    assert abs(score(p1, k1) - score(p1 + shift, k1 + shift)) < 1e-10
    assert abs(score(p1, k1) - score(p1 + 1.0, k1)) > 1e-3


# ------------------------------------------------------------------ norms, activations

def test_layer_norm_matches_library():
    x = rng(4).normal(3.0, 2.0, (9, 256))
    ref = F.layer_norm(torch.tensor(x), (256,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, 1e-6), ref, rtol=0, atol=1e-12)
    y = O.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(-1), 1, atol=1e-12)


def test_rms_norm_matches_library():
    r = rng(5)
    x = r.normal(size=(7, 3, 128))
    w = r.uniform(0.5, 1.5, 128)
    ref = F.rms_norm(torch.tensor(x), (128,), torch.tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref, rtol=0, atol=1e-12)
    y = O.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1, atol=1e-12)


def test_silu_matches_library():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.tensor(z)).numpy(), rtol=1e-13, atol=1e-300)


# ------------------------------------------------------------------ attention

def test_attention_matches_library():
    r = rng(6)
    n, h, d = 13, 2, 128
    q, k, v = (r.normal(size=(n, h, d)) for _ in range(3))
    seg = O.segment_ids(4, 6, 3)
    for mask in (O.MASK_FULL, O.MASK_SEGMENT):
        got = O.attention(q, k, v, seg, mask)
        am = None if mask == O.MASK_FULL else torch.tensor(seg[:, None] == seg[None, :])
        ref = F.scaled_dot_product_attention(
            torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
            torch.tensor(v).transpose(0, 1), attn_mask=am).transpose(0, 1).numpy()
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_invariants():
    r = rng(7)
    n, h, d = 11, 2, 128
    q, k = r.normal(size=(n, h, d)), r.normal(size=(n, h, d))
    seg = O.segment_ids(3, 5, 3)
    # constant values -> constant output
    v = np.full((n, h, d), 0.37)
    np.testing.assert_allclose(O.attention(q, k, v, seg, O.MASK_FULL), 0.37, atol=1e-14)
    # q = 0 -> uniform weights: output is the mean of the allowed values
    v = r.normal(size=(n, h, d))
    z = np.zeros_like(q)
    np.testing.assert_allclose(O.attention(z, k, v, seg, O.MASK_FULL),
                               np.broadcast_to(v.mean(0), (n, h, d)), atol=1e-13)
    o = O.attention(z, k, v, seg, O.MASK_SEGMENT)
    for s in range(3):
        sel = seg == s
        np.testing.assert_allclose(o[sel], np.broadcast_to(v[sel].mean(0), o[sel].shape), atol=1e-13)


# ------------------------------------------------------------------ one block

def torch_block(x, segs, sets, sos, mods, pos, mask, dims, act=None, act2=None):
    """Independent composition of torch float64 library routines for one block; act and act2
    (if given) are applied to the inputs of the first and the second projection."""
    act = act or (lambda t: t)
    act2 = act2 or act
    d, nh, hd, f = dims.hidden, dims.heads, dims.head_dim, dims.mlp_hidden
    seg = torch.tensor(O.segment_ids(*segs))
    n = x.shape[0]
    X = torch.tensor(x)
    M = torch.stack([torch.tensor(mods[int(s)]) for s in seg])          # [n, 3D]
    shift, scale, gate = M[:, :d], M[:, d:2 * d], M[:, 2 * d:]
    xm = act(F.layer_norm(X, (d,), eps=dims.ln_eps) * (1 + scale) + shift)
    W1 = torch.stack([torch.tensor(sets[sos[int(s)]].w1) for s in seg])  # [n, 3D+2F, D]
    h = torch.einsum("nk,nok->no", xm, W1)
    q, k, v = h[:, :d].reshape(n, nh, hd), h[:, d:2 * d].reshape(n, nh, hd), h[:, 2 * d:3 * d].reshape(n, nh, hd)
    qw = torch.stack([torch.tensor(sets[sos[int(s)]].qn) for s in seg])[:, None, :]
    kw = torch.stack([torch.tensor(sets[sos[int(s)]].kn) for s in seg])[:, None, :]
    q = F.rms_norm(q, (hd,), eps=dims.rms_eps) * qw
    k = F.rms_norm(k, (hd,), eps=dims.rms_eps) * kw
    q = torch.tensor(rope_complex(q.numpy(), pos, dims.rope_theta))
    k = torch.tensor(rope_complex(k.numpy(), pos, dims.rope_theta))
    am = None if mask == O.MASK_FULL else (seg[:, None] == seg[None, :])
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       attn_mask=am).transpose(0, 1).reshape(n, d)
    g, u = h[:, 3 * d:3 * d + f], h[:, 3 * d + f:]
    cat = act2(torch.cat([o, F.silu(g) * u], dim=1))
    W2 = torch.stack([torch.tensor(sets[sos[int(s)]].w2) for s in seg])
    return (X + gate * torch.einsum("nk,nok->no", cat, W2)).numpy()


@pytest.mark.parametrize("mask,sos,segs", [
    (O.MASK_FULL, (0, 0, 0), (4, 6, 0)),
    (O.MASK_FULL, (0, 1, 1), (5, 4, 3)),
    (O.MASK_SEGMENT, (0, 1, 2), (3, 6, 4)),
])
def test_block_matches_library_composition(mask, sos, segs):
    r = rng(8)
    dims = TINY
    n = sum(segs)
    sets = [rand_set(r, dims) for _ in range(3)]
    mods = rand_mods(r, dims)
    x = r.normal(size=(n, dims.hidden))
    pos = O.positions(segs[0], (2, segs[1] // 2), ((segs[2], 1),) if segs[2] else ())
    got = O.block_forward(x, segs, sets, sos, mods, pos, mask, dims)
    ref = torch_block(x, segs, sets, sos, mods, pos, mask, dims)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    # computing a subset of rows gives the same rows
    rows = np.array([0, n // 2, n - 1])
    np.testing.assert_allclose(O.block_forward(x, segs, sets, sos, mods, pos, mask, dims, rows=rows),
                               got[rows], rtol=0, atol=1e-12)


def torch_sequential_block(x, segs, sets, sos, mods6, pos, mask, dims, act=None, act2=None):
    """Independent torch float64 composition of a sequentially wired double block: attention
    with (shift1, scale1, gate1), then the SwiGLU MLP on the updated residual with (shift2,
    scale2, gate2); act and act2 (if given) are applied to the inputs of the first and the
    second projection of each half."""
    act = act or (lambda t: t)
    act2 = act2 or act
    d, nh, hd, f = dims.hidden, dims.heads, dims.head_dim, dims.mlp_hidden
    seg = torch.tensor(O.segment_ids(*segs))
    n = x.shape[0]
    X = torch.tensor(x)
    M = torch.stack([torch.tensor(mods6[int(s)]) for s in seg])          # [n, 6D]
    sh1, sc1, g1, sh2, sc2, g2 = (M[:, i * d:(i + 1) * d] for i in range(6))
    W1 = torch.stack([torch.tensor(sets[sos[int(s)]].w1) for s in seg])  # [n, 3D+2F, D]
    W2 = torch.stack([torch.tensor(sets[sos[int(s)]].w2) for s in seg])  # [n, D, D+F]
    xm = act(F.layer_norm(X, (d,), eps=dims.ln_eps) * (1 + sc1) + sh1)
    h = torch.einsum("nk,nok->no", xm, W1[:, :3 * d])
    q, k, v = h[:, :d].reshape(n, nh, hd), h[:, d:2 * d].reshape(n, nh, hd), h[:, 2 * d:].reshape(n, nh, hd)
    qw = torch.stack([torch.tensor(sets[sos[int(s)]].qn) for s in seg])[:, None, :]
    kw = torch.stack([torch.tensor(sets[sos[int(s)]].kn) for s in seg])[:, None, :]
    q = torch.tensor(rope_complex((F.rms_norm(q, (hd,), eps=dims.rms_eps) * qw).numpy(), pos, dims.rope_theta))
    k = torch.tensor(rope_complex((F.rms_norm(k, (hd,), eps=dims.rms_eps) * kw).numpy(), pos, dims.rope_theta))
    am = None if mask == O.MASK_FULL else (seg[:, None] == seg[None, :])
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       attn_mask=am).transpose(0, 1).reshape(n, d)
    X1 = X + g1 * torch.einsum("nk,nok->no", act2(o), W2[:, :, :d])
    xm2 = act(F.layer_norm(X1, (d,), eps=dims.ln_eps) * (1 + sc2) + sh2)
    gu = torch.einsum("nk,nok->no", xm2, W1[:, 3 * d:])
    m = act2(F.silu(gu[:, :f]) * gu[:, f:])
    return (X1 + g2 * torch.einsum("nk,nok->no", m, W2[:, :, d:])).numpy()


@pytest.mark.parametrize("sos,segs", [((0, 1, 1), (5, 4, 3)), ((0, 1, 1), (4, 6, 0))])
def test_sequential_block_matches_library_composition(sos, segs):
    r = rng(60)
    dims = TINY
    n = sum(segs)
    sets = [rand_set(r, dims) for _ in range(2)]
    mods6 = [np.concatenate([a, b]) for a, b in zip(rand_mods(r, dims), rand_mods(r, dims))]
    x = r.normal(size=(n, dims.hidden))
    pos = O.positions(segs[0], (2, segs[1] // 2), ((segs[2], 1),) if segs[2] else ())
    got = O.block_forward_sequential(x, segs, sets, sos, mods6, pos, O.MASK_FULL, dims)
    ref = torch_sequential_block(x, segs, sets, sos, mods6, pos, O.MASK_FULL, dims)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    # differs from the parallel wiring of the same weights
    par = O.block_forward(x, segs, sets, sos, [m[:3 * dims.hidden] for m in mods6], pos,
                          O.MASK_FULL, dims)
    assert not np.allclose(got, par)
    # both gates zero: identity
    z = [np.concatenate([m[:2 * dims.hidden], np.zeros(dims.hidden), m[3 * dims.hidden:5 * dims.hidden],
                         np.zeros(dims.hidden)]) for m in mods6]
    np.testing.assert_array_equal(O.block_forward_sequential(x, segs, sets, sos, z, pos, O.MASK_FULL, dims), x)
    # sampled rows (text, image and reference rows among them) equal those rows of the full block
    rows = np.array([0, segs[0], n - 1])
    np.testing.assert_allclose(
        O.block_forward_sequential(x, segs, sets, sos, mods6, pos, O.MASK_FULL, dims, rows=rows),
        ref[rows], rtol=0, atol=1e-11)


def test_block_gate_zero_is_identity():
    r = rng(9)
    x = r.normal(size=(10, TINY.hidden))
    sets = [rand_set(r, TINY)]
    mods = rand_mods(r, TINY, gate_zero=True)
    pos = O.positions(4, (2, 3))
    out = O.block_forward(x, (4, 6, 0), sets, (0, 0, 0), mods, pos, O.MASK_FULL, TINY)
    np.testing.assert_array_equal(out, x)


def test_double_block_with_equal_sets_is_single_block():
    r = rng(10)
    s = rand_set(r, TINY)
    m = rand_mods(r, TINY, n=1)[0]
    x = r.normal(size=(9, TINY.hidden))
    pos = O.positions(3, (2, 3))
    a = O.block_forward(x, (3, 6, 0), [s, s], (0, 1, 1), [m, m, m], pos, O.MASK_FULL, TINY)
    b = O.block_forward(x, (3, 6, 0), [s], (0, 0, 0), [m, m, m], pos, O.MASK_FULL, TINY)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_per_mode_block_equals_separate_streams():
    """Per-mode blocks = each stream run on its own with its own weights (the stream sees
    only itself)."""
    r = rng(11)
    segs = (4, 6, 6)
    n = sum(segs)
    sets = [rand_set(r, TINY) for _ in range(3)]
    mods = rand_mods(r, TINY)
    x = r.normal(size=(n, TINY.hidden))
    pos = O.positions(4, (2, 3), ((2, 3),))
    joint = O.block_forward(x, segs, sets, (0, 1, 2), mods, pos, O.MASK_SEGMENT, TINY)
    start = 0
    for s in range(3):
        sl = slice(start, start + segs[s])
        alone = O.block_forward(x[sl], (segs[s], 0, 0), [sets[s]], (0, 0, 0),
                                [mods[s]] * 3, pos[sl], O.MASK_FULL, TINY)
        np.testing.assert_allclose(joint[sl], alone, rtol=0, atol=1e-12)
        start += segs[s]


def test_joint_block_with_equal_mods_is_single_block():
    r = rng(12)
    s = rand_set(r, TINY)
    m = rand_mods(r, TINY, n=1)[0]
    x = r.normal(size=(10, TINY.hidden))
    pos = O.positions(2, (2, 2), ((2, 2),))
    a = O.block_forward(x, (2, 4, 4), [s], (0, 0, 0), [m, m, m], pos, O.MASK_FULL, TINY)
    b = O.block_forward(x, (10, 0, 0), [s], (0, 0, 0), [m, m, m], pos, O.MASK_FULL, TINY)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ conditioning, head, Euler

def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(0.0, 256)
    np.testing.assert_array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    e = O.timestep_embedding(0.37, 256)
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-15)
    assert abs(e[0] - math.cos(370.0)) < 1e-12          # f_0 = 1: angle 1000 t
    assert abs(e[128 + 64] - math.sin(370.0 * 10000 ** -0.5)) < 1e-12


def test_modulation_and_cond_match_library():
    r = rng(13)
    d = 64
    w_mod = r.normal(size=(3 * d, d))
    c = r.normal(size=d)
    ref = F.linear(F.silu(torch.tensor(c)), torch.tensor(w_mod)).numpy()
    np.testing.assert_allclose(O.modulation(w_mod, c), ref, atol=1e-12)
    w1, w2 = r.normal(size=(d, 32)), r.normal(size=(d, d))
    e = torch.tensor(O.timestep_embedding(0.5, 32))
    ref = F.linear(F.silu(F.linear(e, torch.tensor(w1))), torch.tensor(w2)).numpy()
    np.testing.assert_allclose(O.cond_vector(0.5, w1, w2), ref, atol=1e-12)


def test_cond_rows_per_token_type():
    r = rng(14)
    w1, w2 = r.normal(size=(16, 32)), r.normal(size=(16, 16))
    c2 = O.cond_rows(O.ARCH_FLUX2, 0.7, w1, w2)
    assert np.array_equal(c2[0], c2[1]) and np.array_equal(c2[1], c2[2])
    c3 = O.cond_rows(O.ARCH_FLUX3, 0.7, w1, w2)
    assert np.array_equal(c3[0], O.cond_vector(0.0, w1, w2))
    assert np.array_equal(c3[2], c3[0]) and not np.allclose(c3[1], c3[0])


def test_final_layer_matches_library():
    r = rng(15)
    d, c = 64, 16
    x = r.normal(size=(5, d))
    cond = r.normal(size=d)
    w_fmod, w_out = r.normal(size=(2 * d, d)), r.normal(size=(c, d))
    fm = F.linear(F.silu(torch.tensor(cond)), torch.tensor(w_fmod))
    y = F.layer_norm(torch.tensor(x), (d,), eps=1e-6) * (1 + fm[d:]) + fm[:d]
    ref = F.linear(y, torch.tensor(w_out)).numpy()
    np.testing.assert_allclose(O.final_layer(x, cond, w_fmod, w_out, 1e-6), ref, atol=1e-12)


def test_euler_closed_forms():
    ts = O.euler_schedule(4)
    assert ts[0] == 1.0 and ts[-1] == 0.0 and np.all(np.diff(ts) < 0)
    lat = rng(16).normal(size=(6, 4))
    c = 0.25
    out = lat.copy()
    for i in range(4):
        out = O.euler_step(out, np.full_like(lat, c), ts[i], ts[i + 1])
    np.testing.assert_allclose(out, lat + c, atol=1e-15)     # sum of steps = 1
    np.testing.assert_array_equal(O.euler_step(lat, np.zeros_like(lat), 1.0, 0.5), lat)


def tiny_model(arch, r, n_stream=1, n_shared=1, zero_out=False):
    dims = TINY
    d, c = dims.hidden, dims.in_channels
    nsets = 2 if arch == O.ARCH_FLUX2 else 3
    m = O.Model(arch=arch, dims=dims, n_stream=n_stream, n_shared=n_shared,
                img_in=r.normal(0, 0.1, (d, c)), temb_l1=r.normal(0, 0.1, (d, dims.time_dim)),
                temb_l2=r.normal(0, 0.1, (d, d)), final_mod=r.normal(0, 0.05, (2 * d, d)),
                final_out=np.zeros((c, d)) if zero_out else r.normal(0, 0.05, (c, d)))
    m.mods = [[r.normal(0, 0.05, (3 * d, d)) for _ in range(nsets)], [r.normal(0, 0.05, (3 * d, d))]]
    m.blocks = [[rand_set(r, dims) for _ in range(nsets)] for _ in range(n_stream)] + \
               [[rand_set(r, dims)] for _ in range(n_shared)]
    return m


def test_denoise_zero_head_keeps_noise():
    r = rng(17)
    m = tiny_model(O.ARCH_FLUX2, r, zero_out=True)
    noise = r.normal(size=(4, TINY.in_channels))
    txt = r.normal(size=(3, TINY.hidden))
    np.testing.assert_array_equal(O.denoise(m, noise, txt, (2, 2), 3), noise)


def test_forward_stack_is_block_composition():
    """forward() = img_in, the planned blocks, then the output head on image rows."""
    r = rng(18)
    for arch in (O.ARCH_FLUX2, O.ARCH_FLUX3):
        m = tiny_model(arch, r)
        lat = r.normal(size=(4, TINY.in_channels))
        ref_lat = r.normal(size=(4, TINY.in_channels))
        txt = r.normal(size=(3, TINY.hidden))
        seen = []
        v = O.forward(m, lat, txt, (2, 2), 0.6, ref_lat, (2, 2), block_hook=lambda b, x: seen.append(x.copy()))
        assert len(seen) == 2
        np.testing.assert_allclose(seen[0][3:7], lat @ m.img_in.T, atol=1e-14)
        np.testing.assert_allclose(seen[0][7:], ref_lat @ m.img_in.T, atol=1e-14)
        assert v.shape == (4, TINY.in_channels)
        # the per-mode block of FLUX.3 keeps streams apart: changing the reference latents
        # does not change the image rows after the first (per-mode) block
        if arch == O.ARCH_FLUX3:
            seen2 = []
            O.forward(m, lat, txt, (2, 2), 0.6, ref_lat * 2.0, (2, 2),
                      block_hook=lambda b, x: seen2.append(x.copy()))
            np.testing.assert_allclose(seen2[1][:7], seen[1][:7], atol=1e-13)
            assert not np.allclose(seen2[1][7:], seen[1][7:])


# ------------------------------------------------------------------ classifier-free guidance

def test_guided_velocity_closed_forms():
    """g = 1 gives the conditional velocity, g = 0 the unconditional one; the result is affine
    in g (g = 2 gives 2 v_c - v_u); equal branches give that velocity at any g."""
    r = rng(30)
    vc, vu = r.normal(size=(5, 4)), r.normal(size=(5, 4))
    np.testing.assert_allclose(O.guided_velocity(vc, vu, 1.0), vc, atol=1e-15)
    np.testing.assert_array_equal(O.guided_velocity(vc, vu, 0.0), vu)
    np.testing.assert_allclose(O.guided_velocity(vc, vu, 2.0), 2 * vc - vu, atol=1e-14)
    np.testing.assert_allclose(O.guided_velocity(vc, vc, 3.5), vc, atol=1e-14)


def test_forward_cfg_branches():
    """The guided call is the conditional call at g = 1 and the unconditional one at g = 0;
    with the same text for both branches it does not depend on g; the guided denoise at g = 1
    is the plain denoise."""
    r = rng(31)
    for arch in (O.ARCH_FLUX2, O.ARCH_FLUX3):
        m = tiny_model(arch, r)
        lat = r.normal(size=(4, TINY.in_channels))
        ref_lat = r.normal(size=(4, TINY.in_channels))
        tc, tu = r.normal(size=(3, TINY.hidden)), r.normal(size=(3, TINY.hidden))
        vc = O.forward(m, lat, tc, (2, 2), 0.7, ref_lat, (2, 2))
        vu = O.forward(m, lat, tu, (2, 2), 0.7, ref_lat, (2, 2))
        assert not np.allclose(vc, vu)
        np.testing.assert_allclose(O.forward_cfg(m, lat, tc, tu, (2, 2), 0.7, 1.0, ref_lat, (2, 2)), vc, atol=1e-13)
        np.testing.assert_allclose(O.forward_cfg(m, lat, tc, tu, (2, 2), 0.7, 0.0, ref_lat, (2, 2)), vu, atol=1e-13)
        np.testing.assert_allclose(O.forward_cfg(m, lat, tc, tc, (2, 2), 0.7, 3.5, ref_lat, (2, 2)), vc, atol=1e-13)
        g = 3.5
        np.testing.assert_allclose(O.forward_cfg(m, lat, tc, tu, (2, 2), 0.7, g, ref_lat, (2, 2)),
                                   vu + g * (vc - vu), atol=1e-12)
        noise = r.normal(size=(4, TINY.in_channels))
        np.testing.assert_allclose(O.denoise_cfg(m, noise, tc, tu, (2, 2), 2, 1.0),
                                   O.denoise(m, noise, tc, (2, 2), 2), atol=1e-12)


# ------------------------------------------------------------------ image-to-image, several references

def test_img2img_schedule_and_mix():
    """The straight path from the clean latents (t = 0) to the noise (t = 1); the loop runs
    the last floor(n s) steps; strength 1 is the plain sampler from the noise."""
    r = rng(50)
    x, e = r.normal(size=(5, 4)), r.normal(size=(5, 4))
    np.testing.assert_array_equal(O.noise_mix(x, e, 0.0), x)
    np.testing.assert_array_equal(O.noise_mix(x, e, 1.0), e)
    np.testing.assert_allclose(O.noise_mix(x, e, 0.25), x + 0.25 * (e - x), atol=1e-15)
    assert [O.img2img_first_step(4, s) for s in (1.0, 0.75, 0.5, 0.25, 0.2)] == [0, 1, 2, 3, 4]
    assert O.img2img_first_step(50, 0.75) == 13          # 37 of 50 steps
    m = tiny_model(O.ARCH_FLUX2, r)
    txt = r.normal(size=(3, TINY.hidden))
    x = r.normal(size=(4, TINY.in_channels))
    e = r.normal(size=(4, TINY.in_channels))
    np.testing.assert_array_equal(O.img2img(m, x, e, txt, (2, 2), 3, 1.0), O.denoise(m, e, txt, (2, 2), 3))
    with pytest.raises(ValueError):
        O.img2img(m, x, e, txt, (2, 2), 4, 0.2)
    # a zero output head: the result is the starting point on the path, t = 3/4
    mz = tiny_model(O.ARCH_FLUX2, r, zero_out=True)
    np.testing.assert_array_equal(O.img2img(mz, x, e, txt, (2, 2), 4, 0.75), O.noise_mix(x, e, 0.75))


def test_several_references_use_their_own_sequence_axis():
    """Two references are two images at l = -1 and l = -2: the same latents laid out as one
    taller reference (all at l = -1) give a different velocity, and a list of one grid is the
    single-reference call."""
    r = rng(51)
    m = tiny_model(O.ARCH_FLUX3, r)
    lat = r.normal(size=(4, TINY.in_channels))
    refs = r.normal(size=(8, TINY.in_channels))
    txt = r.normal(size=(3, TINY.hidden))
    two = O.forward(m, lat, txt, (2, 2), 0.6, refs, [(2, 2), (2, 2)])
    tall = O.forward(m, lat, txt, (2, 2), 0.6, refs, (4, 2))
    assert not np.allclose(two, tall)
    np.testing.assert_array_equal(O.forward(m, lat, txt, (2, 2), 0.6, refs[:4], [(2, 2)]),
                                  O.forward(m, lat, txt, (2, 2), 0.6, refs[:4], (2, 2)))


# ------------------------------------------------------------------ FLUX.3 conditioning preamble

def test_text_feature_layout_matches_printed_values():
    with open(os.path.join(os.path.dirname(GOLDEN), "text_features.json")) as f:
        g = json.load(f)
    assert O.TEXT_ENCODER_DEPTH == g["encoder_layers_total"]
    assert list(O.TEXT_FEATURE_LAYERS) == g["layers"]
    assert O.TEXT_HIDDEN == g["hidden"]
    assert len(O.TEXT_FEATURE_LAYERS) * O.TEXT_HIDDEN == g["stacked_width"]
    # every 4th layer of 36, none past the last
    assert all(l % 4 == 0 and 0 < l <= g["encoder_layers_total"] for l in g["layers"])
    # stacking keeps the listed layer order: layer l's state fills its own column block
    n = 3
    hid = {l: np.full((n, 5), float(l)) for l in O.TEXT_FEATURE_LAYERS}
    st = O.stack_text_features(hid)
    assert st.shape == (n, 8 * 5)
    np.testing.assert_array_equal(st[0], np.repeat(np.array(g["layers"], float), 5))


def test_text_projection_identities():
    """A one-hot feature picks that column of txt_in (catches a transposed weight); the
    projection is additive."""
    r = rng(40)
    w = r.normal(size=(6, 32))
    e = np.zeros((1, 32))
    e[0, 7] = 1.0
    np.testing.assert_array_equal(O.project_text(e, w)[0], w[:, 7])
    a, b = r.normal(size=(4, 32)), r.normal(size=(4, 32))
    np.testing.assert_allclose(O.project_text(a + b, w), O.project_text(a, w) + O.project_text(b, w),
                               atol=1e-13)


def test_flow_map_cond_rows():
    """A zero target-time MLP leaves the plain conditioning; otherwise every segment's row
    moves by the same vector, the target time's own embedding, whatever the segment's time."""
    r = rng(41)
    d, td = 8, 16
    l1, l2 = r.normal(size=(d, td)), r.normal(size=(d, d))
    tl1, tl2 = r.normal(size=(d, td)), r.normal(size=(d, d))
    for arch in (O.ARCH_FLUX2, O.ARCH_FLUX3):
        plain = O.cond_rows(arch, 0.6, l1, l2)
        zero = O.flow_map_cond_rows(arch, 0.6, 0.3, l1, l2, np.zeros_like(tl1), np.zeros_like(tl2))
        for a, b in zip(zero, plain):
            np.testing.assert_array_equal(a, b)
        fm = O.flow_map_cond_rows(arch, 0.6, 0.3, l1, l2, tl1, tl2)
        want = l2 @ O.silu(l1 @ O.timestep_embedding(0.6, td))
        tgt = tl2 @ O.silu(tl1 @ O.timestep_embedding(0.3, td))
        for s in range(3):
            np.testing.assert_allclose(fm[s] - plain[s], tgt, atol=1e-12)
        np.testing.assert_allclose(fm[1], want + tgt, atol=1e-12)
        other = O.flow_map_cond_rows(arch, 0.6, 0.1, l1, l2, tl1, tl2)
        assert not np.allclose(other[1], fm[1])


def test_forward_per_block_modulation():
    """Per-block modulation projections that alias the shared ones give the shared model's
    velocity exactly; with every block's gate rows zero the stack is the identity, so the
    velocity is the output head on the embedded latents; distinct projections change it."""
    r = rng(43)
    for arch in (O.ARCH_FLUX2, O.ARCH_FLUX3):
        m = tiny_model(arch, r)
        lat = r.normal(size=(4, TINY.in_channels))
        txt = r.normal(size=(3, TINY.hidden))
        v_shared = O.forward(m, lat, txt, (2, 2), 0.6)
        m.block_mods = [m.mods[O.block_plan(arch, b, m.n_stream)[0]] for b in range(m.n_stream + m.n_shared)]
        np.testing.assert_array_equal(O.forward(m, lat, txt, (2, 2), 0.6), v_shared)
        d = TINY.hidden
        zero_gate = []
        for sets in m.block_mods:
            zs = []
            for w in sets:
                w = w.copy()
                w[2 * d:3 * d] = 0.0
                zs.append(w)
            zero_gate.append(zs)
        m.block_mods = zero_gate
        cond_img = O.cond_rows(arch, 0.6, m.temb_l1, m.temb_l2)[1]
        want = O.final_layer(lat @ m.img_in.T, cond_img, m.final_mod, m.final_out, TINY.ln_eps)
        np.testing.assert_allclose(O.forward(m, lat, txt, (2, 2), 0.6), want, rtol=0, atol=1e-12)
        m.block_mods = [[r.normal(0, 0.05, w.shape) for w in sets] for sets in m.block_mods]
        assert not np.allclose(O.forward(m, lat, txt, (2, 2), 0.6), v_shared)


def test_flow_map_forward():
    """A flow-map model with a zero target MLP is the plain model; it needs the target time;
    with a real target MLP the velocity depends on the target time."""
    r = rng(42)
    for arch in (O.ARCH_FLUX2, O.ARCH_FLUX3):
        m = tiny_model(arch, r)
        lat = r.normal(size=(4, TINY.in_channels))
        txt = r.normal(size=(3, TINY.hidden))
        v_plain = O.forward(m, lat, txt, (2, 2), 0.6)
        m.temb_tgt_l1 = np.zeros((TINY.hidden, TINY.time_dim))
        m.temb_tgt_l2 = np.zeros((TINY.hidden, TINY.hidden))
        np.testing.assert_array_equal(O.forward(m, lat, txt, (2, 2), 0.6, t_target=0.2), v_plain)
        with pytest.raises(ValueError):
            O.forward(m, lat, txt, (2, 2), 0.6)
        m.temb_tgt_l1 = r.normal(0, 0.1, (TINY.hidden, TINY.time_dim))
        m.temb_tgt_l2 = r.normal(0, 0.1, (TINY.hidden, TINY.hidden))
        assert not np.allclose(O.forward(m, lat, txt, (2, 2), 0.6, t_target=0.2),
                               O.forward(m, lat, txt, (2, 2), 0.6, t_target=0.4))


# ------------------------------------------------------------------ the pins catch planted slips

def _wrong_rope(x, angles):
    n, h, d = x.shape
    xr = x.reshape(n, h, 4, 16, 2)
    c, s = np.cos(angles)[:, None], np.sin(angles)[:, None]
    out = np.empty_like(xr)
    out[..., 0] = xr[..., 0] * c + xr[..., 1] * s      # sign slip
    out[..., 1] = -xr[..., 0] * s + xr[..., 1] * c
    return out.reshape(n, h, d)


# ------------------------------------------------------------------ seeded noise

def test_philox_known_answers():
    """The generator reproduces the published known-answer vectors bit for bit."""
    with open(PHILOX_KAT) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = np.array([int(w, 16) for w in v["counter"]], dtype=np.uint64)
        key = [int(w, 16) for w in v["key"]]
        got = O.philox4x32(ctr, key, rounds=kat["rounds"])
        assert [f"{int(w):08x}" for w in got] == v["output"]


def test_noise_inverts_to_its_uniforms():
    """Box-Muller closed form: z0^2 + z1^2 = -2 ln u0 and atan2(z1, z0) = 2 pi u1 (mod 2 pi),
    with u the Philox words of the element's counter, (w + 1/2) / 2^32."""
    n, seed = 4 * 257 + 3, (7 << 32) | 12345
    z = O.noise(n, seed)
    assert z.shape == (n,)
    g = np.arange((n + 3) // 4, dtype=np.uint64)
    ctr = np.stack([g, np.zeros_like(g), np.zeros_like(g), np.zeros_like(g)], -1)
    u = (O.philox4x32(ctr, (12345, 7)).astype(np.float64) + 0.5) / 2.0 ** 32
    zz = np.concatenate([z, np.zeros(4 * len(g) - n)]).reshape(-1, 4)
    for a in (0, 2):
        r2 = zz[:-1, a] ** 2 + zz[:-1, a + 1] ** 2
        np.testing.assert_allclose(np.exp(-0.5 * r2), u[:-1, a], rtol=1e-12)
        ang = np.mod(np.arctan2(zz[:-1, a + 1], zz[:-1, a]) / (2 * np.pi), 1.0)
        d = np.abs(ang - u[:-1, a + 1])
        assert np.all(np.minimum(d, 1 - d) < 1e-12)


def test_noise_distribution_and_prefix():
    """N(0,1) in distribution (Kolmogorov-Smirnov), pairs uncorrelated, counter-based (a
    shorter draw is a prefix of a longer one), and the seed's high word matters."""
    from scipy import stats
    z = O.noise(200_003, 42)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    assert abs(z.mean()) < 5 / math.sqrt(len(z))
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / len(z))
    assert abs(np.corrcoef(z[0:-3:4], z[1:-2:4])[0, 1]) < 5 / math.sqrt(len(z) / 4)
    np.testing.assert_array_equal(O.noise(1001, 42), z[:1001])
    assert not np.array_equal(O.noise(64, 42), O.noise(64, 42 + (1 << 32)))


# ------------------------------------------------------------------ row-wise FP8 (fp8r)

def _e4m3_ties():
    """Midpoints of neighbouring non-negative E4M3 values (from the decoded code table)."""
    grid = np.unique(O.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    return (grid[:-1] + grid[1:]) / 2


def torch_fp8_rows(X):
    """Row-wise E4M3 values through torch's float8_e4m3fn conversion of the float64 quotients
    X * 448 / max|row| (round to nearest even), independent of the oracle's rounding code.
    torch converts float64 through fp32, which can move a quotient exactly onto a tie of two
    E4M3 values; there the fp32 value is nudged one fp32 step toward the true quotient first,
    so torch rounds it to the side the quotient lies on."""
    X = X.to(torch.float64)
    amax = X.abs().amax(dim=1, keepdim=True)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    q = torch.where(amax > 0, X * 448.0 / safe, torch.zeros_like(X))
    q32 = q.to(torch.float32)
    ties = torch.tensor(_e4m3_ties())
    on_tie = torch.isin(q32.abs().to(torch.float64), ties) & (q32.to(torch.float64) != q)
    toward = torch.where(q > q32.to(torch.float64), torch.tensor(math.inf), torch.tensor(-math.inf))
    q32 = torch.where(on_tie, torch.nextafter(q32, toward.to(torch.float32)), q32)
    return q32.to(torch.float8_e4m3fn).to(torch.float64) * (amax / 448.0)


def _e4m3_torch(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_library():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and np.sum(np.isnan(got)) == 2
    # encoding the finite values gives their codes back (-0 included)
    np.testing.assert_array_equal(O.e4m3_encode(got[ok]), codes[ok])


def test_e4m3_round_matches_library():
    r = rng(70)
    mag = np.exp2(r.uniform(-12, np.log2(448), 20000))
    v = (mag * r.choice([-1, 1], mag.size)).astype(np.float32).astype(np.float64)
    # every code value and every midpoint of neighbouring positive codes, both signs
    grid = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([v, grid, -grid, mids, -mids])
    np.testing.assert_array_equal(O.e4m3_round(v), _e4m3_torch(v))


def test_e4m3_round_closed_forms():
    v = np.array([464.0, 465.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6 - 2.0 ** -10,
                  17.0, 18.0, 19.0, 0.0])
    want = np.array([448.0, 448.0, 448.0, -448.0, 0.0, 2.0 ** -8, 2.0 ** -6,
                     16.0, 18.0, 20.0, 0.0])
    np.testing.assert_array_equal(O.e4m3_round(v), want)


def test_quantize_rows_fp8_properties():
    r = rng(71)
    x = r.normal(size=(6, 300)) * np.array([1e-3, 1, 50, 3e4, 1, 1])[:, None]
    x[4] = 0.0
    codes, scale = O.quantize_rows_fp8(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float64
    # the largest magnitude of each row lands on +-448; a zero row has scale 0 and codes 0
    for i in (0, 1, 2, 3, 5):
        j = np.argmax(np.abs(x[i]))
        assert codes[i, j] & 0x7F == 0x7E
    assert scale[4] == 0 and not codes[4].any()
    # a power-of-two factor changes the scale only
    c2, s2 = O.quantize_rows_fp8(x * 2.0 ** 7)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scale * 2.0 ** 7)
    # each value is within half an E4M3 step (relative 2^-4, or 2^-10 of the scale) of x
    xr = O.fp8_round_rows(x)
    sc = scale[:, None]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-12)
    assert np.all(np.abs(xr - x) <= bound)
    np.testing.assert_array_equal(xr, torch_fp8_rows(torch.tensor(x)).numpy())


def _nearest_e4m3_exact(q):
    """Code of the E4M3 value nearest to the exact rational q (|q| <= 448) by brute force over
    the code table, ties to the code with the even mantissa bit."""
    from fractions import Fraction
    mag = abs(q)
    best = None
    for c in range(0x7F):
        v = Fraction(float(O.e4m3_decode(np.array([c], np.uint8))[0]))
        key = (abs(v - mag), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    return code | (0x80 if q < 0 and code else 0)


def test_quantize_rows_fp8_matches_exact_rational_rounding():
    """Codes equal the E4M3 rounding of the exact quotient value * 448 / max|row| (computed in
    rational arithmetic), including quotients that are exactly ties and quotients a few fp32
    steps on either side of a tie; scales equal max|row| / 448 correctly rounded."""
    from fractions import Fraction
    r = rng(74)
    ties = _e4m3_ties()
    rows = []
    rows.append(r.normal(size=40).astype(np.float32))                 # random values
    t = r.choice(ties, 40) * r.choice([-1, 1], 40)                    # exact ties, max 448
    t[0] = 448.0
    rows.append(t.astype(np.float32))
    amax = np.float32(3.5)                                            # ties after a 2^7 scale
    t2 = (r.choice(ties[ties < 440], 40) * (3.5 / 448)).astype(np.float32)
    t2[0] = amax
    rows.append(t2)
    for sgn in (-1, 1):                                               # near ties, both sides
        near = r.choice(ties[ties < 440], 40) * (1 + sgn * 3 * 2.0 ** -23)
        near[0] = 448.0
        rows.append(near.astype(np.float32))
    # a generic row maximum: the quotients of the fp32 values nearest tie * max / 448 lie
    # within an fp32 rounding of the tie without being on it
    am = np.float64(np.float32(1000.123))
    hz = (r.choice(ties[(ties < 440) & (ties > 2.0 ** -5)], 40) * r.choice([-1, 1], 40) * am / 448)
    hz = hz.astype(np.float32).astype(np.float64)
    hz[0] = am
    q = hz * 448 / am
    q32 = q.astype(np.float32).astype(np.float64)
    assert np.sum(np.isin(np.abs(q32), ties) & (q32 != q)) > 20
    rows.append(hz.astype(np.float32))
    x = np.stack(rows).astype(np.float64)
    codes, scale = O.quantize_rows_fp8(x)
    for i in range(x.shape[0]):
        am = Fraction(float(np.max(np.abs(x[i]))))
        assert scale[i] == float(am / 448)
        for j in range(x.shape[1]):
            qv = Fraction(float(x[i, j])) * 448 / am
            assert codes[i, j] == _nearest_e4m3_exact(qv), (i, j, float(qv))
    # torch's conversion (with its fp32 step moved off the ties it creates) agrees
    np.testing.assert_array_equal(O.fp8_round_rows(x), torch_fp8_rows(torch.tensor(x)).numpy())


def test_fp8_projection_error_bound():
    """x W^T through row-wise E4M3 stays within the first-order bound of the two roundings."""
    r = rng(72)
    x, w = r.normal(size=(9, 256)), r.normal(0, 0.05, size=(40, 256))
    xr, wr = O.fp8_round_rows(x), O.fp8_round_rows(w)
    err = np.abs(xr @ wr.T - x @ w.T)
    bound = np.abs(xr - x) @ np.abs(w).T + np.abs(xr) @ np.abs(wr - w).T
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    assert err.max() > 0


@pytest.mark.parametrize("sequential", [False, True], ids=["parallel", "sequential"])
def test_fp8_block_matches_library_composition(sequential):
    r = rng(73)
    dims = TINY
    segs = (5, 4, 3)
    sos = (0, 1, 1)
    n = sum(segs)
    sets = [rand_set(r, dims) for _ in range(2)]
    x = r.normal(size=(n, dims.hidden))
    pos = O.positions(segs[0], (2, 2), ((3, 1),))
    q_or = O.quantize_weights_fp8(sets)
    q_t = [O.WeightSet(torch_fp8_rows(torch.tensor(ws.w1)).numpy(),
                       torch_fp8_rows(torch.tensor(ws.w2)).numpy(), ws.qn, ws.kn) for ws in sets]
    if sequential:
        mods6 = [np.concatenate([a, b]) for a, b in zip(rand_mods(r, dims), rand_mods(r, dims))]
        got = O.block_forward_sequential(x, segs, q_or, sos, mods6, pos, O.MASK_FULL, dims, act_fp8=True)
        ref = torch_sequential_block(x, segs, q_t, sos, mods6, pos, O.MASK_FULL, dims, act=torch_fp8_rows,
                                     act2=torch_fp8_rows)
        plain = O.block_forward_sequential(x, segs, sets, sos, mods6, pos, O.MASK_FULL, dims)
    else:
        mods = rand_mods(r, dims)
        got = O.block_forward(x, segs, q_or, sos, mods, pos, O.MASK_FULL, dims, act_fp8=True)
        ref = torch_block(x, segs, q_t, sos, mods, pos, O.MASK_FULL, dims, act=torch_fp8_rows,
                          act2=torch_fp8_rows)
        plain = O.block_forward(x, segs, sets, sos, mods, pos, O.MASK_FULL, dims)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    # the E4M3 rounding is visible but small against the unquantized block
    d = np.abs(got - plain).max() / np.abs(plain - x).max()
    assert 1e-3 < d < 0.2


def _per_tensor_quantize(x):
    x = np.asarray(x, np.float64)
    amax = np.max(np.abs(x))
    return O.e4m3_encode(O.e4m3_round(x * 448.0 / amax)), np.full(x.shape[0], amax / 448.0)


def _fp32_reciprocal_quantize(x):
    """The quotient formed in fp32 as value * fp32(448 / max) (two fp32 roundings)."""
    x32 = np.asarray(x, np.float32)
    amax = np.max(np.abs(x32), axis=1)
    rcp = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    q = (x32 * rcp[:, None]).astype(np.float32).astype(np.float64)
    return O.e4m3_encode(O.e4m3_round(q)), amax.astype(np.float64) / 448.0


def _wrong_layer_norm(x, eps):
    return (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, keepdims=True) + eps + 1e-3)


def test_pins_catch_planted_slips(monkeypatch):
    monkeypatch.setattr(O, "apply_rope", _wrong_rope)
    with pytest.raises(AssertionError):
        test_rope_matches_complex_rotation()
    with pytest.raises(AssertionError):
        test_block_matches_library_composition(O.MASK_FULL, (0, 0, 0), (4, 6, 0))
    monkeypatch.undo()
    monkeypatch.setattr(O, "layer_norm", _wrong_layer_norm)
    with pytest.raises(AssertionError):
        test_layer_norm_matches_library()
    monkeypatch.undo()
    # Philox with the two round multipliers swapped
    monkeypatch.setattr(O, "PHILOX_MUL", (O.PHILOX_MUL[1], O.PHILOX_MUL[0]))
    with pytest.raises(AssertionError):
        test_philox_known_answers()
    monkeypatch.undo()
    # the target time added to the image row only
    orig_fm = O.flow_map_cond_rows

    def image_only(arch, t, tt, l1, l2, tl1, tl2):
        rows = O.cond_rows(arch, t, l1, l2)
        rows[1] = rows[1] + O.cond_vector(tt, tl1, tl2)
        return rows
    monkeypatch.setattr(O, "flow_map_cond_rows", image_only)
    with pytest.raises(AssertionError):
        test_flow_map_cond_rows()
    monkeypatch.setattr(O, "flow_map_cond_rows", orig_fm)
    # the sequential block's MLP half normalising the block input instead of the updated residual
    def parallel_halves(x, segs, sets, sos, mods6, pos, mask, dims):
        d = dims.hidden
        a = O.block_forward(x, segs, sets, sos, [m[:3 * d] for m in mods6], pos, mask, dims)
        mlp_only = [O.WeightSet(np.concatenate([np.zeros((3 * d, d)), ws.w1[3 * d:]]),
                                np.concatenate([np.zeros((d, d)), ws.w2[:, d:]], axis=1), ws.qn, ws.kn)
                    for ws in sets]
        b = O.block_forward(x, segs, mlp_only, sos, [m[3 * d:] for m in mods6], pos, mask, dims)
        return a + b - x
    monkeypatch.setattr(O, "block_forward_sequential", parallel_halves)
    with pytest.raises(AssertionError):
        test_sequential_block_matches_library_composition((0, 1, 1), (5, 4, 3))
    monkeypatch.undo()
    # one scale per tensor instead of one per row
    monkeypatch.setattr(O, "quantize_rows_fp8", _per_tensor_quantize)
    with pytest.raises(AssertionError):
        test_fp8_block_matches_library_composition(False)
    monkeypatch.undo()
    # the quotient rounded through fp32 before its E4M3 rounding
    monkeypatch.setattr(O, "quantize_rows_fp8", _fp32_reciprocal_quantize)
    with pytest.raises(AssertionError):
        test_quantize_rows_fp8_matches_exact_rational_rounding()
    monkeypatch.undo()
    # guidance with the branches swapped
    monkeypatch.setattr(O, "guided_velocity", lambda vc, vu, g: vc + g * (vu - vc))
    with pytest.raises(AssertionError):
        test_guided_velocity_closed_forms()
    monkeypatch.undo()
    # a slightly wrong activation
    orig = O.silu
    monkeypatch.setattr(O, "silu", lambda z: orig(z) * 1.0001)
    with pytest.raises(AssertionError):
        test_silu_matches_library()
