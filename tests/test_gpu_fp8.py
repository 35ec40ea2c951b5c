"""GPU parity of the row-wise FP8 (E4M3) path against the oracle's E4M3 definitions.

The quantizer is compared with the oracle's float64 quantization: scales to one fp32 rounding,
codes bit for bit except where the exact quotient value * 448 / max|row| lies within two fp32
roundings of a tie between two E4M3 values (the kernel forms the quotient in fp32); there the
codes may be the two neighbours of the tie, and the test counts such cases.  The E4M3 GEMM
runs on codes and scales made by the oracle and is compared with their exact product: the MFMA
truncates products more than about 12 bits below the largest one of its group of k, so the
bar is 2^-12 of the sum of |products| per output.  Blocks are judged on their update against
the oracle's E4M3 block, with the bars of the error model in tests/golden/fp8_error_model.py
(written to tests/golden/fp8_error_model.json before any GPU run); forwards on the velocity
(FP8_TOL).
"""
from dataclasses import replace

import numpy as np
import pytest

from latent_flow_matching_amd import synth as S
from oracle import dit_oracle as O
from tests.helpers import (FP8_TOL, TINY2, TINY3, f64, fp8_bars, oracle_block, oracle_model,
                           rel_err, seg_cond)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests.test_gpu_parity import TINY3_FM, _cfg_inputs, _forward_case, _rows, context, dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_flow_matching_amd import dit
    dit.load_library()


def _matrix(rows, cols, seed):
    r = np.random.default_rng(seed)
    x = r.normal(size=(rows, cols)).astype(np.float32)
    ties = _ties()
    if rows > 3:
        x[1] *= np.float32(1e-30)       # scale far below 1 (tiny values, subnormal codes)
        x[2] *= np.float32(3e4)         # large values
        x[3] = 0.0                      # zero row: scale 0, codes 0
    if rows > 4:
        # max 448 (quotients equal the values): every midpoint of neighbouring E4M3 values,
        # an exact tie
        row = np.resize(np.concatenate([ties, -ties]), cols).astype(np.float32)
        row[0] = 448.0
        x[4] = row
    if rows > 5:
        # a generic maximum: quotients within an fp32 rounding of a tie, not on it
        am = np.float32(1000.123)
        row = (r.choice(ties[(ties < 440) & (ties > 2.0 ** -5)], cols) * r.choice([-1, 1], cols)
               * (float(am) / 448)).astype(np.float32)
        row[0] = am
        x[5] = row
    return x


def _ties():
    grid = np.unique(O.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    return (grid[:-1] + grid[1:]) / 2


def _near_tie(x, rel):
    """Elements whose exact quotient x * 448 / max|row| lies within rel (relative) of a tie."""
    x = np.asarray(x, np.float64)
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    q = np.abs(np.where(amax > 0, x * 448.0 / np.where(amax > 0, amax, 1.0), 0.0))
    ties = _ties()
    i = np.clip(np.searchsorted(ties, q), 1, len(ties) - 1)
    dist = np.minimum(np.abs(q - ties[i - 1]), np.abs(q - ties[i]))
    return (dist <= rel * q) & (q > 0)


@pytest.mark.parametrize("rows,cols", [(7, 256), (33, 3072), (6, 12288), (300, 136)])
def test_quantize_rows_matches_oracle(rows, cols):
    from latent_flow_matching_amd import dit
    x = _matrix(rows, cols, rows + cols)
    print(f"[fp8 quantize] {rows} x {cols}", flush=True)
    q, sc = dit.quantize_rows_fp8(dev(x))
    torch.cuda.synchronize()
    want_q, want_s = O.quantize_rows_fp8(x)
    got_q, got_s = q.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_s, want_s, rtol=2.0 ** -24, atol=0)
    # the kernel's quotient is two fp32 roundings from the exact one (relative 2^-23)
    near = _near_tie(x, 2.0 ** -22)
    diff = got_q != want_q
    assert not np.any(diff & ~near), np.argwhere(diff & ~near)[:5]
    same_sign = (got_q[diff] & 0x80) == (want_q[diff] & 0x80)
    adjacent = np.abs((got_q[diff] & 0x7F).astype(int) - (want_q[diff] & 0x7F).astype(int)) == 1
    assert np.all(same_sign & adjacent)
    print(f"    {int(near.sum())} quotients near a tie, {int(diff.sum())} codes on the other "
          f"neighbour; every other code bit for bit", flush=True)


@pytest.mark.parametrize("m,n,k", [(1, 256, 128), (300, 512, 384), (513, 256, 3072), (256, 768, 12288)])
def test_gemm_fp8_matches_exact_product(m, n, k):
    """The GEMM on the oracle's codes and scales (fp32) against their exact product."""
    from latent_flow_matching_amd import dit
    x = _matrix(m, k, 11 + m)
    w = (np.random.default_rng(12 + n).normal(size=(n, k)) * 0.02).astype(np.float32)
    print(f"[fp8 gemm] m={m} n={n} k={k}", flush=True)
    qx, sx = O.quantize_rows_fp8(x)
    qw, sw = O.quantize_rows_fp8(w)
    sx32, sw32 = sx.astype(np.float32), sw.astype(np.float32)
    mp = (m + 255) // 256 * 256                 # rows readable up to a multiple of 256
    qx_pad = np.zeros((mp, k), np.uint8)
    qx_pad[:m] = qx
    qx_d = torch.tensor(qx_pad, device="cuda")
    y = dit.gemm_fp8(qx_d[:m], dev(sx32), torch.tensor(qw, device="cuda"), dev(sw32))
    torch.cuda.synchronize()
    xr = O.e4m3_decode(qx) * sx32.astype(np.float64)[:, None]
    wr = O.e4m3_decode(qw) * sw32.astype(np.float64)[:, None]
    want = xr @ wr.T
    bound = 2.0 ** -12 * (np.abs(xr) @ np.abs(wr).T) + 1e-30
    got = y.cpu().numpy().astype(np.float64)
    ratio = np.max(np.abs(got - want) / bound)
    print(f"    max |err| / bound = {ratio:.3f}", flush=True)
    assert ratio <= 1.0


def test_gemm_fp8_argument_checks():
    from latent_flow_matching_amd import dit
    lib = dit.load_library()
    z = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    f = torch.zeros(256, device="cuda")
    P = dit._ptr
    assert lib.dit_gemm_fp8(P(z), P(f), 4, 128, P(z), P(f), 128, 128, 128, P(f), 128, None) != 0
    assert lib.dit_gemm_fp8(P(z), P(f), 4, 128, P(z), P(f), 256, 128, 64, P(f), 256, None) != 0
    assert lib.dit_quantize_rows_fp8(P(f), 2, 12, 12, P(z), 12, P(f), None) != 0


FP8 = [replace(TINY2, compute="fp8"), replace(TINY3, compute="fp8")]


def _call_bar(case):
    """Whole calls add code flips to the 16-bit path's own error, which is held to FP8_TOL:
    the bar is the larger of FP8_TOL and twice the error model's emulated error."""
    b = fp8_bars(case)
    print(f"    error model: emulated {b['emulated_max']:.3e}", flush=True)
    return max(FP8_TOL, b["bar_max"])


def check_block(case, cfg, b, n_txt, grid, ref_grid=None, rows=None, max_tokens=None):
    """Run block b on seeded inputs and compare its update with the oracle's E4M3 block,
    against the bars of the named error-model case."""
    from latent_flow_matching_amd import dit
    n_img = grid[0] * grid[1]
    n_ref = 0 if ref_grid is None else ref_grid[0] * ref_grid[1]
    segs = (n_txt, n_img, n_ref)
    n = sum(segs)
    ctx, w = context(cfg, max_tokens or n)
    x = S.gen_tokens(n, cfg.hidden, key=(0,))
    cond = S.gen_cond(3, cfg.hidden)
    pos = O.positions(n_txt, grid, (ref_grid,) if ref_grid else ())
    xt = dev(x)
    print(f"[fp8 block] {case}: arch={cfg.arch} b={b} segs={segs} D={cfg.hidden} "
          f"seq={cfg.double_wiring}", flush=True)
    ctx.block_forward(b, xt, n_txt, n_img, n_ref, dev(pos), dev(seg_cond(cond, segs)), dit.DIT_MASK_DEFAULT)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    got = xt.cpu().numpy()[sel].astype(np.float64)
    ref = oracle_block(cfg, w, b, x, segs, pos, cond, rows=rows)
    u_got, u_ref = got - f64(x[sel]), ref - f64(x[sel])
    rms_u = float(np.sqrt(np.mean(u_ref ** 2)))
    e_rms = float(np.sqrt(np.mean((u_got - u_ref) ** 2))) / rms_u
    e_max = float(np.max(np.abs(u_got - u_ref))) / rms_u
    bar = fp8_bars(case)
    print(f"    update error: RMS {e_rms:.3e} (emulated {bar['emulated_rms']:.3e}, bar {bar['bar_rms']:.3e}), "
          f"max {e_max:.3e} (emulated {bar['emulated_max']:.3e}, bar {bar['bar_max']:.3e}); "
          f"output max/RMS {rel_err(got, ref):.3e}", flush=True)
    assert e_rms <= bar["bar_rms"] and e_max <= bar["bar_max"]


@pytest.mark.parametrize("cfg", FP8, ids=["flux2", "flux3"])
@pytest.mark.parametrize("b", [0, 1], ids=["stream_block", "shared_block"])
def test_fp8_block_tiny_ragged(cfg, b):
    case = f"tiny_flux{2 if cfg.arch == S.ARCH_FLUX2 else 3}_{'stream' if b == 0 else 'shared'}"
    check_block(case, cfg, b, 77, (13, 11), (9, 10) if cfg.arch == S.ARCH_FLUX3 else None)


def test_fp8_sequential_block_tiny():
    check_block("tiny_sequential_double", replace(TINY2, compute="fp8", double_wiring=True), 0, 37,
                (9, 11), (5, 6))


@pytest.mark.parametrize("cfg", FP8, ids=["flux2", "flux3"])
def test_fp8_forward_tiny(cfg):
    err = _forward_case(cfg, 50, (9, 7), (6, 5), 0.75)
    bar = _call_bar(f"tiny_forward_flux{2 if cfg.arch == S.ARCH_FLUX2 else 3}")
    print(f"fp8 forward err {err:.3e} (bar {bar:.1e})")
    assert err <= bar


@pytest.mark.parametrize("n_img,grid", [(4096, (64, 64)), (1024, (32, 32))], ids=["4096img", "1024img"])
@pytest.mark.parametrize("b", [0, 1], ids=["double", "single"])
def test_fp8_flux2_block_full_width_sampled_rows(b, n_img, grid):
    """Full-width FLUX.2 blocks at 512 text tokens; at 1024 image tokens linear2 runs as
    k-slices."""
    cfg = replace(S.FLUX2_KLEIN, n_stream_blocks=1, n_shared_blocks=1, compute="fp8")
    n = 512 + n_img
    case = f"flux2_{'double' if b == 0 else 'single'}_512txt_{n_img}img"
    check_block(case, cfg, b, 512, grid, rows=_rows(n), max_tokens=n)


def test_fp8_denoise_cfg_matches_oracle():
    """Guidance (a batch of two sequences) on the E4M3 path: FLUX.3 with a reference image."""
    cfg = replace(TINY3, compute="fp8")
    ctx, w = context(cfg, 600)
    grid = (8, 6)
    noise = S.gen_latents(48, cfg.in_channels, key=(2,))
    _, ref, txt, txt_u = _cfg_inputs(cfg, 20, grid, (4, 4))
    lat = dev(noise)
    print("[fp8 denoise_cfg] FLUX.3 tiny", flush=True)
    ctx.denoise_cfg(lat, dev(txt), dev(txt_u), grid, 3, 2.5, -1, dev(ref), (4, 4))
    torch.cuda.synchronize()
    want = O.denoise_cfg(oracle_model(cfg, w), f64(noise), f64(txt), f64(txt_u), grid, 3, 2.5,
                         f64(ref), (4, 4))
    err = rel_err(lat.cpu().numpy() - f64(noise), want - f64(noise))
    bar = _call_bar("tiny_denoise_cfg_flux3")
    print(f"    fp8 denoise_cfg update err {err:.3e} (bar {bar:.1e})", flush=True)
    assert err <= bar


def test_fp8_flow_map_denoise_matches_oracle():
    """A flow-map model on the E4M3 path: each step's target time, one reference image."""
    cfg = replace(TINY3_FM, compute="fp8")
    ctx, w = context(cfg, 600)
    grid, ref_grid = (8, 6), (4, 4)
    noise = S.gen_latents(48, cfg.in_channels, key=(2,))
    ref = S.gen_latents(16, cfg.in_channels, key=(3,))
    txt = S.gen_text(20, cfg.hidden)
    lat = dev(noise)
    print("[fp8 flow-map denoise] FLUX.3 tiny", flush=True)
    ctx.denoise(lat, dev(txt), grid, 4, -1, dev(ref), ref_grid)
    torch.cuda.synchronize()
    want = O.denoise(oracle_model(cfg, w), f64(noise), f64(txt), grid, 4, f64(ref), ref_grid)
    err = rel_err(lat.cpu().numpy() - f64(noise), want - f64(noise))
    bar = _call_bar("tiny_flow_map_denoise_flux3")
    print(f"    fp8 flow-map denoise update err {err:.3e} (bar {bar:.1e})", flush=True)
    assert err <= bar


@pytest.mark.parametrize("b", [0, 1], ids=["per_mode", "joint"])
def test_fp8_flux3_block_1024px_ref_sampled_rows(b):
    """Full-width FLUX.3 per-mode (three weight sets, block-diagonal) and joint blocks at
    512 text + 4096 image + 4096 reference tokens on the E4M3 path."""
    cfg = replace(S.FLUX3_KLEIN, n_stream_blocks=1, n_shared_blocks=1, compute="fp8")
    n = 512 + 4096 + 4096
    case = f"flux3_{'per_mode' if b == 0 else 'joint'}_512txt_4096img_4096ref"
    check_block(case, cfg, b, 512, (64, 64), (64, 64), rows=_rows(n), max_tokens=n)
