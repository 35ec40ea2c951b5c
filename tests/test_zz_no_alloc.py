"""dit_gemm_fp8_static, the allocation-free variant of dit_gemm_fp8 (its k-slice partials in the
library's static device array), against dit_gemm_fp8 and the exact product of the same codes:
two calls in a row, the second smaller, so the second reuses the array the first filled."""
import numpy as np
import pytest

from oracle import dit_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_flow_matching_amd import dit
    dit.load_library()


def _case(m, n, k, seed):
    """Oracle codes and fp32 scales of seeded operands, and their exact product and bound."""
    r = np.random.default_rng(seed)
    x = r.normal(size=(m, k))
    w = r.normal(0, 0.02, size=(n, k))
    qx, sx = O.quantize_rows_fp8(x)
    qw, sw = O.quantize_rows_fp8(w)
    sx32, sw32 = sx.astype(np.float32), sw.astype(np.float32)
    xr = O.e4m3_decode(qx) * sx32.astype(np.float64)[:, None]
    wr = O.e4m3_decode(qw) * sw32.astype(np.float64)[:, None]
    mp = (m + 255) // 256 * 256
    qx_pad = np.zeros((mp, k), np.uint8)
    qx_pad[:m] = qx
    dev = lambda a: torch.tensor(a, device="cuda")
    return (dev(qx_pad)[:m], dev(sx32), dev(qw), dev(sw32)), xr @ wr.T, 2.0 ** -12 * (np.abs(xr) @ np.abs(wr).T)


def test_static_gemm_matches_allocating_gemm_twice():
    from latent_flow_matching_amd import dit
    for m, n, k, seed in [(300, 512, 12288, 1), (100, 256, 3072, 2)]:
        print(f"[fp8 gemm static] m={m} n={n} k={k}", flush=True)
        args, exact, bound = _case(m, n, k, seed)
        y_plain = dit.gemm_fp8(*args)
        y_static = dit.gemm_fp8(*args, static=True)
        torch.cuda.synchronize()
        yp = y_plain.cpu().numpy().astype(np.float64)
        ys = y_static.cpu().numpy().astype(np.float64)
        r_static = float(np.max(np.abs(ys - exact) / (bound + 1e-30)))
        r_pair = float(np.max(np.abs(ys - yp) / (2 * bound + 1e-30)))
        print(f"    static vs exact: {r_static:.3f} of the bound; static vs dit_gemm_fp8: "
              f"{r_pair:.3f} of twice the bound; identical: {np.array_equal(ys, yp)}", flush=True)
        assert r_static <= 1.0 and r_pair <= 1.0
