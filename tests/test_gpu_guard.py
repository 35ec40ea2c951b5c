"""The DIT_DEBUG_SYNC numeric guard: with the environment variable set at context creation, a
call fails with DIT_ENUMERIC at the first launch whose output holds fp16 values at the
saturation limit +-65504 or NaN / Inf values, naming the block and the launch; ordinary inputs
pass and give the same result as without the guard (the error reporting of the C library:
negative return and a message, hakusoku FLUX.2-klein-4B article, "エラーハンドリング")."""
import numpy as np
import pytest

from latent_flow_matching_amd import synth as S
from oracle import dit_oracle as O
from tests.helpers import TINY2, gpu_weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_flow_matching_amd import dit
    dit.load_library()


def _ctx(monkeypatch, debug):
    from latent_flow_matching_amd import dit
    if debug:
        monkeypatch.setenv("DIT_DEBUG_SYNC", "1")
    else:
        monkeypatch.delenv("DIT_DEBUG_SYNC", raising=False)
    return dit.DiT(TINY2, gpu_weights(TINY2, S.gen_weights(TINY2)), 256)


def _block_inputs(scale_cond=1.0, nan_at=None):
    n_txt, grid = 20, (6, 5)
    n = n_txt + 30
    x = S.gen_tokens(n, TINY2.hidden)
    if nan_at is not None:
        x[nan_at] = np.nan
    cond = (S.gen_cond(2, TINY2.hidden) * scale_cond).astype(np.float32)
    pos = O.positions(n_txt, grid).astype(np.float32)
    dev = lambda a: torch.tensor(a, device="cuda")
    return dev(x), n_txt, 30, dev(pos), dev(cond)


def test_guard_passes_ordinary_inputs_bitwise(monkeypatch):
    outs = []
    for debug in (False, True):
        ctx = _ctx(monkeypatch, debug)
        x, n_txt, n_img, pos, cond = _block_inputs()
        for b in (0, 1):
            ctx.block_forward(b, x, n_txt, n_img, 0, pos, cond)
        torch.cuda.synchronize()
        outs.append(x.cpu().numpy())
        ctx.close()
    assert np.array_equal(outs[0], outs[1])


def test_guard_reports_saturated_activations(monkeypatch):
    """A conditioning vector scaled by 1e5 makes the adaLN shift and scale huge, so the
    modulated LayerNorm output overflows the fp16 range."""
    from latent_flow_matching_amd import dit
    ctx = _ctx(monkeypatch, True)
    x, n_txt, n_img, pos, cond = _block_inputs(scale_cond=1e5)
    print("[guard] saturating cond", flush=True)
    with pytest.raises(dit.DitError) as ei:
        ctx.block_forward(0, x, n_txt, n_img, 0, pos, cond)
    ctx.close()
    msg = str(ei.value)
    print("   ", msg, flush=True)
    assert ei.value.code == dit.DIT_ENUMERIC
    assert "block 0, ln_modulate -> xm" in msg and "+-65504" in msg


def test_guard_reports_nonfinite_input(monkeypatch):
    from latent_flow_matching_amd import dit
    ctx = _ctx(monkeypatch, True)
    x, n_txt, n_img, pos, cond = _block_inputs(nan_at=(7, 11))
    print("[guard] NaN in the residual", flush=True)
    with pytest.raises(dit.DitError) as ei:
        ctx.block_forward(1, x, n_txt, n_img, 0, pos, cond)
    ctx.close()
    msg = str(ei.value)
    print("   ", msg, flush=True)
    assert ei.value.code == dit.DIT_ENUMERIC
    assert "block 1, input residual x" in msg and "1 NaN/Inf" in msg


def test_guard_is_off_without_the_variable(monkeypatch):
    """Without DIT_DEBUG_SYNC the same saturating call returns normally (no checks, no syncs)."""
    ctx = _ctx(monkeypatch, False)
    x, n_txt, n_img, pos, cond = _block_inputs(scale_cond=1e5)
    ctx.block_forward(0, x, n_txt, n_img, 0, pos, cond)
    torch.cuda.synchronize()
    ctx.close()
