"""The C-ABI library builds, loads and exports every symbol include/dit.h declares; host-side
validation and error paths work without a GPU (no compute calls here)."""
import ctypes
import os

import numpy as np
import pytest

from latent_flow_matching_amd import dit, synth as S
from tests.helpers import TINY2, lib_built


@pytest.fixture(scope="module")
def lib():
    if not lib_built():
        from latent_flow_matching_amd import build
        build.build()
    return dit.load_library()


def test_exports_every_declared_symbol(lib):
    names = dit.header_functions()
    assert {"dit_ctx_create", "dit_ctx_free", "dit_block_forward", "dit_forward", "dit_denoise",
            "dit_get_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_header_compiles_as_c_and_links(lib, tmp_path):
    """include/dit.h is plain C: a C99 translation unit that takes the address of every
    declared function compiles and links against the built library."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = dit.header_functions()
    src = tmp_path / "abi.c"
    src.write_text('#include "dit.h"\n#include <stdio.h>\n'
                   "typedef void (*fn)(void);\n"
                   "static fn table[] = {" + ", ".join(f"(fn){n}" for n in names) + "};\n"
                   "int main(void) { printf(\"%d\\n\", (int)(sizeof table / sizeof table[0])); "
                   "return 0; }\n")
    libdir = os.path.dirname(dit.LIB_PATH)
    out = tmp_path / "abi"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-Wno-pedantic",
                        "-I", os.path.join(os.path.dirname(libdir), "include"), str(src),
                        "-L", libdir, "-ldit", f"-Wl,-rpath,{libdir}", "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(out)], capture_output=True, text=True)
    assert run.returncode == 0 and int(run.stdout) == len(names), run.stderr


def _cfg(**kw):
    c = dit.make_config(TINY2, 512)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _table(cfg=TINY2, drop=None, extra=None, bad_numel=None, w=None):
    w = S.gen_weights(cfg, bits=True) if w is None else w
    if drop:
        w.pop(drop)
    if extra:
        w[extra] = np.zeros(4, np.uint16)
    if bad_numel:
        w[bad_numel] = w[bad_numel][:-1]
    names = [k.encode() for k in w]
    arr = (dit.DitTensor * len(w))()
    keep = list(w.values())
    for i, (n, a) in enumerate(zip(names, keep)):
        arr[i] = dit.DitTensor(n, a.ctypes.data, a.size, dit.DIT_BF16)
    return arr, len(w), (names, keep)


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 64, "head_dim must be 128"),
    ("hidden", 300, "hidden"),
    ("mlp_hidden", 100, "mlp_hidden"),
    ("in_channels", 100, "in_channels"),
    ("arch", 7, "unknown arch"),
    ("compute", 9, "unknown compute"),
    ("max_tokens", 0, "max_tokens"),
    ("n_stream_blocks", -1, "block"),
    ("rope_theta", 0.0, "positive"),
    ("time_dim", 8192, "time_dim"),
])
def test_bad_config_rejected(lib, field, value, msg):
    arr, n, keep = _table()
    h = lib.dit_ctx_create(ctypes.byref(_cfg(**{field: value})), arr, n)
    assert not h
    assert msg in dit.last_error()


@pytest.mark.parametrize("fields,msg", [
    ({"double_wiring": 2}, "double_wiring must be 0 or 1"),
    ({"double_wiring": 1, "arch": dit.DIT_FLUX3}, "DIT_FLUX2 double blocks only"),
    ({"compute": dit.DIT_FP8, "mlp_hidden": 16384}, "at most 16384 values"),
])
def test_bad_config_combination_rejected(lib, fields, msg):
    arr, n, keep = _table()
    h = lib.dit_ctx_create(ctypes.byref(_cfg(**fields)), arr, n)
    assert not h
    assert msg in dit.last_error()


@pytest.mark.parametrize("kw,msg", [
    ({"drop": "blk0.s1.w2"}, "missing weight 'blk0.s1.w2'"),
    ({"extra": "blk9.s0.w1"}, "unknown weight 'blk9.s0.w1'"),
    ({"bad_numel": "final.out"}, "'final.out' has"),
])
def test_bad_weight_table_rejected(lib, kw, msg):
    arr, n, keep = _table(**kw)
    assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
    assert msg in dit.last_error()


def _no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")


def test_per_block_modulation_tables_pass_the_weight_checks(lib):
    """Each block's own blk{b}.s{s}.mod (distinct, aliased to one array, or mixed with the
    shared names) passes every weight check: create then fails only for want of a device."""
    from dataclasses import replace
    _no_gpu()
    own = S.gen_weights(replace(TINY2, mod_per_block=True), bits=True)
    shared = S.gen_weights(TINY2, bits=True)
    aliased = {k: v for k, v in shared.items() if not k.startswith("mod.")}
    aliased.update({"blk0.s0.mod": shared["mod.0.s0"], "blk0.s1.mod": shared["mod.0.s0"],
                    "blk1.s0.mod": shared["mod.1.s0"]})
    mixed = dict(shared)
    mixed.pop("mod.1.s0")
    mixed["blk1.s0.mod"] = own["blk1.s0.mod"]
    for w in (own, aliased, mixed):
        arr, n, keep = _table(w=w)
        assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
        assert "no HIP device" in dit.last_error(), dit.last_error()


def test_modulation_table_rules(lib):
    from dataclasses import replace
    own = S.gen_weights(replace(TINY2, mod_per_block=True), bits=True)
    shared = S.gen_weights(TINY2, bits=True)
    # a shared projection that no block uses
    w = dict(own)
    w["mod.1.s0"] = shared["mod.1.s0"]
    arr, n, keep = _table(w=w)
    assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
    assert "'mod.1.s0' is used by no block" in dit.last_error()
    # neither the block's own projection nor the shared one
    w = dict(own)
    w.pop("blk1.s0.mod")
    arr, n, keep = _table(w=w)
    assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
    assert "missing weight 'blk1.s0.mod' (or the shared 'mod.1.s0')" in dit.last_error()
    # a block's own projection of the wrong size
    w = dict(own)
    w["blk0.s1.mod"] = w["blk0.s1.mod"][:-1]
    arr, n, keep = _table(w=w)
    assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
    assert "'blk0.s1.mod' has" in dit.last_error()


def test_no_device_is_an_error_not_a_fallback(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    arr, n, keep = _table()
    assert not lib.dit_ctx_create(ctypes.byref(_cfg()), arr, n)
    assert "no HIP device" in dit.last_error()


def test_null_context_calls_fail(lib):
    assert lib.dit_block_forward(None, 0, None, 1, 1, 0, None, None, -1, None) == dit.DIT_EINVAL
    assert "ctx is NULL" in dit.last_error()
    assert lib.dit_forward(None, None, None, None, 1, 1, 1, 0, 0, 0.5, None, None) == dit.DIT_EINVAL
    assert lib.dit_denoise(None, None, None, 1, 1, 1, None, 0, 0, 4, -1, None) == dit.DIT_EINVAL
    assert lib.dit_fill_noise(None, 4, 1, None) == dit.DIT_EINVAL
    assert lib.dit_debug_buffer(None, b"xm", None, None) is None
    assert lib.dit_profile_start(None, 10) == dit.DIT_EINVAL
    assert lib.dit_profile_select(None, b"linear1") == dit.DIT_EINVAL
    assert lib.dit_profile_stop(None) == dit.DIT_EINVAL
    lib.dit_ctx_free(None)   # no-op


def test_fp8_entries_check_arguments_before_any_launch(lib):
    """Argument errors of the row-wise FP8 entries come back as codes, with no device touched."""
    P = ctypes.c_void_p
    buf = P(64)  # never dereferenced: every call below fails its checks first
    assert lib.dit_quantize_rows_fp8(None, 2, 16, 16, buf, 16, buf, None) == dit.DIT_EINVAL
    assert lib.dit_quantize_rows_fp8(buf, 2, 12, 12, buf, 12, buf, None) == dit.DIT_EINVAL
    assert lib.dit_quantize_rows_fp8(buf, 2, 32, 16, buf, 32, buf, None) == dit.DIT_EINVAL
    assert lib.dit_quantize_rows_fp8(buf, 2, 16392, 16392, buf, 16392, buf, None) == dit.DIT_EINVAL
    assert "cols" in dit.last_error()
    assert lib.dit_gemm_fp8(None, buf, 4, 128, buf, buf, 256, 128, 128, buf, 256, None) == dit.DIT_EINVAL
    assert lib.dit_gemm_fp8(buf, buf, -1, 128, buf, buf, 256, 128, 128, buf, 256, None) == dit.DIT_EINVAL
    assert lib.dit_gemm_fp8(buf, buf, 4, 128, buf, buf, 128, 128, 128, buf, 128, None) == dit.DIT_EUNSUPPORTED
    assert lib.dit_gemm_fp8(buf, buf, 4, 64, buf, buf, 256, 64, 64, buf, 256, None) == dit.DIT_EUNSUPPORTED
    assert lib.dit_gemm_fp8(buf, buf, 4, 120, buf, buf, 256, 128, 128, buf, 256, None) == dit.DIT_EINVAL
    assert "strides" in dit.last_error()


def test_binding_refuses_to_run_without_library(tmp_path):
    saved = dit._lib
    try:
        dit._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            dit.load_library(str(tmp_path / "missing.so"))
    finally:
        dit._lib = saved
