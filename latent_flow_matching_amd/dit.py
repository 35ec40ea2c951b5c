"""Thin ctypes binding of libdit.so (include/dit.h).  Argument marshalling only: every step of
the forward pass runs in the library's HIP kernels.  torch tensors provide device memory and
streams.  There is no CPU fallback: without the built library on a gfx950 GPU every call
raises."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

from .synth import ModelConfig

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdit.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dit.h")

DIT_F32, DIT_BF16, DIT_F16, DIT_FP8 = 0, 1, 2, 3
COMPUTE = {"f32": DIT_F32, "bf16": DIT_BF16, "f16": DIT_F16, "fp8": DIT_FP8}
DIT_FLUX2, DIT_FLUX3 = 0, 1
DIT_MASK_DEFAULT, DIT_MASK_FULL, DIT_MASK_SEGMENT = -1, 0, 1
DIT_OK, DIT_EINVAL, DIT_ENOMEM, DIT_EHIP, DIT_EUNSUPPORTED, DIT_ENUMERIC = 0, -1, -2, -3, -4, -5


class DitConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "arch", "hidden", "heads", "head_dim", "mlp_hidden", "in_channels", "time_dim",
        "n_stream_blocks", "n_shared_blocks", "max_tokens", "compute")] + \
        [(n, ctypes.c_float) for n in ("rope_theta", "ln_eps", "rms_eps")] + \
        [(n, ctypes.c_int) for n in ("txt_feat_dim", "flow_map", "double_wiring")]


class DitTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("dtype", ctypes.c_int)]


class DitRequest(ctypes.Structure):
    _fields_ = [("txt", ctypes.c_void_p), ("txt_uncond", ctypes.c_void_p), ("n_txt", ctypes.c_int),
                ("guidance", ctypes.c_float), ("gh", ctypes.c_int), ("gw", ctypes.c_int),
                ("ref_lat", ctypes.c_void_p), ("n_refs", ctypes.c_int),
                ("ref_grids", ctypes.POINTER(ctypes.c_int))]


class DitError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"dit error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = None):
    """Load libdit.so (LIB_PATH unless given) and declare its signatures.  Raises if it is
    not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (run __graft_entry__.build() or "
                           "python -m latent_flow_matching_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, F, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.dit_ctx_create.restype = P
    lib.dit_ctx_create.argtypes = [ctypes.POINTER(DitConfig), ctypes.POINTER(DitTensor), I]
    lib.dit_ctx_free.restype = None
    lib.dit_ctx_free.argtypes = [P]
    lib.dit_block_forward.restype = I
    lib.dit_block_forward.argtypes = [P, I, P, I, I, I, P, P, I, P]
    lib.dit_forward.restype = I
    lib.dit_forward.argtypes = [P, P, P, P, I, I, I, I, I, F, P, P]
    lib.dit_denoise.restype = I
    lib.dit_denoise.argtypes = [P, P, P, I, I, I, P, I, I, I, I64, P]
    lib.dit_forward_ex.restype = I
    lib.dit_forward_ex.argtypes = [P, ctypes.POINTER(DitRequest), P, F, F, P, P]
    lib.dit_denoise_ex.restype = I
    lib.dit_denoise_ex.argtypes = [P, ctypes.POINTER(DitRequest), P, I, F, P, I64, P]
    lib.dit_forward_flow.restype = I
    lib.dit_forward_flow.argtypes = [P, P, P, P, I, I, I, I, I, F, F, P, P]
    lib.dit_text_features.restype = I
    lib.dit_text_features.argtypes = [P, P, I, P, P]
    lib.dit_forward_cfg.restype = I
    lib.dit_forward_cfg.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, P, P]
    lib.dit_denoise_cfg.restype = I
    lib.dit_denoise_cfg.argtypes = [P, P, P, P, I, I, I, P, I, I, I, F, I64, P]
    lib.dit_fill_noise.restype = I
    lib.dit_fill_noise.argtypes = [P, I64, I64, P]
    lib.dit_quantize_rows_fp8.restype = I
    lib.dit_quantize_rows_fp8.argtypes = [P, I, I, I, P, I, P, P]
    lib.dit_gemm_fp8.restype = I
    lib.dit_gemm_fp8.argtypes = [P, P, I, I, P, P, I, I, I, P, I, P]
    lib.dit_gemm_fp8_static.restype = I
    lib.dit_gemm_fp8_static.argtypes = [P, P, I, I, P, P, I, I, I, P, I, P]
    lib.dit_mfma_rate.restype = I
    lib.dit_mfma_rate.argtypes = [I, I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), P]
    lib.dit_debug_buffer.restype = P
    lib.dit_debug_buffer.argtypes = [P, ctypes.c_char_p, ctypes.POINTER(I), ctypes.POINTER(I64)]
    lib.dit_profile_start.restype = I
    lib.dit_profile_start.argtypes = [P, I]
    lib.dit_profile_select.restype = I
    lib.dit_profile_select.argtypes = [P, ctypes.c_char_p]
    lib.dit_profile_stop.restype = I
    lib.dit_profile_stop.argtypes = [P]
    D = ctypes.POINTER(ctypes.c_double)
    lib.dit_profile_get.restype = I
    lib.dit_profile_get.argtypes = [P, ctypes.c_char_p, D, ctypes.POINTER(I64), D, D]
    lib.dit_get_error.restype = ctypes.c_char_p
    lib.dit_get_error.argtypes = []
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/dit.h declares."""
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z_0-9]+)\s*\(", txt)))


def last_error() -> str:
    return load_library().dit_get_error().decode()


def _check(rc: int):
    if rc != 0:
        raise DitError(rc, last_error())


def make_config(cfg: ModelConfig, max_tokens: int) -> DitConfig:
    return DitConfig(cfg.arch, cfg.hidden, cfg.heads, cfg.head_dim, cfg.mlp_hidden,
                     cfg.in_channels, cfg.time_dim, cfg.n_stream_blocks, cfg.n_shared_blocks,
                     max_tokens, COMPUTE[cfg.compute], cfg.rope_theta, cfg.ln_eps,
                     cfg.rms_eps, cfg.txt_feat_dim, int(cfg.flow_map), int(cfg.double_wiring))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype_name, what):
    import torch
    if t is None:
        return
    if not t.is_cuda or t.dtype != getattr(torch, dtype_name) or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype_name} CUDA tensor")


class DiT:
    """One library context (weights uploaded, workspace allocated)."""

    def __init__(self, cfg: ModelConfig, weights: dict, max_tokens: int):
        lib = load_library()
        self.cfg = cfg
        self.max_tokens = max_tokens
        names, keep = [], []
        arr = (DitTensor * len(weights))()
        for i, (name, a) in enumerate(weights.items()):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                dt = DIT_BF16
            elif a.dtype == np.float32:
                dt = DIT_F32
            else:
                raise ValueError(f"weight {name}: dtype {a.dtype} (want float32 or uint16 bf16 bits)")
            keep.append(a)
            names.append(name.encode())
            arr[i] = DitTensor(names[-1], a.ctypes.data, a.size, dt)
        c = make_config(cfg, max_tokens)
        h = lib.dit_ctx_create(ctypes.byref(c), arr, len(weights))
        if not h:
            raise DitError(-1, last_error())
        self._h = ctypes.c_void_p(h)

    def close(self):
        if getattr(self, "_h", None):
            load_library().dit_ctx_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def block_forward(self, block, x, n_txt, n_img, n_ref, pos, cond, mask=DIT_MASK_DEFAULT,
                      stream=None):
        for t, w in ((x, "x"), (pos, "pos"), (cond, "cond")):
            _need(t, "float32", w)
        _check(load_library().dit_block_forward(self._h, block, _ptr(x), n_txt, n_img, n_ref,
                                                _ptr(pos), _ptr(cond), mask, _stream(stream)))

    def forward(self, lat, txt, grid, t, v, ref_lat=None, ref_grid=(0, 0), stream=None):
        for a, w in ((lat, "lat"), (txt, "txt"), (v, "v"), (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        _check(load_library().dit_forward(self._h, _ptr(lat), _ptr(ref_lat), _ptr(txt),
                                          txt.shape[0], grid[0], grid[1], ref_grid[0],
                                          ref_grid[1], float(t), _ptr(v), _stream(stream)))

    def denoise(self, lat, txt, grid, n_steps, seed=-1, ref_lat=None, ref_grid=(0, 0),
                stream=None):
        for a, w in ((lat, "lat"), (txt, "txt"), (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        _check(load_library().dit_denoise(self._h, _ptr(lat), _ptr(txt), txt.shape[0], grid[0],
                                          grid[1], _ptr(ref_lat), ref_grid[0], ref_grid[1],
                                          n_steps, seed, _stream(stream)))

    @staticmethod
    def _request(txt, grid, txt_uncond, guidance, ref_lat, ref_grids):
        for a, w in ((txt, "txt"), (txt_uncond, "txt_uncond"), (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        if txt_uncond is not None and tuple(txt_uncond.shape) != tuple(txt.shape):
            raise ValueError("txt and txt_uncond must have the same shape")
        grids = [int(v) for g in ref_grids for v in g]
        arr = (ctypes.c_int * max(1, len(grids)))(*grids)
        req = DitRequest(txt.data_ptr() if txt.numel() else None,
                         None if txt_uncond is None else (txt_uncond.data_ptr() or None),
                         txt.shape[0], float(guidance), grid[0], grid[1],
                         None if ref_lat is None else ref_lat.data_ptr(), len(ref_grids), arr)
        return req, arr

    def forward_ex(self, lat, txt, grid, t, v, t_target=None, txt_uncond=None, guidance=1.0,
                   ref_lat=None, ref_grids=(), stream=None):
        """One call for a request: optional guidance (txt_uncond), any number of reference
        images (ref_lat = their latents one after another, ref_grids = [(rows, cols), ...])."""
        _need(lat, "float32", "lat")
        _need(v, "float32", "v")
        req, keep = self._request(txt, grid, txt_uncond, guidance, ref_lat, ref_grids)
        _check(load_library().dit_forward_ex(self._h, ctypes.byref(req), _ptr(lat), float(t),
                                             float(t if t_target is None else t_target), _ptr(v),
                                             _stream(stream)))

    def denoise_ex(self, lat, txt, grid, n_steps, strength=1.0, noise=None, seed=-1,
                   txt_uncond=None, guidance=1.0, ref_lat=None, ref_grids=(), stream=None):
        """Sampling for a request; strength < 1 is image-to-image from the clean latents in lat."""
        _need(lat, "float32", "lat")
        _need(noise, "float32", "noise")
        req, keep = self._request(txt, grid, txt_uncond, guidance, ref_lat, ref_grids)
        _check(load_library().dit_denoise_ex(self._h, ctypes.byref(req), _ptr(lat), n_steps,
                                             float(strength), _ptr(noise), seed, _stream(stream)))

    def forward_flow(self, lat, txt, grid, t, t_target, v, ref_lat=None, ref_grid=(0, 0),
                     stream=None):
        """Velocity of a flow-map model for the step from t to t_target."""
        for a, w in ((lat, "lat"), (txt, "txt"), (v, "v"), (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        _check(load_library().dit_forward_flow(self._h, _ptr(lat), _ptr(ref_lat), _ptr(txt),
                                               txt.shape[0], grid[0], grid[1], ref_grid[0],
                                               ref_grid[1], float(t), float(t_target), _ptr(v),
                                               _stream(stream)))

    def text_features(self, feat, txt, stream=None):
        """txt [n, D] = feat [n, txt_feat_dim] . txt_in^T."""
        _need(feat, "float32", "feat")
        _need(txt, "float32", "txt")
        if feat.shape[0] != txt.shape[0] or feat.dim() != 2 or txt.dim() != 2:
            raise ValueError("feat [n, txt_feat_dim] and txt [n, D] need the same row count")
        _check(load_library().dit_text_features(self._h, _ptr(feat), feat.shape[0], _ptr(txt),
                                                _stream(stream)))

    def forward_cfg(self, lat, txt, txt_uncond, grid, t, guidance, v, ref_lat=None,
                    ref_grid=(0, 0), stream=None):
        """Guided velocity v_u + guidance * (v_c - v_u) from one batch-of-two call."""
        for a, w in ((lat, "lat"), (txt, "txt"), (txt_uncond, "txt_uncond"), (v, "v"),
                     (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        if tuple(txt_uncond.shape) != tuple(txt.shape):
            raise ValueError("txt and txt_uncond must have the same shape")
        _check(load_library().dit_forward_cfg(self._h, _ptr(lat), _ptr(ref_lat), _ptr(txt),
                                              _ptr(txt_uncond), txt.shape[0], grid[0], grid[1],
                                              ref_grid[0], ref_grid[1], float(t), float(guidance),
                                              _ptr(v), _stream(stream)))

    def denoise_cfg(self, lat, txt, txt_uncond, grid, n_steps, guidance, seed=-1, ref_lat=None,
                    ref_grid=(0, 0), stream=None):
        for a, w in ((lat, "lat"), (txt, "txt"), (txt_uncond, "txt_uncond"), (ref_lat, "ref_lat")):
            _need(a, "float32", w)
        if tuple(txt_uncond.shape) != tuple(txt.shape):
            raise ValueError("txt and txt_uncond must have the same shape")
        _check(load_library().dit_denoise_cfg(self._h, _ptr(lat), _ptr(txt), _ptr(txt_uncond),
                                              txt.shape[0], grid[0], grid[1], _ptr(ref_lat),
                                              ref_grid[0], ref_grid[1], n_steps, float(guidance),
                                              seed, _stream(stream)))

    KERNELS = ("ln_modulate", "linear1", "qk_norm_rope", "attention", "linear2", "conditioning",
               "embed", "final", "fp8_quant")

    def profile_start(self, max_launches: int = 100000, kernels: str | None = None):
        """Time the following launches; kernels = comma-separated classes (None: all)."""
        lib = load_library()
        _check(lib.dit_profile_select(self._h, None if kernels is None else kernels.encode()))
        _check(lib.dit_profile_start(self._h, max_launches))

    def profile_stop(self) -> dict:
        """Stop timing; {kernel: (ms, launches, flops, bytes)} over the recorded launches."""
        lib = load_library()
        _check(lib.dit_profile_stop(self._h))
        out = {}
        for k in self.KERNELS:
            ms, n, fl, by = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
            _check(lib.dit_profile_get(self._h, k.encode(), ctypes.byref(ms), ctypes.byref(n),
                                       ctypes.byref(fl), ctypes.byref(by)))
            out[k] = (ms.value, n.value, fl.value, by.value)
        return out

    def debug_buffer(self, name: str, rows: int, cols: int | None = None):
        """Copy a workspace buffer (see dit_debug_buffer) into a new float32 CUDA tensor."""
        import torch
        lib = load_library()
        dt, rs = ctypes.c_int(), ctypes.c_int64()
        p = lib.dit_debug_buffer(self._h, name.encode(), ctypes.byref(dt), ctypes.byref(rs))
        if not p:
            raise KeyError(name)
        cols = rs.value if cols is None else cols
        if dt.value == DIT_FP8:
            raise ValueError(f"{name} holds E4M3 codes")
        tdt = {DIT_BF16: torch.bfloat16, DIT_F16: torch.float16}.get(dt.value, torch.float32)
        out = torch.empty((rows, rs.value), dtype=tdt, device="cuda")
        torch.cuda.synchronize()
        _hip_memcpy_dtod(out.data_ptr(), p, out.numel() * out.element_size())
        return out[:, :cols].float()


def quantize_rows_fp8(x, stream=None):
    """(codes uint8 [rows, cols], scales float32 [rows]) of the row-wise E4M3 quantization of
    a float32 CUDA matrix x (dit_quantize_rows_fp8)."""
    import torch
    _need(x, "float32", "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sc = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(load_library().dit_quantize_rows_fp8(_ptr(x), rows, cols, x.stride(0), _ptr(q), cols,
                                                _ptr(sc), _stream(stream)))
    return q, sc


def gemm_fp8(qx, sx, qw, sw, stream=None, y=None, static=False):
    """y = sx[:, None] * sw[None, :] * (qx . qw^T) over E4M3 codes (dit_gemm_fp8, or
    dit_gemm_fp8_static with static=True); qx must have rows readable up to its row count
    rounded up to 256 (pass a padded tensor's view).  y: an output to fill, else a new one."""
    import torch
    m, k = qx.shape
    n = qw.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=qx.device)
    fn = load_library().dit_gemm_fp8_static if static else load_library().dit_gemm_fp8
    _check(fn(_ptr(qx), _ptr(sx), m, qx.stride(0), _ptr(qw), _ptr(sw), n, qw.stride(0), k, _ptr(y),
              y.stride(0), _stream(stream)))
    return y


def mfma_rate(compute: str = "f16", iters: int = 100000, stream=None):
    """(sustained TFLOP/s, clock GHz) of the 16x16x32 MFMA on the current device (dit_mfma_rate)."""
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(load_library().dit_mfma_rate(COMPUTE[compute], iters, ctypes.byref(tf), ctypes.byref(ghz),
                                        _stream(stream)))
    return tf.value, ghz.value


def fill_noise(dst, seed: int, stream=None):
    _need(dst, "float32", "dst")
    _check(load_library().dit_fill_noise(_ptr(dst), dst.numel(), seed, _stream(stream)))


_hip = None


def _hip_memcpy_dtod(dst: int, src: int, nbytes: int):
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    rc = _hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 3)  # device to device
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed: {rc}")
