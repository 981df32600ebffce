"""ctypes binding of liblens.so: the structs of include/lens.h and the entry
points under the same names.  Argument marshalling only; every step of the
denoiser runs in the library's HIP kernels.  Loading fails loudly when the
library has not been built."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LENS_LIBRARY names another build of the same library (the tests' host
# sanitizer build); the default is the in-tree liblens.so
LIB_PATH = os.environ.get("LENS_LIBRARY") or os.path.join(_HERE, "liblens.so")

LENS_OK, LENS_ERR_INVALID_ARG, LENS_ERR_UNSUPPORTED, LENS_ERR_WORKSPACE, LENS_ERR_HIP = 0, -1, -2, -3, -4
LENS_F32, LENS_BF16 = 0, 1
LENS_MX_ROWS, LENS_MX_SLABS = 0, 1
LENS_KERNEL_GEMM, LENS_KERNEL_ATTENTION, LENS_KERNEL_NORM, LENS_KERNEL_QKNORM_ROPE, LENS_KERNEL_ADALN = range(5)
LENS_KERNEL_COUNT = 5
KERNEL_NAMES = ("gemm", "attention", "norm", "qknorm_rope", "adaln")

# every function lens.h declares (checked against the header by the tests)
EXPORTS = (
    "lens_default_config", "lens_block_workspace_bytes", "lens_dit_workspace_bytes", "lens_block_forward",
    "lens_dit_forward", "lens_dit_forward_noalloc", "lens_flow_step", "lens_flow_step_rescaled", "lens_quantize_mxfp8", "lens_timer_start",
    "lens_timer_stop", "lens_time_grid", "lens_mu_for_tokens",
    "lens_status_string",
    "lens_last_error", "lens_version",
)


class LensConfig(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("mlp_hidden", C.c_int32),
        ("n_blocks", C.c_int32), ("rope_axes", C.c_int32 * 3), ("in_ch", C.c_int32), ("out_ch", C.c_int32),
        ("txt_feat_dim", C.c_int32), ("txt_layers", C.c_int32), ("t_freq_dim", C.c_int32),
        ("rope_theta", C.c_float), ("eps", C.c_float), ("t_scale", C.c_float), ("act_dtype", C.c_int),
        ("gemm_fp8", C.c_int32),
    ]


class LensLinear(C.Structure):
    _fields_ = [("w", C.c_void_p), ("b", C.c_void_p), ("w_scale", C.c_void_p)]


class LensStreamW(C.Structure):
    _fields_ = [("mod", LensLinear), ("qkv", LensLinear), ("out", LensLinear), ("w1", LensLinear),
                ("w3", LensLinear), ("w2", LensLinear), ("q_gain", C.c_void_p), ("k_gain", C.c_void_p)]


class LensBlockW(C.Structure):
    _fields_ = [("img", LensStreamW), ("txt", LensStreamW)]


class LensDitW(C.Structure):
    _fields_ = [("t_fc1", LensLinear), ("t_fc2", LensLinear), ("img_in", LensLinear), ("txt_in", LensLinear),
                ("norm_out", LensLinear), ("proj_out", LensLinear), ("txt_gain", C.c_void_p),
                ("blocks", C.POINTER(LensBlockW))]


class LensError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -m text_image_flow_amd.build)")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, SZ, F, D = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float, C.c_double
        cfgp = C.POINTER(LensConfig)
        sig = {
            "lens_default_config": (None, [cfgp, C.c_int]),
            "lens_block_workspace_bytes": (SZ, [cfgp, I32, I32, I32]),
            "lens_dit_workspace_bytes": (SZ, [cfgp, I32, I32, I32]),
            "lens_block_forward": (C.c_int, [cfgp, C.POINTER(LensBlockW), P, P, P, P, P, P, I32, I32, I32, P, SZ, P]),
            "lens_dit_forward": (C.c_int, [cfgp, C.POINTER(LensDitW), P, P, P, P, P, P, I32, I32, I32, P, P, SZ, P]),
            "lens_dit_forward_noalloc": (C.c_int, [cfgp, C.POINTER(LensDitW), P, P, P, P, P, P, I32, I32, I32, P, P]),
            "lens_flow_step": (C.c_int, [P, P, P, I64, F, F, P, C.c_int, P]),
            "lens_flow_step_rescaled": (C.c_int, [P, P, P, I64, I32, F, F, P, C.c_int, P]),
            "lens_quantize_mxfp8": (C.c_int, [P, C.c_int, I64, I32, I32, P, P, P]),
            "lens_timer_start": (C.c_int, [C.c_uint32]),
            "lens_timer_stop": (C.c_int, [C.POINTER(D), C.POINTER(I64)]),
            "lens_time_grid": (C.c_int, [I32, F, I32, P, P]),
            "lens_mu_for_tokens": (C.c_int, [I64, D, D, D, D, C.POINTER(D)]),
            "lens_status_string": (C.c_char_p, [C.c_int]),
            "lens_last_error": (C.c_char_p, []),
            "lens_version": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().lens_status_string(int(s)).decode()


def last_error() -> str:
    return lib().lens_last_error().decode()


def check(status: int) -> int:
    if status != LENS_OK:
        raise LensError(status, last_error())
    return status


def version() -> str:
    return lib().lens_version().decode()


def default_config(act_dtype: int = LENS_BF16) -> LensConfig:
    c = LensConfig()
    lib().lens_default_config(C.byref(c), act_dtype)
    return c


def lens_block_workspace_bytes(cfg, B, S_img, S_txt) -> int:
    return lib().lens_block_workspace_bytes(C.byref(cfg), B, S_img, S_txt)


def lens_dit_workspace_bytes(cfg, B, S_img, S_txt) -> int:
    return lib().lens_dit_workspace_bytes(C.byref(cfg), B, S_img, S_txt)


def lens_block_forward(cfg, w, h_img, h_txt, temb, img_pos, txt_pos, txt_len, B, S_img, S_txt, workspace,
                       ws_bytes, stream) -> int:
    return lib().lens_block_forward(C.byref(cfg), C.byref(w), h_img, h_txt, temb, img_pos, txt_pos, txt_len, B,
                                    S_img, S_txt, workspace, ws_bytes, stream)


def lens_dit_forward(cfg, w, x, txt_feats, t, img_pos, txt_pos, txt_len, B, S_img, S_txt, v_out, workspace,
                     ws_bytes, stream) -> int:
    return lib().lens_dit_forward(C.byref(cfg), C.byref(w), x, txt_feats, t, img_pos, txt_pos, txt_len, B, S_img,
                                  S_txt, v_out, workspace, ws_bytes, stream)


NOALLOC_SCRATCH_BYTES = 384 << 20   # LENS_NOALLOC_SCRATCH_BYTES of lens.h


def lens_dit_forward_noalloc(cfg, w, x, txt_feats, t, img_pos, txt_pos, txt_len, B, S_img, S_txt, v_out,
                             stream) -> int:
    return lib().lens_dit_forward_noalloc(C.byref(cfg), C.byref(w), x, txt_feats, t, img_pos, txt_pos, txt_len, B,
                                          S_img, S_txt, v_out, stream)


def lens_flow_step(x, v_cond, v_uncond, n, dt, cfg_scale, x_lowp_out, lowp_dtype, stream) -> int:
    return lib().lens_flow_step(x, v_cond, v_uncond, n, dt, cfg_scale, x_lowp_out, lowp_dtype, stream)


def lens_flow_step_rescaled(x, v_cond, v_uncond, n_tokens, channels, dt, cfg_scale, x_lowp_out, lowp_dtype,
                            stream) -> int:
    return lib().lens_flow_step_rescaled(x, v_cond, v_uncond, n_tokens, channels, dt, cfg_scale, x_lowp_out,
                                         lowp_dtype, stream)


def lens_quantize_mxfp8(src, src_dtype, rows, cols, scale_layout, q_out, scale_out, stream) -> int:
    return lib().lens_quantize_mxfp8(src, src_dtype, rows, cols, scale_layout, q_out, scale_out, stream)


def lens_time_grid(steps, mu, has_mu, t_out, dt_out) -> int:
    """t_out / dt_out: host addresses (or None) of steps + 1 / steps floats."""
    return lib().lens_time_grid(steps, mu, has_mu, t_out, dt_out)


def lens_mu_for_tokens(n_tokens, n0, mu0, n1, mu1, mu_out) -> int:
    return lib().lens_mu_for_tokens(n_tokens, n0, mu0, n1, mu1, mu_out)


def lens_timer_start(kind_mask: int) -> int:
    return lib().lens_timer_start(kind_mask)


def lens_timer_stop():
    """-> (status, [ms per kernel family], [launches per kernel family])"""
    ms, n = (C.c_double * LENS_KERNEL_COUNT)(), (C.c_int64 * LENS_KERNEL_COUNT)()
    st = lib().lens_timer_stop(ms, n)
    return st, list(ms), list(n)
