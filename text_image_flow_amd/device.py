"""Device-side plumbing around the C ABI: upload weights, allocate the
workspace, and call lens_block_forward / lens_dit_forward / lens_flow_step
on torch's current HIP stream.  PyTorch supplies device memory and streams
only; no arithmetic of the denoiser runs here."""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib as L

STREAMS = ("img", "txt")
_LINEARS = ("mod", "qkv", "out", "w1", "w3", "w2")


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible: the Lens library runs on an MI355X (gfx950) GPU only")
    L.lib()


def torch_dtype(act_dtype: int):
    return torch.bfloat16 if act_dtype == L.LENS_BF16 else torch.float32


def upload(a, act_dtype: int | None = None, device="cuda") -> torch.Tensor:
    """numpy -> device tensor.  Floats go to the activation type (bf16 values
    are already bf16-representable, so the conversion is exact); ints stay int32."""
    a = np.ascontiguousarray(a)
    if a.dtype.kind in "iu":
        return torch.from_numpy(a.astype(np.int32)).to(device)
    t = torch.from_numpy(a.astype(np.float32, copy=False))
    if act_dtype is not None:
        t = t.to(torch_dtype(act_dtype))
    return t.to(device)


def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def stream_handle(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


FP8_LINEARS = ("qkv", "out", "w1", "w3", "w2")   # the projections an MX fp8 model quantizes


def quantize_mxfp8(w: torch.Tensor, stream=None, layout: int = L.LENS_MX_SLABS):
    """MX fp8 copy of a bf16 / f32 device matrix [rows, cols] (lens_quantize_mxfp8):
    -> (e4m3 bytes [rows, cols] uint8, E8M0 scales uint8), the scales
    [cols / 128, rows, 4] in the slab-major layout the fp8 GEMMs read
    (LENS_MX_SLABS, the default) or [rows, cols / 32] (LENS_MX_ROWS)."""
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    shape = (cols // 128, rows, 4) if layout == L.LENS_MX_SLABS else (rows, cols // 32)
    s = torch.empty(shape, dtype=torch.uint8, device=w.device)
    dt = L.LENS_BF16 if w.dtype == torch.bfloat16 else L.LENS_F32
    L.check(L.lens_quantize_mxfp8(ptr(w), dt, rows, cols, layout, ptr(q), ptr(s), stream_handle(stream)))
    return q, s


class DeviceBlock:
    """One block's weights on the device plus its lens_block_w table.  With
    gemm_fp8 the projections in FP8_LINEARS are stored as MX fp8 (quantized
    on the device from the act_dtype upload)."""

    def __init__(self, w: dict, act_dtype: int, device="cuda", gemm_fp8: bool = False):
        self.t = {s: {k: upload(v, act_dtype, device) if v is not None else None for k, v in w[s].items()}
                  for s in STREAMS}
        if gemm_fp8:
            for s in STREAMS:
                for name in FP8_LINEARS:
                    q, sc = quantize_mxfp8(self.t[s][f"{name}_w"])
                    self.t[s][f"{name}_w"], self.t[s][f"{name}_s"] = q, sc
            torch.cuda.synchronize(device)
        self._table()

    @classmethod
    def fp8_copy(cls, blk: "DeviceBlock") -> "DeviceBlock":
        """An MX fp8 version of a bf16 device block, quantized on the device
        (biases, gains and the AdaLN weight are shared, not copied)."""
        new = object.__new__(cls)
        new.t = {s: dict(blk.t[s]) for s in STREAMS}
        for s in STREAMS:
            for name in FP8_LINEARS:
                new.t[s][f"{name}_w"], new.t[s][f"{name}_s"] = quantize_mxfp8(blk.t[s][f"{name}_w"])
        torch.cuda.synchronize()
        new._table()
        return new

    def _table(self):
        self.table = L.LensBlockW()
        for s in STREAMS:
            sw = getattr(self.table, s)
            for name in _LINEARS:
                lin = getattr(sw, name)
                lin.w = ptr(self.t[s][f"{name}_w"])
                lin.b = ptr(self.t[s].get(f"{name}_b"))
                lin.w_scale = ptr(self.t[s].get(f"{name}_s"))
            sw.q_gain = ptr(self.t[s]["q_gain"])
            sw.k_gain = ptr(self.t[s]["k_gain"])


class DeviceDit:
    """All denoiser weights on the device plus the lens_dit_w table."""

    def __init__(self, top: dict, blocks, act_dtype: int, device="cuda", gemm_fp8: bool = False):
        self.top = {k: upload(v, act_dtype, device) if v is not None else None for k, v in top.items()}
        self.blocks = [b if isinstance(b, DeviceBlock) else DeviceBlock(b, act_dtype, device, gemm_fp8)
                       for b in blocks]
        self._tables()

    def with_blocks(self, order):
        """The same weights run as the block sequence `order` (indices into
        this model's blocks; repeats and omissions allowed): block swap and
        block removal without copying weights.  Set cfg.n_blocks = len(order)."""
        view = object.__new__(DeviceDit)
        view.top = self.top
        view.blocks = [self.blocks[i] for i in order]
        view._tables()
        return view

    def _tables(self):
        self.block_array = (L.LensBlockW * max(1, len(self.blocks)))()
        for i, b in enumerate(self.blocks):
            self.block_array[i] = b.table
        self.table = L.LensDitW()
        for name in ("t_fc1", "t_fc2", "img_in", "txt_in", "norm_out", "proj_out"):
            lin = getattr(self.table, name)
            lin.w = ptr(self.top[f"{name}_w"])
            lin.b = ptr(self.top.get(f"{name}_b"))
        self.table.txt_gain = ptr(self.top["txt_gain"])
        self.table.blocks = C.cast(self.block_array, C.POINTER(L.LensBlockW))

    @property
    def n_blocks(self):
        return len(self.blocks)


class Workspace:
    """Grow-only device workspace (256-byte aligned by the caching allocator)."""

    def __init__(self, device="cuda"):
        self.buf = None
        self.device = device

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def block_forward(cfg, blk: DeviceBlock, h_img, h_txt, temb, img_pos, txt_pos, txt_len, ws: Workspace, stream=None):
    B, Si = h_img.shape[0], h_img.shape[1]
    St = h_txt.shape[1] if h_txt is not None else 0
    need = L.lens_block_workspace_bytes(cfg, B, Si, St)
    if need == 0:
        raise L.LensError(L.LENS_ERR_INVALID_ARG, L.last_error())
    buf = ws.get(need)
    L.check(L.lens_block_forward(cfg, blk.table, ptr(h_img), ptr(h_txt), ptr(temb), ptr(img_pos), ptr(txt_pos),
                                 ptr(txt_len), B, Si, St, ptr(buf), buf.numel(), stream_handle(stream)))


def dit_forward(cfg, dit: DeviceDit, x, txt_feats, t, img_pos, txt_pos, txt_len, v_out, ws: Workspace, stream=None):
    B, Si = x.shape[0], x.shape[1]
    St = txt_feats.shape[1] if txt_feats is not None else 0
    need = L.lens_dit_workspace_bytes(cfg, B, Si, St)
    if need == 0:
        raise L.LensError(L.LENS_ERR_INVALID_ARG, L.last_error())
    buf = ws.get(need)
    L.check(L.lens_dit_forward(cfg, dit.table, ptr(x), ptr(txt_feats), ptr(t), ptr(img_pos), ptr(txt_pos),
                               ptr(txt_len), B, Si, St, ptr(v_out), ptr(buf), buf.numel(), stream_handle(stream)))


def flow_step(x, v_cond, v_uncond, dt, cfg_scale, x_lowp=None, lowp_dtype=L.LENS_BF16, stream=None):
    L.check(L.lens_flow_step(ptr(x), ptr(v_cond), ptr(v_uncond), x.numel(), float(dt), float(cfg_scale),
                             ptr(x_lowp), lowp_dtype, stream_handle(stream)))


def flow_step_rescaled(x, v_cond, v_uncond, dt, cfg_scale, x_lowp=None, lowp_dtype=L.LENS_BF16, stream=None):
    """Norm-rescaled CFG Euler step over the tokens of x (channels = last dim)."""
    C = int(x.shape[-1])
    L.check(L.lens_flow_step_rescaled(ptr(x), ptr(v_cond), ptr(v_uncond), x.numel() // C, C, float(dt),
                                      float(cfg_scale), ptr(x_lowp), lowp_dtype, stream_handle(stream)))


def time_grid(steps: int, mu: float | None = None):
    """(t, dt) of the sampling loop from lens_time_grid: t [steps + 1] and
    dt [steps] float32 host arrays (uniform grid from t = 1 to 0, or moved
    by mu in logit space)."""
    t = np.empty(steps + 1, np.float32)
    dt = np.empty(max(steps, 0), np.float32)
    L.check(L.lens_time_grid(int(steps), float(mu if mu is not None else 0.0), int(mu is not None),
                             t.ctypes.data, dt.ctypes.data))
    return t, dt


def mu_for_tokens(n: int, n0: float, mu0: float, n1: float, mu1: float) -> float:
    """mu on the line through (n0, mu0) and (n1, mu1) at n tokens (lens_mu_for_tokens)."""
    out = C.c_double()
    L.check(L.lens_mu_for_tokens(int(n), float(n0), float(mu0), float(n1), float(mu1), C.byref(out)))
    return out.value


class Sampler:
    """Flow-matching Euler loop with optional CFG on one device.

    The batch of lens_dit_forward holds the n cond samples in [0, n) and, with
    CFG, n uncond samples in [n, 2n) that share x and t; lens_flow_step then
    combines the two halves of v and advances x.  Nothing synchronises with
    the host inside the loop."""

    def __init__(self, cfg, dit: DeviceDit, img_pos, txt_pos, n: int, S_img: int, S_txt: int, cfg_scale: float,
                 use_cfg: bool, device="cuda", mu: float | None = None, norm_rescale: bool = False):
        """mu: timestep shift of the grid (None: uniform grid); norm_rescale:
        norm-rescaled CFG (lens_flow_step_rescaled) instead of the plain one."""
        self.mu, self.norm_rescale = mu, bool(norm_rescale)
        self.cfg, self.dit = cfg, dit
        self.img_pos, self.txt_pos = img_pos, txt_pos
        self.n, self.S_img, self.S_txt = n, S_img, S_txt
        self.cfg_scale, self.use_cfg = float(cfg_scale), bool(use_cfg)
        self.B = 2 * n if use_cfg else n
        act = torch_dtype(cfg.act_dtype)
        self.x_act = torch.empty((self.B, S_img, cfg.in_ch), dtype=act, device=device)
        self.v = torch.empty((self.B, S_img, cfg.out_ch), dtype=torch.float32, device=device)
        self.ws = Workspace(device)
        self.device = device

    def run(self, x: torch.Tensor, x_act0: torch.Tensor, txt_feats: torch.Tensor, txt_len, steps: int,
            step_hook=None):
        """x: [n, S_img, in_ch] float32 latent tokens, updated in place;
        x_act0: the same values in the activation type (the first DiT input).
        txt_feats: [B, S_txt, F] act type (cond rows first); txt_len [B] or None."""
        ts, dts = time_grid(steps, self.mu)
        t_tab = upload(np.repeat(ts[:, None], self.B, axis=1), None, self.device)   # [steps+1, B]
        # first input, duplicated for the uncond half (plain copies)
        for h in range(self.B // self.n):
            self.x_act[h * self.n:(h + 1) * self.n].copy_(x_act0)
        for k in range(steps):
            if step_hook is not None:
                step_hook(k, x, self.x_act)
            dit_forward(self.cfg, self.dit, self.x_act, txt_feats, t_tab[k], self.img_pos, self.txt_pos, txt_len,
                        self.v, self.ws)
            vc = self.v[:self.n]
            vu = self.v[self.n:] if self.use_cfg else None
            step = flow_step_rescaled if self.norm_rescale else flow_step
            step(x, vc, vu, float(dts[k]), self.cfg_scale, self.x_act[:self.n], self.cfg.act_dtype)
            if self.use_cfg:
                self.x_act[self.n:].copy_(self.x_act[:self.n])
        return x
