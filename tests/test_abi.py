"""The C ABI on the CPU: the library loads, exports every function the header
declares, fills the Lens config, sizes workspaces, and rejects bad arguments
before touching the GPU (no compute call is made here)."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import text_image_flow_amd as T
from text_image_flow_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lens.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "lens_config.json")))


def header_functions():
    txt = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"\b(lens_[a-z_0-9]+)\s*\(", txt))


def test_library_exports_every_header_function():
    names = header_functions()
    assert names == set(L.EXPORTS), names ^ set(L.EXPORTS)
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_default_config_matches_pages():
    c = T.default_config(T.LENS_BF16)
    g = lambda k: GOLD[k]["value"]
    assert (c.n_blocks, c.hidden, c.heads, c.head_dim) == (g("n_blocks"), g("hidden"), g("heads"), g("head_dim"))
    assert list(c.rope_axes) == g("rope_axes") and c.mlp_hidden == g("mlp_hidden")
    assert c.in_ch == g("in_channels") and c.txt_feat_dim == g("enc_hidden_dim") and c.txt_layers == g("txt_layers")
    assert c.act_dtype == T.LENS_BF16 and T.default_config(T.LENS_F32).act_dtype == T.LENS_F32
    assert "gfx950" in T.version()


def test_status_strings():
    for s, n in [(0, "LENS_OK"), (-1, "LENS_ERR_INVALID_ARG"), (-2, "LENS_ERR_UNSUPPORTED"),
                 (-3, "LENS_ERR_WORKSPACE"), (-4, "LENS_ERR_HIP")]:
        assert T.status_string(s) == n
    assert T.status_string(42) == "unknown lens_status"


def test_workspace_sizes():
    c = T.default_config(T.LENS_BF16)
    a = T.lens_block_workspace_bytes(c, 1, 4096, 512)
    b = T.lens_block_workspace_bytes(c, 2, 4096, 512)
    assert a > 0 and b > a and a % 256 == 0
    f = T.default_config(T.LENS_F32)
    assert T.lens_block_workspace_bytes(f, 1, 4096, 512) > a           # 4-byte activations
    assert T.lens_dit_workspace_bytes(c, 2, 4096, 512) > b
    assert T.lens_block_workspace_bytes(c, 0, 4096, 512) == 0           # invalid sizes
    assert T.lens_block_workspace_bytes(c, 1, 0, 512) == 0
    assert T.lens_block_workspace_bytes(c, 1, 16, 0) > 0                # no text is valid


def _bad(cfg_mut=None, **kw):
    c = T.default_config(T.LENS_BF16)
    if cfg_mut:
        cfg_mut(c)
    w = T.LensBlockW()
    for s in ("img", "txt"):
        sw = getattr(w, s)
        for n in ("mod", "qkv", "out", "w1", "w3", "w2"):
            getattr(sw, n).w = 0x1000
        sw.q_gain = sw.k_gain = 0x1000
    args = dict(h_img=0x1000, h_txt=0x1000, temb=0x1000, img_pos=0x1000, txt_pos=0x1000, txt_len=None,
                B=1, S_img=16, S_txt=8, ws=0x1000, ws_bytes=1 << 40)
    args.update(kw)
    st = T.lens_block_forward(c, w, args["h_img"], args["h_txt"], args["temb"], args["img_pos"], args["txt_pos"],
                              args["txt_len"], args["B"], args["S_img"], args["S_txt"], args["ws"],
                              args["ws_bytes"], None)
    return st, T.last_error()


@pytest.mark.parametrize("mut,kw,status,frag", [
    (lambda c: setattr(c, "head_dim", 32), {}, L.LENS_ERR_INVALID_ARG, "hidden"),
    (lambda c: (setattr(c, "heads", 48), setattr(c, "head_dim", 32),
                c.rope_axes.__setitem__(0, 4), c.rope_axes.__setitem__(1, 14), c.rope_axes.__setitem__(2, 14)),
     {}, L.LENS_ERR_UNSUPPORTED, "head_dim"),
    (lambda c: c.rope_axes.__setitem__(0, 7), {}, L.LENS_ERR_INVALID_ARG, "rope_axes"),
    (lambda c: setattr(c, "act_dtype", 7), {}, L.LENS_ERR_INVALID_ARG, "act_dtype"),
    (None, {"B": 0}, L.LENS_ERR_INVALID_ARG, "B >= 1"),
    (None, {"S_img": 0}, L.LENS_ERR_INVALID_ARG, "S_img"),
    (None, {"S_txt": -1}, L.LENS_ERR_INVALID_ARG, "S_txt"),
    (None, {"h_img": None}, L.LENS_ERR_INVALID_ARG, "NULL"),
    (None, {"ws_bytes": 100}, L.LENS_ERR_WORKSPACE, "workspace"),
    (None, {"ws": None}, L.LENS_ERR_WORKSPACE, "workspace"),
    (None, {"ws": 0x1001}, L.LENS_ERR_WORKSPACE, "aligned"),
    (None, {"h_img": 0x1008}, L.LENS_ERR_INVALID_ARG, "16-byte aligned"),
    (None, {"h_txt": 0x1004}, L.LENS_ERR_INVALID_ARG, "16-byte aligned"),
])
def test_block_forward_argument_checks(mut, kw, status, frag):
    st, msg = _bad(mut, **kw)
    assert st == status and frag in msg, (st, msg)


def test_null_weight_is_rejected():
    c = T.default_config(T.LENS_BF16)
    w = T.LensBlockW()
    st = T.lens_block_forward(c, w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 1, 16, 8, 0x1000, 1 << 40, None)
    assert st == L.LENS_ERR_INVALID_ARG and "NULL" in T.last_error()
    st = L.lib().lens_block_forward(None, None, None, None, None, None, None, None, 1, 1, 1, None, 0, None)
    assert st == L.LENS_ERR_INVALID_ARG and "cfg" in T.last_error()


def test_misaligned_tensors_are_rejected_before_any_device_work():
    """Tensors the kernels read in 16-byte pieces must start on a 16-byte
    boundary: a weight, bias or gain that does not is an argument error (the
    pointers are never dereferenced on the host)."""
    def block_call(edit):
        c = T.default_config(T.LENS_BF16)
        w = T.LensBlockW()
        for s in ("img", "txt"):
            sw = getattr(w, s)
            for n in ("mod", "qkv", "out", "w1", "w3", "w2"):
                getattr(sw, n).w = 0x1000
            sw.q_gain = sw.k_gain = 0x1000
        edit(w)
        st = T.lens_block_forward(c, w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 1, 16, 8, 0x1000, 1 << 40,
                                  None)
        return st, T.last_error()

    for edit, frag in ((lambda w: setattr(w.txt.w2, "w", 0x1002), "txt.w2"),
                       (lambda w: setattr(w.img.qkv, "b", 0x1008), "img.qkv"),
                       (lambda w: setattr(w.img, "k_gain", 0x1002), "gains")):
        st, msg = block_call(edit)
        assert st == L.LENS_ERR_INVALID_ARG and "16-byte aligned" in msg and frag in msg, (st, msg)
    # the denoiser's inputs and output, and the quantizer's source
    c = T.default_config(T.LENS_BF16)
    c.n_blocks = 0
    d = T.LensDitW()
    for n in ("t_fc1", "t_fc2", "img_in", "txt_in", "norm_out", "proj_out"):
        getattr(d, n).w = 0x1000
    d.txt_gain = 0x1000
    for x, f, v in ((0x1001, 0x1000, 0x1000), (0x1000, 0x1004, 0x1000), (0x1000, 0x1000, 0x100c)):
        st = T.lens_dit_forward(c, d, x, f, 0x1000, 0x1000, 0x1000, None, 1, 16, 8, v, 0x1000, 1 << 40, None)
        assert st == L.LENS_ERR_INVALID_ARG and "16-byte aligned" in T.last_error(), T.last_error()
    st = T.lens_quantize_mxfp8(0x1002, L.LENS_BF16, 4, 128, L.LENS_MX_SLABS, 0x1000, 0x1000, None)
    assert st == L.LENS_ERR_INVALID_ARG and "16-byte aligned" in T.last_error()


def test_dit_and_flow_argument_checks():
    c = T.default_config(T.LENS_BF16)
    d = T.LensDitW()
    st = T.lens_dit_forward(c, d, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 1, 16, 8, 0x1000, 0x1000, 1 << 40,
                            None)
    assert st == L.LENS_ERR_INVALID_ARG and "t_fc1" in T.last_error()
    c2 = T.default_config(T.LENS_BF16)
    c2.out_ch = 96
    assert T.lens_dit_workspace_bytes(c2, 1, 16, 8) == 0
    assert T.lens_flow_step(None, None, None, -1, 0.1, 1.0, None, 1, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_flow_step(None, None, None, 5, 0.1, 1.0, None, 1, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_flow_step(0x1000, 0x1000, None, 5, 0.1, 1.0, 0x1000, 9, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_flow_step(None, None, None, 0, 0.1, 1.0, None, 1, None) == L.LENS_OK   # empty: nothing to do
    R = T.lens_flow_step_rescaled
    assert R(None, None, None, -1, 128, 0.1, 1.0, None, 1, None) == L.LENS_ERR_INVALID_ARG
    assert R(None, None, None, 5, 0, 0.1, 1.0, None, 1, None) == L.LENS_ERR_INVALID_ARG
    assert R(None, None, None, 5, 128, 0.1, 1.0, None, 1, None) == L.LENS_ERR_INVALID_ARG
    assert R(0x1000, 0x1000, None, 5, 128, 0.1, 1.0, 0x1000, 9, None) == L.LENS_ERR_INVALID_ARG
    assert R(None, None, None, 0, 128, 0.1, 1.0, None, 1, None) == L.LENS_OK   # empty: nothing to do


def test_timer_argument_check():
    assert T.lens_timer_start(1 << 7) == L.LENS_ERR_INVALID_ARG
    assert T.lens_timer_start(0b11) == L.LENS_OK
    st, ms, n = T.lens_timer_stop()
    assert st == L.LENS_OK and n == [0] * 5 and ms == [0.0] * 5


def test_time_grid_through_the_abi_matches_oracle():
    """lens_time_grid (host code in the library) against the oracle's fp64
    grid, uniform and shifted: t and dt = t[k + 1] - t[k] within one float
    rounding, exact end points; lens_mu_for_tokens against the oracle's line."""
    import oracle as O
    from text_image_flow_amd import device as dv
    for steps in (1, 4, 20, 50):
        for mu in (None, 0.0, 1.06, -0.5, 3.0):
            t, dt = dv.time_grid(steps, mu)
            assert t.dtype == np.float32 and t.shape == (steps + 1,) and dt.shape == (steps,)
            ref = O.time_grid(steps, mu)
            np.testing.assert_allclose(t, ref, rtol=0, atol=6e-8)
            np.testing.assert_allclose(dt, np.diff(ref), rtol=0, atol=6e-8)
            assert t[0] == 1.0 and t[-1] == 0.0 and np.all(dt < 0)
    for n in (256, 1024, 2560, 4096, 8100):
        assert abs(dv.mu_for_tokens(n, 1024, 1.06, 4096, 1.5) - O.mu_for_tokens(n, 1024, 1.06, 4096, 1.5)) < 1e-12


def test_time_grid_argument_checks():
    out = C.c_double()
    t = np.zeros(8, np.float32)
    assert T.lens_time_grid(0, 0.0, 0, t.ctypes.data, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_time_grid(-3, 0.0, 0, t.ctypes.data, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_time_grid(4, float("nan"), 1, t.ctypes.data, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_time_grid(4, float("nan"), 0, t.ctypes.data, None) == L.LENS_OK   # mu unused
    assert T.lens_time_grid(4, 1.0, 1, None, None) == L.LENS_OK
    assert T.lens_mu_for_tokens(10, 5.0, 1.0, 5.0, 2.0, C.byref(out)) == L.LENS_ERR_INVALID_ARG
    assert T.lens_mu_for_tokens(10, 5.0, 1.0, 6.0, 2.0, None) == L.LENS_ERR_INVALID_ARG
    assert T.lens_mu_for_tokens(10, 5.0, float("inf"), 6.0, 2.0, C.byref(out)) == L.LENS_ERR_INVALID_ARG
    assert T.lens_mu_for_tokens(10, 5.0, 1.0, 6.0, 2.0, C.byref(out)) == L.LENS_OK and out.value == 6.0


def test_fp8_argument_checks():
    Q = T.lens_quantize_mxfp8
    R, S = T.LENS_MX_ROWS, T.LENS_MX_SLABS
    assert Q(None, 1, -1, 64, R, None, None, None) == L.LENS_ERR_INVALID_ARG
    assert Q(None, 1, 4, 48, R, None, None, None) == L.LENS_ERR_INVALID_ARG    # cols not a multiple of 32
    assert Q(None, 1, 4, 64, S, None, None, None) == L.LENS_ERR_INVALID_ARG    # slabs: cols % 128
    assert Q(None, 1, 4, 128, 2, None, None, None) == L.LENS_ERR_INVALID_ARG   # bad layout
    assert Q(None, 7, 4, 64, R, None, None, None) == L.LENS_ERR_INVALID_ARG    # bad dtype
    assert Q(None, 1, 4, 64, R, None, None, None) == L.LENS_ERR_INVALID_ARG    # NULL pointers
    assert Q(None, 1, 0, 64, R, None, None, None) == L.LENS_OK                 # empty: nothing to do
    assert Q(None, 1, 0, 256, S, None, None, None) == L.LENS_OK
    cfg = T.default_config(L.LENS_F32)
    assert cfg.gemm_fp8 == 0
    cfg.gemm_fp8 = 1                                                          # needs bf16 activations
    assert T.lens_block_workspace_bytes(cfg, 1, 16, 8) == 0
    cfg = T.default_config(L.LENS_BF16)
    cfg.gemm_fp8 = 2
    assert T.lens_block_workspace_bytes(cfg, 1, 16, 8) == 0
    cfg.gemm_fp8 = 1
    assert T.lens_block_workspace_bytes(cfg, 1, 16, 8) > T.lens_block_workspace_bytes(T.default_config(L.LENS_BF16), 1, 16, 8)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """lens_dit_forward_noalloc checks the call's scratch need against the
    static array before any device work: 2:1 at batch 8 (1.08 GiB) is
    refused with LENS_ERR_WORKSPACE; invalid arguments as lens_dit_forward."""
    c = T.default_config(T.LENS_BF16)
    c.n_blocks = 1
    blk = (T.LensBlockW * 1)()
    for s in ("img", "txt"):
        sw = getattr(blk[0], s)
        for n in ("mod", "qkv", "out", "w1", "w3", "w2"):
            getattr(sw, n).w = 0x1000
        sw.q_gain = sw.k_gain = 0x1000
    d = T.LensDitW()
    for n in ("t_fc1", "t_fc2", "img_in", "txt_in", "norm_out", "proj_out"):
        getattr(d, n).w = 0x1000
    d.txt_gain = 0x1000
    d.blocks = C.cast(blk, C.POINTER(T.LensBlockW))
    assert T.lens_dit_workspace_bytes(c, 8, 4050, 512) > L.NOALLOC_SCRATCH_BYTES
    st = L.lens_dit_forward_noalloc(c, d, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 8, 4050, 512, 0x1000, None)
    assert st == L.LENS_ERR_WORKSPACE and "static scratch" in T.last_error(), T.last_error()
    st = L.lens_dit_forward_noalloc(c, d, None, 0x1000, 0x1000, 0x1000, 0x1000, None, 1, 16, 8, 0x1000, None)
    assert st == L.LENS_ERR_INVALID_ARG
    st = L.lens_dit_forward_noalloc(c, d, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 0, 16, 8, 0x1000, None)
    assert st == L.LENS_ERR_INVALID_ARG
