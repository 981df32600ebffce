"""lens_dit_forward_noalloc (the allocation-free variant of lens_dit_forward,
whose scratch is the library's static per-device array) against
lens_dit_forward on a caller workspace: the same results, bit for bit, on
two calls in a row, the second with a smaller input than the first (the
first fills most of the static scratch: the 1024^2 cond + uncond launch)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _call_both(dit, cfg, B, gh, gw, St, txt_len, t):
    from text_image_flow_amd import _lib as L
    from text_image_flow_amd import device as dv
    Si = gh * gw
    print(f"noalloc vs workspace: B={B} grid={gh}x{gw} S_txt={St} txt_len={txt_len}", flush=True)
    x = synth.bf16_round(synth.latents(B, Si))
    feats = synth.text_features(B, St, txt_len=txt_len)
    d_x, d_f = dv.upload(x, L.LENS_BF16), dv.upload(feats, L.LENS_BF16)
    d_t, d_ip, d_tp = dv.upload(np.asarray(t, np.float32)), dv.upload(synth.image_positions(gh, gw)), \
        dv.upload(synth.text_positions(St))
    d_tl = dv.upload(np.asarray(txt_len, np.int32)) if txt_len is not None else None
    need = L.lens_dit_workspace_bytes(cfg, B, Si, St)
    assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
    v_ws = torch.full((B, Si, 128), float("nan"), dtype=torch.float32, device="cuda")
    v_na = torch.full((B, Si, 128), float("nan"), dtype=torch.float32, device="cuda")
    dv.dit_forward(cfg, dit, d_x, d_f, d_t, d_ip, d_tp, d_tl, v_ws, dv.Workspace())
    L.check(L.lens_dit_forward_noalloc(cfg, dit.table, dv.ptr(d_x), dv.ptr(d_f), dv.ptr(d_t), dv.ptr(d_ip),
                                       dv.ptr(d_tp), dv.ptr(d_tl), B, Si, St, dv.ptr(v_na), dv.stream_handle()))
    torch.cuda.synchronize()
    a, b = v_ws.cpu().numpy(), v_na.cpu().numpy()
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b), f"max |diff| {np.nanmax(np.abs(a - b))}"


def test_noalloc_matches_workspace_call_twice_shrinking():
    import text_image_flow_amd as T
    from text_image_flow_amd import device as dv
    dv.require_gpu()
    cfg = T.default_config(T.LENS_BF16)
    cfg.n_blocks = 2
    dit = dv.DeviceDit(synth.top_weights(), [synth.block_weights(i) for i in range(2)], T.LENS_BF16)
    _call_both(dit, cfg, 2, 64, 64, 512, None, [0.7, 0.7])          # 274 MiB of the 384 MiB scratch
    _call_both(dit, cfg, 1, 6, 7, 24, [11], [0.3])                   # smaller, masked text
