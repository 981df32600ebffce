"""GPU parity of lens_block_forward against the fp64 oracle on the same
seeded inputs: block outputs and block deltas (h_out - h_in), valid rows
only (rows of masked text queries are unspecified)."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.parity import DELTA_REL, SHARP_DELTA_REL, assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    from text_image_flow_amd import device as dv
    dv.require_gpu()
    return dv


def run_case(dtype, B, gh, gw, St, txt_len=None, variant="canonical", block=0, seed_h=1):
    dv = _dev()
    import text_image_flow_amd as T
    act = T.LENS_BF16 if dtype == "bf16" else T.LENS_F32
    cfg = T.default_config(act)
    Si = gh * gw
    print(f"case dtype={dtype} B={B} grid={gh}x{gw} S_txt={St} txt_len={txt_len} variant={variant}", flush=True)
    w = synth.block_weights(block, dtype=dtype, variant=variant)
    h_img, h_txt, temb = synth.block_inputs(B, Si, St, dtype=dtype, seed=seed_h)
    ip, tp = synth.image_positions(gh, gw), synth.text_positions(St)

    blk = dv.DeviceBlock(w, act)
    d_hi = dv.upload(h_img)
    d_ht = dv.upload(h_txt) if St > 0 else None
    d_temb = dv.upload(temb)
    d_ip, d_tp = dv.upload(ip), (dv.upload(tp) if St > 0 else None)
    d_tl = dv.upload(np.asarray(txt_len, np.int32)) if txt_len is not None else None
    ws = dv.Workspace()
    dv.block_forward(cfg, blk, d_hi, d_ht, d_temb, d_ip, d_tp, d_tl, ws)
    torch.cuda.synchronize()
    gi = d_hi.cpu().numpy()
    gt = d_ht.cpu().numpy() if St > 0 else np.zeros((B, 0, cfg.hidden), np.float32)

    ri, rt = O.block_forward(w, h_img, h_txt, temb, ip, tp, txt_len)
    tl = np.full(B, St) if txt_len is None else np.asarray(txt_len)
    # fp32 runs hold block deltas to the output bar; bf16 runs to DELTA_REL.
    # With the 'wide' stress weights (N(0,1) modulation biases) the block
    # update is several times larger than h, so bf16 outputs inherit the
    # delta budget as well.
    drel = DELTA_REL if dtype == "bf16" else 2e-2
    orel = DELTA_REL if (dtype == "bf16" and variant in ("wide", "sharp")) else 2e-2
    if dtype == "bf16" and variant == "sharp":
        drel = orel = SHARP_DELTA_REL
    assert_parity(gi, ri, "h_img", rel=orel)
    assert_parity(gi - h_img, ri - h_img, "delta_img", rel=drel)
    vt = np.concatenate([gt[b, :tl[b]] for b in range(B)]) if St else np.zeros((0, cfg.hidden))
    rv = np.concatenate([rt[b, :tl[b]] for b in range(B)]) if St else np.zeros((0, cfg.hidden))
    hv = np.concatenate([h_txt[b, :tl[b]] for b in range(B)]) if St else np.zeros((0, cfg.hidden))
    if vt.size:
        assert_parity(vt, rv, "h_txt", rel=orel)
        assert_parity(vt - hv, rv - hv, "delta_txt", rel=drel)


def test_block_f32_config0():
    """fp32, 16x16 image grid + 32 text tokens, B = 1, canonical init."""
    run_case("f32", 1, 16, 16, 32)


def test_block_f32_wide_masked():
    run_case("f32", 2, 9, 11, 13, txt_len=[13, 5], variant="wide")


def test_block_bf16_ragged_masked_wide():
    """Tails everywhere: 2 x 130 image rows (not a tile multiple), 45 text
    tokens with lengths 45 and 17, large gains and biases."""
    run_case("bf16", 2, 10, 13, 45, txt_len=[45, 17], variant="wide")


def test_block_bf16_sharp_attention_online_max():
    """q/k gains near 2.05: the score bound from the gains (about 52 in log2
    units) is too large to serve as a fixed softmax offset, so the kernel
    tracks the running max and rescales (the path every other bf16 case,
    with gains <= 1.5, skips)."""
    run_case("bf16", 2, 10, 13, 45, txt_len=[45, 17], variant="sharp")


def test_block_bf16_no_text():
    run_case("bf16", 1, 8, 8, 0)


def test_block_bf16_empty_and_single_text():
    run_case("bf16", 3, 8, 12, 20, txt_len=[0, 20, 1])


def test_block_bf16_two_tiles_exact():
    run_case("bf16", 1, 16, 16, 64, txt_len=[64])


def test_block_bf16_config1_full():
    """bf16, 64x64 image grid (4096 tokens, 1024^2) + 512 text tokens, B = 1."""
    run_case("bf16", 1, 64, 64, 512)
