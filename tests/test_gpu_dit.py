"""GPU parity of lens_dit_forward, lens_flow_step and the sampler loop
against the fp64 oracle on the same seeded inputs.

Whole-model parity: two blocks at small token counts; one block at the real
1024^2 / 1440^2 / 2:1 and 1:2 shapes (embeddings, a block and the final
layer all at full size); the full 48-block model's v at 1024^2 (B = 1)
against the oracle's 48-block forward (about two minutes of fp64 on the
host); and, teacher-forced, blocks 0, 23 and 47 of the 48-block model at the
benchmarked cond + uncond launch (1024^2, B = 2), at 1440^2 (B = 1) and at
2:1 and 1:2 with batch 8 and masked text: the GPU chains lens_block_forward
through all 48 blocks from the oracle's embeddings, and the oracle runs each
sampled block from the GPU's own input to it, so block outputs and block
deltas are compared at the model's own modulation scale.  The 48-block
model at the benchmarked launch is also checked through properties that
hold at any size: bit-identical reruns and exact sample-swap symmetry
(batch independence); its MX fp8 variant by the same properties, its cosine
to the bf16 model and, at B = 1, to the oracle's exact v."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.parity import MAXABS_REL, MODEL_DELTA_REL, SAMPLER_DX_REL, assert_parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _env():
    import text_image_flow_amd as T
    from text_image_flow_amd import device as dv
    dv.require_gpu()
    return T, dv


def make_inputs(B, gh, gw, St, dtype, txt_len=None, t=None, seed_lat=synth.SEED_LATENT):
    x = synth.latents(B, gh * gw, seed=seed_lat)
    x = synth.bf16_round(x) if dtype == "bf16" else x
    feats = synth.text_features(B, St, dtype=dtype, txt_len=txt_len) if St else np.zeros((B, 0, 11520), np.float32)
    t = np.linspace(0.9, 0.2, B).astype(np.float32) if t is None else np.asarray(t, np.float32)
    return x, feats, t, synth.image_positions(gh, gw), synth.text_positions(St)


def gpu_dit(n_blocks, dtype, x, feats, t, ip, tp, txt_len, blocks=None, top=None):
    T, dv = _env()
    act = T.LENS_BF16 if dtype == "bf16" else T.LENS_F32
    cfg = T.default_config(act)
    cfg.n_blocks = n_blocks
    top = synth.top_weights(dtype=dtype) if top is None else top
    blocks = [synth.block_weights(i, dtype=dtype) for i in range(n_blocks)] if blocks is None else blocks
    dit = dv.DeviceDit(top, blocks, act)
    B, Si = x.shape[:2]
    St = feats.shape[1]
    v = torch.empty((B, Si, cfg.out_ch), dtype=torch.float32, device="cuda")
    d_tl = dv.upload(np.asarray(txt_len, np.int32)) if txt_len is not None else None
    dv.dit_forward(cfg, dit, dv.upload(x, act), dv.upload(feats, act) if St else None, dv.upload(t), dv.upload(ip),
                   dv.upload(tp) if St else None, d_tl, v, dv.Workspace())
    torch.cuda.synchronize()
    return v.cpu().numpy(), top, blocks


def check_dit(n_blocks, dtype, B, gh, gw, St, txt_len=None, t=None):
    print(f"dit n_blocks={n_blocks} {dtype} B={B} grid={gh}x{gw} S_txt={St} txt_len={txt_len}", flush=True)
    x, feats, t, ip, tp = make_inputs(B, gh, gw, St, dtype, txt_len, t)
    v, top, blocks = gpu_dit(n_blocks, dtype, x, feats, t, ip, tp, txt_len)
    ref = O.dit_forward(top, blocks, x, feats, t, ip, tp, txt_len)
    assert_parity(v, ref, f"v ({n_blocks} blocks, {dtype})")


def test_dit_two_blocks_bf16_masked():
    check_dit(2, "bf16", 2, 8, 10, 24, txt_len=[24, 9])


@pytest.mark.parametrize("order", [[2, 0, 2], [1], [2, 1, 0]])
def test_dit_block_list(order):
    """Block removal / swap / repeat: the model built with blocks 0..2 run as
    the block sequence `order` against the oracle on that sequence."""
    T, dv = _env()
    print(f"dit block list {order}", flush=True)
    x, feats, t, ip, tp = make_inputs(2, 8, 10, 24, "bf16", [24, 9])
    top = synth.top_weights(dtype="bf16")
    blocks = [synth.block_weights(i, dtype="bf16") for i in range(3)]
    dit = dv.DeviceDit(top, blocks, T.LENS_BF16).with_blocks(order)
    cfg = T.default_config(T.LENS_BF16)
    cfg.n_blocks = len(order)
    v = torch.empty((2, 80, cfg.out_ch), dtype=torch.float32, device="cuda")
    dv.dit_forward(cfg, dit, dv.upload(x, T.LENS_BF16), dv.upload(feats, T.LENS_BF16), dv.upload(t), dv.upload(ip),
                   dv.upload(tp), dv.upload(np.array([24, 9], np.int32)), v, dv.Workspace())
    torch.cuda.synchronize()
    ref = O.dit_forward(top, [blocks[i] for i in order], x, feats, t, ip, tp, [24, 9])
    assert_parity(v.cpu().numpy(), ref, f"v (blocks {order})")


def test_dit_two_blocks_f32():
    check_dit(2, "f32", 1, 7, 9, 16)


def test_dit_no_blocks_1024():
    """Embeddings and final layer alone at 1024^2, B = 2."""
    check_dit(0, "bf16", 2, 64, 64, 512)


def test_dit_one_block_1024_cfg_batch():
    """img_in / txt_in / one block / final layer at 1024^2 with the cond and
    uncond text of the CFG batch (independent seeded feature draws)."""
    T, dv = _env()
    x, _, t, ip, tp = make_inputs(2, 64, 64, 512, "bf16", t=[0.55, 0.55])
    x[1] = x[0]
    feats = np.concatenate([synth.text_features(1, 512, seed=synth.SEED_TEXT_COND),
                            synth.text_features(1, 512, seed=synth.SEED_TEXT_UNCOND)])
    v, top, blocks = gpu_dit(1, "bf16", x, feats, t, ip, tp, None)
    ref = O.dit_forward(top, blocks, x, feats, t, ip, tp, None)
    assert_parity(v, ref, "v (1 block, 1024^2, cond+uncond)")


def test_dit_one_block_1440():
    """1440^2: 90 x 90 = 8100 image tokens + 512 text tokens, B = 1."""
    check_dit(1, "bf16", 1, 90, 90, 512, t=[1.0])


@pytest.mark.parametrize("gh,gw", [(45, 90), (90, 45)])
def test_dit_one_block_aspect_masked_batch8(gh, gw):
    """2:1 and 1:2 aspect (4050 image tokens), batch 8 (4 cond + 4 uncond),
    text lengths drawn from 64..512 and padded to 512 with the key mask."""
    tl = np.concatenate([synth.text_lengths(4, 64, 512, stream=0), synth.text_lengths(4, 64, 512, stream=1)])
    check_dit(1, "bf16", 8, gh, gw, 512, txt_len=tl, t=[0.8] * 8)


def lazy_blocks(n, variant="canonical", ahead=6, threads=8):
    """Weights of blocks 0 .. n-1 in order, generated on a thread pool a few
    blocks ahead of their use (the oracle holds one block at a time)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        futs = {i: ex.submit(synth.block_weights, i, variant=variant) for i in range(min(ahead, n))}
        for i in range(n):
            if i + ahead < n:
                futs[i + ahead] = ex.submit(synth.block_weights, i + ahead, variant=variant)
            yield futs.pop(i).result()


class _Progress(dict):
    """capture= target of oracle.dit_forward that prints a line per block
    (the 48-block oracle pass is long) and keeps nothing."""

    def __setitem__(self, i, value):
        print(f"  oracle block {i} done", flush=True)


@pytest.fixture(scope="module")
def full_inputs_b1():
    """Inputs of the 1024^2 B = 1 forward and the oracle's 48-block v for them."""
    import time
    x, feats, t, ip, tp = make_inputs(1, 64, 64, 512, "bf16", t=[0.6])
    t0 = time.time()
    print("oracle: 48-block forward at 1024^2, B = 1", flush=True)
    ref = O.dit_forward(synth.top_weights(), lazy_blocks(48), x, feats, t, ip, tp, capture=_Progress())
    print(f"oracle: done in {time.time() - t0:.1f} s", flush=True)
    return x, feats, t, ip, tp, ref


@pytest.fixture(scope="module")
def full_dit():
    """The 48-block bf16 model at the benchmarked shapes, uploaded once for
    the full-size tests of this module."""
    T, dv = _env()
    return dv.DeviceDit(synth.top_weights(), [w for _, w in synth.all_block_weights(threads=16)], T.LENS_BF16)


def _full_run_props(cfg, dit):
    """Runs the 1024^2 cond + uncond launch: returns v, after checking that
    it is finite, that a rerun is bit-identical and that swapping the two
    samples' inputs swaps the outputs exactly (no cross-sample leakage)."""
    T, dv = _env()
    x0 = synth.bf16_round(synth.latents(1, 4096))
    xa = np.concatenate([x0, synth.bf16_round(synth.latents(1, 4096, sample=1))])
    fa = np.concatenate([synth.text_features(1, 512, seed=synth.SEED_TEXT_COND),
                         synth.text_features(1, 512, seed=synth.SEED_TEXT_UNCOND)])
    ip, tp = dv.upload(synth.image_positions(64, 64)), dv.upload(synth.text_positions(512))
    ws = dv.Workspace()

    def run(x, f, t):
        v = torch.empty((2, 4096, 128), dtype=torch.float32, device="cuda")
        dv.dit_forward(cfg, dit, dv.upload(x, T.LENS_BF16), dv.upload(f, T.LENS_BF16), dv.upload(t), ip, tp, None,
                       v, ws)
        torch.cuda.synchronize()
        return v.cpu().numpy()

    t = np.array([0.75, 0.35], np.float32)
    v1 = run(xa, fa, t)
    assert np.all(np.isfinite(v1)) and np.std(v1) > 0
    v2 = run(xa, fa, t)
    assert np.array_equal(v1, v2), "rerun is not bit-identical"
    vs = run(xa[::-1].copy(), fa[::-1].copy(), t[::-1].copy())
    assert np.array_equal(vs[0], v1[1]) and np.array_equal(vs[1], v1[0]), "sample swap changed the outputs"
    return v1


def test_dit_full_48_blocks_1024_properties(full_dit):
    """The benchmarked launch: 48 blocks, 1024^2, cond + uncond batch of 2
    (finite, bit-identical rerun, exact sample swap)."""
    T, dv = _env()
    print("dit 48 blocks bf16 1024^2 B=2", flush=True)
    _full_run_props(T.default_config(T.LENS_BF16), full_dit)


def _run_b1(cfg, dit, x, feats, t, ip, tp):
    T, dv = _env()
    v = torch.empty((1, x.shape[1], 128), dtype=torch.float32, device="cuda")
    dv.dit_forward(cfg, dit, dv.upload(x, T.LENS_BF16), dv.upload(feats, T.LENS_BF16), dv.upload(t), dv.upload(ip),
                   dv.upload(tp), None, v, dv.Workspace())
    torch.cuda.synchronize()
    return v.cpu().numpy()


@pytest.mark.timeout(1200)
def test_dit_full_48_blocks_1024_b1_against_oracle(full_dit, full_inputs_b1):
    """v of the whole 48-block bf16 denoiser at 1024^2 (4096 image + 512 text
    tokens, B = 1) against the oracle's 48-block fp64 forward on the same
    inputs, at the parity bar."""
    T, dv = _env()
    x, feats, t, ip, tp, ref = full_inputs_b1
    print("dit 48 blocks bf16 1024^2 B=1 vs oracle", flush=True)
    v = _run_b1(T.default_config(T.LENS_BF16), full_dit, x, feats, t, ip, tp)
    assert_parity(v, ref, "v (48 blocks, 1024^2, B = 1)")


@pytest.mark.timeout(1200)
def test_dit_fp8_full_48_blocks_1024_b1_cosine_gate(full_dit, full_inputs_b1):
    """The MX fp8 variant of the same forward against the oracle's exact v:
    the pages' low-precision gate, cosine >= 0.9976 (Lens-3.8B-4bit article,
    section 4: a single quantized DiT pass against the unquantized one)."""
    T, dv = _env()
    x, feats, t, ip, tp, ref = full_inputs_b1
    dit8 = dv.DeviceDit(synth.top_weights(), [dv.DeviceBlock.fp8_copy(b) for b in full_dit.blocks], T.LENS_BF16)
    cfg8 = T.default_config(T.LENS_BF16)
    cfg8.gemm_fp8 = 1
    v = _run_b1(cfg8, dit8, x, feats, t, ip, tp).ravel().astype(np.float64)
    r = ref.ravel()
    cos = float(v @ r / np.linalg.norm(v) / np.linalg.norm(r))
    print(f"v cosine, fp8 48-block model vs exact fp64 model: {cos:.6f}", flush=True)
    assert np.all(np.isfinite(v)) and cos >= 0.9976


def _teacher_forced_blocks(full_dit, x, feats, t, gh, gw, St, txt_len, rows=None, sample=(0, 23, 47)):
    """Chains lens_block_forward through the 48 blocks from the oracle's
    embeddings (img_in, txt_norm + txt_in, timestep MLP, fp32 as the residual
    stream holds them) and, for each sampled block, runs the oracle block on
    the GPU's own input to it: outputs at the parity bar, deltas at
    MODEL_DELTA_REL (the rounding budget of a block at the model's own
    modulation, 0.043 x RMS(delta), with margin), over valid rows (rows:
    optional (image, text) row subsets)."""
    T, dv = _env()
    top = synth.top_weights()
    B = x.shape[0]
    ip, tp = synth.image_positions(gh, gw), synth.text_positions(St)
    temb = O.timestep_embedding(top, t).astype(np.float32)
    h_img = O.linear(x, top["img_in_w"], top["img_in_b"]).astype(np.float32)
    h_txt = O.text_embed(top, feats).astype(np.float32)
    cfg = T.default_config(T.LENS_BF16)
    d_hi, d_ht = dv.upload(h_img), dv.upload(h_txt)
    d_temb, d_ip, d_tp = dv.upload(temb), dv.upload(ip), dv.upload(tp)
    d_tl = dv.upload(np.asarray(txt_len, np.int32)) if txt_len is not None else None
    ws = dv.Workspace()
    got = {}
    for i, blk in enumerate(full_dit.blocks):
        if i in sample:
            torch.cuda.synchronize()
            got[i] = [d_hi.cpu().numpy(), d_ht.cpu().numpy()]
        dv.block_forward(cfg, blk, d_hi, d_ht, d_temb, d_ip, d_tp, d_tl, ws)
        if i in sample:
            torch.cuda.synchronize()
            got[i] += [d_hi.cpu().numpy(), d_ht.cpu().numpy()]
    assert np.all(np.isfinite(d_hi.cpu().numpy()))
    ri_sel = np.arange(gh * gw) if rows is None else np.asarray(rows[0])
    rt_sel = np.arange(St) if rows is None else np.asarray(rows[1])
    tl = np.full(B, St) if txt_len is None else np.asarray(txt_len)
    for i in sample:
        hi_in, ht_in, hi_out, ht_out = got[i]
        print(f"oracle block {i} (teacher-forced)", flush=True)
        ri, rt = O.block_forward(synth.block_weights(i), hi_in, ht_in, temb, ip, tp, txt_len, rows=rows)
        gi, hi0 = hi_out[:, ri_sel], hi_in[:, ri_sel]
        assert_parity(gi, ri, f"block {i} h_img", rel=MAXABS_REL)
        assert_parity(gi - hi0, ri - hi0, f"block {i} delta_img", rel=MODEL_DELTA_REL)
        if St:
            keep = [rt_sel < tl[b] for b in range(B)]
            pick = lambda a: np.concatenate([a[b][keep[b]] for b in range(B)])
            gt, ht0 = pick(ht_out[:, rt_sel]), pick(ht_in[:, rt_sel])
            rv = pick(rt)
            assert_parity(gt, rv, f"block {i} h_txt", rel=MAXABS_REL)
            assert_parity(gt - ht0, rv - ht0, f"block {i} delta_txt", rel=MODEL_DELTA_REL)


@pytest.mark.timeout(900)
def test_dit_teacher_forced_blocks_1024_cfg_batch(full_dit):
    """Blocks 0, 23, 47 of the benchmarked launch: 1024^2, cond + uncond
    (shared latent and t, independent text features), all rows."""
    print("teacher-forced blocks 0/23/47, 1024^2, B = 2 (CFG)", flush=True)
    x0 = synth.bf16_round(synth.latents(1, 4096))
    x = np.concatenate([x0, x0])
    feats = np.concatenate([synth.text_features(1, 512, seed=synth.SEED_TEXT_COND),
                            synth.text_features(1, 512, seed=synth.SEED_TEXT_UNCOND)])
    _teacher_forced_blocks(full_dit, x, feats, np.array([0.75, 0.75]), 64, 64, 512, None)


@pytest.mark.timeout(900)
def test_dit_teacher_forced_blocks_1440_turbo(full_dit):
    """1440^2 (90 x 90 = 8100 image + 512 text tokens), B = 1, the first
    Turbo step (t = 1, no CFG); every 4th image row and all text rows."""
    print("teacher-forced blocks 0/23/47, 1440^2, B = 1", flush=True)
    x = synth.bf16_round(synth.latents(1, 8100))
    feats = synth.text_features(1, 512, seed=synth.SEED_TEXT_COND)
    _teacher_forced_blocks(full_dit, x, feats, np.array([1.0]), 90, 90, 512, None,
                           rows=(np.arange(0, 8100, 4), np.arange(512)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("gh,gw", [(45, 90), (90, 45)])
def test_dit_teacher_forced_blocks_aspect_batch8(full_dit, gh, gw):
    """2:1 and 1:2 aspect (4050 image tokens), 4 latents with CFG (batch 8),
    text lengths drawn from 64..512 and padded to 512 with the key mask, at
    the middle of a 50-step loop (t = 0.5); every 8th image row and all
    valid text rows."""
    print(f"teacher-forced blocks 0/23/47, {gh}x{gw}, B = 8 (CFG), masked text", flush=True)
    xs = synth.bf16_round(synth.latents(4, gh * gw))
    x = np.concatenate([xs, xs])
    tl = np.concatenate([synth.text_lengths(4, 64, 512, stream=0), synth.text_lengths(4, 64, 512, stream=1)])
    fc = synth.text_features(4, 512, seed=synth.SEED_TEXT_COND, txt_len=tl[:4])
    fu = synth.text_features(4, 512, seed=synth.SEED_TEXT_UNCOND, txt_len=tl[4:])
    _teacher_forced_blocks(full_dit, x, np.concatenate([fc, fu]), np.full(8, 0.5), gh, gw, 512, tl,
                           rows=(np.arange(0, gh * gw, 8), np.arange(512)))


def test_dit_fp8_full_48_blocks_1024(full_dit):
    """The MX fp8 variant of the benchmarked launch (projection weights
    quantized on the device from the same bf16 model): the same properties,
    and per sample the pages' low-precision gate (cosine >= 0.9976 of the
    quantized DiT's output against the unquantized one, Lens-3.8B-4bit
    article, section 4) against the bf16 model (measured 0.9992-0.9993; at
    B = 1 the same fp8 model is held to the gate against the exact fp64
    model above)."""
    T, dv = _env()
    print("dit 48 blocks fp8 1024^2 B=2", flush=True)
    v16 = _full_run_props(T.default_config(T.LENS_BF16), full_dit)
    dit8 = dv.DeviceDit(synth.top_weights(), [dv.DeviceBlock.fp8_copy(b) for b in full_dit.blocks], T.LENS_BF16)
    cfg8 = T.default_config(T.LENS_BF16)
    cfg8.gemm_fp8 = 1
    v8 = _full_run_props(cfg8, dit8)
    for b in range(2):
        a, c = v8[b].ravel().astype(np.float64), v16[b].ravel().astype(np.float64)
        cos = float(a @ c / np.linalg.norm(a) / np.linalg.norm(c))
        print(f"sample {b}: v cosine fp8 vs bf16 {cos:.6f}", flush=True)
        assert cos >= 0.9976


# ------------------------------------------------------------ flow step
@pytest.mark.parametrize("cfg_scale,use_uncond", [(5.0, True), (1.0, False), (1.0, True)])
def test_flow_step_1024(cfg_scale, use_uncond):
    T, dv = _env()
    n = 4096 * 128
    x = synth.gaussian((n,), 2, 0)
    vc, vu = synth.gaussian((n,), 2, 1), synth.gaussian((n,), 2, 2)
    dx = dv.upload(x)
    lowp = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dv.flow_step(dx, dv.upload(vc), dv.upload(vu) if use_uncond else None, -0.05, cfg_scale, lowp)
    torch.cuda.synchronize()
    ref = O.flow_step(x, vc, vu if use_uncond else None, -0.05, cfg_scale)
    g = dx.cpu().numpy()
    assert_parity(g, ref, f"flow step s={cfg_scale} uncond={use_uncond}")
    assert np.max(np.abs(g - ref)) <= 4e-6 * np.max(np.abs(ref))
    # the bf16 copy is the round-to-nearest-even of the new x
    assert np.array_equal(lowp.float().cpu().numpy(), synth.bf16_round(g))


@pytest.mark.parametrize("ntok,C,cfg_scale,use_uncond", [(8192, 128, 5.0, True), (4097, 128, 1.0, True),
                                                      (4096, 128, 5.0, False), (1001, 96, 2.5, True),
                                                      (333, 200, 5.0, True)])
def test_flow_step_rescaled(ntok, C, cfg_scale, use_uncond):
    """Norm-rescaled CFG step against the oracle: 1024^2 cond+uncond latents
    (2 x 4096 tokens of 128 channels), a ragged token count, no uncond, and
    channel counts that are not multiples of the wave width."""
    T, dv = _env()
    x = synth.gaussian((ntok, C), 3, 0)
    vc, vu = synth.gaussian((ntok, C), 3, 1), synth.gaussian((ntok, C), 3, 2)
    # token 0: u + 5 (c - u) = 1.25 + 5 (1 - 1.25) = 0 exactly in fp32 -> unchanged
    vc[0], vu[0] = 1.0, 1.25
    dx = dv.upload(x)
    lowp = torch.empty((ntok, C), dtype=torch.bfloat16, device="cuda")
    dv.flow_step_rescaled(dx, dv.upload(vc), dv.upload(vu) if use_uncond else None, -0.05, cfg_scale, lowp)
    torch.cuda.synchronize()
    ref = O.flow_step_rescaled(x, vc, vu if use_uncond else None, -0.05, cfg_scale)
    g = dx.cpu().numpy()
    assert_parity(g, ref, f"rescaled flow step n={ntok} C={C} s={cfg_scale} uncond={use_uncond}")
    assert np.max(np.abs(g - ref)) <= 4e-6 * np.max(np.abs(ref))
    if use_uncond and cfg_scale == 5.0:
        assert np.array_equal(g[0], x[0])
    assert np.array_equal(lowp.float().cpu().numpy(), synth.bf16_round(g))


# ------------------------------------------------------------ sampler
def _small_sampler_setup(use_cfg, **smp_kw):
    T, dv = _env()
    gh, gw, St = 8, 8, 16
    cfg = T.default_config(T.LENS_BF16)
    cfg.n_blocks = 2
    top = synth.top_weights()
    blocks = [synth.block_weights(i) for i in range(2)]
    dit = dv.DeviceDit(top, blocks, T.LENS_BF16)
    n = 1
    fc = synth.text_features(1, St, seed=synth.SEED_TEXT_COND)
    fu = synth.text_features(1, St, seed=synth.SEED_TEXT_UNCOND)
    feats = np.concatenate([fc, fu]) if use_cfg else fc
    ip, tp = synth.image_positions(gh, gw), synth.text_positions(St)
    x0 = synth.latents(n, gh * gw)
    smp = dv.Sampler(cfg, dit, dv.upload(ip), dv.upload(tp), n, gh * gw, St, 5.0 if use_cfg else 1.0, use_cfg,
                     **smp_kw)
    return dv, top, blocks, feats, ip, tp, x0, smp


def test_sampler_cfg_teacher_forced():
    """Each CFG Euler step from the GPU's own state: x_{k+1} - x_k against
    dt * (v_u + 5 (v_c - v_u)) from the oracle at the same bf16 input."""
    dv, top, blocks, feats, ip, tp, x0, smp = _small_sampler_setup(True)
    steps = 3
    states = []
    x = dv.upload(x0)
    smp.run(x, dv.upload(synth.bf16_round(x0), 1), dv.upload(feats, 1), None, steps,
            step_hook=lambda k, xs, xa: states.append((xs.cpu().numpy().copy(), xa.float().cpu().numpy().copy())))
    torch.cuda.synchronize()
    states.append((x.cpu().numpy(), None))
    ts = O.time_grid(steps)
    for k in range(steps):
        xk, xa = states[k]
        assert np.array_equal(xa[0], synth.bf16_round(xk[0])) and np.array_equal(xa[1], xa[0])
        t = np.array([ts[k], ts[k]])
        v = O.dit_forward(top, blocks, xa, feats, t, ip, tp)
        ref = O.flow_step(xk[0], v[0], v[1], ts[k + 1] - ts[k], 5.0)
        assert_parity(states[k + 1][0][0], ref, f"x_{k + 1}")
        # the increment carries the whole step; CFG 5 amplifies velocity
        # rounding by up to 5 + 4, so it gets the bar derived for it
        assert_parity(states[k + 1][0][0] - xk[0], ref - xk[0], f"dx_{k}", rel=SAMPLER_DX_REL)


def test_sampler_rescaled_cfg_shifted_grid_teacher_forced():
    """Sampler with the norm-rescaled CFG step and the shifted grid (mu =
    1.06): each step against the oracle's rescaled combine of its own dit
    velocities at the GPU's bf16 input, on the oracle's shifted grid."""
    dv, top, blocks, feats, ip, tp, x0, smp = _small_sampler_setup(True, mu=1.06, norm_rescale=True)
    steps = 3
    states = []
    x = dv.upload(x0)
    smp.run(x, dv.upload(synth.bf16_round(x0), 1), dv.upload(feats, 1), None, steps,
            step_hook=lambda k, xs, xa: states.append((xs.cpu().numpy().copy(), xa.float().cpu().numpy().copy())))
    torch.cuda.synchronize()
    states.append((x.cpu().numpy(), None))
    ts = O.time_grid(steps, mu=1.06)
    for k in range(steps):
        xk, xa = states[k]
        t = np.array([ts[k], ts[k]])
        v = O.dit_forward(top, blocks, xa, feats, t, ip, tp)
        ref = O.flow_step_rescaled(xk[0], v[0], v[1], ts[k + 1] - ts[k], 5.0)
        assert_parity(states[k + 1][0][0], ref, f"x_{k + 1}")
        assert_parity(states[k + 1][0][0] - xk[0], ref - xk[0], f"dx_{k}", rel=SAMPLER_DX_REL)


def test_sampler_turbo_free_running():
    """Four Euler steps without CFG from the same N(0,1) latent: final x."""
    dv, top, blocks, feats, ip, tp, x0, smp = _small_sampler_setup(False)
    x = dv.upload(x0)
    smp.run(x, dv.upload(synth.bf16_round(x0), 1), dv.upload(feats, 1), None, 4)
    torch.cuda.synchronize()

    def vel(xs, t):
        return O.dit_forward(top, blocks, synth.bf16_round(xs.astype(np.float32)), feats, np.array([t]), ip, tp)

    ref = O.sample(vel, x0, 4)
    assert_parity(x.cpu().numpy(), ref, "x after 4 steps")


def test_empty_inputs_touch_nothing():
    """Zero tokens / rows: the entry points return LENS_OK and write nothing
    (buffers around them keep a sentinel)."""
    T, dv = _env()
    from text_image_flow_amd import _lib as L
    from text_image_flow_amd.device import ptr, stream_handle
    x = torch.full((64, 128), 7.0, dtype=torch.float32, device="cuda")
    v = torch.full((64, 128), 1.0, dtype=torch.float32, device="cuda")
    lowp = torch.full((64, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    L.check(L.lens_flow_step(ptr(x), ptr(v), ptr(v), 0, 0.5, 5.0, ptr(lowp), L.LENS_BF16, stream_handle(None)))
    L.check(L.lens_flow_step_rescaled(ptr(x), ptr(v), ptr(v), 0, 128, 0.5, 5.0, ptr(lowp), L.LENS_BF16,
                                      stream_handle(None)))
    q = torch.full((64, 128), 5, dtype=torch.uint8, device="cuda")
    s = torch.full((64, 4), 9, dtype=torch.uint8, device="cuda")
    for layout in (L.LENS_MX_ROWS, L.LENS_MX_SLABS):
        L.check(L.lens_quantize_mxfp8(ptr(lowp), L.LENS_BF16, 0, 128, layout, ptr(q), ptr(s), stream_handle(None)))
    torch.cuda.synchronize()
    assert bool((x == 7.0).all()) and bool((lowp.float() == 3.0).all())
    assert bool((q == 5).all()) and bool((s == 9).all())
    # empty tensors through the Python wrappers
    e = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    dv.flow_step(e, e, e, 0.5, 5.0)
    dv.flow_step_rescaled(e, e, e, 0.5, 5.0)
    q0, s0 = dv.quantize_mxfp8(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), layout=L.LENS_MX_ROWS)
    q1, s1 = dv.quantize_mxfp8(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert q0.shape == (0, 64) and s0.shape == (0, 2)
    assert q1.shape == (0, 256) and s1.shape == (2, 0, 4)
