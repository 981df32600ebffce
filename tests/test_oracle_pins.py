"""Pins of the fp64 oracle against facts that do not come from the oracle:
numbers the pages print, closed forms, invariants, textbook/library routines
and brute force on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lens_config.json")))
EPS = 1e-6


def g(name):
    return GOLD[name]["value"]


# ----------------------------------------------------------------- tiny model
TD = dict(D=16, H=2, d=8, axes=(2, 2, 4), mlp=16)


def tiny_stream(rs, mlp=TD["mlp"], D=TD["D"], d=TD["d"]):
    return {
        "mod_w": rs.standard_normal((6 * D, D)) * 0.3, "mod_b": rs.standard_normal(6 * D) * 0.3,
        "qkv_w": rs.standard_normal((3 * D, D)) * 0.3, "qkv_b": rs.standard_normal(3 * D) * 0.3,
        "out_w": rs.standard_normal((D, D)) * 0.3, "out_b": rs.standard_normal(D) * 0.3,
        "w1_w": rs.standard_normal((mlp, D)) * 0.3, "w1_b": rs.standard_normal(mlp) * 0.3,
        "w3_w": rs.standard_normal((mlp, D)) * 0.3, "w3_b": rs.standard_normal(mlp) * 0.3,
        "w2_w": rs.standard_normal((D, mlp)) * 0.3, "w2_b": rs.standard_normal(D) * 0.3,
        "q_gain": rs.uniform(0.5, 1.5, d), "k_gain": rs.uniform(0.5, 1.5, d),
    }


def tiny_block(seed=0):
    rs = np.random.default_rng(seed)
    return {"img": tiny_stream(rs), "txt": tiny_stream(rs)}


def tiny_inputs(B=2, gh=3, gw=4, St=5, seed=1):
    rs = np.random.default_rng(seed)
    Si = gh * gw
    return (rs.standard_normal((B, Si, TD["D"])), rs.standard_normal((B, St, TD["D"])),
            rs.standard_normal((B, TD["D"])), synth.image_positions(gh, gw), synth.text_positions(St))


def run_block(w, hi, ht, temb, ip, tp, tl=None, **kw):
    return O.block_forward(w, hi, ht, temb, ip, tp, tl, heads=TD["H"], axes=TD["axes"], eps=EPS, **kw)


def set_mod(ws, **chunks):
    """Zero the AdaLN weight and put constant chunks into its bias."""
    D = ws["out_w"].shape[0]
    ws["mod_w"] = np.zeros_like(ws["mod_w"])
    b = np.zeros(6 * D)
    order = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    for k, v in chunks.items():
        i = order.index(k)
        b[i * D:(i + 1) * D] = v
    ws["mod_b"] = b


# ------------------------------------------------------- pages' numbers (pins)
def test_config_constants_from_pages():
    d = synth.LENS
    assert d.n_blocks == g("n_blocks") and d.hidden == g("hidden") and d.heads == g("heads")
    assert d.head_dim == g("head_dim") and d.heads * d.head_dim == d.hidden
    assert list(d.rope_axes) == g("rope_axes") and sum(d.rope_axes) == d.head_dim
    assert d.mlp == g("mlp_hidden") and 6 * d.hidden == g("adaln_out")
    assert d.in_ch == g("in_channels") == g("patch_size") ** 2 * g("latent_channels")
    assert d.txt_feat == g("enc_hidden_dim") and d.txt_layers == g("txt_layers")


def test_parameter_count_matches_pages():
    shapes = synth.stream_tensor_shapes()
    per_stream = O.stream_param_count(shapes)
    assert per_stream == 42_467_328
    n = lambda k: int(np.prod(shapes[k]))
    # the blog's components: 4 x 1536^2 ~ 9.43M; 3 x 1536x4096 ~ 18.8M; 1536x9216 ~ 14.1M
    assert abs((n("qkv_w") + n("out_w")) / 1e6 - g("attn_params_per_stream_M")) < 0.01
    assert abs((n("w1_w") + n("w3_w") + n("w2_w")) / 1e6 - g("mlp_params_per_stream_M")) < 0.1
    assert abs(n("mod_w") / 1e6 - g("adaln_params_per_stream_M")) < 0.1
    # the blog rounds each component before summing (9.43 + 18.8 + 14.1)
    assert abs(per_stream / 1e6 - g("params_per_stream_M")) < 0.25
    assert abs(2 * per_stream / 1e6 - g("params_per_block_M")) < 0.5
    top = sum(int(np.prod(s)) for k, s in synth.top_tensor_shapes().items() if k.endswith("_w"))
    total_blocks = 48 * 2 * per_stream
    # bf16 checkpoint ~ 8.2 GB
    assert abs((total_blocks + top) * 2 / 1e9 - g("dit_bytes_bf16_GB")) < 0.05
    # int4 group-64 (a 16-bit scale and 16-bit bias per group) for block weights,
    # the listed sensitive layers in bf16: ~ 2.35 GB.  A modulation network
    # shared across blocks would give ~2.0 GB instead.
    int4 = total_blocks * (0.5 + 4 / 64) + top * 2
    assert abs(int4 / 1e9 - g("dit_bytes_int4_g64_GB")) < 0.02


# ---------------------------------------------------------------- primitives
def test_linear_triple_loop():
    rs = np.random.default_rng(0)
    x, w, b = rs.standard_normal((3, 5)), rs.standard_normal((4, 5)), rs.standard_normal(4)
    y = O.linear(x, w, b)
    for i in range(3):
        for j in range(4):
            assert y[i, j] == pytest.approx(sum(x[i, k] * w[j, k] for k in range(5)) + b[j], abs=1e-12)


def test_silu_library():
    x = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(O.silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)


def test_rms_norm_unit_rms_and_closed_forms():
    rs = np.random.default_rng(0)
    x = rs.standard_normal((7, 64)) * 5
    y = O.rms_norm(x, EPS)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, atol=1e-6)
    np.testing.assert_allclose(O.rms_norm(3 * x, EPS), y, atol=1e-7)   # scale invariance
    c = 0.01
    np.testing.assert_allclose(O.rms_norm(np.full((1, 8), c), EPS), c / math.sqrt(c * c + EPS), rtol=1e-14)
    gain = rs.uniform(0.5, 1.5, 64)
    np.testing.assert_allclose(O.rms_norm(x, EPS, gain), y * gain, rtol=1e-14)
    assert np.all(O.rms_norm(np.zeros((2, 8)), EPS) == 0)


def test_modulate_special_cases():
    rs = np.random.default_rng(0)
    xn, sh = rs.standard_normal((2, 3, 8)), rs.standard_normal((2, 8))
    np.testing.assert_allclose(O.modulate(xn, sh, -np.ones((2, 8))), np.broadcast_to(sh[:, None], (2, 3, 8)))
    np.testing.assert_allclose(O.modulate(xn, np.zeros((2, 8)), np.zeros((2, 8))), xn)
    np.testing.assert_allclose(O.modulate(xn, np.zeros((2, 8)), np.ones((2, 8))), 2 * xn)


def test_adaln_chunk_order_from_blog():
    D = 4
    w = np.zeros((6 * D, D))
    b = np.repeat(np.arange(6.0), D)
    m = O.adaln(np.ones((1, D)), w, b)
    for i, k in enumerate(("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")):
        assert np.all(m[k] == i)
    # SiLU applied to temb before the Linear
    w = np.zeros((6 * D, D)); w[0, 0] = 1.0
    m = O.adaln(np.array([[2.0, 0, 0, 0]]), w, np.zeros(6 * D))
    assert m["shift1"][0, 0] == pytest.approx(2.0 * scipy.special.expit(2.0), rel=1e-14)


# ---------------------------------------------------------------------- RoPE
AX = (8, 28, 28)


def test_rope_preserves_norms_and_zero_is_identity():
    rs = np.random.default_rng(0)
    x = rs.standard_normal((10, 3, 64))
    pos = rs.integers(0, 90, (10, 3))
    y = O.rope(x, pos, AX, 1e4)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(O.rope(x, np.zeros((10, 3), int), AX, 1e4), x)


def test_rope_relative_position_property():
    rs = np.random.default_rng(1)
    q, k = rs.standard_normal((1, 1, 64)), rs.standard_normal((1, 1, 64))
    p, p2 = np.array([[3, 17, 41]]), np.array([[5, 2, 60]])
    lhs = np.sum(O.rope(q, p, AX, 1e4) * O.rope(k, p2, AX, 1e4))
    rhs = np.sum(q * O.rope(k, p2 - p, AX, 1e4))
    assert lhs == pytest.approx(rhs, rel=1e-11)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_single_axis_is_textbook_1d_rope(axis):
    """With one non-zero axis, the rotation equals multiplying the complex
    pairs of that axis' segment by exp(i p theta^(-2j/d_a)); others untouched."""
    rs = np.random.default_rng(axis)
    x = rs.standard_normal((4, 2, 64))
    p = rs.integers(1, 100, 4)
    pos = np.zeros((4, 3), int)
    pos[:, axis] = p
    y = O.rope(x, pos, AX, 1e4)
    lo = sum(AX[:axis]); da = AX[axis]
    z = x[..., lo:lo + da:2] + 1j * x[..., lo + 1:lo + da:2]
    w = np.power(1e4, -np.arange(0, da, 2) / da)
    zr = z * np.exp(1j * p[:, None, None] * w[None, None, :])
    np.testing.assert_allclose(y[..., lo:lo + da:2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[..., lo + 1:lo + da:2], zr.imag, atol=1e-12)
    mask = np.ones(64, bool); mask[lo:lo + da] = False
    np.testing.assert_array_equal(y[..., mask], x[..., mask])


def test_rope_angle_table_values():
    ang = O.rope_angles(np.array([[2, 3, 5]]), AX, 1e4)[0]
    assert ang.shape == (32,)
    assert ang[0] == 2 and ang[4] == 3 and ang[18] == 5          # first pair of each axis: omega = 1
    assert ang[3] == pytest.approx(2 * 1e4 ** (-6 / 8))
    assert ang[17] == pytest.approx(3 * 1e4 ** (-26 / 28))
    assert ang[31] == pytest.approx(5 * 1e4 ** (-26 / 28))


# ----------------------------------------------------------------- attention
def test_attention_brute_force_tiny():
    rs = np.random.default_rng(0)
    q, k, v = rs.standard_normal((3, 2, 4)), rs.standard_normal((5, 2, 4)), rs.standard_normal((5, 2, 4))
    valid = np.array([1, 0, 1, 1, 0], bool)
    o = O.attention(q, k, v, valid)
    for h in range(2):
        for i in range(3):
            e = [math.exp(sum(q[i, h, t] * k[j, h, t] for t in range(4)) / 2.0) if valid[j] else 0.0 for j in range(5)]
            z = sum(e)
            for t in range(4):
                assert o[i, h, t] == pytest.approx(sum(e[j] * v[j, h, t] for j in range(5)) / z, abs=1e-12)


def test_attention_scipy_softmax_and_rows_sum_to_one():
    rs = np.random.default_rng(1)
    q, k, v = rs.standard_normal((6, 3, 64)) * 3, rs.standard_normal((9, 3, 64)) * 3, rs.standard_normal((9, 3, 64))
    o, p = O.attention(q, k, v, return_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-13)
    for h in range(3):
        ref = scipy.special.softmax(q[:, h] @ k[:, h].T / 8.0, axis=1) @ v[:, h]
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)


def test_attention_identical_keys_mean_v_and_mask_zero():
    rs = np.random.default_rng(2)
    q = rs.standard_normal((4, 1, 8))
    k = np.repeat(rs.standard_normal((1, 1, 8)), 6, 0)
    v = rs.standard_normal((6, 1, 8))
    np.testing.assert_allclose(O.attention(q, k, v)[:, 0], np.broadcast_to(v[:, 0].mean(0), (4, 8)), atol=1e-13)
    valid = np.array([1, 1, 0, 1, 0, 0], bool)
    o, p = O.attention(q, rs.standard_normal((6, 1, 8)), v, valid, return_probs=True)
    assert np.all(p[..., ~valid] == 0)


# ------------------------------------------------------------------- SwiGLU
def test_swiglu_closed_form():
    D = 5
    a = np.linspace(-2, 2, D)[None]
    I = np.eye(D)
    y = O.swiglu_mlp(a, I, None, 2 * I, None, I, None)
    np.testing.assert_allclose(y, a * scipy.special.expit(a) * 2 * a, rtol=1e-14)
    rs = np.random.default_rng(0)
    b2 = rs.standard_normal(D)
    y = O.swiglu_mlp(rs.standard_normal((3, D)), rs.standard_normal((7, D)), None,
                     rs.standard_normal((7, D)), None, np.zeros((D, 7)), b2)
    np.testing.assert_allclose(y, np.broadcast_to(b2, (3, D)))


# --------------------------------------------------------------------- block
def test_block_adaln_zero_is_identity():
    w = tiny_block()
    for s in ("img", "txt"):
        set_mod(w[s])
    hi, ht, temb, ip, tp = tiny_inputs()
    oi, ot = run_block(w, hi, ht, temb, ip, tp, np.array([5, 2]))
    np.testing.assert_array_equal(oi, hi)
    np.testing.assert_array_equal(ot, ht)


def test_block_mlp_branch_closed_form():
    """scale2 = -1 makes the MLP input shift2 for every token; W1 = I,
    W3 = 2I, W2 = I give out = silu(c) * 2c; gate1 = 0 switches attention off."""
    w = tiny_block()
    D = TD["D"]
    rs = np.random.default_rng(5)
    res = {}
    for s in ("img", "txt"):
        c, gt = rs.standard_normal(D), rs.standard_normal(D)
        set_mod(w[s], shift1=rs.standard_normal(D), scale1=rs.standard_normal(D), scale2=-1.0, shift2=c, gate2=gt)
        w[s].update(w1_w=np.eye(D), w1_b=None, w3_w=2 * np.eye(D), w3_b=None, w2_w=np.eye(D), w2_b=None)
        res[s] = gt * (c * scipy.special.expit(c) * 2 * c)
    hi, ht, temb, ip, tp = tiny_inputs()
    oi, ot = run_block(w, hi, ht, temb, ip, tp)
    np.testing.assert_allclose(oi - hi, np.broadcast_to(res["img"], oi.shape), atol=1e-12)
    np.testing.assert_allclose(ot - ht, np.broadcast_to(res["txt"], ot.shape), atol=1e-12)


def test_block_attention_branch_value_path_closed_form():
    """scale1 = -1 makes every token of a stream the same vector c, so all
    values of the stream are W_v c + b_v; with both streams equal the joint
    attention output is that vector whatever the scores, and with W_o = I the
    attention branch adds gate1 * (W_v c + b_v + b_o)."""
    w = tiny_block()
    D = TD["D"]
    rs = np.random.default_rng(6)
    c, g1 = rs.standard_normal(D), rs.standard_normal(D)
    for s in ("img", "txt"):
        set_mod(w[s], scale1=-1.0, shift1=c, gate1=g1)
        w[s]["out_w"] = np.eye(D)
    w["txt"]["qkv_w"][2 * D:] = w["img"]["qkv_w"][2 * D:]
    w["txt"]["qkv_b"][2 * D:] = w["img"]["qkv_b"][2 * D:]
    hi, ht, temb, ip, tp = tiny_inputs()
    v = w["img"]["qkv_w"][2 * D:] @ c + w["img"]["qkv_b"][2 * D:]
    oi, ot = run_block(w, hi, ht, temb, ip, tp, np.array([5, 1]))
    np.testing.assert_allclose(oi - hi, np.broadcast_to(g1 * (v + w["img"]["out_b"]), oi.shape), atol=1e-12)
    np.testing.assert_allclose(ot - ht, np.broadcast_to(g1 * (v + w["txt"]["out_b"]), ot.shape), atol=1e-12)


def test_block_uniform_attention_is_mean_over_valid_joint_tokens():
    """q = k = 0 gives uniform attention over the sample's valid keys (all
    image tokens and the first txt_len text tokens); with W_v = I and W_o = I
    every query receives the mean of the valid tokens' normalised inputs."""
    w = tiny_block()
    D = TD["D"]
    rs = np.random.default_rng(7)
    g1 = rs.standard_normal(D)
    for s in ("img", "txt"):
        set_mod(w[s], gate1=g1)
        w[s]["qkv_w"] = np.concatenate([np.zeros((2 * D, D)), np.eye(D)])
        w[s]["qkv_b"] = np.zeros(3 * D)
        w[s]["out_w"], w[s]["out_b"] = np.eye(D), np.zeros(D)
    hi, ht, temb, ip, tp = tiny_inputs(B=3)
    tl = np.array([5, 0, 3])
    oi, ot = run_block(w, hi, ht, temb, ip, tp, tl)
    for b in range(3):
        toks = np.concatenate([ht[b, :tl[b]], hi[b]])
        m = O.rms_norm(toks, EPS).mean(0)
        np.testing.assert_allclose(oi[b] - hi[b], np.broadcast_to(g1 * m, hi[b].shape), atol=1e-12)
        np.testing.assert_allclose(ot[b] - ht[b], np.broadcast_to(g1 * m, ht[b].shape), atol=1e-12)


def test_block_no_text_reduces_to_single_stream_self_attention():
    """S_txt = 0: the image stream alone, written here as a single-stream
    block with scipy's softmax and numpy's complex rotation for RoPE."""
    w = tiny_block(3)
    hi, _, temb, ip, _ = tiny_inputs(B=2)
    ht = np.zeros((2, 0, TD["D"]))
    oi, ot = run_block(w, hi, ht, temb, ip, np.zeros((0, 3), int))
    assert ot.shape == (2, 0, TD["D"])
    ws, D, H, d = w["img"], TD["D"], TD["H"], TD["d"]
    for b in range(2):
        m = ws["mod_w"] @ (temb[b] * scipy.special.expit(temb[b])) + ws["mod_b"]
        sh1, sc1, g1, sh2, sc2, g2 = np.split(m, 6)
        nrm = lambda x: x / np.sqrt((x ** 2).mean(-1, keepdims=True) + EPS)
        a = nrm(hi[b]) * (1 + sc1) + sh1
        qkv = a @ ws["qkv_w"].T + ws["qkv_b"]
        q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, d) for i in range(3))
        q, k = nrm(q) * ws["q_gain"], nrm(k) * ws["k_gain"]
        ang = np.concatenate([ip[:, [a_]] * np.power(1e4, -np.arange(0, n, 2) / n)
                              for a_, n in enumerate(TD["axes"])], 1)
        rot = lambda x: (lambda z: np.stack([z.real, z.imag], -1).reshape(x.shape))(
            (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)[:, None, :])
        q, k = rot(q), rot(k)
        o = np.concatenate([scipy.special.softmax(q[:, h] @ k[:, h].T / math.sqrt(d), 1) @ v[:, h]
                            for h in range(H)], 1)
        h1 = hi[b] + g1 * (o @ ws["out_w"].T + ws["out_b"])
        a2 = nrm(h1) * (1 + sc2) + sh2
        f = (a2 @ ws["w1_w"].T + ws["w1_b"])
        mlp = (f * scipy.special.expit(f) * (a2 @ ws["w3_w"].T + ws["w3_b"])) @ ws["w2_w"].T + ws["w2_b"]
        np.testing.assert_allclose(oi[b], h1 + g2 * mlp, atol=1e-11)


def test_block_padding_invariance():
    """Masked text keys act exactly like text that was never there."""
    w = tiny_block(4)
    hi, ht, temb, ip, tp = tiny_inputs(B=2, St=7)
    tl = np.array([4, 6])
    oi, ot = run_block(w, hi, ht, temb, ip, tp, tl)
    for b in range(2):
        n = tl[b]
        ri, rt = run_block(w, hi[b:b + 1], ht[b:b + 1, :n], temb[b:b + 1], ip, tp[:n])
        np.testing.assert_allclose(oi[b], ri[0], atol=1e-12)
        np.testing.assert_allclose(ot[b, :n], rt[0], atol=1e-12)


def test_block_permutation_equivariance_and_batch_independence():
    w = tiny_block(5)
    hi, ht, temb, ip, tp = tiny_inputs(B=2)
    oi, ot = run_block(w, hi, ht, temb, ip, tp)
    perm = np.random.default_rng(0).permutation(hi.shape[1])
    pi, pt = run_block(w, hi[:, perm], ht, temb, ip[perm], tp)
    np.testing.assert_allclose(pi, oi[:, perm], atol=1e-12)
    np.testing.assert_allclose(pt, ot, atol=1e-12)
    hi2 = hi.copy(); hi2[1] += 3.0
    qi, qt = run_block(w, hi2, ht, temb, ip, tp)
    np.testing.assert_allclose(qi[0], oi[0], atol=1e-12)
    np.testing.assert_allclose(qt[0], ot[0], atol=1e-12)


def test_block_sampled_rows_match_full():
    w = tiny_block(6)
    hi, ht, temb, ip, tp = tiny_inputs(B=2, St=6)
    tl = np.array([6, 3])
    oi, ot = run_block(w, hi, ht, temb, ip, tp, tl)
    ri, rt = np.array([0, 5, 11]), np.array([1, 2])
    si, st = run_block(w, hi, ht, temb, ip, tp, tl, rows=(ri, rt))
    np.testing.assert_allclose(si, oi[:, ri], atol=1e-12)
    np.testing.assert_allclose(st, ot[:, rt], atol=1e-12)


# --------------------------------------------------------- embeddings, DiT
def test_timestep_features_values():
    phi = O.timestep_features(np.array([0.0, 0.25]))
    np.testing.assert_array_equal(phi[0], np.r_[np.ones(128), np.zeros(128)])
    assert phi[1, 0] == pytest.approx(math.cos(250.0)) and phi[1, 128] == pytest.approx(math.sin(250.0))
    assert phi[1, 64] == pytest.approx(math.cos(2.5)) and phi[1, 192] == pytest.approx(math.sin(2.5))


def test_timestep_embedding_mlp_closed_form():
    D = 256
    top = {"t_fc1_w": np.eye(D), "t_fc1_b": None, "t_fc2_w": 3 * np.eye(D), "t_fc2_b": np.ones(D)}
    t = np.array([0.3])
    phi = O.timestep_features(t)
    np.testing.assert_allclose(O.timestep_embedding(top, t), 3 * phi * scipy.special.expit(phi) + 1, rtol=1e-14)


def test_text_embed_normalises_each_layer_separately():
    rs = np.random.default_rng(0)
    L, F, D = 4, 6, 5
    top = {"txt_gain": rs.uniform(0.5, 1.5, (L, F)), "txt_in_w": rs.standard_normal((D, L * F)),
           "txt_in_b": rs.standard_normal(D)}
    f = rs.standard_normal((2, 3, L * F))
    y = O.text_embed(top, f, layers=L)
    f2 = f.copy(); f2[..., F:2 * F] *= 7.0           # rescale one layer only (invariant up to eps)
    np.testing.assert_allclose(O.text_embed(top, f2, layers=L), y, rtol=1e-4, atol=1e-4)
    f3 = f.copy(); f3[..., :F] *= 7.0; f3[..., F:] *= 0.5   # not invariant if normalised jointly
    assert np.max(np.abs(O.text_embed(top, f3, layers=L) - y)) < 1e-4
    # identity projection exposes the per-layer normalised, gained features in layer order
    top2 = dict(top, txt_in_w=np.eye(L * F), txt_in_b=None)
    z = O.text_embed(top2, f, layers=L)
    for l in range(L):
        seg = z[..., l * F:(l + 1) * F] / top["txt_gain"][l]
        np.testing.assert_allclose(np.sqrt((seg ** 2).mean(-1)), 1.0, atol=1e-5)


def test_final_layer_scale_minus_one_gives_projected_shift():
    D, C = 6, 4
    rs = np.random.default_rng(1)
    sh = rs.standard_normal(D)
    top = {"norm_out_w": np.zeros((2 * D, D)), "norm_out_b": np.r_[sh, -np.ones(D)],
           "proj_out_w": rs.standard_normal((C, D)), "proj_out_b": rs.standard_normal(C)}
    v = O.final_layer(top, rs.standard_normal((2, 3, D)), rs.standard_normal((2, D)))
    np.testing.assert_allclose(v, np.broadcast_to(top["proj_out_w"] @ sh + top["proj_out_b"], (2, 3, C)), atol=1e-13)


def test_dit_with_identity_blocks_is_embed_then_final_layer():
    rs = np.random.default_rng(2)
    D = TD["D"]
    top = {"t_fc1_w": rs.standard_normal((D, 8)), "t_fc1_b": rs.standard_normal(D),
           "t_fc2_w": rs.standard_normal((D, D)), "t_fc2_b": rs.standard_normal(D),
           "img_in_w": rs.standard_normal((D, 4)), "img_in_b": rs.standard_normal(D),
           "txt_gain": rs.uniform(0.5, 1.5, (2, 3)), "txt_in_w": rs.standard_normal((D, 6)),
           "txt_in_b": rs.standard_normal(D), "norm_out_w": rs.standard_normal((2 * D, D)),
           "norm_out_b": rs.standard_normal(2 * D), "proj_out_w": rs.standard_normal((4, D)),
           "proj_out_b": rs.standard_normal(4)}
    blocks = [tiny_block(i) for i in range(2)]
    for wb in blocks:
        for s in ("img", "txt"):
            set_mod(wb[s])
    x, f, t = rs.standard_normal((2, 12, 4)), rs.standard_normal((2, 5, 6)), np.array([0.9, 0.4])
    kw = dict(heads=TD["H"], axes=TD["axes"], t_freq=8, txt_layers=2)
    v = O.dit_forward(top, blocks, x, f, t, synth.image_positions(3, 4), synth.text_positions(5), **kw)
    temb = O.timestep_embedding(top, t, t_freq=8)
    np.testing.assert_allclose(v, O.final_layer(top, O.linear(x, top["img_in_w"], top["img_in_b"]), temb), atol=1e-12)


# ------------------------------------------------------------ CFG, sampler
def test_cfg_special_cases():
    rs = np.random.default_rng(0)
    c, u = rs.standard_normal(50), rs.standard_normal(50)
    np.testing.assert_allclose(O.cfg_combine(c, u, 1.0), c, rtol=0, atol=1e-15)   # exact up to rounding
    np.testing.assert_array_equal(O.cfg_combine(c, u, 0.0), u)
    a, b = O.cfg_combine(c, u, 2.0), O.cfg_combine(c, u, 5.0)
    np.testing.assert_allclose(O.cfg_combine(c, u, 3.5), 0.5 * (a + b), atol=1e-12)   # affine in s


def test_euler_constant_velocity_closed_form():
    rs = np.random.default_rng(1)
    x0, v = rs.standard_normal(40), rs.standard_normal(40)
    for steps in (1, 4, 20, 50):
        ts = O.time_grid(steps)
        assert ts[0] == 1.0 and ts[-1] == 0.0 and np.allclose(np.diff(ts), -1.0 / steps)
        x = O.sample(lambda x, t: v, x0, steps)
        np.testing.assert_allclose(x, x0 - v, atol=1e-13)


def test_euler_linear_path_is_exact():
    """On the straight path x_t = (1-t) x0 + t x1 the velocity x1 - x0 is
    constant, so Euler from x1 at t = 1 lands on x0 at t = 0 in any number
    of steps; with CFG on two such fields the end point is the guided mix."""
    rs = np.random.default_rng(2)
    x0c, x0u, x1 = rs.standard_normal(30), rs.standard_normal(30), rs.standard_normal(30)
    x = O.sample(lambda x, t: (x1 - x0c, x1 - x0u), x1, 7, scale=5.0, use_uncond=True)
    np.testing.assert_allclose(x, x0u + 5.0 * (x0c - x0u), atol=1e-12)


# ------------------------------------------------------------ norm-rescaled CFG
def test_rescaled_cfg_worked_example():
    """c = (3, 4), u = 0, s = 2: comb = (6, 8) with norm 10, rescaled to the
    conditional norm 5 -> (3, 4); a second token with u = c stays c."""
    c = np.array([[3.0, 4.0], [1.0, -2.0]])
    u = np.array([[0.0, 0.0], [1.0, -2.0]])
    np.testing.assert_allclose(O.cfg_combine_rescaled(c, u, 2.0), [[3.0, 4.0], [1.0, -2.0]], atol=1e-15)
    # direction comes from the combination, length from c
    c2 = np.array([[1.0, 0.0]])
    u2 = np.array([[0.0, 1.0]])
    out = O.cfg_combine_rescaled(c2, u2, 3.0)          # comb = (3, -2)
    np.testing.assert_allclose(out, np.array([[3.0, -2.0]]) / math.sqrt(13.0), atol=1e-15)


def test_rescaled_cfg_properties():
    rs = np.random.default_rng(3)
    c, u = rs.standard_normal((5, 7, 128)), rs.standard_normal((5, 7, 128))
    # s = 1: comb = c (up to rounding), so the rescale factor is 1
    np.testing.assert_allclose(O.cfg_combine_rescaled(c, u, 1.0), c, atol=1e-13)
    for s in (0.0, 2.5, 5.0):
        out = O.cfg_combine_rescaled(c, u, s)
        # per-token norm equals the conditional norm
        np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(c, axis=-1), rtol=1e-12)
        # per-token direction equals the plain guided direction
        comb = O.cfg_combine(c, u, s)
        cosv = np.sum(out * comb, -1) / (np.linalg.norm(out, axis=-1) * np.linalg.norm(comb, axis=-1))
        np.testing.assert_allclose(cosv, 1.0, atol=1e-12)
    # no uncond: identity
    np.testing.assert_array_equal(O.cfg_combine_rescaled(c, None, 5.0), c)


def test_rescaled_cfg_zero_norm_token_and_euler():
    c = np.array([[1.0, 1.0], [2.0, 0.0]])
    u = np.array([[1.25, 1.25], [0.0, 0.0]])
    # token 0: s = 5 gives comb = 1.25 + 5 (1 - 1.25) = 0 exactly -> kept at 0
    out = O.cfg_combine_rescaled(c, u, 5.0)
    np.testing.assert_array_equal(out[0], [0.0, 0.0])
    np.testing.assert_allclose(out[1], [2.0, 0.0], atol=1e-15)   # comb = (10, 0) rescaled to norm 2
    x = np.array([[0.5, -0.5], [1.0, 1.0]])
    np.testing.assert_allclose(O.flow_step_rescaled(x, c, u, -0.25, 5.0), x - 0.25 * out, atol=1e-15)


# ------------------------------------------------------------ timestep shift
def test_time_shift_is_a_logit_translation():
    t = np.linspace(0.0, 1.0, 41)[1:-1]
    for mu in (-0.7, 0.5, 1.06, 2.0):
        ts = O.time_shift(t, mu)
        np.testing.assert_allclose(scipy.special.logit(ts), scipy.special.logit(t) + mu, atol=1e-12)
        assert np.all(np.diff(ts) > 0)                                      # order kept
        np.testing.assert_allclose(O.time_shift(ts, -mu), t, atol=1e-14)    # -mu undoes mu
    np.testing.assert_array_equal(O.time_shift(np.array([0.0, 1.0]), 1.06), [0.0, 1.0])
    np.testing.assert_allclose(O.time_shift(t, 0.0), t, rtol=0, atol=1e-15)   # identity up to rounding
    assert abs(O.time_shift(0.5, 1.06) - scipy.special.expit(1.06)) < 1e-15


def test_shifted_grid_and_mu_line():
    ts = O.time_grid(20, mu=1.06)
    assert ts[0] == 1.0 and ts[-1] == 0.0 and np.all(np.diff(ts) < 0)
    np.testing.assert_allclose(ts, O.time_shift(O.time_grid(20), 1.06), rtol=0, atol=0)
    # a positive shift spends more of the steps at high noise
    assert np.all(ts[1:-1] > O.time_grid(20)[1:-1])
    assert O.mu_for_tokens(1024, 1024, 1.06, 4096, 1.5) == 1.06
    assert abs(O.mu_for_tokens(4096, 1024, 1.06, 4096, 1.5) - 1.5) < 1e-15
    assert abs(O.mu_for_tokens(2560, 1024, 1.06, 4096, 1.5) - 1.28) < 1e-12


# ------------------------------------------------------------ MX fp8 (e4m3)
def _e4m3_decode(code):
    """OCP e4m3 (fn) decode from its bit fields: sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 is subnormal; 0x7f / 0xff are NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_grid_is_fixed_and_ties_go_to_even():
    pos = np.array([_e4m3_decode(c) for c in range(1, 0x7F)])          # all positive finite codes
    assert len(set(pos)) == 126 and pos.max() == 448.0 and pos.min() == 2.0 ** -9
    assert np.all(np.diff(pos) > 0)
    grid = np.concatenate([-pos[::-1], [0.0], pos])
    np.testing.assert_array_equal(O.round_e4m3(grid), grid)
    # midpoints go to the neighbour whose code is even (mantissa LSB 0)
    codes = np.arange(1, 0x7E)
    mid = 0.5 * (pos[:-1] + pos[1:])
    want = np.where(codes % 2 == 0, pos[:-1], pos[1:])
    np.testing.assert_array_equal(O.round_e4m3(mid), want)
    np.testing.assert_array_equal(O.round_e4m3(-mid), -want)
    # just off the midpoints: the nearer neighbour
    np.testing.assert_array_equal(O.round_e4m3(mid * (1 - 1e-9)), pos[:-1])
    np.testing.assert_array_equal(O.round_e4m3(mid * (1 + 1e-9)), pos[1:])
    assert O.round_e4m3(2.0 ** -10) == 0.0 and O.round_e4m3(2.0 ** -10 * 1.0001) == 2.0 ** -9


def test_mx_scale_exponent_closed_form():
    for k in (-100, -9, -1, 0, 1, 7, 100):
        assert O.mx_scale_exponent(448.0 * 2.0 ** k) == k
        assert O.mx_scale_exponent(448.0 * 2.0 ** k * (1 + 2e-16 * 8)) == k + 1
        assert O.mx_scale_exponent(448.0 * 2.0 ** (k - 1) * (1 + 1e-12)) == k
    assert O.mx_scale_exponent(0.0) == -127
    assert O.mx_scale_exponent(1e-60) == -127 and O.mx_scale_exponent(1e60) == 127


def test_mx_quantize_bounds_and_idempotence():
    rs = np.random.default_rng(5)
    x = rs.standard_normal((6, 128)) * np.exp(rs.uniform(-8, 8, (6, 1)))
    x[0, :32] = 0.0                                       # an all-zero block
    x[1, 5] = 1e4                                         # an outlier block
    q, e = O.mx_quantize(x)
    assert e.shape == (6, 4) and e[0, 0] == -127 and np.all(q[0, :32] == 0)
    np.testing.assert_array_equal(O.round_e4m3(q), q)                 # on the grid
    assert np.all(np.abs(q) <= 448.0)
    blockmax = np.abs(x).reshape(6, 4, 32).max(-1) / 2.0 ** e
    assert np.all(((blockmax > 224.0) & (blockmax <= 448.0)) | (e == -127))   # the tightest scale
    dq = O.mx_dequantize(q, e)
    # error: half a step of the element's binade (relative 2^-4), or half a
    # subnormal step
    scale = 2.0 ** np.repeat(e, 32, axis=1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 0.5 * 2.0 ** -9 * scale)
    assert np.all(np.abs(dq - x) <= bound * (1 + 1e-12))
    np.testing.assert_array_equal(O.mx_roundtrip(dq), dq)            # idempotent


def test_block_fp8_variant_reduces_to_quantized_operands():
    """With gemm_fp8 the block equals the plain block run on weights and
    activations that are already MX-quantized where the projections read
    them: quantizing the weights beforehand changes nothing (the roundtrip
    is idempotent), and the output stays close to the exact block."""
    rs = np.random.default_rng(7)
    D, H, F = 128, 2, 256
    def stream(seed):
        g = np.random.default_rng(seed)
        n = lambda *s: g.standard_normal(s) * 0.05
        return {"mod_w": n(6 * D, D), "mod_b": n(6 * D), "qkv_w": n(3 * D, D), "qkv_b": n(3 * D),
                "out_w": n(D, D), "out_b": n(D), "w1_w": n(F, D), "w1_b": n(F), "w3_w": n(F, D), "w3_b": n(F),
                "w2_w": n(D, F), "w2_b": n(D), "q_gain": 1 + n(64), "k_gain": 1 + n(64)}
    w = {"img": stream(1), "txt": stream(2)}
    hi, ht, temb = rs.standard_normal((1, 12, D)), rs.standard_normal((1, 5, D)), rs.standard_normal((1, D))
    ip = np.stack([np.zeros(12, int), np.arange(12) // 4, np.arange(12) % 4], 1)
    tp = np.zeros((5, 3), int)
    kw = dict(heads=H, axes=(8, 28, 28))
    a8 = O.block_forward(w, hi, ht, temb, ip, tp, gemm_fp8=True, **kw)
    wq = {s: {k: (O.mx_roundtrip(v) if k in ("qkv_w", "out_w", "w1_w", "w3_w", "w2_w") else v)
              for k, v in w[s].items()} for s in w}
    b8 = O.block_forward(wq, hi, ht, temb, ip, tp, gemm_fp8=True, **kw)
    for x, y in zip(a8, b8):
        np.testing.assert_array_equal(x, y)
    ex = O.block_forward(w, hi, ht, temb, ip, tp, **kw)
    for x, y, h in zip(a8, ex, (hi, ht)):
        dx, dy = (x - h).ravel(), (y - h).ravel()
        assert dx @ dy / np.linalg.norm(dx) / np.linalg.norm(dy) > 0.998     # block update direction kept
        assert not np.array_equal(x, y)                                        # and it is a different path
