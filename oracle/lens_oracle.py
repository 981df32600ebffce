"""Plain, slow, fp64 reference of the Lens double-stream MM-DiT denoiser, its
embeddings, and the flow-matching Euler sampler with classifier-free guidance.

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the HIP library, with which
it shares no code.  Inputs are whatever float32 arrays the caller holds (for
bf16 runs, the bf16-rounded values the GPU receives); everything here is
computed in float64, step by step, in the order the definition states, with
an explicit S x S score matrix per head.

Sources (pages on Lens; cited by page and section):
  [blog]   Lens blog post (zjwfufu.github.io), sections "Overview",
           "Exploring Text Encoder", "Exploring Image Editing".
  [paper]  Chinese summary of "Lens: Rethinking Training Efficiency for
           Foundational Text-to-Image Models", sections 前置知识 (MMDiT; Flow
           Matching training objective) and 方法步骤详情.
  [turbo]  Lens-Turbo-3.8B-bf16 article (wmrh.cn): architecture table,
           "双流注意力机制", "自适应调制与 RMSNorm", "3D RoPE",
           "多层级文本特征融合", "Patchify 补丁化与输出投影", "guidance 1.0".
  [4bit]   Lens-3.8B-4bit pipeline article (2kiu.com), section 4.
  [survey] SOTA image generation survey (youngju.dev), sections on text
           conditioning (joint attention), CFG, and rectified flow.

Where the pages leave a step open, the plainest reading is taken; each such
reading is marked READING below.  Parity against the real Lens weights is
unpinned: the pages print no tensors.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f(x):
    return np.asarray(x, dtype=F64)


# --------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------

def linear(x, w, b=None):
    """y = x W^T + b, W stored [out, in] (the per-stream Linear layers named
    in [turbo] "双流注意力机制" / "自适应调制与 RMSNorm")."""
    y = _f(x) @ _f(w).T
    if b is not None:
        y = y + _f(b)
    return y


def silu(x):
    x = _f(x)
    return x / (1.0 + np.exp(-x))


def rms_norm(x, eps, gain=None):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) (* gain).
    [turbo] "自适应调制与 RMSNorm" (rms_norm: true).  READING: eps = 1e-6."""
    x = _f(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if gain is not None:
        y = y * _f(gain)
    return y


def adaln(temb, w, b):
    """Per-stream modulation from the timestep embedding: Linear(SiLU(temb))
    of width 6*D, split in the order the [blog] Overview gives: shift, scale,
    gate before attention, then shift, scale, gate before the gated MLP.
    READING: SiLU before the Linear (standard DiT AdaLN).
    temb [B, D] -> dict of six [B, D] arrays."""
    m = linear(silu(temb), w, b)
    D = m.shape[-1] // 6
    names = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    return {n: m[..., i * D:(i + 1) * D] for i, n in enumerate(names)}


def modulate(xn, shift, scale):
    """xn * (1 + scale) + shift, one (shift, scale) row per sample broadcast
    over that sample's tokens.  xn [B, S, D]; shift, scale [B, D]."""
    return _f(xn) * (1.0 + _f(scale)[:, None, :]) + _f(shift)[:, None, :]


def rope_angles(pos, axes, theta):
    """Rotation angle of every (token, pair) for the 3-axis RoPE of [turbo]
    "3D RoPE" (axes_dims_rope [8, 28, 28], summing to the 64-d head).
    READING: head dims are split into contiguous segments of widths axes[a];
    inside segment a, pair j (dims 2j, 2j+1 of the segment) turns by
    pos[a] * theta^(-2j / axes[a]).  pos [S, 3] -> angles [S, sum(axes)//2]."""
    pos = _f(pos)
    cols = []
    for a, da in enumerate(axes):
        j = np.arange(da // 2, dtype=F64)
        omega = theta ** (-2.0 * j / da)
        cols.append(pos[:, a:a + 1] * omega[None, :])
    return np.concatenate(cols, axis=1)


def rope(x, pos, axes, theta):
    """Rotate interleaved pairs: (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
    x [S, H, d] with d = sum(axes); pos [S, 3]."""
    x = _f(x)
    ang = rope_angles(pos, axes, theta)[:, None, :]          # [S, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def attention(q, k, v, key_valid=None, return_probs=False):
    """Softmax attention per head: O = softmax(Q K^T / sqrt(d) + M) V, with
    M = -inf on invalid keys and no causal mask ([survey] joint attention;
    [turbo] "双流注意力机制").  READING: scale 1/sqrt(head_dim).
    q [Sq, H, d], k/v [Skv, H, d], key_valid [Skv] bool -> O [Sq, H, d]."""
    q, k, v = _f(q), _f(k), _f(v)
    Sq, H, d = q.shape
    Skv = k.shape[0]
    valid = np.ones(Skv, bool) if key_valid is None else np.asarray(key_valid, bool)
    out = np.empty((Sq, H, v.shape[-1]), F64)
    probs = [] if return_probs else None
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(d)          # [Sq, Skv]
        s[:, ~valid] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
        if return_probs:
            probs.append(p)
    if return_probs:
        return out, np.stack(probs)
    return out


def swiglu_mlp(a, w1, b1, w3, b3, w2, b2):
    """Gated MLP: W2 (SiLU(W1 a + b1) * (W3 a + b3)) + b2.  READING: w1 is the
    gate and w3 the up projection ([blog] Overview names gate/up/down of
    1536x4096; [turbo] names w1/w2/w3)."""
    return linear(silu(linear(a, w1, b1)) * linear(a, w3, b3), w2, b2)


# --------------------------------------------------------------------------
# one double-stream block
# --------------------------------------------------------------------------

def _proj(x, w, b, fp8):
    """A block projection; with fp8, both operands as the MX fp8 GEMM sees
    them (mx_roundtrip along the reduction axis)."""
    if fp8:
        return linear(mx_roundtrip(x), mx_roundtrip(w), b)
    return linear(x, w, b)


def _stream_qkv(ws, a, heads, eps, fp8=False):
    """QKV projection, then per-head RMSNorm of q and k with the stream's
    64-d gains ([turbo] norm_q/norm_k for the image stream,
    norm_added_q/norm_added_k for the text stream).  READING: output columns
    are q | k | v, each heads x head_dim; the norm comes before RoPE."""
    B, S, D = a.shape
    qkv = _proj(a, ws["qkv_w"], ws.get("qkv_b"), fp8)
    q, k, v = (qkv[..., i * D:(i + 1) * D].reshape(B, S, heads, D // heads) for i in range(3))
    q = rms_norm(q, eps, ws["q_gain"])
    k = rms_norm(k, eps, ws["k_gain"])
    return q, k, v


def block_forward(w, h_img, h_txt, temb, img_pos, txt_pos, txt_len=None, *,
                  heads=24, axes=(8, 28, 28), theta=10000.0, eps=1e-6, rows=None, gemm_fp8=False):
    """One double-stream MM-DiT block ([paper] 前置知识, MMDiT: each stream
    runs its own RMSNorm-attention-MLP branch and the two meet in joint
    attention; [turbo] "双流注意力机制", "自适应调制与 RMSNorm").

    w: {'img': {...}, 'txt': {...}} with mod_w/b, qkv_w/b, out_w/b, w1_w/b,
    w3_w/b, w2_w/b, q_gain, k_gain.  h_img [B, Si, D], h_txt [B, St, D],
    temb [B, D], img_pos [Si, 3], txt_pos [St, 3], txt_len [B] or None.

    rows: None, or (img_rows, txt_rows) index arrays; then only those query
    rows are carried through attention, the projections and the MLP (keys
    and values still come from every token), and the result is
    (h_img[:, img_rows], h_txt[:, txt_rows]) of the full block.

    gemm_fp8: the qkv, out, w1, w3 and w2 projections take MX fp8 operands
    (the low-precision variant above); everything else is unchanged.

    Text keys j >= txt_len[b] are masked ([blog] "Exploring Text Encoder":
    the DiT never sees the zero padding).  Rows of padded text queries are
    computed but carry no meaning.  READING: joint order text then image
    ([survey] text tokens concatenated with image tokens); the order does not
    change any result.  Returns (h_img_new, h_txt_new) in float64."""
    h = {"img": _f(h_img), "txt": _f(h_txt)}
    pos = {"img": np.asarray(img_pos), "txt": np.asarray(txt_pos)}
    B, Si, D = h["img"].shape
    St = h["txt"].shape[1]
    d = D // heads
    assert sum(axes) == d and all(a % 2 == 0 for a in axes)
    tl = np.full(B, St) if txt_len is None else np.clip(np.asarray(txt_len), 0, St)

    mod = {s: adaln(temb, w[s]["mod_w"], w[s].get("mod_b")) for s in ("img", "txt")}

    if rows is None:
        sel = {"img": np.arange(Si), "txt": np.arange(St)}
    else:
        sel = {"img": np.asarray(rows[0], int), "txt": np.asarray(rows[1], int)}

    # pre-attention RMSNorm + modulation, QKV, QK-norm, RoPE
    qkv = {}
    for s in ("img", "txt"):
        a = modulate(rms_norm(h[s], eps), mod[s]["shift1"], mod[s]["scale1"])
        q, k, v = _stream_qkv(w[s], a, heads, eps, gemm_fp8)
        q = np.stack([rope(q[b], pos[s], axes, theta) for b in range(B)])
        k = np.stack([rope(k[b], pos[s], axes, theta) for b in range(B)])
        qkv[s] = (q, k, v)

    out = {s: h[s][:, sel[s]].copy() for s in ("img", "txt")}
    for b in range(B):
        # joint sequence: text tokens, then image tokens
        K = np.concatenate([qkv["txt"][1][b], qkv["img"][1][b]], 0)
        V = np.concatenate([qkv["txt"][2][b], qkv["img"][2][b]], 0)
        valid = np.concatenate([np.arange(St) < tl[b], np.ones(Si, bool)])
        Q = np.concatenate([qkv["txt"][0][b][sel["txt"]], qkv["img"][0][b][sel["img"]]], 0)
        O = attention(Q, K, V, valid).reshape(Q.shape[0], D)
        nt = len(sel["txt"])
        O_s = {"txt": O[:nt], "img": O[nt:]}
        for s in ("img", "txt"):
            y = _proj(O_s[s], w[s]["out_w"], w[s].get("out_b"), gemm_fp8)
            out[s][b] = out[s][b] + mod[s]["gate1"][b] * y

    # pre-MLP RMSNorm + modulation, gated SwiGLU MLP
    for s in ("img", "txt"):
        a = modulate(rms_norm(out[s], eps), mod[s]["shift2"], mod[s]["scale2"])
        if gemm_fp8:
            u = silu(_proj(a, w[s]["w1_w"], w[s].get("w1_b"), True)) * _proj(a, w[s]["w3_w"], w[s].get("w3_b"), True)
            y = _proj(u, w[s]["w2_w"], w[s].get("w2_b"), True)
        else:
            y = swiglu_mlp(a, w[s]["w1_w"], w[s].get("w1_b"), w[s]["w3_w"], w[s].get("w3_b"),
                           w[s]["w2_w"], w[s].get("w2_b"))
        out[s] = out[s] + mod[s]["gate2"][:, None, :] * y
    return out["img"], out["txt"]


# --------------------------------------------------------------------------
# embeddings, whole denoiser
# --------------------------------------------------------------------------

def timestep_features(t, dim=256, scale=1000.0, theta=10000.0):
    """Sinusoidal features of the timestep feeding the timestep-embedder MLP
    ([turbo] time_text_embed.timestep_embedder).  READING: phi(t) =
    [cos(scale*t*w_k) | sin(scale*t*w_k)], w_k = theta^(-k/(dim/2)),
    k < dim/2.  t [B] -> [B, dim]."""
    half = dim // 2
    wk = theta ** (-np.arange(half, dtype=F64) / half)
    arg = scale * _f(t)[:, None] * wk[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def timestep_embedding(top, t, *, t_freq=256, t_scale=1000.0):
    """temb = fc2(SiLU(fc1(phi(t)))).  READING: two Linear layers with a SiLU."""
    phi = timestep_features(t, t_freq, t_scale)
    return linear(silu(linear(phi, top["t_fc1_w"], top.get("t_fc1_b"))),
                  top["t_fc2_w"], top.get("t_fc2_b"))


def text_embed(top, feats, *, layers=4, eps=1e-6):
    """RMSNorm each encoder layer's feature slice with its own gain
    ([turbo] "多层级文本特征融合": txt_norm.0..3 normalise the four feature
    streams), concatenate them along features in layer order and project
    with txt_in to the hidden width ([paper] 核心方法: the layers are
    concatenated to D = 1536).  feats [B, S, layers*F] -> [B, S, D]."""
    feats = _f(feats)
    F = feats.shape[-1] // layers
    parts = [rms_norm(feats[..., l * F:(l + 1) * F], eps, top["txt_gain"][l]) for l in range(layers)]
    return linear(np.concatenate(parts, -1), top["txt_in_w"], top.get("txt_in_b"))


def final_layer(top, h_img, temb, *, eps=1e-6):
    """norm_out + proj_out ([turbo] "Patchify 补丁化与输出投影"): (shift,
    scale) = norm_out.linear(SiLU(temb)), in that order; v = proj_out(
    RMSNorm(h) * (1 + scale) + shift).  READING: order and SiLU as in AdaLN."""
    m = linear(silu(temb), top["norm_out_w"], top.get("norm_out_b"))
    D = m.shape[-1] // 2
    a = modulate(rms_norm(h_img, eps), m[:, :D], m[:, D:])
    return linear(a, top["proj_out_w"], top.get("proj_out_b"))


def dit_forward(top, blocks, x, txt_feats, t, img_pos, txt_pos, txt_len=None, *,
                heads=24, axes=(8, 28, 28), theta=10000.0, eps=1e-6, t_freq=256,
                t_scale=1000.0, txt_layers=4, capture=None, gemm_fp8=False):
    """Whole denoiser: v = proj_out(norm_out(blocks(img_in(x), txt_in(f)))).
    blocks: iterable of block weight dicts (generated lazily by the caller).
    x [B, Si, in_ch] patchified tokens (a 2x2 patch of the 32-channel latent
    is 128 features: [turbo] "Patchify"), txt_feats [B, St, 4*2880], t [B].
    capture: optional dict; capture[i] = (h_img, h_txt) after block i."""
    temb = timestep_embedding(top, t, t_freq=t_freq, t_scale=t_scale)
    h_img = linear(x, top["img_in_w"], top.get("img_in_b"))
    h_txt = text_embed(top, txt_feats, layers=txt_layers, eps=eps)
    for i, wb in enumerate(blocks):
        h_img, h_txt = block_forward(wb, h_img, h_txt, temb, img_pos, txt_pos, txt_len,
                                     heads=heads, axes=axes, theta=theta, eps=eps, gemm_fp8=gemm_fp8)
        if capture is not None:
            capture[i] = (h_img, h_txt)
    return final_layer(top, h_img, temb, eps=eps)


# --------------------------------------------------------------------------
# sampler
# --------------------------------------------------------------------------

def time_grid(steps, mu=None):
    """t_k = 1 - k/N, k = 0..N.  [paper] 前置知识 (Flow Matching): the path
    x_t = (1 - t) x0 + t x1 with target x1 - x0, so t = 1 is the noise end
    when x1 is noise and sampling starts from N(0, 1) latents.  READING: a
    uniform grid; with mu, each point is moved by time_shift(t, mu)."""
    t = 1.0 - np.arange(steps + 1, dtype=F64) / steps
    return t if mu is None else time_shift(t, mu)


def time_shift(t, mu):
    """Resolution-dependent timestep shift ([paper] 前置知识 and 方法步骤详情:
    logit-normal timesteps with a location mu(n) interpolated linearly in
    the token count, mu = 1.06 for the 512^2 stage).  READING: the inference
    grid is shifted by the same mu as t' = e^mu t / (e^mu t + 1 - t), i.e. a
    translation by mu in logit space; t = 0 and t = 1 stay fixed."""
    t = _f(t)
    e = math.exp(mu)
    return e * t / (e * t + 1.0 - t)


def mu_for_tokens(n, n0, mu0, n1, mu1):
    """mu(n) on the straight line through (n0, mu0) and (n1, mu1) ([paper]
    方法步骤详情: linear interpolation in the token count).  The pages give
    one point only (mu = 1.06 at 512^2, 1024 tokens); the other is the
    caller's."""
    return mu0 + (float(n) - n0) * (mu1 - mu0) / (n1 - n0)


def cfg_combine(v_cond, v_uncond, scale):
    """guided = uncond + scale * (cond - uncond) ([survey] CFG; [blog]
    "Exploring Image Editing")."""
    vc, vu = _f(v_cond), _f(v_uncond)
    return vu + scale * (vc - vu)


def euler_step(x, v, dt):
    """One explicit Euler step of the flow ODE dx/dt = v: x + dt * v
    ([survey] rectified flow: integrate the learned velocity field)."""
    return _f(x) + dt * _f(v)


def flow_step(x, v_cond, v_uncond, dt, scale):
    """CFG combine (skipped when v_uncond is None) then the Euler update."""
    v = _f(v_cond) if v_uncond is None else cfg_combine(v_cond, v_uncond, scale)
    return euler_step(x, v, dt)


def cfg_combine_rescaled(v_cond, v_uncond, scale):
    """Norm-rescaled CFG ([blog] "Exploring Image Editing": Lens's inference
    rescales the guided velocity by norms; the printed formula keeps only the
    plain combination).  READING: per token (the last axis, the 128 latent
    channels of a patch token), comb = u + s (c - u), then
    comb <- comb * ||c|| / ||comb||, so the guided velocity keeps the
    conditional velocity's per-token norm.  A token with ||comb|| = 0 keeps
    comb (= 0)."""
    vc = _f(v_cond)
    comb = vc if v_uncond is None else cfg_combine(v_cond, v_uncond, scale)
    nc = np.sqrt(np.sum(vc * vc, axis=-1, keepdims=True))
    nb = np.sqrt(np.sum(comb * comb, axis=-1, keepdims=True))
    factor = np.where(nb > 0.0, nc / np.where(nb > 0.0, nb, 1.0), 1.0)
    return comb * factor


def flow_step_rescaled(x, v_cond, v_uncond, dt, scale):
    """Norm-rescaled CFG combine then the Euler update (x, v: [..., C])."""
    return euler_step(x, cfg_combine_rescaled(v_cond, v_uncond, scale), dt)


def sample(velocity, x0, steps, scale=1.0, use_uncond=False):
    """Euler loop over time_grid(steps).  velocity(x, t) returns v_cond, or
    (v_cond, v_uncond) when use_uncond; returns the final x (float64)."""
    ts = time_grid(steps)
    x = _f(x0)
    for k in range(steps):
        out = velocity(x, ts[k])
        vc, vu = (out if use_uncond else (out, None))
        x = flow_step(x, vc, vu, ts[k + 1] - ts[k], scale)
    return x


# --------------------------------------------------------------------------
# low-precision GEMM variant (MX fp8)
# --------------------------------------------------------------------------
# [4bit] section 4: the DiT's projection weights are quantized (int4, groups
# of 64) while img_in, txt_in, proj_out, the timestep/text embedders and
# norm_out stay bf16; a single DiT pass keeps cosine 0.9976 against the
# reference.  READING (MI355X analogue): the per-block projections (qkv, out,
# w1, w3, w2) take MX fp8 operands -- e4m3 elements with one power-of-two
# scale per 32 consecutive elements along the reduction axis -- for both the
# weights and the activations entering them; AdaLN and everything outside
# the blocks stay as they are.

E4M3_MAX = 448.0     # largest finite e4m3 value (1.75 * 2^8)
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUB_STEP = 2.0 ** -9


def round_e4m3(y):
    """Round to the nearest e4m3 value (ties to even), for |y| <= 448: 3
    mantissa bits on normals (exponents -6..8), steps of 2^-9 below 2^-6."""
    y = _f(y)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a >= E4M3_MIN_NORMAL, a, 1.0)))
    step = np.where(a >= E4M3_MIN_NORMAL, 2.0 ** (e - 3), E4M3_SUB_STEP)
    q = np.round(a / step) * step          # np.round: ties to even
    return np.sign(y) * q


def mx_scale_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (amax > 0), clamped to the
    E8M0 range [-127, 127]; -127 for amax = 0.  READING: the scale is chosen
    so that no element saturates."""
    amax = _f(amax)
    e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX))
    # log2 of an exact power-of-two ratio can land a hair off an integer
    e = np.where(amax > E4M3_MAX * 2.0 ** e, e + 1, e)
    e = np.where(amax <= E4M3_MAX * 2.0 ** (e - 1), e - 1, e)
    return np.clip(np.where(amax > 0, e, -127), -127, 127).astype(np.int64)


def mx_quantize(x, block=32):
    """MX fp8 along the last axis: per block of 32, e = mx_scale_exponent of
    the block's max |x|, elements round_e4m3(x / 2^e).  Returns (q, e) with q
    on the e4m3 grid and e of shape [..., n / 32]."""
    x = _f(x)
    n = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (n // block, block))
    e = mx_scale_exponent(np.max(np.abs(xb), axis=-1))
    q = round_e4m3(xb / 2.0 ** e[..., None])
    return q.reshape(x.shape), e


def mx_dequantize(q, e, block=32):
    q = _f(q)
    n = q.shape[-1]
    return (q.reshape(q.shape[:-1] + (n // block, block)) * 2.0 ** _f(e)[..., None]).reshape(q.shape)


def mx_roundtrip(x, block=32):
    """The value an MX fp8 GEMM sees for x: dequantize(quantize(x))."""
    return mx_dequantize(*mx_quantize(x, block), block)


def stream_param_count(shapes):
    """Weights of one stream (biases and 64-d gains excluded), from the shape
    table of the tensors the block above reads."""
    return sum(int(np.prod(shapes[n])) for n in ("mod_w", "qkv_w", "out_w", "w1_w", "w3_w", "w2_w"))


__all__ = [
    "linear", "silu", "rms_norm", "adaln", "modulate", "rope_angles", "rope", "attention",
    "swiglu_mlp", "block_forward", "timestep_features", "timestep_embedding", "text_embed",
    "final_layer", "dit_forward", "time_grid", "cfg_combine", "euler_step", "flow_step",
    "cfg_combine_rescaled", "flow_step_rescaled", "time_shift", "mu_for_tokens", "sample", "stream_param_count",
    "E4M3_MAX", "round_e4m3", "mx_scale_exponent", "mx_quantize", "mx_dequantize", "mx_roundtrip",
]
