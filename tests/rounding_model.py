"""Error budget of the bf16 block: the fp64 oracle block with bf16
round-to-nearest-even inserted at every point where the HIP path stores a
bf16 tensor, and nothing else changed.

The whole-model variant (dit_forward_rounded) adds the two bf16 storage
points outside the blocks: the normalised text features before txt_in and
the norm_out-modulated image rows before proj_out (the latent x arrives in
bf16 already; temb, the modulations and the residual stream stay float).

Test infrastructure only (CPU).  It shows how far from the exact block a
computation can land that differs from it only by those storage roundings,
which is what the GPU parity bars for bf16 block outputs and deltas are
derived from (tests/test_parity_budget.py).  It uses the oracle's
primitives for every step and the input module's bf16 rounding; the
storage points are those of the bf16 kernels:

  a   = RMSNorm(h)(1 + scale) + shift            -> bf16 (norm + modulate)
  q   = RoPE(RMSNorm_64(q) g_q) * log2(e) / 8    -> bf16 (QKV epilogue; the
        attention takes q in log2 units, so the rounding is of the scaled q)
  k   = RoPE(RMSNorm_64(k) g_k)                  -> bf16
  v                                              -> bf16
  p   = 2^(s - m)                                -> bf16 (the PV product's
        operand; the row sum adds the unrounded values)
  O   = sum(p v) / sum(p)                        -> bf16
  u   = SiLU(W1 a + b1)(W3 a + b3)               -> bf16 (SwiGLU epilogue)
  residual updates h += gate * (.) stay float (fp32 on the GPU).

The GEMM accumulations (fp32 on the GPU) are taken exact here: their
rounding is orders of magnitude below the bf16 storage terms.
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O
import synth

LOG2E = 1.0 / math.log(2.0)


def bf16(x):
    """fp64 -> the nearest float32 -> the nearest bf16 (RNE), back as fp64."""
    return synth.bf16_round(np.asarray(x, np.float64).astype(np.float32)).astype(np.float64)


def _attention_rounded(q2, k, v, key_valid):
    """q2 in log2 units (already rounded), k, v rounded; probabilities
    rounded to bf16 before the product with V, while the row sum adds them
    unrounded."""
    Sq, H, d = q2.shape
    out = np.empty((Sq, H, d))
    for h in range(H):
        s = q2[:, h, :] @ k[:, h, :].T
        s[:, ~key_valid] = -np.inf
        e = np.exp2(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (bf16(e) @ v[:, h, :]) / e.sum(axis=1, keepdims=True)
    return out


def block_forward_rounded(w, h_img, h_txt, temb, img_pos, txt_pos, txt_len=None, *, heads=24, axes=(8, 28, 28),
                          theta=10000.0, eps=1e-6):
    """The oracle block (oracle.block_forward) with the bf16 storage points
    above; same arguments and outputs (float64)."""
    h = {"img": np.asarray(h_img, np.float64), "txt": np.asarray(h_txt, np.float64)}
    pos = {"img": np.asarray(img_pos), "txt": np.asarray(txt_pos)}
    B, Si, D = h["img"].shape
    St = h["txt"].shape[1]
    tl = np.full(B, St) if txt_len is None else np.clip(np.asarray(txt_len), 0, St)
    mod = {s: O.adaln(temb, w[s]["mod_w"], w[s].get("mod_b")) for s in ("img", "txt")}
    qkv = {}
    for s in ("img", "txt"):
        a = bf16(O.modulate(O.rms_norm(h[s], eps), mod[s]["shift1"], mod[s]["scale1"]))
        y = O.linear(a, w[s]["qkv_w"], w[s].get("qkv_b"))
        q, k, v = (y[..., i * D:(i + 1) * D].reshape(B, -1, heads, D // heads) for i in range(3))
        q = O.rms_norm(q, eps, w[s]["q_gain"])
        k = O.rms_norm(k, eps, w[s]["k_gain"])
        q = np.stack([O.rope(q[b], pos[s], axes, theta) for b in range(B)])
        k = np.stack([O.rope(k[b], pos[s], axes, theta) for b in range(B)])
        qkv[s] = (bf16(q * (LOG2E / 8.0)), bf16(k), bf16(v))
    out = {s: h[s].copy() for s in ("img", "txt")}
    for b in range(B):
        Q = np.concatenate([qkv["txt"][0][b], qkv["img"][0][b]], 0)
        K = np.concatenate([qkv["txt"][1][b], qkv["img"][1][b]], 0)
        V = np.concatenate([qkv["txt"][2][b], qkv["img"][2][b]], 0)
        valid = np.concatenate([np.arange(St) < tl[b], np.ones(Si, bool)])
        Ob = bf16(_attention_rounded(Q, K, V, valid).reshape(St + Si, D))
        for s, rows in (("txt", Ob[:St]), ("img", Ob[St:])):
            out[s][b] = out[s][b] + mod[s]["gate1"][b] * O.linear(rows, w[s]["out_w"], w[s].get("out_b"))
    for s in ("img", "txt"):
        a = bf16(O.modulate(O.rms_norm(out[s], eps), mod[s]["shift2"], mod[s]["scale2"]))
        u = bf16(O.silu(O.linear(a, w[s]["w1_w"], w[s].get("w1_b"))) * O.linear(a, w[s]["w3_w"], w[s].get("w3_b")))
        out[s] = out[s] + mod[s]["gate2"][:, None, :] * O.linear(u, w[s]["w2_w"], w[s].get("w2_b"))
    return out["img"], out["txt"]


def budget(variant, B, gh, gw, St, txt_len=None, block=0, seed_h=1, biases=True):
    """Max |rounded - exact| of the block outputs and deltas (h_out - h_in),
    each relative to the RMS of the exact tensor, over the valid rows of
    both streams: {'out': ratio, 'delta': ratio}."""
    w = synth.block_weights(block, dtype="bf16", variant=variant)
    if not biases:
        w = synth.without_biases(w)
    hi, ht, temb = synth.block_inputs(B, gh * gw, St, dtype="bf16", seed=seed_h)
    ip, tp = synth.image_positions(gh, gw), synth.text_positions(St)
    xi, xt = O.block_forward(w, hi, ht, temb, ip, tp, txt_len)
    ri, rt = block_forward_rounded(w, hi, ht, temb, ip, tp, txt_len)
    n = np.full(B, St) if txt_len is None else np.asarray(txt_len)
    pick = lambda a: np.concatenate([a[b, :n[b]] for b in range(B)]) if St else np.zeros((0, a.shape[-1]))
    res = {"out": 0.0, "delta": 0.0}
    for x, r, h in ((xi, ri, hi), (pick(xt), pick(rt), pick(ht))):
        if x.size == 0:
            continue
        err = float(np.max(np.abs(r - x)))
        res["out"] = max(res["out"], err / float(np.sqrt(np.mean(x * x))))
        res["delta"] = max(res["delta"], err / float(np.sqrt(np.mean((x - h) ** 2))))
    return res


def budget_model_block(block=0, t=0.75):
    """The same budget for a block of the whole model at its own modulation:
    the 1024^2 cond + uncond launch (B = 2, one latent, cond and uncond text),
    h from the oracle's img_in / txt_in and temb from its timestep MLP at t
    (fp32, as the residual stream holds them), block `block` of the seeded
    model.  Returns {'out': ratio, 'delta': ratio} as budget()."""
    top = synth.top_weights()
    x0 = synth.bf16_round(synth.latents(1, 4096))
    x = np.concatenate([x0, x0])
    feats = np.concatenate([synth.text_features(1, 512, seed=synth.SEED_TEXT_COND),
                            synth.text_features(1, 512, seed=synth.SEED_TEXT_UNCOND)])
    temb = O.timestep_embedding(top, np.array([t, t])).astype(np.float32)
    hi = O.linear(x, top["img_in_w"], top["img_in_b"]).astype(np.float32)
    ht = O.text_embed(top, feats).astype(np.float32)
    ip, tp = synth.image_positions(64, 64), synth.text_positions(512)
    w = synth.block_weights(block)
    xi, xt = O.block_forward(w, hi, ht, temb, ip, tp)
    ri, rt = block_forward_rounded(w, hi, ht, temb, ip, tp)
    res = {"out": 0.0, "delta": 0.0}
    for x_, r_, h_ in ((xi, ri, hi), (xt, rt, ht)):
        err = float(np.max(np.abs(r_ - x_)))
        res["out"] = max(res["out"], err / float(np.sqrt(np.mean(x_ * x_))))
        res["delta"] = max(res["delta"], err / float(np.sqrt(np.mean((x_ - h_) ** 2))))
    return res


def dit_forward_rounded(top, blocks, x, feats, t, img_pos, txt_pos, txt_len=None, *, layers=4, eps=1e-6):
    """The oracle denoiser (oracle.dit_forward) with the bf16 storage points
    of the blocks (block_forward_rounded) and of the text-feature norm and
    the final layer's modulation; same arguments and output (float64)."""
    temb = O.timestep_embedding(top, t)
    h_img = O.linear(x, top["img_in_w"], top.get("img_in_b"))
    f = np.asarray(feats, np.float64)
    F = f.shape[-1] // layers
    tn = bf16(np.concatenate([O.rms_norm(f[..., l * F:(l + 1) * F], eps, top["txt_gain"][l]) for l in range(layers)],
                             -1))
    h_txt = O.linear(tn, top["txt_in_w"], top.get("txt_in_b"))
    for wb in blocks:
        h_img, h_txt = block_forward_rounded(wb, h_img, h_txt, temb, img_pos, txt_pos, txt_len, eps=eps)
    m = O.linear(O.silu(temb), top["norm_out_w"], top.get("norm_out_b"))
    D = m.shape[-1] // 2
    a = bf16(O.modulate(O.rms_norm(h_img, eps), m[:, :D], m[:, D:]))
    return O.linear(a, top["proj_out_w"], top.get("proj_out_b"))


def budget_sampler_step(norm_rescale=False, mu=None, steps=3, scale=5.0, gh=8, gw=8, St=16, n_blocks=2):
    """Max |dx_rounded - dx_exact| / RMS(dx_exact) over the steps of a CFG
    Euler run (one latent, cond + uncond text in one B = 2 call, the seeded
    model cut to n_blocks blocks): at each step the velocities of
    dit_forward_rounded and of the oracle at the same bf16 input, combined
    by the plain or norm-rescaled CFG step; the trajectory is the oracle's."""
    top = synth.top_weights()
    blocks = [synth.block_weights(i) for i in range(n_blocks)]
    feats = np.concatenate([synth.text_features(1, St, seed=synth.SEED_TEXT_COND),
                            synth.text_features(1, St, seed=synth.SEED_TEXT_UNCOND)])
    ip, tp = synth.image_positions(gh, gw), synth.text_positions(St)
    x = np.asarray(synth.latents(1, gh * gw), np.float64)[0]
    ts = O.time_grid(steps, mu=mu)
    step = O.flow_step_rescaled if norm_rescale else O.flow_step
    worst = 0.0
    for k in range(steps):
        xa = np.stack([synth.bf16_round(x.astype(np.float32))] * 2)
        t = np.array([ts[k], ts[k]])
        dt = ts[k + 1] - ts[k]
        ve = O.dit_forward(top, blocks, xa, feats, t, ip, tp)
        vr = dit_forward_rounded(top, blocks, xa, feats, t, ip, tp)
        xe = step(x, ve[0], ve[1], dt, scale)
        xr = step(x, vr[0], vr[1], dt, scale)
        dxe = xe - x
        worst = max(worst, float(np.max(np.abs(xr - xe))) / float(np.sqrt(np.mean(dxe * dxe))))
        x = xe
    return worst
