"""Seeded synthetic inputs for the Lens MM-DiT denoiser.

This module only draws random numbers and rounds them to the storage type.
It holds none of the denoiser's arithmetic, so both the fp64 oracle (through
the tests) and the HIP path (through the tests, the bench and the smoke run)
can take their inputs from it without sharing any computation.

Every tensor comes from its own stream
``numpy.random.default_rng(SeedSequence([seed, block, tensor_id]))`` drawn
in float32, so one block's weights can be regenerated on the host without
drawing the other 47.  bf16 tensors are rounded to nearest-even and kept as
float32 arrays holding bf16-representable values (``bf16_bits`` gives the raw
16-bit patterns for upload).

Seeds by role: 0 weights, 1 hidden states / temb, 2 latents, 3 cond text,
4 uncond text, 5 text lengths.

Shapes follow the model the pages describe: 48 double-stream blocks, hidden
1536 = 24 heads x 64, SwiGLU 4096, per-stream AdaLN 1536 -> 6 x 1536, RoPE axes
[8, 28, 28], 2x2 patches of a 32-channel latent (128 per token), four 2880-d
text-encoder layers (Lens-Turbo-3.8B-bf16 article, architecture table and
config fields; Lens blog, Overview).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_WEIGHTS = 0
SEED_HIDDEN = 1
SEED_LATENT = 2
SEED_TEXT_COND = 3
SEED_TEXT_UNCOND = 4
SEED_TEXT_LEN = 5


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int = 1536
    heads: int = 24
    head_dim: int = 64
    mlp: int = 4096
    n_blocks: int = 48
    rope_axes: tuple = (8, 28, 28)
    rope_theta: float = 10000.0
    eps: float = 1e-6
    in_ch: int = 128
    out_ch: int = 128
    txt_feat: int = 2880
    txt_layers: int = 4
    t_freq: int = 256
    t_scale: float = 1000.0


LENS = Dims()

# tensor ids inside a block; stream offset 0 (image) or 100 (text)
_STREAM_TENSORS = (
    # name,  kind,  shape(dims) -> tuple
    ("mod_w", "w", lambda d: (6 * d.hidden, d.hidden)),
    ("mod_b", "b", lambda d: (6 * d.hidden,)),
    ("qkv_w", "w", lambda d: (3 * d.hidden, d.hidden)),
    ("qkv_b", "b", lambda d: (3 * d.hidden,)),
    ("out_w", "w", lambda d: (d.hidden, d.hidden)),
    ("out_b", "b", lambda d: (d.hidden,)),
    ("w1_w", "w", lambda d: (d.mlp, d.hidden)),
    ("w1_b", "b", lambda d: (d.mlp,)),
    ("w3_w", "w", lambda d: (d.mlp, d.hidden)),
    ("w3_b", "b", lambda d: (d.mlp,)),
    ("w2_w", "w", lambda d: (d.hidden, d.mlp)),
    ("w2_b", "b", lambda d: (d.hidden,)),
    ("q_gain", "g", lambda d: (d.head_dim,)),
    ("k_gain", "g", lambda d: (d.head_dim,)),
)
STREAMS = ("img", "txt")

# non-block tensors (block index = n_blocks, i.e. after the last block)
_TOP_TENSORS = (
    ("t_fc1_w", "w", lambda d: (d.hidden, d.t_freq)),
    ("t_fc1_b", "b", lambda d: (d.hidden,)),
    ("t_fc2_w", "w", lambda d: (d.hidden, d.hidden)),
    ("t_fc2_b", "b", lambda d: (d.hidden,)),
    ("img_in_w", "w", lambda d: (d.hidden, d.in_ch)),
    ("img_in_b", "b", lambda d: (d.hidden,)),
    ("txt_gain", "g", lambda d: (d.txt_layers, d.txt_feat)),
    ("txt_in_w", "w", lambda d: (d.hidden, d.txt_layers * d.txt_feat)),
    ("txt_in_b", "b", lambda d: (d.hidden,)),
    ("norm_out_w", "w", lambda d: (2 * d.hidden, d.hidden)),
    ("norm_out_b", "b", lambda d: (2 * d.hidden,)),
    ("proj_out_w", "w", lambda d: (d.out_ch, d.hidden)),
    ("proj_out_b", "b", lambda d: (d.out_ch,)),
)


def rng(*keys: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in keys]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 patterns, round to nearest even (NaN kept NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


# 'late' variant: base of the q / k RMSNorm gains per (stream, tensor)
_LATE_GAINS = {("img", "q_gain"): 2.0, ("txt", "q_gain"): 2.0, ("img", "k_gain"): 0.5, ("txt", "k_gain"): 2.5}


def _draw(kind: str, shape, g: np.random.Generator, variant: str, stream: str = "", name: str = "") -> np.ndarray:
    """One weight tensor.  'canonical': linear weights and biases N(0, 0.02),
    norm gains 1 + N(0, 0.02).  'wide': the same weights, but gains U(0.5, 1.5)
    and biases N(0, 1), so gain and bias paths carry visible signal.
    'sharp': canonical, but norm gains 2.05 + N(0, 0.02): q.k logits about 4x
    larger, so attention is sharp and its running max moves often.
    'late': canonical, but q gains 2, image k gains 0.5 and text k gains 2.5
    (+ N(0, 0.02)): keys of the text stream score far above image keys, so
    a softmax pass that meets the image keys first (in key order) sees its
    running maximum jump when it reaches the text keys."""
    if kind == "w":
        return g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    if kind == "b":
        s = 1.0 if variant == "wide" else 0.02
        return g.standard_normal(shape, dtype=np.float32) * np.float32(s)
    if kind == "g":
        if variant == "wide":
            return g.uniform(0.5, 1.5, size=shape).astype(np.float32)
        if variant == "late" and (stream, name) in _LATE_GAINS:
            base = np.float32(_LATE_GAINS[(stream, name)])
        else:
            base = np.float32(2.05) if variant == "sharp" else np.float32(1.0)
        return base + g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    raise ValueError(kind)


def stream_tensor_shapes(d: Dims = LENS) -> dict:
    return {name: shape(d) for name, _, shape in _STREAM_TENSORS}


def top_tensor_shapes(d: Dims = LENS) -> dict:
    return {name: shape(d) for name, _, shape in _TOP_TENSORS}


def block_weights(block: int, d: Dims = LENS, dtype: str = "bf16", seed: int = SEED_WEIGHTS,
                  variant: str = "canonical") -> dict:
    """{'img': {name: array}, 'txt': {...}} for one block (float32 arrays)."""
    out = {}
    for si, s in enumerate(STREAMS):
        ws = {}
        for ti, (name, kind, shape) in enumerate(_STREAM_TENSORS):
            g = rng(seed, block, 100 * si + ti)
            ws[name] = _store(_draw(kind, shape(d), g, variant, s, name), dtype)
        out[s] = ws
    return out


def without_biases(w: dict) -> dict:
    """The same block weights with every Linear bias removed (None): the
    bias-free Linear layers a checkpoint may carry."""
    return {s: {k: (None if k.endswith("_b") else v) for k, v in ws.items()} for s, ws in w.items()}


def top_weights(d: Dims = LENS, dtype: str = "bf16", seed: int = SEED_WEIGHTS,
                variant: str = "canonical") -> dict:
    out = {}
    for ti, (name, kind, shape) in enumerate(_TOP_TENSORS):
        g = rng(seed, 10_000, ti)
        out[name] = _store(_draw(kind, shape(d), g, variant), dtype)
    return out


def all_block_weights(d: Dims = LENS, dtype: str = "bf16", seed: int = SEED_WEIGHTS,
                      variant: str = "canonical", threads: int = 8, blocks=None):
    """Yield (block, weights) in block order, generated on a thread pool."""
    blocks = list(range(d.n_blocks)) if blocks is None else list(blocks)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for b, w in zip(blocks, ex.map(lambda i: block_weights(i, d, dtype, seed, variant), blocks)):
            yield b, w


def block_inputs(B: int, S_img: int, S_txt: int, d: Dims = LENS, dtype: str = "bf16",
                 seed: int = SEED_HIDDEN):
    """h_img [B,S_img,D], h_txt [B,S_txt,D] ~ N(0,1) (float32 residual streams,
    values rounded to the activation type) and temb [B,D] ~ N(0,1)."""
    h_img = _store(rng(seed, 0).standard_normal((B, S_img, d.hidden), dtype=np.float32), dtype)
    h_txt = _store(rng(seed, 1).standard_normal((B, S_txt, d.hidden), dtype=np.float32), dtype)
    temb = _store(rng(seed, 2).standard_normal((B, d.hidden), dtype=np.float32), dtype)
    return h_img, h_txt, temb


def image_positions(grid_h: int, grid_w: int) -> np.ndarray:
    """[grid_h*grid_w, 3] int32 positions (0, h, w), row-major over the grid."""
    hh, ww = np.meshgrid(np.arange(grid_h), np.arange(grid_w), indexing="ij")
    return np.stack([np.zeros_like(hh), hh, ww], -1).reshape(-1, 3).astype(np.int32)


def text_positions(S_txt: int) -> np.ndarray:
    return np.zeros((S_txt, 3), np.int32)


def latents(B: int, S_img: int, d: Dims = LENS, seed: int = SEED_LATENT, sample: int = 0) -> np.ndarray:
    """Patchified N(0,1) latent tokens [B,S_img,in_ch] (float32)."""
    return rng(seed, sample).standard_normal((B, S_img, d.in_ch), dtype=np.float32)


def text_features(B: int, S_txt: int, d: Dims = LENS, dtype: str = "bf16", seed: int = SEED_TEXT_COND,
                  txt_len=None) -> np.ndarray:
    """N(0,1) stand-ins for the four encoder-layer features, [B,S_txt,layers*feat]
    in layer-major order; rows past txt_len[b] are zero padding."""
    f = rng(seed, 0).standard_normal((B, S_txt, d.txt_layers * d.txt_feat), dtype=np.float32)
    if txt_len is not None:
        for b, n in enumerate(np.asarray(txt_len)):
            f[b, int(n):] = 0.0
    return _store(f, dtype)


def text_lengths(B: int, lo: int, hi: int, seed: int = SEED_TEXT_LEN, stream: int = 0) -> np.ndarray:
    """Valid text lengths drawn uniformly from {lo..hi}, int32 [B]."""
    return rng(seed, stream).integers(lo, hi + 1, size=B).astype(np.int32)


def gaussian(shape, seed: int, *keys: int, dtype: str = "f32") -> np.ndarray:
    return _store(rng(seed, *keys).standard_normal(shape, dtype=np.float32), dtype)
