"""Seeded synthetic inputs for the generation-pass attention block.

This module only draws random numbers and lays them out in the shapes the
pages describe; it holds none of the method's arithmetic (no norm, no rotary,
no attention, no flow-matching update).  Both the fp64 oracle and the HIP
library consume what it returns.

Shapes follow the pages:
  * each backbone token stands for a 32x32 block of pixels (SenseNova-U1.5
    (NEO-unify) architecture, §Vision tower), so 512^2 -> 256, 1024^2 -> 1024 and
    2048^2 -> 4096 image tokens;
  * head_dim 128 split into a temporal [0:64), height [64:96) and width
    [96:128) slice, each fed by its own row of a 3-row position index; every
    token of an image carries the same temporal position, the number of text
    tokens before it (same page, §Three rotary axes);
  * the generation pass reads a frozen understanding-branch K/V prefix
    (same page, §Mixture of Transformers), stored token-major [S, H, D]
    (SenseNova-U1 paper notes, §4.4 KV cache reuse).

Every floating-point tensor is returned as float32; for the bf16 workloads the
values are already rounded to bf16 (round-to-nearest-even on the host), so the
same bits reach both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

HEAD_DIM = 128
HALF = 64
PIXELS_PER_TOKEN = 32  # 16x16 patchify followed by a 2x2 merge


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16": dtype of q/k/v/o
    B: int
    Hq: int
    Hkv: int
    grids: list                   # per sample (gh, gw) image-token grid
    n_img: list                   # per sample image-token count N_b
    n_prefix: list                # per sample prefix length P_b
    # generation block, pre-norm, token-major [Tq, H, 128]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    # generation-branch norm weights, each [64]
    wq_t: np.ndarray
    wq_hw: np.ndarray
    wk_t: np.ndarray
    wk_hw: np.ndarray
    pos_img: np.ndarray           # int32 [3, Tq]
    cu_q: np.ndarray              # int32 [B+1]
    cu_p: np.ndarray              # int32 [B+1]
    # frozen prefix: either drawn directly as the cache ("direct"), or raw
    # pre-norm keys plus understanding-branch norm weights and positions that
    # the consumer turns into a rotated cache ("built")
    prefix_kind: str
    v_prefix: np.ndarray          # [Tp, Hkv, 128]
    k_prefix: Optional[np.ndarray] = None      # direct: the cache keys
    k_prefix_pre: Optional[np.ndarray] = None  # built: pre-norm keys
    wk_und_t: Optional[np.ndarray] = None
    wk_und_hw: Optional[np.ndarray] = None
    pos_prefix: Optional[np.ndarray] = None    # int32 [3, Tp]
    # pixel-space flow matching
    pixel_shape: tuple = ()       # (B, 3, H, W)
    eps_pixels: Optional[np.ndarray] = None    # N(0,1) noise, fp32
    x_hat: Optional[np.ndarray] = None         # synthetic x0 prediction, fp32
    z_start: Optional[np.ndarray] = None       # given z at t_grid[0] (tiny only)
    sigma_R: float = 1.0
    t_grid: tuple = ()            # (t_0, ..., t_S): step k goes t_k -> t_{k+1}
    eps: float = 1e-6
    rope_theta: float = 5.0e6
    rope_theta_hw: float = 1.0e4
    t_eps: float = 0.02
    extras: dict = dataclasses.field(default_factory=dict)

    @property
    def Tq(self) -> int:
        return int(self.cu_q[-1])

    @property
    def Tp(self) -> int:
        return int(self.cu_p[-1])


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _uniform(rng, lo, hi, shape):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def _image_positions(temporal: int, gh: int, gw: int) -> np.ndarray:
    """[3, gh*gw]: one shared temporal index, height/width tile the grid row-major."""
    hh, ww = np.meshgrid(np.arange(gh, dtype=np.int32), np.arange(gw, dtype=np.int32),
                         indexing="ij")
    t = np.full(gh * gw, temporal, dtype=np.int32)
    return np.stack([t, hh.reshape(-1), ww.reshape(-1)]).astype(np.int32)


def _text_positions(start: int, n: int) -> np.ndarray:
    """[3, n]: text tokens count up on the temporal axis, height = width = 0."""
    t = np.arange(start, start + n, dtype=np.int32)
    z = np.zeros(n, dtype=np.int32)
    return np.stack([t, z, z]).astype(np.int32)


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


CONFIG_NAMES = ("tiny", "small", "mid", "large", "editing")


def make(name: str, seed: int = 0, *, pixels: bool = True) -> Workload:
    """Build one of the five named workloads.

    Draw order from one PCG64 stream: q, k, v (generation block); prefix keys
    and values; norm weights q_t, q_hw, k_t, k_hw; understanding-branch key
    norm weights where the prefix is built; per-sample text lengths (editing);
    pixel noise; synthetic x0 prediction.
    """
    if name not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {name!r}; expected one of {CONFIG_NAMES}")
    rng = np.random.default_rng(seed)

    if name == "tiny":
        dtype, B, Hq, Hkv = "f32", 1, 4, 1
        grids = [(4, 4)]
        text_len = [16]
        prefix_kind = "built"
        n_steps, img_px = 1, 128
    elif name == "small":
        dtype, B, Hq, Hkv = "bf16", 1, 32, 8
        grids = [(16, 16)]
        text_len = [64]
        prefix_kind = "built"
        n_steps, img_px = 8, 512
    elif name == "mid":
        dtype, B, Hq, Hkv = "bf16", 1, 32, 8
        grids = [(32, 32)]
        text_len = [256]
        prefix_kind = "direct"
        n_steps, img_px = 20, 1024
    elif name == "large":
        dtype, B, Hq, Hkv = "bf16", 1, 32, 8
        grids = [(64, 64)]
        text_len = [512]
        prefix_kind = "direct"
        n_steps, img_px = 20, 2048
    else:  # editing
        dtype, B, Hq, Hkv = "bf16", 4, 32, 8
        grids = [(32, 32)] * 4
        text_len = None  # drawn below, after the tensors that do not depend on it
        prefix_kind = "built"
        n_steps, img_px = 20, 1024

    n_img = [gh * gw for gh, gw in grids]
    Tq = sum(n_img)
    q = _normal(rng, (Tq, Hq, HEAD_DIM), dtype)
    k = _normal(rng, (Tq, Hkv, HEAD_DIM), dtype)
    v = _normal(rng, (Tq, Hkv, HEAD_DIM), dtype)

    if name == "editing":
        # the text length must be known before the prefix is drawn
        L = rng.integers(64, 257, size=B).astype(np.int32)
        text_len = [int(x) for x in L]
        ref_grid, suffix = (32, 32), 32
        n_prefix = [l + ref_grid[0] * ref_grid[1] + suffix for l in text_len]
    else:
        n_prefix = list(text_len)
    Tp = sum(n_prefix)

    k_prefix_raw = _normal(rng, (Tp, Hkv, HEAD_DIM), dtype)
    v_prefix = _normal(rng, (Tp, Hkv, HEAD_DIM), dtype)
    wq_t = _uniform(rng, 0.5, 1.5, HALF)
    wq_hw = _uniform(rng, 0.5, 1.5, HALF)
    wk_t = _uniform(rng, 0.5, 1.5, HALF)
    wk_hw = _uniform(rng, 0.5, 1.5, HALF)

    wl = dict(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, grids=grids, n_img=n_img,
              n_prefix=n_prefix, q=q, k=k, v=v, wq_t=wq_t, wq_hw=wq_hw, wk_t=wk_t,
              wk_hw=wk_hw, cu_q=_cu(n_img), cu_p=_cu(n_prefix), prefix_kind=prefix_kind,
              v_prefix=v_prefix)

    # generation-block positions: temporal index = prefix length of that sample
    wl["pos_img"] = np.concatenate(
        [_image_positions(P, gh, gw) for P, (gh, gw) in zip(n_prefix, grids)], axis=1)

    if prefix_kind == "direct":
        wl["k_prefix"] = k_prefix_raw
    else:
        wl["k_prefix_pre"] = k_prefix_raw
        wl["wk_und_t"] = _uniform(rng, 0.5, 1.5, HALF)
        wl["wk_und_hw"] = _uniform(rng, 0.5, 1.5, HALF)
        parts = []
        for b in range(B):
            L = text_len[b]
            if name == "editing":
                parts += [_text_positions(0, L), _image_positions(L, 32, 32),
                          _text_positions(L + 1, 32)]
            else:
                parts.append(_text_positions(0, L))
        wl["pos_prefix"] = np.concatenate(parts, axis=1).astype(np.int32)
    wl["extras"] = {"text_len": text_len}

    # pixel-space flow-matching tensors
    wl["pixel_shape"] = (B, 3, img_px, img_px)
    wl["sigma_R"] = float(np.sqrt(n_img[0] / 256.0))
    wl["t_grid"] = tuple(k_ / n_steps for k_ in range(n_steps + 1))
    if name == "tiny":
        wl["t_grid"] = (0.6, 0.7)
    if pixels:
        npx = B * 3 * img_px * img_px
        wl["eps_pixels"] = rng.standard_normal(size=npx, dtype=np.float32)
        wl["x_hat"] = rng.standard_normal(size=npx, dtype=np.float32)
        if name == "tiny":
            # the tiny workload starts from a given z ~ N(0,1) at t = 0.6
            wl["z_start"] = wl["eps_pixels"]
    return Workload(**wl)


def cfg_branches(w: Workload, seed: int = 0) -> tuple:
    """x0 predictions of the two extra guidance branches (text-uncond, then full
    uncond) for the pixel tensors of workload w: independent N(0,1) fp32 draws of the
    same size as x_hat, from their own PCG64 stream so the workload's draws are unchanged.
    """
    assert w.x_hat is not None, "workload made without pixel tensors"
    rng = np.random.default_rng([seed, 0x6366])
    x_tu = rng.standard_normal(size=w.x_hat.size, dtype=np.float32)
    x_u = rng.standard_normal(size=w.x_hat.size, dtype=np.float32)
    return x_tu, x_u


def prefill_inputs(w: Workload, seed: int = 0) -> dict:
    """Inputs of the understanding-pass (prefill) attention over workload w's prefix
    tokens: the temporal index of every prefix token (its layout's first rotary axis when
    the workload builds the prefix by structure; 0..P_b-1, pure text, when the workload
    draws the frozen cache directly), and Q [Tp, Hq, 128], K and V [Tp, Hkv, 128] as
    N(0,1) fp32 draws from their own PCG64 stream (q, then k, then v)."""
    rng = np.random.default_rng([seed, 0x7066])
    Tp = int(w.cu_p[-1])
    if w.pos_prefix is not None:
        idx = np.ascontiguousarray(w.pos_prefix[0], dtype=np.int32)
    else:
        idx = np.concatenate([np.arange(p, dtype=np.int32) for p in w.n_prefix])
    q = rng.standard_normal(size=(Tp, w.Hq, 128), dtype=np.float32)
    k = rng.standard_normal(size=(Tp, w.Hkv, 128), dtype=np.float32)
    v = rng.standard_normal(size=(Tp, w.Hkv, 128), dtype=np.float32)
    return {"q": q, "k": k, "v": v, "idx": idx, "cu": np.asarray(w.cu_p, dtype=np.int32),
            "max_len": int(max(w.n_prefix))}


def prefill_layout(segments, Hq: int, Hkv: int, seed: int = 0) -> dict:
    """A hand-made prefill case: `segments` lists, per sample, runs of ("text", n) or
    ("image", n); text tokens take consecutive temporal indices, an image's n tokens share
    the next one.  Q/K/V are N(0,1) fp32 draws as in prefill_inputs."""
    rng = np.random.default_rng([seed, 0x706c])
    idx, cu = [], [0]
    for sample in segments:
        t = 0
        for kind, n in sample:
            if kind == "text":
                idx += list(range(t, t + n))
                t += n
            else:
                idx += [t] * n
                t += 1
        cu.append(len(idx))
    T = len(idx)
    q = rng.standard_normal(size=(T, Hq, 128), dtype=np.float32)
    k = rng.standard_normal(size=(T, Hkv, 128), dtype=np.float32)
    v = rng.standard_normal(size=(T, Hkv, 128), dtype=np.float32)
    lens = np.diff(cu)
    return {"q": q, "k": k, "v": v, "idx": np.asarray(idx, dtype=np.int32),
            "cu": np.asarray(cu, dtype=np.int32), "max_len": int(lens.max()) if len(lens) else 0}


def proj_inputs(w: Workload, seed: int = 0) -> dict:
    """Inputs of the generation branch's q/k/v projection for workload w's image tokens:
    hidden states x [Tq, Hq * 128] ~ N(0,1) and stacked weights w_qkv [(Hq + 2 Hkv) * 128,
    Hq * 128] ~ N(0, 1/hidden) (q heads, then k, then v), fp32 draws from their own PCG64
    stream; the workload's norm weights and image positions complete the inputs."""
    rng = np.random.default_rng([seed, 0x7170])
    hidden = w.Hq * 128
    x = rng.standard_normal(size=(w.Tq, hidden), dtype=np.float32)
    wq = rng.standard_normal(size=((w.Hq + 2 * w.Hkv) * 128, hidden), dtype=np.float32)
    wq *= np.float32(1.0 / np.sqrt(hidden))
    return {"x": x, "w_qkv": wq, "hidden": hidden}


def embed_inputs(w: Workload, seed: int = 0, *, C1: int = 1024, D: int = 4096) -> dict:
    """Inputs of the generation branch's embedding front end for workload w's pixel shape,
    from their own PCG64 stream (seed key [seed, 0x656d]), all fp32:
      z   [B, 3, H, W] = sigma_R * N(0,1) (the noisy image at the start of sampling);
      w1  [C1, 3, 16, 16] ~ N(0, 1/768), b1 [C1] ~ N(0, 0.1^2)  (patch convolution);
      w2  [D, C1, 2, 2] ~ N(0, 1/(4 C1)), b2 [D] ~ N(0, 0.1^2)  (2x2 merge convolution);
      time and noise-scale embedders, each wa [D, 256] ~ N(0, 1/256), ba [D], wb [D, D]
      ~ N(0, 1/D), bb [D] (biases ~ N(0, 0.1^2));
      t (the second point of the time grid), noise_scale = sigma_R, noise_scale_max = 16.
    The 1/fan-in variances keep every stage's outputs near unit size."""
    rng = np.random.default_rng([seed, 0x656D])
    Bn, C, H, Wd = w.pixel_shape
    f32 = np.float32

    def nrm(shape, var):
        return (rng.standard_normal(size=shape, dtype=f32) * f32(np.sqrt(var))).astype(f32)

    d = {"z": nrm((Bn, C, H, Wd), w.sigma_R ** 2)}
    d["w1"], d["b1"] = nrm((C1, C, 16, 16), 1.0 / (C * 256)), nrm((C1,), 0.01)
    d["w2"], d["b2"] = nrm((D, C1, 2, 2), 1.0 / (4 * C1)), nrm((D,), 0.01)
    for e in ("t", "s"):
        d[f"emb_{e}"] = (nrm((D, 256), 1.0 / 256), nrm((D,), 0.01), nrm((D, D), 1.0 / D),
                         nrm((D,), 0.01))
    d["t"] = float(w.t_grid[1]) if len(w.t_grid) > 1 else 0.5
    d["noise_scale"], d["noise_scale_max"] = float(w.sigma_R), 16.0
    return d
