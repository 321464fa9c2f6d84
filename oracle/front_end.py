"""fp64 oracle of the generation branch's embedding front end (numpy).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
use it; the HIP library never imports, links or calls it, and it never imports the library.
Every step is written from its plain definition, with library primitives (a matmul, erf)
as the only building blocks.  Channel counts are taken from the weights' shapes, so the same
code serves the model's sizes and the small pinned cases.

Pages cited:
  [A] "SenseNova-U1.5 (NEO-unify) architecture": §Vision tower -- no transformer blocks (a
      16x16 stride-16 patch convolution, GELU, interleaved two-axis rotary with base 1e4 --
      the first half of the channels rotated by the column position, the second half by the
      row position -- then a 2x2 stride-2 convolution into the backbone width; one token per
      32x32 pixels; the generation branch has its own instance); §Timestep and noise-scale
      conditioning (two embedders over a 256-wide [cos, sin] sinusoid basis, the noise scale
      normalised by its maximum, the two embeddings summed and added to every image token);
      §Timestep schedule (the shift of the time grid).
  [B] "SenseNova-U1: ... NEO-unify Architecture" §2.1 (NEOVisionEmbeddings: the two
      convolutions, the GELU and the rotary position code between them).

Layouts: pixels z [B, 3, H, W]; convolution weights in the usual [out, in, kh, kw] order;
patch grid (H/16, W/16) and token grid (H/32, W/32), both row-major; features [B, rows, C].
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

PATCH = 16   # first convolution: kernel = stride = 16
MERGE = 2    # second convolution: kernel = stride = 2
SIN_DIM = 256


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def patchify(z) -> np.ndarray:
    """[B, C, H, W] -> [B, (H/16)(W/16), C*16*16]: patch (py, px) row-major, each row ordered
    (channel, ky, kx) like a flattened [out, in, kh, kw] convolution weight.  A pure
    rearrangement ([A] §Flow matching without a VAE calls patchify a permutation)."""
    z = _f64(z)
    B, C, H, W = z.shape
    assert H % PATCH == 0 and W % PATCH == 0
    gh, gw = H // PATCH, W // PATCH
    p = z.reshape(B, C, gh, PATCH, gw, PATCH).transpose(0, 2, 4, 1, 3, 5)
    return np.ascontiguousarray(p.reshape(B, gh * gw, C * PATCH * PATCH))


def patch_conv(z, w1, b1) -> np.ndarray:
    """Conv2d(C, C1, kernel=16, stride=16) with bias ([B] §2.1's patch embedding): each
    output is the bias plus the sum over the patch's C*16*16 pixels times the weights.
    Returns [B, P, C1] over the row-major patch grid."""
    w1 = _f64(w1)
    return patchify(z) @ w1.reshape(w1.shape[0], -1).T + _f64(b1)


def gelu(x) -> np.ndarray:
    """GELU, x * Phi(x) with the normal CDF written through erf ([A] §Vision tower)."""
    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def rope2d_interleaved(h, gh, gw, theta=1.0e4) -> np.ndarray:
    """Two-axis interleaved rotary on [B, gh*gw, C] features of the row-major (gh, gw) grid
    ([A] §Vision tower): channels (2i, 2i+1) of the first C/2 form a pair rotated by the
    column position x, those of the last C/2 by the row position y; pair i of a half of
    width d = C/2 turns by position * theta^(-2i/d):
        (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi)."""
    h = _f64(h).copy()
    B, P, C = h.shape
    assert P == gh * gw and C % 4 == 0
    d = C // 2
    yy, xx = np.meshgrid(np.arange(gh, dtype=np.float64), np.arange(gw, dtype=np.float64),
                         indexing="ij")
    freq = theta ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)      # [d/2]
    for half, pos in ((0, xx.reshape(-1)), (1, yy.reshape(-1))):
        phi = pos[:, None] * freq[None, :]                                  # [P, d/2]
        c, s = np.cos(phi), np.sin(phi)
        a = h[:, :, half * d:(half + 1) * d:2].copy()
        b = h[:, :, half * d + 1:(half + 1) * d:2].copy()
        h[:, :, half * d:(half + 1) * d:2] = a * c - b * s
        h[:, :, half * d + 1:(half + 1) * d:2] = a * s + b * c
    return h


def merge_conv(h, gh, gw, w2, b2, tokens=None) -> np.ndarray:
    """Conv2d(C1, C2, kernel=2, stride=2) with bias on features h [B, gh*gw, C1] of the
    row-major patch grid ([A] §Vision tower's 2x2 merge): token (ty, tx) of the (gh/2, gw/2)
    grid is the bias plus the sum over channels c and offsets (dy, dy) of
    w2[o, c, dy, dx] * h[(2ty + dy, 2tx + dx), c].  tokens: optional token rows (indices
    into the row-major token grid) to evaluate.  Returns [B, n_tokens, C2]."""
    h, w2 = _f64(h), _f64(w2)
    B, P, C1 = h.shape
    assert P == gh * gw and gh % MERGE == 0 and gw % MERGE == 0
    th, tw = gh // MERGE, gw // MERGE
    n = np.arange(th * tw) if tokens is None else np.asarray(tokens, dtype=np.int64)
    ty, tx = n // tw, n % tw
    # gathered rows ordered (c, dy, dx) like the flattened weight
    g = np.empty((B, len(n), C1, MERGE, MERGE))
    for dy in range(MERGE):
        for dx in range(MERGE):
            g[:, :, :, dy, dx] = h[:, (MERGE * ty + dy) * gw + MERGE * tx + dx, :]
    return g.reshape(B, len(n), -1) @ w2.reshape(w2.shape[0], -1).T + _f64(b2)


def sinusoid(t, dim=SIN_DIM, max_period=10000.0) -> np.ndarray:
    """[cos, sin] sinusoid basis of a scalar ([A] §Timestep and noise-scale conditioning:
    256 wide, cosines first): frequencies exp(-ln(max_period) * i / (dim/2)), i < dim/2."""
    half = dim // 2
    freqs = np.exp(-math.log(max_period) * np.arange(half, dtype=np.float64) / half)
    args = float(t) * freqs
    return np.concatenate([np.cos(args), np.sin(args)])


def silu(x) -> np.ndarray:
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def embedder_mlp(e, wa, ba, wb, bb) -> np.ndarray:
    """The embedder's two layers: wb @ silu(wa @ e + ba) + bb (wa [D, 256], wb [D, D])."""
    return _f64(wb) @ silu(_f64(wa) @ _f64(e) + _f64(ba)) + _f64(bb)


def cond_embed(t, noise_scale, noise_scale_max, emb_t, emb_s) -> np.ndarray:
    """The conditioning vector added to every image token: the time embedder of t plus the
    noise-scale embedder of noise_scale / noise_scale_max ([A] §Timestep and noise-scale
    conditioning).  emb_t, emb_s: (wa, ba, wb, bb) each."""
    return (embedder_mlp(sinusoid(t), *emb_t)
            + embedder_mlp(sinusoid(float(noise_scale) / float(noise_scale_max)), *emb_s))


def gen_embed(z, w1, b1, w2, b2, cond, theta=1.0e4, tokens=None) -> np.ndarray:
    """The whole front end: tokens = merge_conv(rope2d(gelu(patch_conv(z)))) + cond, over
    the row-major (H/32, W/32) token grid.  tokens: optional token rows; only the patches
    they cover are evaluated.  Returns [B, n_tokens, C2]."""
    z = _f64(z)
    B, C, H, W = z.shape
    gh, gw = H // PATCH, W // PATCH
    if tokens is None:
        h = rope2d_interleaved(gelu(patch_conv(z, w1, b1)), gh, gw, theta)
        return merge_conv(h, gh, gw, w2, b2) + _f64(cond)
    # evaluate only the patches under the requested tokens: build a sparse copy of the
    # feature grid holding those patches (the others are never read)
    tokens = np.asarray(tokens, dtype=np.int64)
    tw = gw // MERGE
    ty, tx = tokens // tw, tokens % tw
    pts = np.unique(np.concatenate([(MERGE * ty + dy) * gw + MERGE * tx + dx
                                    for dy in range(MERGE) for dx in range(MERGE)]))
    w1 = _f64(w1)
    rows = patchify(z)[:, pts, :] @ w1.reshape(w1.shape[0], -1).T + _f64(b1)
    g = gelu(rows)
    # rotary of the selected patches at their own grid positions
    d = g.shape[2] // 2
    freq = theta ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    for half, pos in ((0, (pts % gw).astype(np.float64)), (1, (pts // gw).astype(np.float64))):
        phi = pos[:, None] * freq[None, :]
        c, s = np.cos(phi), np.sin(phi)
        a = g[:, :, half * d:(half + 1) * d:2].copy()
        b = g[:, :, half * d + 1:(half + 1) * d:2].copy()
        g[:, :, half * d:(half + 1) * d:2] = a * c - b * s
        g[:, :, half * d + 1:(half + 1) * d:2] = a * s + b * c
    h = np.zeros((B, gh * gw, g.shape[2]))
    h[:, pts, :] = g
    return merge_conv(h, gh, gw, w2, b2, tokens) + _f64(cond)


def shift_time(t, shift) -> float:
    """[A] §Timestep schedule: sigma = 1 - t, sigma <- shift sigma / (1 + (shift - 1) sigma),
    t <- 1 - sigma."""
    sigma = 1.0 - float(t)
    sigma = shift * sigma / (1.0 + (shift - 1.0) * sigma)
    return 1.0 - sigma
