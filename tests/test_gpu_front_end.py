"""GPU parity of the embedding front end (through the C ABI) against the fp64 oracle.

Per stage, on inputs both sides take from the seeded generators (no stage reads another
stage's GPU output): patchify bit-exact (a permutation plus one bf16 rounding); the patch
convolution + GELU + rotary, the merge convolution and the whole chain within the front
end's tolerance (tests/harness.py); the conditioning vector (fp32 products of bf16
weights) within max-abs 1e-4 relative to its size.
"""
import sys
import time

import numpy as np
import pytest

import workloads as W
from oracle import front_end as fe
from tests import harness as H

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch


def _say(msg):
    print(f"[gpu-front-end] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def neo():
    _cuda()
    import pixel_space_flow_amd as P
    P.lib()  # raises if the library is missing
    return P


def _weights(rng, C1, D):
    """Small seeded weight sets for the shape cases (fp32, bf16-exact)."""
    r = W.bf16_round
    w1 = r((rng.standard_normal((C1, 3, 16, 16)) / np.sqrt(768)).astype(np.float32))
    b1 = (0.1 * rng.standard_normal(C1)).astype(np.float32)
    w2 = r((rng.standard_normal((D, C1, 2, 2)) / np.sqrt(4 * C1)).astype(np.float32))
    b2 = (0.1 * rng.standard_normal(D)).astype(np.float32)
    return w1, b1, w2, b2


def _emb(rng, D):
    r = W.bf16_round
    return tuple((r((rng.standard_normal((D, 256)) / 16.0).astype(np.float32)),
                  (0.1 * rng.standard_normal(D)).astype(np.float32),
                  r((rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)),
                  (0.1 * rng.standard_normal(D)).astype(np.float32)) for _ in range(2))


def _dev_emb(e):
    wa, ba, wb, bb = e
    return (H.dev(wa, "bf16"), H.dev_f32(ba), H.dev(wb, "bf16"), H.dev_f32(bb))


def _w2_dev(w2):
    """[D, C1, 2, 2] convolution weight -> the call's [D, 2, 2, C1] layout."""
    return H.dev(np.ascontiguousarray(w2.transpose(0, 2, 3, 1)), "bf16")


def _chain(neo, z, w1, b1, w2, b2, emb_t, emb_s, t, ns, ns_max, what, tokens=None):
    torch = _cuda()
    B, _, Hh, Ww = z.shape
    _say(f"chain {what}: z {z.shape} C1={w1.shape[0]} D={w2.shape[0]}")
    out = neo.gen_embed(H.dev_f32(z), H.dev(w1.reshape(w1.shape[0], -1), "bf16"), H.dev_f32(b1),
                        _w2_dev(w2), H.dev_f32(b2), _dev_emb(emb_t), _dev_emb(emb_s), t, ns, ns_max)
    torch.cuda.synchronize()
    cond = fe.cond_embed(t, ns, ns_max, emb_t, emb_s)
    n = (Hh // 32) * (Ww // 32)
    got = H.host(out).reshape(B, n, -1)
    t0 = time.perf_counter()
    ref = fe.gen_embed(z, w1, b1, w2, b2, cond, tokens=tokens)
    _say(f"chain {what}: oracle {time.perf_counter() - t0:.1f} s")
    if tokens is not None:
        got = got[:, tokens]
    H.assert_front_end(got, ref, f"front end {what}")


# --------------------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hh,Ww", [(1, 128, 128), (2, 64, 96), (1, 48, 80)])
def test_patchify_bit_exact(neo, B, Hh, Ww):
    """A rearrangement plus one round-to-nearest-even per pixel: every bit equal to the
    oracle's patch rows rounded on the host."""
    torch = _cuda()
    rng = np.random.default_rng(B * Hh + Ww)
    z = (3.0 * rng.standard_normal((B, 3, Hh, Ww))).astype(np.float32)
    _say(f"patchify {z.shape}")
    p = neo.gen_patchify(H.dev_f32(z))
    torch.cuda.synchronize()
    want = W.bf16_round(fe.patchify(z).reshape(-1, 768).astype(np.float32))
    got = p.view(torch.int16).cpu().numpy()
    ref = (want.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("B,Hh,Ww,C1", [(1, 256, 256, 1024), (2, 64, 96, 192), (1, 32, 32, 64),
                                         (3, 160, 48, 320)])
def test_patch_embed(neo, B, Hh, Ww, C1):
    """Convolution + bias, GELU, rotary on bf16-exact patches: partial feature tiles (C1 not
    a multiple of 256), patch counts below one tile and across several."""
    torch = _cuda()
    rng = np.random.default_rng(C1 + Hh)
    z = W.bf16_round((2.0 * rng.standard_normal((B, 3, Hh, Ww))).astype(np.float32))
    w1, b1, _, _ = _weights(rng, C1, 32)
    _say(f"patch embed z {z.shape} C1={C1}")
    patches = H.dev(fe.patchify(z).reshape(-1, 768), "bf16")
    h = neo.gen_patch_embed(patches, B, Hh, Ww, H.dev(w1.reshape(C1, -1), "bf16"), H.dev_f32(b1))
    torch.cuda.synchronize()
    gh, gw = Hh // 16, Ww // 16
    ref = fe.rope2d_interleaved(fe.gelu(fe.patch_conv(z, w1, b1)), gh, gw)
    H.assert_front_end(H.host(h).reshape(ref.shape), ref, f"patch embed {z.shape} C1={C1}")


@pytest.mark.parametrize("B,Hh,Ww,C1", [(1, 256, 256, 1024), (2, 64, 96, 192), (1, 32, 32, 64),
                                         (3, 160, 48, 320), (1, 2080, 2048, 1024)])
def test_patch_embed_px(neo, B, Hh, Ww, C1):
    """The one-launch form from the pixels: every bit equal to patchify followed by the
    patch convolution (the same RNE rounding of the same pixels, the same products in the
    same order), on pixels that are not bf16-exact; 2080 x 2048 gives 260 tiles, so half
    tiles run too.  The smaller shapes are also compared with the oracle on the rounded
    pixels."""
    torch = _cuda()
    rng = np.random.default_rng(C1 + Hh + 7)
    z = (2.0 * rng.standard_normal((B, 3, Hh, Ww))).astype(np.float32)
    w1, b1, _, _ = _weights(rng, C1, 32)
    _say(f"patch embed from pixels z {z.shape} C1={C1}")
    zd, w1d, b1d = H.dev_f32(z), H.dev(w1.reshape(C1, -1), "bf16"), H.dev_f32(b1)
    h_px = neo.gen_patch_embed_px(zd, w1d, b1d)
    h_two = neo.gen_patch_embed(neo.gen_patchify(zd), B, Hh, Ww, w1d, b1d)
    torch.cuda.synchronize()
    assert torch.equal(h_px.view(torch.int16), h_two.view(torch.int16)), "differs from the two calls"
    if Hh * Ww <= 256 * 256:
        zr = W.bf16_round(z)
        ref = fe.rope2d_interleaved(fe.gelu(fe.patch_conv(zr, w1, b1)), Hh // 16, Ww // 16)
        H.assert_front_end(H.host(h_px).reshape(ref.shape), ref, f"patch embed px {z.shape} C1={C1}")


@pytest.mark.parametrize("D,t,ns", [(4096, 0.35, 4.0), (96, 0.0, 1.0), (512, 0.95, 16.0)])
def test_cond_embed(neo, D, t, ns):
    """Both embedders, summed: fp32 results of bf16 weights against fp64."""
    torch = _cuda()
    rng = np.random.default_rng(D)
    emb_t, emb_s = _emb(rng, D)
    _say(f"cond D={D} t={t} noise {ns}/16")
    cond, hidden = neo.gen_cond_embed(t, ns, 16.0, _dev_emb(emb_t), _dev_emb(emb_s))
    torch.cuda.synchronize()
    ref = fe.cond_embed(t, ns, 16.0, emb_t, emb_s)
    got = H.host(cond)
    scale = max(1.0, float(np.sqrt(np.mean(ref ** 2))))
    err = float(np.max(np.abs(got - ref)))
    assert err <= 1e-4 * scale, f"cond max-abs {err:.3e} > {1e-4 * scale:.3e}"
    href = np.stack([fe.silu(emb_t[0] @ fe.sinusoid(t) + emb_t[1]),
                     fe.silu(emb_s[0] @ fe.sinusoid(ns / 16.0) + emb_s[1])])
    errh = float(np.max(np.abs(H.host(hidden) - href)))
    assert errh <= 1e-4, f"hidden max-abs {errh:.3e}"
    print(f"[parity] cond D={D}: max-abs {err:.3e}, hidden {errh:.3e}", flush=True)


@pytest.mark.parametrize("B,Hh,Ww,C1,D", [(1, 512, 512, 1024, 4096), (2, 64, 96, 192, 96),
                                           (1, 32, 32, 64, 32), (3, 160, 224, 128, 288)])
def test_merge_embed(neo, B, Hh, Ww, C1, D):
    """2x2 merge + bias + cond on seeded bf16 features: token counts below one tile and
    across several, D not a multiple of 256 (partial feature tiles), several images."""
    torch = _cuda()
    rng = np.random.default_rng(D + C1)
    gh, gw = Hh // 16, Ww // 16
    h = W.bf16_round(rng.standard_normal((B, gh * gw, C1)).astype(np.float32))
    _, _, w2, b2 = _weights(rng, C1, D)
    cond = rng.standard_normal(D).astype(np.float32)
    _say(f"merge B={B} {Hh}x{Ww} C1={C1} D={D}")
    tok = neo.gen_merge_embed(H.dev(h.reshape(-1, C1), "bf16"), B, Hh, Ww, _w2_dev(w2),
                              H.dev_f32(b2), H.dev_f32(cond))
    torch.cuda.synchronize()
    ref = fe.merge_conv(h, gh, gw, w2, b2) + cond
    H.assert_front_end(H.host(tok).reshape(ref.shape), ref, f"merge {Hh}x{Ww} C1={C1} D={D}")


# --------------------------------------------------------------------------------------
# the whole front end
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_front_end_configs(neo, name):
    """Each workload's pixel shape with the model's widths (C1 = 1024, D = 4096); every
    token of every image."""
    w = W.make(name, pixels=False)
    d = W.embed_inputs(w)
    r = W.bf16_round
    emb = [tuple(r(a) if a.ndim == 2 else a for a in d[k]) for k in ("emb_t", "emb_s")]
    B, _, Hh, Ww = d["z"].shape
    _chain(neo, d["z"], r(d["w1"]), d["b1"], r(d["w2"]), d["b2"], emb[0], emb[1], d["t"],
           d["noise_scale"], d["noise_scale_max"], name)


@pytest.mark.parametrize("B,Hh,Ww,C1,D", [(2, 96, 64, 192, 160), (1, 32, 32, 64, 32)])
def test_front_end_shapes(neo, B, Hh, Ww, C1, D):
    """Non-square images, one-token images, several images, narrow widths."""
    rng = np.random.default_rng(Hh * Ww + C1)
    z = (2.0 * rng.standard_normal((B, 3, Hh, Ww))).astype(np.float32)
    w1, b1, w2, b2 = _weights(rng, C1, D)
    emb_t, emb_s = _emb(rng, D)
    _chain(neo, z, w1, b1, w2, b2, emb_t, emb_s, 0.6, 2.0, 16.0, f"B={B} {Hh}x{Ww} C1={C1} D={D}")
