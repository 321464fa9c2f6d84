"""Pins of the embedding front end's oracle (oracle/front_end.py) against what the pages and
the mathematics fix: brute-force convolutions on tiny inputs, one-hot weights, closed forms
and table values, and the invariants of the rotary and of the sinusoid basis.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import front_end as fe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# -- patch convolution: [B] §2.1, [A] §Vision tower ---------------------------------------

def test_patch_conv_brute_force():
    """Explicit loops over every output, input channel and kernel tap on a 2-image, 3-channel
    32x48 input with 3 output channels."""
    rng = np.random.default_rng(0)
    z = rng.standard_normal((2, 3, 32, 48))
    w = rng.standard_normal((3, 3, 16, 16))
    b = rng.standard_normal(3)
    got = fe.patch_conv(z, w, b)                       # [2, 2*3, 3]
    for bi in range(2):
        for py in range(2):
            for px in range(3):
                for o in range(3):
                    acc = [b[o]]
                    for c in range(3):
                        for ky in range(16):
                            for kx in range(16):
                                acc.append(w[o, c, ky, kx] * z[bi, c, 16 * py + ky, 16 * px + kx])
                    assert got[bi, py * 3 + px, o] == pytest.approx(math.fsum(acc), abs=1e-11)


def test_patch_conv_one_hot_picks_a_pixel():
    """A weight with a single 1 at (c, ky, kx) copies that pixel of every patch (plus bias):
    catches a transposed kernel, a swapped channel/row order or a wrong patch stride."""
    rng = np.random.default_rng(1)
    z = rng.standard_normal((1, 3, 48, 32))
    for c, ky, kx in [(0, 0, 0), (2, 15, 3), (1, 4, 15)]:
        w = np.zeros((1, 3, 16, 16))
        w[0, c, ky, kx] = 1.0
        got = fe.patch_conv(z, w, [0.5])[0, :, 0]
        want = np.array([z[0, c, 16 * py + ky, 16 * px + kx] + 0.5
                         for py in range(3) for px in range(2)])
        np.testing.assert_array_equal(got, want)


# -- GELU -------------------------------------------------------------------------------

def test_gelu_table_values():
    """x Phi(x) with Phi from the standard normal table (Phi(1) = 0.8413447460685429,
    Phi(2) = 0.9772498680518208, Phi(3) = 0.9986501019683699); GELU(0) = 0; and
    GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1)."""
    for x, phi in [(1.0, 0.8413447460685429), (2.0, 0.9772498680518208),
                   (3.0, 0.9986501019683699)]:
        assert fe.gelu(x) == pytest.approx(x * phi, rel=1e-14)
        assert fe.gelu(-x) == pytest.approx(-x * (1.0 - phi), rel=1e-12)
    assert fe.gelu(0.0) == 0.0
    xs = np.linspace(-6, 6, 49)
    np.testing.assert_allclose(fe.gelu(xs) - fe.gelu(-xs), xs, atol=1e-14)


# -- interleaved two-axis rotary: [A] §Vision tower ----------------------------------------

def _one_hot_rows(C, ch, n):
    h = np.zeros((1, n, C))
    h[0, :, ch] = 1.0
    return h


def test_rope2d_first_pair_turns_by_the_position():
    """Pair 0 of each half has frequency 1 whatever the base: e_0 at grid column x becomes
    (cos x, sin x) in channels (0, 1); e_{C/2} at row y becomes (cos y, sin y) in channels
    (C/2, C/2 + 1); the partner e_1 goes to (-sin, cos).  Catches a sign, a pairing that is
    not interleaved, or the two axes swapped."""
    C, gh, gw = 16, 3, 5
    for ch, axis in [(0, "x"), (C // 2, "y")]:
        out = fe.rope2d_interleaved(_one_hot_rows(C, ch, gh * gw), gh, gw, theta=7.0)[0]
        out1 = fe.rope2d_interleaved(_one_hot_rows(C, ch + 1, gh * gw), gh, gw, theta=7.0)[0]
        for p in range(gh * gw):
            pos = (p % gw) if axis == "x" else (p // gw)
            assert out[p, ch] == pytest.approx(math.cos(pos), abs=1e-15)
            assert out[p, ch + 1] == pytest.approx(math.sin(pos), abs=1e-15)
            assert out1[p, ch] == pytest.approx(-math.sin(pos), abs=1e-15)
            assert out1[p, ch + 1] == pytest.approx(math.cos(pos), abs=1e-15)
            others = np.delete(out[p], [ch, ch + 1])
            assert np.all(others == 0.0)


def test_rope2d_axes_and_frequency_ladder():
    """The first half moves only with the column, the second only with the row; the angle of
    pair i (read back with atan2 from a one-hot input at position 1) falls by the same factor
    base^(-2/d) from pair to pair, d = C/2, reaching base^(-2(d/2 - 1)/d) at the last pair."""
    C, gh, gw, theta = 64, 2, 2, 1.0e4
    rng = np.random.default_rng(3)
    h = rng.standard_normal((1, gh * gw, C))
    out = fe.rope2d_interleaved(h, gh, gw, theta)[0]
    d = C // 2
    # grid (0,0) unchanged; (0,1) changes only the first half; (1,0) only the second
    np.testing.assert_array_equal(out[0], h[0, 0])
    np.testing.assert_array_equal(out[1, d:], h[0, 1, d:])
    np.testing.assert_array_equal(out[2, :d], h[0, 2, :d])
    ang = []
    for i in range(d // 2):
        o = fe.rope2d_interleaved(_one_hot_rows(C, 2 * i, gh * gw), gh, gw, theta)[0]
        ang.append(math.atan2(o[1, 2 * i + 1], o[1, 2 * i]))       # column 1, row 0
    ang = np.array(ang)
    assert ang[0] == pytest.approx(1.0, abs=1e-15)
    np.testing.assert_allclose(ang[1:] / ang[:-1], theta ** (-2.0 / d), rtol=1e-12)
    assert ang[-1] == pytest.approx(theta ** (-2.0 * (d // 2 - 1) / d), rel=1e-12)


def test_rope2d_norms_and_relative_position():
    """Rotations keep each pair's length, and the product of two rotated rows depends only on
    the difference of their grid positions (per axis)."""
    C, gh, gw = 32, 4, 6
    rng = np.random.default_rng(4)
    a, b = rng.standard_normal(C), rng.standard_normal(C)
    ha = np.tile(a, (1, gh * gw, 1))
    hb = np.tile(b, (1, gh * gw, 1))
    ra, rb = fe.rope2d_interleaved(ha, gh, gw)[0], fe.rope2d_interleaved(hb, gh, gw)[0]
    np.testing.assert_allclose(ra[:, 0::2] ** 2 + ra[:, 1::2] ** 2,
                               np.tile(a[0::2] ** 2 + a[1::2] ** 2, (gh * gw, 1)), rtol=1e-13)
    # positions (y, x): (1, 2) vs (2, 5) and (0, 0) vs (1, 3): same difference (1, 3)
    idx = lambda y, x: y * gw + x
    np.testing.assert_allclose(ra[idx(1, 2)] @ rb[idx(2, 5)], ra[idx(0, 0)] @ rb[idx(1, 3)],
                               rtol=1e-12)


# -- 2x2 merge convolution -------------------------------------------------------------------

def test_merge_conv_brute_force_and_token_subset():
    """Explicit sums over channels and the 2x2 window on a 4x6 patch grid; a token subset
    returns the same rows."""
    rng = np.random.default_rng(5)
    gh, gw, C1, C2 = 4, 6, 5, 3
    h = rng.standard_normal((2, gh * gw, C1))
    w = rng.standard_normal((C2, C1, 2, 2))
    b = rng.standard_normal(C2)
    got = fe.merge_conv(h, gh, gw, w, b)
    tw = gw // 2
    for bi in range(2):
        for n in range(got.shape[1]):
            ty, tx = divmod(n, tw)
            for o in range(C2):
                acc = [b[o]] + [w[o, c, dy, dx] * h[bi, (2 * ty + dy) * gw + 2 * tx + dx, c]
                                for c in range(C1) for dy in range(2) for dx in range(2)]
                assert got[bi, n, o] == pytest.approx(math.fsum(acc), abs=1e-12)
    sub = fe.merge_conv(h, gh, gw, w, b, tokens=[5, 0, 3])
    np.testing.assert_allclose(sub, got[:, [5, 0, 3]], atol=1e-14)


def test_merge_conv_one_hot_picks_a_window_cell():
    """A weight with a single 1 at (c, dy, dx) copies channel c of patch (2ty+dy, 2tx+dx)."""
    rng = np.random.default_rng(6)
    gh, gw = 4, 4
    h = rng.standard_normal((1, gh * gw, 3))
    for c, dy, dx in [(0, 0, 0), (2, 1, 0), (1, 0, 1), (2, 1, 1)]:
        w = np.zeros((1, 3, 2, 2))
        w[0, c, dy, dx] = 1.0
        got = fe.merge_conv(h, gh, gw, w, [0.0])[0, :, 0]
        want = [h[0, (2 * ty + dy) * gw + 2 * tx + dx, c] for ty in range(2) for tx in range(2)]
        np.testing.assert_array_equal(got, want)


# -- time and noise-scale conditioning: [A] §Timestep and noise-scale conditioning ----------

def test_sinusoid_basis():
    """Cosines first: t = 0 gives 128 ones then 128 zeros; entry 0 / 128 is (cos t, sin t)
    (frequency 1); entry 127 / 255 turns at 10000^(-127/128); the first half is even in t,
    the second odd; cos^2 + sin^2 = 1 per frequency."""
    e0 = fe.sinusoid(0.0)
    assert e0.shape == (256,)
    np.testing.assert_array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    t = 0.37
    e = fe.sinusoid(t)
    assert (e[0], e[128]) == (pytest.approx(math.cos(t), abs=1e-16), pytest.approx(math.sin(t), abs=1e-16))
    f = 10000.0 ** (-127.0 / 128.0)
    assert e[255] == pytest.approx(math.sin(t * f), rel=1e-13)
    em = fe.sinusoid(-t)
    np.testing.assert_allclose(em[:128], e[:128], atol=1e-16)
    np.testing.assert_allclose(em[128:], -e[128:], atol=1e-16)
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-15)


def test_silu_and_embedder_mlp():
    """SiLU(1) = 1 / (1 + e^-1) = 0.7310585786300049 and SiLU(x) - SiLU(-x) = x; zero second
    layer weights leave the second bias; selection weights route one sinusoid entry."""
    assert fe.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    xs = np.linspace(-5, 5, 21)
    np.testing.assert_allclose(fe.silu(xs) - fe.silu(-xs), xs, atol=1e-14)
    rng = np.random.default_rng(7)
    D = 8
    wa, ba = rng.standard_normal((D, 256)), rng.standard_normal(D)
    bb = rng.standard_normal(D)
    e = fe.sinusoid(0.3)
    np.testing.assert_array_equal(fe.embedder_mlp(e, wa, ba, np.zeros((D, D)), bb), bb)
    wa = np.zeros((D, 256)); wa[np.arange(D), 128 + np.arange(D)] = 1.0   # sin entries 0..7
    wb = np.eye(D)
    got = fe.embedder_mlp(e, wa, np.zeros(D), wb, np.zeros(D))
    np.testing.assert_allclose(got, fe.silu(e[128:128 + D]), rtol=1e-15)


def test_cond_embed_sums_the_two_embedders():
    """The time embedder sees t; the noise embedder sees noise_scale / noise_scale_max; the
    result is their sum (a zero noise embedder leaves its bias)."""
    rng = np.random.default_rng(8)
    D = 6
    mk = lambda: (rng.standard_normal((D, 256)), rng.standard_normal(D),
                  rng.standard_normal((D, D)), rng.standard_normal(D))
    et, es = mk(), mk()
    got = fe.cond_embed(0.25, 3.0, 12.0, et, es)
    want = fe.embedder_mlp(fe.sinusoid(0.25), *et) + fe.embedder_mlp(fe.sinusoid(0.25), *es)
    np.testing.assert_allclose(got, want, rtol=1e-14)
    zero = (np.zeros((D, 256)), np.zeros(D), np.zeros((D, D)), es[3])
    np.testing.assert_allclose(fe.cond_embed(0.6, 3.0, 12.0, et, zero),
                               fe.embedder_mlp(fe.sinusoid(0.6), *et) + es[3], rtol=1e-14)


def test_shift_time_worked_values():
    """Hand-worked schedule values (tests/golden/time_shift.json); shift 1 is the identity;
    the shifted grid stays increasing."""
    with open(os.path.join(GOLDEN, "time_shift.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert fe.shift_time(c["t"], c["shift"]) == pytest.approx(float(Fraction(c["t_shifted"])), abs=1e-15)
    for t in np.linspace(0, 1, 11):
        assert fe.shift_time(t, 1.0) == pytest.approx(t, abs=1e-15)
    ts = [fe.shift_time(k / 20, 3.0) for k in range(21)]
    assert all(b > a for a, b in zip(ts, ts[1:]))


# -- the whole front end -------------------------------------------------------------------

def test_gen_embed_composition_and_subset():
    """The front end is merge(rope(gelu(conv))) + cond over the token grid, and a token
    subset (evaluating only its patches) gives the same rows."""
    rng = np.random.default_rng(9)
    z = rng.standard_normal((2, 3, 64, 96))
    C1, C2 = 8, 5
    w1, b1 = rng.standard_normal((C1, 3, 16, 16)) / 27.0, rng.standard_normal(C1)
    w2, b2 = rng.standard_normal((C2, C1, 2, 2)), rng.standard_normal(C2)
    cond = rng.standard_normal(C2)
    full = fe.gen_embed(z, w1, b1, w2, b2, cond)
    gh, gw = 4, 6
    h = fe.rope2d_interleaved(fe.gelu(fe.patch_conv(z, w1, b1)), gh, gw)
    np.testing.assert_allclose(full, fe.merge_conv(h, gh, gw, w2, b2) + cond, atol=1e-13)
    rows = [4, 0, 5, 2]
    np.testing.assert_allclose(fe.gen_embed(z, w1, b1, w2, b2, cond, tokens=rows),
                               full[:, rows], atol=1e-13)
