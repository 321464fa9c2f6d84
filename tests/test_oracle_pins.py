"""Pins for the fp64 oracle: values and properties fixed by the pages and by
mathematics, independent of the oracle's own code.

Each test names what it would catch.  Pages:
  [A] "SenseNova-U1.5 (NEO-unify) architecture" (Mobius design note)
  [B] "SenseNova-U1: Unifying Multimodal Understanding and Generation with
      NEO-unify Architecture" (paper notes)
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------------------
# Euler update: [A] §Flow matching without a VAE; [B] §2.2 and §2.7
# --------------------------------------------------------------------------------------

def test_euler_worked_example():
    """[B] §2.2 numeric example: t=0.6, x=1, eps=0, sigma_R=1 gives z_t=0.6, v*=1.0.

    A perfect x0 prediction (x0 = x) taken from z_t must move z by dt * v*; with
    t_next = 1 it lands exactly on x.  Catches a wrong divisor (t instead of 1-t),
    a wrong sign in (x0 - z) or a dropped dt."""
    g = _golden("fm_worked_example.json")
    z_t = g["t"] * g["x"] + (1 - g["t"]) * g["sigma_R"] * g["epsilon"]
    assert z_t == pytest.approx(g["z_t"], abs=1e-15)
    for t_next in (0.7, 0.8, 1.0):
        z1 = oracle.euler_step([g["z_t"]], [g["x"]], g["t"], t_next)[0]
        v = (z1 - g["z_t"]) / (t_next - g["t"])
        assert v == pytest.approx(g["v_star"], abs=1e-12)
    assert oracle.euler_step([g["z_t"]], [g["x"]], g["t"], 1.0)[0] == pytest.approx(g["x"], abs=1e-15)


def test_euler_clamp_cases():
    """max(1 - t, t_eps) divisor: the clamp branch and the plain branch at fixed values."""
    for c in _golden("euler_clamp.json")["cases"]:
        got = oracle.euler_step([c["z"]], [c["x0"]], c["t"], c["t_next"], c["t_eps"])[0]
        assert got == pytest.approx(c["z_next"], abs=1e-12), c["why"]


def test_euler_trajectory_stays_on_interpolant():
    """Closed form: with x0 fixed to the clean x, Euler from z_0 = sigma*eps at t=0
    reproduces z_t = t x + (1 - t) sigma eps at every grid point and ends at x.
    Catches any error in the step that a single-point check could hide."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000)
    eps = rng.standard_normal(1000)
    sigma = 2.0
    S = 20
    z = sigma * eps
    for k in range(S):
        t, tn = k / S, (k + 1) / S
        z = oracle.euler_step(z, x, t, tn)
        np.testing.assert_allclose(z, tn * x + (1 - tn) * sigma * eps, atol=1e-12, rtol=0)
    np.testing.assert_allclose(z, x, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------------------
# Split-half RMSNorm: [A] §Three rotary axes, last paragraph
# --------------------------------------------------------------------------------------

def test_norm_constant_halves_closed_form():
    """x = c1 on [0:64), c2 on [64:128) gives w_t*c1/sqrt(c1^2+eps) and
    w_hw*c2/sqrt(c2^2+eps).  Catches normalising over all 128 dims, swapping the
    two weights, or forgetting eps."""
    eps = 0.25
    c1, c2 = 3.0, -0.5
    x = np.concatenate([np.full(64, c1), np.full(64, c2)])[None]
    w_t = np.linspace(0.5, 1.5, 64)
    w_hw = np.linspace(2.0, -1.0, 64)
    y = oracle.split_rmsnorm(x, w_t, w_hw, eps)[0]
    np.testing.assert_allclose(y[:64], w_t * c1 / math.sqrt(c1 * c1 + eps), rtol=1e-14)
    np.testing.assert_allclose(y[64:], w_hw * c2 / math.sqrt(c2 * c2 + eps), rtol=1e-14)


def test_norm_unit_weight_rms():
    """With unit weights each half's output RMS is sqrt(ms / (ms + eps))."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * 0.01
    eps = 1e-4
    y = oracle.split_rmsnorm(x, np.ones(64), np.ones(64), eps)
    for s in (slice(0, 64), slice(64, 128)):
        ms = np.mean(x[:, s] ** 2, axis=1)
        np.testing.assert_allclose(np.sqrt(np.mean(y[:, s] ** 2, axis=1)),
                                   np.sqrt(ms / (ms + eps)), rtol=1e-12)


def test_norm_halves_independent_and_scale_invariant():
    """Changing one half leaves the other half's output unchanged; scaling a half by
    alpha leaves its output unchanged when eps is negligible."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128))
    w_t, w_hw = rng.uniform(0.5, 1.5, 64), rng.uniform(0.5, 1.5, 64)
    y = oracle.split_rmsnorm(x, w_t, w_hw, 1e-6)
    x2 = x.copy()
    x2[:, 64:] *= 7.0
    x2[:, 64:] += 1.0
    y2 = oracle.split_rmsnorm(x2, w_t, w_hw, 1e-6)
    np.testing.assert_array_equal(y[:, :64], y2[:, :64])
    y0 = oracle.split_rmsnorm(x, w_t, w_hw, 0.0)
    y3 = oracle.split_rmsnorm(x * 1000.0, w_t, w_hw, 0.0)
    np.testing.assert_allclose(y3, y0, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------------------
# Three-axis rotary: [A] §Three rotary axes (table), §Vision tower (half-split backbone)
# --------------------------------------------------------------------------------------

def _one_hot(d):
    x = np.zeros((1, 1, 128))
    x[0, 0, d] = 1.0
    return x


def test_rope_one_hot_closed_form():
    """Rotating the unit vector e_d gives cos(phi) at d and +-sin(phi) at its partner
    d +- w/2, with phi = p * base^(-2i/w) for slice (start, width w, base, position
    row) from the page's table.  Checks, per slice: the slice boundaries, which
    position row drives it, its base, the frequency exponent, the half-split
    pairing and the rotation's sign."""
    table = _golden("rope_axes.json")["slices"]
    theta = [s_["base"] for s_ in table if s_["axis"] == "temporal"][0]
    theta_hw = [s_["base"] for s_ in table if s_["axis"] == "height"][0]
    assert [s_["base"] for s_ in table if s_["axis"] == "width"][0] == theta_hw
    pos = np.array([[37], [11], [5]], dtype=np.int32)  # temporal, height, width
    for sl in table:
        o, w, base = sl["start"], sl["stop"] - sl["start"], sl["base"]
        p = float(pos[sl["position_row"], 0])
        half = w // 2
        for i in (0, 1, half // 2, half - 1):
            phi = p * base ** (-2.0 * i / w)
            # first element of the pair: (a, b) = (1, 0) -> (cos, sin)
            y = oracle.rope3(_one_hot(o + i), pos, theta, theta_hw)[0, 0]
            expect = np.zeros(128)
            expect[o + i] = math.cos(phi)
            expect[o + i + half] = math.sin(phi)
            np.testing.assert_allclose(y, expect, atol=1e-13)
            # second element of the pair: (a, b) = (0, 1) -> (-sin, cos)
            y = oracle.rope3(_one_hot(o + i + half), pos, theta, theta_hw)[0, 0]
            expect = np.zeros(128)
            expect[o + i] = -math.sin(phi)
            expect[o + i + half] = math.cos(phi)
            np.testing.assert_allclose(y, expect, atol=1e-13)


def test_rope_position_zero_is_identity():
    """Text tokens sit at h = w = 0, so their spatial dims are left unrotated; at
    p = 0 on every axis the whole row is unchanged."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 2, 128))
    pos = np.array([[0, 5, 9], [0, 0, 0], [0, 0, 0]], dtype=np.int32)
    y = oracle.rope3(x, pos)
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_array_equal(y[1:, :, 64:], x[1:, :, 64:])
    assert not np.allclose(y[1:, :, :64], x[1:, :, :64])


def test_rope_pair_norms_preserved():
    """Every rotated pair keeps its length (orthogonality; catches a sign slip)."""
    rng = np.random.default_rng(5)
    T, H = 6, 3
    x = rng.standard_normal((T, H, 128))
    pos = rng.integers(0, 3000, size=(3, T)).astype(np.int32)
    y = oracle.rope3(x, pos)
    for o, w in ((0, 64), (64, 32), (96, 32)):
        h = w // 2
        n_x = x[..., o:o + h] ** 2 + x[..., o + h:o + w] ** 2
        n_y = y[..., o:o + h] ** 2 + y[..., o + h:o + w] ** 2
        np.testing.assert_allclose(n_y, n_x, rtol=1e-12)


def test_rope_composition():
    """R(a) R(b) = R(a + b) on every axis."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 2, 128))
    a = rng.integers(0, 500, size=(3, 4)).astype(np.int32)
    b = rng.integers(0, 500, size=(3, 4)).astype(np.int32)
    np.testing.assert_allclose(oracle.rope3(oracle.rope3(x, a), b), oracle.rope3(x, a + b),
                               atol=1e-11)


def test_rope_relative_position():
    """Per axis slice, <R(p) q, R(p') k> depends only on p - p': shifting one axis of
    both positions by a constant leaves every slice's score unchanged."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    pq = np.array([[700], [13], [40]], dtype=np.int32)
    pk = np.array([[512], [3], [61]], dtype=np.int32)

    def slice_scores(pq_, pk_):
        a, b = oracle.rope3(q, pq_)[0, 0], oracle.rope3(k, pk_)[0, 0]
        return [float(a[s] @ b[s]) for s in (slice(0, 64), slice(64, 96), slice(96, 128))]

    base = slice_scores(pq, pk)
    for axis, shift in ((0, 1234), (1, 50), (2, 7)):
        dq, dk = pq.copy(), pk.copy()
        dq[axis] += shift
        dk[axis] += shift
        np.testing.assert_allclose(slice_scores(dq, dk), base, atol=1e-10)
    # and a change of the difference on one axis changes exactly that slice
    dq = pq.copy()
    dq[1] += 1
    moved = slice_scores(dq, pk)
    assert moved[0] == pytest.approx(base[0], abs=1e-12)
    assert moved[2] == pytest.approx(base[2], abs=1e-12)
    assert abs(moved[1] - base[1]) > 1e-6


def test_norm_rope_order():
    """norm_rope is the norm followed by the rotary (the rotary preserves pair
    lengths, so the per-half RMS after both steps still equals the norm's)."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 2, 128))
    pos = rng.integers(0, 100, size=(3, 5)).astype(np.int32)
    w1, w2 = np.ones(64), np.ones(64)
    y = oracle.norm_rope(x, w1, w2, pos, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y[..., :64] ** 2, -1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean(y[..., 64:] ** 2, -1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(y, oracle.rope3(oracle.split_rmsnorm(x, w1, w2, 0.0), pos),
                               atol=1e-14)


# --------------------------------------------------------------------------------------
# Generation-pass attention: [A] §Mixture of Transformers, §GQA fusion does not apply
# --------------------------------------------------------------------------------------

def _attn_inputs(rng, n_img, n_pre, Hq, Hkv, D=128):
    Tq, Tp = sum(n_img), sum(n_pre)
    return dict(q=rng.standard_normal((Tq, Hq, D)), k_img=rng.standard_normal((Tq, Hkv, D)),
                v_img=rng.standard_normal((Tq, Hkv, D)), k_pre=rng.standard_normal((Tp, Hkv, D)),
                v_pre=rng.standard_normal((Tp, Hkv, D)),
                cu_q=np.concatenate([[0], np.cumsum(n_img)]).astype(np.int32),
                cu_p=np.concatenate([[0], np.cumsum(n_pre)]).astype(np.int32))


def test_attn_two_key_closed_form():
    """One prefix key with score ln 3 (after the 1/sqrt(128) scale) and one image key
    with score 0: weights 3/4 and 1/4, so O = 0.75*v1 + 0.25*v2 and lse = ln 4.
    Catches a missing or wrong softmax scale and a wrong lse."""
    D = 128
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = math.sqrt(D)
    k_pre = np.zeros((1, 1, D))
    k_pre[0, 0, 0] = math.log(3.0)
    k_img = np.zeros((1, 1, D))
    v_pre = np.full((1, 1, D), 2.0)
    v_img = np.full((1, 1, D), -6.0)
    out, lse = oracle.gen_attn(q, k_img, v_img, k_pre, v_pre, [0, 1], [0, 1], with_lse=True)
    np.testing.assert_allclose(out[0, 0], 0.75 * 2.0 + 0.25 * -6.0, atol=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(4.0), abs=1e-14)


def test_attn_gqa_head_map():
    """V of KV head g is the constant g + 1, so query head h must return
    h // (Hq/Hkv) + 1.  Catches h % Hkv or any other head map."""
    rng = np.random.default_rng(9)
    Hq, Hkv = 8, 2
    a = _attn_inputs(rng, [5], [3], Hq, Hkv)
    for g in range(Hkv):
        a["v_img"][:, g, :] = g + 1
        a["v_pre"][:, g, :] = g + 1
    out = oracle.gen_attn(**a)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h, :], h // (Hq // Hkv) + 1, atol=1e-13)


def test_attn_key_set_per_sample():
    """Sample b sees exactly its own prefix rows and its own image rows: with q = 0
    every key weighs the same, so O = (P_b*a_b + N_b*c_b)/(P_b + N_b) for prefix
    value a_b and image value c_b.  Catches dropping a segment, off-by-one ranges
    and leakage across samples."""
    rng = np.random.default_rng(10)
    n_img, n_pre = [3, 5, 2], [4, 0, 7]
    a = _attn_inputs(rng, n_img, n_pre, 2, 1)
    a["q"][:] = 0.0
    for b in range(3):
        a["v_pre"][a["cu_p"][b]:a["cu_p"][b + 1]] = 10.0 * b + 1
        a["v_img"][a["cu_q"][b]:a["cu_q"][b + 1]] = -(10.0 * b + 3)
    out = oracle.gen_attn(**a)
    for b in range(3):
        P, N = n_pre[b], n_img[b]
        expect = (P * (10.0 * b + 1) - N * (10.0 * b + 3)) / (P + N)
        np.testing.assert_allclose(out[a["cu_q"][b]:a["cu_q"][b + 1]], expect, atol=1e-12)


def test_attn_brute_force_tiny():
    """Brute force on a tiny case with numpy: scores as a matrix product, softmax,
    weighted sum over the concatenated key set."""
    rng = np.random.default_rng(11)
    a = _attn_inputs(rng, [6], [5], 4, 2)
    out, lse = oracle.gen_attn(**a, with_lse=True)
    for h in range(4):
        g = h // 2
        K = np.concatenate([a["k_pre"][:, g], a["k_img"][:, g]])
        V = np.concatenate([a["v_pre"][:, g], a["v_img"][:, g]])
        S = a["q"][:, h] @ K.T / math.sqrt(128)
        P = np.exp(S - S.max(1, keepdims=True))
        np.testing.assert_allclose(out[:, h], (P / P.sum(1, keepdims=True)) @ V, atol=1e-13)
        np.testing.assert_allclose(lse[:, h], np.log(np.exp(S).sum(1)), atol=1e-12)


def test_attn_single_key_and_constant_v():
    """A single key returns its value; a constant V returns that constant."""
    rng = np.random.default_rng(12)
    a = _attn_inputs(rng, [1], [0], 2, 1)
    np.testing.assert_allclose(oracle.gen_attn(**a)[0, 0], a["v_img"][0, 0], atol=1e-15)
    b = _attn_inputs(rng, [4], [3], 2, 1)
    b["v_img"][:] = 0.3
    b["v_pre"][:] = 0.3
    np.testing.assert_allclose(oracle.gen_attn(**b), 0.3, atol=1e-14)


def test_attn_invariants():
    """GQA equals MHA with repeated KV heads; a ragged batch equals separate calls;
    permuting image tokens permutes the outputs; the order of prefix keys is
    irrelevant."""
    rng = np.random.default_rng(13)
    Hq, Hkv = 6, 2
    a = _attn_inputs(rng, [7, 3], [4, 9], Hq, Hkv)
    out = oracle.gen_attn(**a)
    rep = {k_: (np.repeat(v_, Hq // Hkv, axis=1) if k_ in ("k_img", "v_img", "k_pre", "v_pre")
                else v_) for k_, v_ in a.items()}
    np.testing.assert_allclose(oracle.gen_attn(**rep), out, atol=1e-13)
    for b in range(2):
        qs = slice(a["cu_q"][b], a["cu_q"][b + 1])
        ps = slice(a["cu_p"][b], a["cu_p"][b + 1])
        nq, npf = qs.stop - qs.start, ps.stop - ps.start
        single = oracle.gen_attn(a["q"][qs], a["k_img"][qs], a["v_img"][qs], a["k_pre"][ps],
                                 a["v_pre"][ps], [0, nq], [0, npf])
        np.testing.assert_allclose(single, out[qs], atol=1e-13)
    perm = rng.permutation(7)
    p = dict(a)
    for k_ in ("q", "k_img", "v_img"):
        p[k_] = a[k_].copy()
        p[k_][:7] = a[k_][:7][perm]
    np.testing.assert_allclose(oracle.gen_attn(**p)[:7], out[:7][perm], atol=1e-13)
    one = _attn_inputs(rng, [4], [5], 2, 1)
    ref = oracle.gen_attn(**one)
    order = rng.permutation(5)
    swapped = dict(one)
    swapped["k_pre"], swapped["v_pre"] = one["k_pre"][order], one["v_pre"][order]
    np.testing.assert_allclose(oracle.gen_attn(**swapped), ref, atol=1e-13)


def test_attn_streaming_formulation_agrees():
    """A second, independent fp64 formulation: streaming (online) softmax over keys in
    blocks of 3, keeping a running maximum, a rescaled running sum and a rescaled running
    output, the prefix keys first and then the image keys.  It must agree with the
    oracle's two-pass evaluation to ~1e-12, output and log-sum-exp."""
    rng = np.random.default_rng(15)
    Hq, Hkv = 4, 2
    a = _attn_inputs(rng, [9, 4], [7, 11], Hq, Hkv)
    a["q"] *= 3.0  # spread the scores so the running maximum moves
    out, lse = oracle.gen_attn(**a, with_lse=True)
    scale = 1.0 / math.sqrt(128)
    for b in range(2):
        q0, q1 = a["cu_q"][b], a["cu_q"][b + 1]
        p0, p1 = a["cu_p"][b], a["cu_p"][b + 1]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [(a["k_pre"][j, g], a["v_pre"][j, g]) for j in range(p0, p1)]
            keys += [(a["k_img"][j, g], a["v_img"][j, g]) for j in range(q0, q1)]
            for i in range(q0, q1):
                m, l, acc = -math.inf, 0.0, np.zeros(128)
                for blk in range(0, len(keys), 3):
                    s = [scale * float(a["q"][i, h] @ k_) for k_, _ in keys[blk:blk + 3]]
                    m_new = max(m, max(s))
                    c = math.exp(m - m_new)  # 0 on the first block
                    l = l * c + sum(math.exp(x - m_new) for x in s)
                    acc = acc * c + sum(math.exp(x - m_new) * v_ for x, (_, v_)
                                        in zip(s, keys[blk:blk + 3]))
                    m = m_new
                np.testing.assert_allclose(out[i, h], acc / l, rtol=0, atol=1e-12)
                assert abs(lse[i, h] - (m + math.log(l))) < 1e-12


def test_attn_score_shift_invariance():
    """Adding the same vector u to every key of a KV head adds q.u (times the scale) to all
    of a query's scores: the output is unchanged and the log-sum-exp moves by exactly that
    amount.  Catches a softmax without its normalisation and an lse taken before the
    maximum is restored."""
    rng = np.random.default_rng(16)
    Hq, Hkv = 4, 2
    a = _attn_inputs(rng, [6, 5], [3, 8], Hq, Hkv)
    out, lse = oracle.gen_attn(**a, with_lse=True)
    u = rng.standard_normal((Hkv, 128))
    s = dict(a)
    s["k_img"] = a["k_img"] + u[None]
    s["k_pre"] = a["k_pre"] + u[None]
    out_s, lse_s = oracle.gen_attn(**s, with_lse=True)
    np.testing.assert_allclose(out_s, out, atol=1e-12)
    shift = np.einsum("thd,hd->th", a["q"], np.repeat(u, Hq // Hkv, axis=0)) / math.sqrt(128)
    np.testing.assert_allclose(lse_s - lse, shift, atol=1e-11)


def test_attn_sampled_rows_match_full():
    """Evaluating a sampled set of query rows returns the same values as the full call."""
    rng = np.random.default_rng(14)
    a = _attn_inputs(rng, [5, 6], [3, 2], 4, 1)
    full, lse = oracle.gen_attn(**a, with_lse=True)
    rows = np.array([10, 0, 7, 5])
    part, lse_p = oracle.gen_attn(**a, tokens=rows, with_lse=True)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(lse_p, lse[rows])


# --------------------------------------------------------------------------------------
# Classifier-free guidance + Euler step: [B] §2.7 (three branches, four code paths)
# --------------------------------------------------------------------------------------

def test_cfg_worked_examples():
    """Hand-worked step on every guidance path and both interval rules (golden fixture);
    catches a wrong sign, a swapped branch or a wrong interval rule."""
    g = _golden("cfg_worked.json")
    for c in g["cases"]:
        iv = tuple(c["cfg_interval"])
        assert oracle.cfg_path(g["t"], c["cfg_scale"], c["img_cfg_scale"], iv) == c["path"], c
        z1 = oracle.euler_step_cfg([g["z"]], [g["x0_cond"]], [g["x0_text_uncond"]],
                                   [g["x0_uncond"]], t=g["t"], t_next=g["t_next"],
                                   t_eps=g["t_eps"], cfg_scale=c["cfg_scale"],
                                   img_cfg_scale=c["img_cfg_scale"], cfg_interval=iv)[0]
        assert z1 == c["z_next"], (c, z1)


def test_cfg_weights_sum_to_one():
    """Invariant: every path is an affine combination of the branch velocities, so when
    all branches predict the same x0 the step is the single-branch Euler step."""
    rng = np.random.default_rng(7)
    z, x = rng.standard_normal(257), rng.standard_normal(257)
    for gam, gim, iv in [(4.0, 1.0, (0, 1)), (3.0, 3.0, (0, 1)), (4.0, 1.5, (0, 1)),
                         (7.5, -2.0, (0, 1)), (4.0, 1.5, (0.7, 1.0))]:
        for t, tn in [(0.1, 0.15), (0.6, 0.7), (0.99, 1.0)]:
            got = oracle.euler_step_cfg(z, x, x, x, t=t, t_next=tn, cfg_scale=gam,
                                        img_cfg_scale=gim, cfg_interval=iv)
            ref = oracle.euler_step(z, x, t, tn)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_cfg_paths_are_continuous():
    """Paths 1-3 are the reductions of the full three-branch formula named on the pages
    (gamma_img = 1; gamma = gamma_img; both 1); the fast paths must agree with the full
    formula just off those lines -- catches a fast path with a wrong branch or term."""
    rng = np.random.default_rng(11)
    z, xc, xtu, xu = (rng.standard_normal(129) for _ in range(4))
    kw = dict(t=0.3, t_next=0.35)
    eps = 1e-9
    pairs = [((4.0, 1.0), (4.0, 1.0 + eps)), ((3.0, 3.0), (3.0, 3.0 + eps)),
             ((1.0, 1.0), (1.0 + eps, 1.0 + 2 * eps))]
    for (g1, i1), (g2, i2) in pairs:
        fast = oracle.euler_step_cfg(z, xc, xtu, xu, cfg_scale=g1, img_cfg_scale=i1, **kw)
        full = oracle.euler_step_cfg(z, xc, xtu, xu, cfg_scale=g2, img_cfg_scale=i2, **kw)
        assert oracle.cfg_path(kw["t"], g2, i2) == 4 and oracle.cfg_path(kw["t"], g1, i1) != 4
        np.testing.assert_allclose(fast, full, rtol=0, atol=1e-6)


def test_cfg_in_x0_space():
    """Property: the guidance weights of each path sum to one, so guiding the x0
    predictions with the same weights and then taking one plain Euler step gives the
    same z (the combine can be fused into the Euler pass)."""
    rng = np.random.default_rng(3)
    z, xc, xtu, xu = (rng.standard_normal(300) for _ in range(4))
    t, tn = 0.42, 0.47
    for gam, gim, w in [(4.0, 1.0, (4.0, -3.0, 0.0)), (2.5, 2.5, (2.5, 0.0, -1.5)),
                        (4.0, 1.5, (4.0, -2.5, -0.5))]:
        assert abs(sum(w) - 1.0) < 1e-15
        xg = w[0] * xc + w[1] * xtu + w[2] * xu
        got = oracle.euler_step_cfg(z, xc, xtu, xu, t=t, t_next=tn, cfg_scale=gam,
                                    img_cfg_scale=gim)
        np.testing.assert_allclose(got, oracle.euler_step(z, xg, t, tn), rtol=0, atol=1e-12)


def test_cfg_missing_branch_is_an_error():
    with pytest.raises(ValueError):
        oracle.euler_step_cfg([0.0], [1.0], None, None, t=0.5, t_next=0.6, cfg_scale=4.0,
                              img_cfg_scale=1.0)
    # path 1 reads the conditional branch only
    assert oracle.euler_step_cfg([0.0], [1.0], None, None, t=0.5, t_next=0.75, cfg_scale=1.0,
                                 img_cfg_scale=1.0)[0] == 0.5


# --------------------------------------------------------------------------------------
# Understanding-pass attention with the block-causal mask: [A] §Block-causal attention
# --------------------------------------------------------------------------------------

def _by_key_sets(q, k, v, cu, key_sets):
    """Reference by reduction: each query row through the (separately pinned) unmasked
    attention oracle with exactly its allowed keys -- its own key as the one-token image
    block, the others as the prefix."""
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    for i in range(T):
        others = [j for j in key_sets[i] if j != i]
        assert i in key_sets[i]
        kp = k[others] if others else np.zeros((0,) + k.shape[1:])
        vp = v[others] if others else np.zeros((0,) + v.shape[1:])
        out[i] = oracle.gen_attn(q[i:i + 1], k[i:i + 1], v[i:i + 1], kp, vp, [0, 1],
                                 [0, len(others)])[0]
    return out


def _qkv(T, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Hq, 128)), rng.standard_normal((T, Hkv, 128)),
            rng.standard_normal((T, Hkv, 128)))


def test_prefill_pure_text_is_causal():
    """The pages: with every index distinct (pure text) the mask is plain causal."""
    T = 9
    q, k, v = _qkv(T, 4, 2, 1)
    idx = np.arange(T) + 3
    got = oracle.prefill_attn(q, k, v, idx, [0, T])
    ref = _by_key_sets(q, k, v, [0, T], [list(range(i + 1)) for i in range(T)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefill_one_image_block_is_bidirectional():
    """Tokens sharing one temporal index see each other both ways: a sample that is one
    image block is full (unmasked) attention."""
    T = 7
    q, k, v = _qkv(T, 2, 1, 2)
    got = oracle.prefill_attn(q, k, v, np.full(T, 5), [0, T])
    ref = _by_key_sets(q, k, v, [0, T], [list(range(T))] * T)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefill_text_image_text_by_structure():
    """Two ragged samples laid out text, image block (one shared index), text: text rows
    are causal; image rows see the text before and the whole block, not the text after;
    GQA with 2 query heads per KV head; no key crosses a sample boundary."""
    # sample 0: 4 text, 6 image, 3 text; sample 1: 2 text, 5 image, 1 text
    layouts = [(4, 6, 3), (2, 5, 1)]
    idx, sets, cu = [], [], [0]
    for (a, n, c) in layouts:
        base = cu[-1]
        idx += list(range(a)) + [a] * n + list(range(a + 1, a + 1 + c))
        for i in range(a + n + c):
            end = a + n - 1 if a <= i < a + n else i
            sets.append([base + j for j in range(end + 1)])
        cu.append(base + a + n + c)
    T = cu[-1]
    q, k, v = _qkv(T, 4, 2, 3)
    got = oracle.prefill_attn(q, k, v, np.array(idx), cu)
    np.testing.assert_allclose(got, _by_key_sets(q, k, v, cu, sets), rtol=0, atol=1e-12)


def test_prefill_first_token_and_lse():
    """A sample's first text token sees only itself: output = its v, lse = scale q.k."""
    T = 5
    q, k, v = _qkv(T, 2, 2, 4)
    out, lse = oracle.prefill_attn(q, k, v, np.arange(T), [0, T], with_lse=True)
    np.testing.assert_allclose(out[0], v[0], rtol=0, atol=1e-14)
    for h in range(2):
        assert lse[0, h] == pytest.approx(q[0, h] @ k[0, h] / math.sqrt(128), abs=1e-12)


def test_prefill_block_permutation_equivariance():
    """Inside an image block every token sees the same keys, so permuting the block's
    tokens (q, k, v together) permutes its output rows and leaves the others unchanged."""
    a, n, c = 3, 6, 2
    T = a + n + c
    idx = np.array(list(range(a)) + [a] * n + list(range(a + 1, a + 1 + c)))
    q, k, v = _qkv(T, 2, 1, 5)
    perm = np.arange(T)
    perm[a:a + n] = a + np.random.default_rng(6).permutation(n)
    o1 = oracle.prefill_attn(q, k, v, idx, [0, T])
    o2 = oracle.prefill_attn(q[perm], k[perm], v[perm], idx, [0, T])
    np.testing.assert_allclose(o2[a:a + n], o1[perm[a:a + n]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2[a + n:], o1[a + n:], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# Generation-branch q/k/v projection fused with the prologue: [A] §Mixture of Transformers
# --------------------------------------------------------------------------------------

def _proj_inputs(N=6, hidden=256, Hq=2, Hkv=1, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, hidden))
    w = rng.standard_normal(((Hq + 2 * Hkv) * 128, hidden)) / np.sqrt(hidden)
    nw = [rng.uniform(0.5, 1.5, 64) for _ in range(4)]
    pos = np.stack([np.full(N, 7), np.arange(N) % 3, np.arange(N) // 3]).astype(np.int32)
    return x, w, nw, pos


def test_qkv_proj_selection_rows():
    """With w_qkv rows selecting (permuted) columns of x, the projection is x[:, perm]: q and
    k are the pinned prologue of those slices and v the slice itself -- catches a
    transposed weight, a wrong q/k/v row order or a head reshaped the wrong way."""
    N, hidden, Hq, Hkv = 5, 512, 2, 1
    rng = np.random.default_rng(1)
    x = rng.standard_normal((N, hidden))
    perm = rng.permutation(hidden)
    w = np.zeros(((Hq + 2 * Hkv) * 128, hidden))
    w[np.arange(512), perm] = 1.0
    _, _, nw, pos = _proj_inputs(N, hidden, Hq, Hkv)
    q, k, v = oracle.qkv_proj_norm_rope(x, w, Hq, Hkv, *nw, pos)
    xs = x[:, perm]
    np.testing.assert_allclose(q, oracle.norm_rope(xs[:, :256].reshape(N, 2, 128), nw[0], nw[1], pos), atol=1e-13)
    np.testing.assert_allclose(k, oracle.norm_rope(xs[:, 256:384].reshape(N, 1, 128), nw[2], nw[3], pos), atol=1e-13)
    np.testing.assert_array_equal(v, xs[:, 384:].reshape(N, 1, 128))


def test_qkv_proj_value_brute_force():
    """v elements by explicit sums over the hidden dim (fsum), against the library matmul."""
    x, w, nw, pos = _proj_inputs(seed=2)
    _, _, v = oracle.qkv_proj_norm_rope(x, w, 2, 1, *nw, pos)
    for t, f in [(0, 0), (3, 77), (5, 127)]:
        ref = math.fsum(x[t, h] * w[(2 + 1) * 128 + f, h] for h in range(x.shape[1]))
        assert v[t, 0, f] == pytest.approx(ref, abs=1e-12)


def test_qkv_proj_scale_invariance_and_token_subset():
    """RMSNorm makes q and k invariant to scaling x (up to eps) while v scales linearly;
    evaluating a subset of tokens gives the same rows."""
    x, w, nw, pos = _proj_inputs(N=9, seed=3)
    q1, k1, v1 = oracle.qkv_proj_norm_rope(x, w, 2, 1, *nw, pos, eps=0.0)
    q2, k2, v2 = oracle.qkv_proj_norm_rope(3.0 * x, w, 2, 1, *nw, pos, eps=0.0)
    np.testing.assert_allclose(q2, q1, atol=1e-12)
    np.testing.assert_allclose(k2, k1, atol=1e-12)
    np.testing.assert_allclose(v2, 3.0 * v1, atol=1e-12)
    rows = [8, 0, 4]
    qs, ks, vs = oracle.qkv_proj_norm_rope(x, w, 2, 1, *nw, pos, eps=0.0, tokens=rows)
    np.testing.assert_allclose(qs, q1[rows], atol=1e-13)
    np.testing.assert_allclose(vs, v1[rows], atol=1e-13)
