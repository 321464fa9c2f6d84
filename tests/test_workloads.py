"""The seeded input generator: shapes the pages imply, determinism, bf16 rounding."""
import numpy as np
import pytest

import workloads as W


def test_bf16_round_ties_to_even_and_exact():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    y = W.bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert y.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    b = W.bf16_round(r)
    assert np.all(b.view(np.uint32) & 0xFFFF == 0)
    assert np.max(np.abs(b - r) / np.abs(r)) <= 2 ** -8
    np.testing.assert_array_equal(W.bf16_round(b), b)


@pytest.mark.parametrize("name,Tq,Tp,Hq,Hkv", [("tiny", 16, 16, 4, 1), ("small", 256, 64, 32, 8),
                                                ("mid", 1024, 256, 32, 8),
                                                ("large", 4096, 512, 32, 8)])
def test_shapes(name, Tq, Tp, Hq, Hkv):
    w = W.make(name, pixels=False)
    assert (w.Tq, w.Tp, w.Hq, w.Hkv) == (Tq, Tp, Hq, Hkv)
    assert w.q.shape == (Tq, Hq, 128) and w.k.shape == (Tq, Hkv, 128)
    assert w.v_prefix.shape == (Tp, Hkv, 128)
    # every image token shares the temporal index = prefix length; h, w tile the grid
    gh, gw = w.grids[0]
    assert np.all(w.pos_img[0] == Tp)
    assert w.pos_img[1].max() == gh - 1 and w.pos_img[2].max() == gw - 1
    assert len(set(zip(w.pos_img[1].tolist(), w.pos_img[2].tolist()))) == Tq
    if w.dtype == "bf16":
        assert np.all(w.q.view(np.uint32) & 0xFFFF == 0)


def test_editing_ragged():
    w = W.make("editing", pixels=False)
    assert w.B == 4 and w.n_img == [1024] * 4
    for b in range(4):
        L = w.extras["text_len"][b]
        assert 64 <= L <= 256
        assert w.n_prefix[b] == L + 1024 + 32
        seg = w.pos_prefix[:, w.cu_p[b]:w.cu_p[b + 1]]
        np.testing.assert_array_equal(seg[0, :L], np.arange(L))
        assert np.all(seg[0, L:L + 1024] == L) and seg[1, L:L + 1024].max() == 31
        np.testing.assert_array_equal(seg[0, L + 1024:], np.arange(L + 1, L + 33))
        assert np.all(w.pos_img[0, w.cu_q[b]:w.cu_q[b + 1]] == w.n_prefix[b])
    assert len(set(w.n_prefix)) > 1


def test_deterministic():
    a, b = W.make("small"), W.make("small")
    for f in ("q", "k", "v", "v_prefix", "k_prefix_pre", "wq_t", "eps_pixels", "x_hat"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = W.make("small", seed=1)
    assert not np.array_equal(a.q, c.q)


def test_pixel_grid_and_sigma():
    w = W.make("large")
    assert w.pixel_shape == (1, 3, 2048, 2048) and w.x_hat.size == 3 * 2048 * 2048
    assert w.sigma_R == 4.0 and len(w.t_grid) == 21 and w.t_grid[-1] == 1.0
    assert W.make("small", pixels=False).sigma_R == 1.0
    assert W.make("mid", pixels=False).sigma_R == 2.0
