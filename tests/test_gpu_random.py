"""Seeded random sweep of the step kernels against the fp64 oracle.

The other GPU tests pick their shapes by hand (the five workloads, edges, launch forms).
Here each case draws its shape from a fixed seed: a ragged batch of 1-6 samples with
0-640 image tokens and 0-640 prefix tokens each (both attention launch forms occur), one
of several head groupings (G = 1, 2, 3, 4, 8), bf16 or fp32, score scales from flat to
peaky; prologue row counts, scales and positions, in place or not; Euler and guided Euler
lengths, offsets, scales and intervals; prefill layouts of text and image runs; fused
projection token counts, widths and head groups; whole front ends of several image sizes
and widths.  Every case prints its
parameters before it runs and is held to the same bounds as the hand-picked ones: fp32
max-abs 1e-4; bf16 max-abs 2e-2 and relative L2 5e-3; log-sum-exp as in test_gpu_parity.
"""
import sys

import numpy as np
import pytest

import oracle
from tests import harness as H
from tests.test_gpu_parity import _check_lse, _random_case

pytestmark = pytest.mark.gpu

HEADS = [(32, 8), (8, 2), (4, 1), (12, 4), (16, 16), (6, 3), (16, 2)]


def _say(msg):
    print(f"[gpu-random] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def neo():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import pixel_space_flow_amd as P
    P.lib()  # raises if the library is missing
    return P


def _attn_shape(seed):
    rng = np.random.default_rng([seed, 0x6174])
    B = int(rng.integers(1, 7))
    n_img = [int(x) for x in rng.integers(0, 641, size=B)]
    n_pre = [int(x) for x in rng.integers(0, 641, size=B)]
    if rng.random() < 0.3:
        n_img[int(rng.integers(0, B))] = 0
    if rng.random() < 0.3:
        n_pre[int(rng.integers(0, B))] = 0
    if sum(n_img) == 0:
        n_img[0] = int(rng.integers(1, 641))
    Hq, Hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    wscale = float(rng.choice([0.5, 1.0, 2.5]))
    return rng, n_img, n_pre, Hq, Hkv, dtype, wscale


def _launch(n_img, Hq, Hkv):
    """The launch form the library picks: 64-token workgroups above 128 of them, else the
    split-key form."""
    G = Hq // Hkv
    chunks = G * ((max(n_img) + 31) // 32)
    return "64-token" if (chunks + 7) // 8 * Hkv * len(n_img) > 128 else "split-key"


@pytest.mark.parametrize("seed", range(16))
def test_random_attention(neo, seed):
    import torch
    rng, n_img, n_pre, Hq, Hkv, dtype, wscale = _attn_shape(seed)
    _say(f"attention seed={seed} n_img={n_img} n_pre={n_pre} Hq={Hq} Hkv={Hkv} {dtype} "
         f"scale={wscale} ({_launch(n_img, Hq, Hkv)} launch)")
    c = _random_case(rng, n_img, n_pre, Hq, Hkv, dtype, wscale=wscale)
    d = dtype
    out, lse = neo.gen_attn_fwd(H.dev(c["q"], d), H.dev(c["k"], d), H.dev(c["v"], d),
                                H.dev(c["kp"], d), H.dev(c["vp"], d), H.dev_i32(c["cu_q"]),
                                H.dev_i32(c["cu_p"]), max(n_img), max(n_pre), return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"],
                                   c["cu_p"], with_lse=True)
    H.assert_close(H.host(out), ref, dtype, f"random attention {seed}")
    _check_lse(H.host(lse).T, lse_ref, dtype, f"random attention {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_prologue(neo, seed):
    import torch
    rng = np.random.default_rng([seed, 0x7072])
    T = int(rng.integers(1, 2049))
    Hq, Hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    in_place = bool(rng.random() < 0.3)
    _say(f"prologue seed={seed} T={T} Hq={Hq} Hkv={Hkv} {dtype} in_place={in_place}")
    q = H.round_to(rng.standard_normal((T, Hq, 128)) * float(rng.choice([0.01, 1.0, 30.0])), dtype)
    k = H.round_to(rng.standard_normal((T, Hkv, 128)) * float(rng.choice([0.01, 1.0, 30.0])), dtype)
    ws = [rng.uniform(0.5, 1.5, 64).astype(np.float32) for _ in range(4)]
    pos = np.stack([rng.integers(0, 20001, T), rng.integers(0, 256, T),
                    rng.integers(0, 256, T)]).astype(np.int32)
    qd, kd = H.dev(q, dtype), H.dev(k, dtype)
    kw = dict(q_out=qd, k_out=kd) if in_place else {}
    qo, ko = neo.qknorm_rope3(qd, kd, *[H.dev_f32(x) for x in ws], H.dev_i32(pos), 5e6, 1e4,
                              1e-6, **kw)
    torch.cuda.synchronize()
    qr, kr = oracle.qknorm_rope3(q, k, *ws, pos, 5e6, 1e4, 1e-6)
    H.assert_close(H.host(qo), qr, dtype, f"random prologue q {seed}")
    H.assert_close(H.host(ko), kr, dtype, f"random prologue k {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_euler(neo, seed):
    import torch
    rng = np.random.default_rng([seed, 0x6575])
    n = int(rng.integers(1, 300000))
    off = int(rng.integers(0, 4))
    t = float(rng.uniform(0.0, 1.0))
    tn = float(min(1.0, t + rng.uniform(0.0, 0.2)))
    _say(f"euler seed={seed} n={n} offset={off} t={t:.4f} t_next={tn:.4f}")
    z0 = rng.standard_normal(n + off).astype(np.float32)
    x0 = rng.standard_normal(n + off).astype(np.float32)
    zb, xb = H.dev_f32(z0), H.dev_f32(x0)
    neo.fm_euler_step(zb[off:], xb[off:], t, tn, 0.02)
    torch.cuda.synchronize()
    ref = oracle.euler_step(z0[off:], x0[off:], t, tn, 0.02)
    got = H.host(zb)
    H.assert_close(got[off:], ref, "f32", f"random euler {seed}")
    assert np.array_equal(got[:off], z0[:off]), "euler wrote before its start"


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill(neo, seed):
    import torch
    import workloads as W
    rng = np.random.default_rng([seed, 0x7066])
    B = int(rng.integers(1, 4))
    segments = []
    for _ in range(B):
        runs = []
        for _ in range(int(rng.integers(1, 5))):
            if rng.random() < 0.5:
                runs.append(("text", int(rng.integers(1, 100))))
            else:
                runs.append(("image", int(rng.integers(1, 260))))
        segments.append(runs)
    Hq, Hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    _say(f"prefill seed={seed} segments={segments} Hq={Hq} Hkv={Hkv}")
    d = W.prefill_layout(segments, Hq, Hkv, seed=seed)
    qb, kb, vb = (W.bf16_round(d[x]) for x in ("q", "k", "v"))
    out, lse = neo.prefill_attn_fwd(H.dev(qb, "bf16"), H.dev(kb, "bf16"), H.dev(vb, "bf16"),
                                    H.dev_i32(d["idx"]), H.dev_i32(d["cu"]), d["max_len"],
                                    return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_attn(qb, kb, vb, d["idx"], d["cu"], with_lse=True)
    H.assert_close(H.host(out), ref, "bf16", f"random prefill {seed}")
    _check_lse(H.host(lse).T, ref_lse, "bf16", f"random prefill {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_cfg_euler(neo, seed):
    import torch
    rng = np.random.default_rng([seed, 0x6366])
    n = int(rng.integers(1, 200000))
    off = int(rng.integers(0, 4))
    t = float(rng.uniform(0.0, 1.0))
    tn = float(min(1.0, t + rng.uniform(0.0, 0.2)))
    g = float(rng.choice([1.0, 2.0, 4.0, 7.5]))
    gi = float(rng.choice([1.0, 1.5, 2.0]))
    iv = (0.0, 1.0)  # the whole trajectory guided, or a drawn interval
    if rng.random() < 0.5:
        iv = tuple(sorted(float(x) for x in rng.uniform(0, 1, 2)))
    path = neo.cfg_path(t, g, gi, iv)
    _say(f"cfg euler seed={seed} n={n} offset={off} t={t:.4f} t_next={tn:.4f} gamma={g} "
         f"gamma_img={gi} interval={iv} path={path}")
    z0, xc, xtu, xu = (rng.standard_normal(n + off).astype(np.float32) for _ in range(4))
    d = [H.dev_f32(a) for a in (z0, xc, xtu, xu)]
    # branches the path does not read are passed as None
    args = [d[1][off:], d[2][off:] if path in (2, 4) else None,
            d[3][off:] if path in (3, 4) else None]
    neo.fm_euler_step_cfg(d[0][off:], *args, t=t, t_next=tn, cfg_scale=g, img_cfg_scale=gi,
                          cfg_interval=iv)
    torch.cuda.synchronize()
    assert path == oracle.cfg_path(np.float32(t), g, gi, iv)
    ref = oracle.euler_step_cfg(z0[off:], xc[off:], xtu[off:], xu[off:], t=t, t_next=tn,
                                cfg_scale=g, img_cfg_scale=gi, cfg_interval=iv)
    got = H.host(d[0])
    H.assert_close(got[off:], ref, "f32", f"random cfg euler {seed}")
    assert np.array_equal(got[:off], z0[:off]), "guided step wrote before its start"


@pytest.mark.parametrize("seed", range(5))
def test_random_projection(neo, seed):
    import torch
    import workloads as W
    rng = np.random.default_rng([seed, 0x716b])
    N = int(rng.integers(1, 701))
    hidden = 64 * int(rng.integers(1, 17))
    Hq, Hkv = [(1, 1), (3, 1), (4, 2), (6, 3), (8, 2), (12, 4)][int(rng.integers(0, 6))]
    _say(f"projection seed={seed} N={N} hidden={hidden} Hq={Hq} Hkv={Hkv}")
    x = W.bf16_round(rng.standard_normal((N, hidden)).astype(np.float32))
    wq = W.bf16_round((rng.standard_normal(((Hq + 2 * Hkv) * 128, hidden)) /
                       np.sqrt(hidden)).astype(np.float32))
    nw = tuple(rng.uniform(0.5, 1.5, 64).astype(np.float32) for _ in range(4))
    pos = np.stack([np.full(N, int(rng.integers(0, 20001))), rng.integers(0, 64, N),
                    rng.integers(0, 64, N)]).astype(np.int32)
    q, k, v = neo.qkv_proj_norm_rope(H.dev(x, "bf16"), H.dev(wq, "bf16"), Hq, Hkv,
                                     *[H.dev_f32(a) for a in nw], H.dev_i32(pos), 5e6, 1e4, 1e-6)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj_norm_rope(x, wq, Hq, Hkv, *nw, pos, 5e6, 1e4, 1e-6)
    H.assert_close(H.host(q), rq, "bf16", f"random projection q {seed}")
    H.assert_close(H.host(k), rk, "bf16", f"random projection k {seed}")
    H.assert_close(H.host(v), rv, "bf16", f"random projection v {seed}")


@pytest.mark.parametrize("seed", range(4))
def test_random_front_end(neo, seed):
    from tests.test_gpu_front_end import _chain, _emb, _weights
    rng = np.random.default_rng([seed, 0x6665])
    B = int(rng.integers(1, 4))
    Hh, Ww = 32 * int(rng.integers(1, 9)), 32 * int(rng.integers(1, 9))
    C1 = 64 * int(rng.integers(1, 5))
    D = 32 * int(rng.integers(1, 11))
    z = (float(rng.choice([0.5, 2.0, 8.0])) * rng.standard_normal((B, 3, Hh, Ww))).astype(np.float32)
    w1, b1, w2, b2 = _weights(rng, C1, D)
    emb_t, emb_s = _emb(rng, D)
    t = float(rng.uniform(0.0, 1.0))
    ns = float(rng.uniform(1.0, 16.0))
    _chain(neo, z, w1, b1, w2, b2, emb_t, emb_s, t, ns, 16.0,
           f"seed={seed} B={B} {Hh}x{Ww} C1={C1} D={D}")
