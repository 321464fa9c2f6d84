"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case feeds both sides the same seeded inputs and compares element by
element.  All five workloads, including the 4096-token and editing ones in the
benchmark's launch configuration, are compared on every output row against the
oracle's full evaluation; only the 16384-token maximum-size sample is compared on
one query row of every 32-row block (every workgroup's share).  Tolerances
(per call): fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and relative L2 <= 5e-3;
log-sum-exp 4e-3 (bf16: ln(1 + 2^-8), one weight's rounding) or 1e-4 (fp32, the fp32
output bound) absolute, its mean error within four standard deviations of unbiased rounding.  Each case prints the time the
oracle took.
"""
import sys
import time

import numpy as np
import pytest

import oracle
import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _timed(what, fn, *args, **kw):
    """Run an oracle call and report how long it took."""
    t0 = time.perf_counter()
    r = fn(*args, **kw)
    _say(f"{what}: oracle {time.perf_counter() - t0:.1f} s")
    return r


# Log-sum-exp.  The bf16 kernels add up the weights exactly as rounded to bf16 for the PV
# product (so the normalised weights sum to one).  One RNE rounding to bf16 (8 significant
# bits) moves a weight by at most 2^-8 of its size, so the row sum is within a factor
# 1 +- 2^-8 of the exact one and its log within ln(1 + 2^-8) = 3.90e-3: reached when one
# weight dominates (peaky scores).  The fp32 score and exp errors add ~1e-5.  Rounding to
# nearest is unbiased, so the mean error over n values must also stay within four standard
# deviations of a mean of n roundings, each with rms <= 2^-8 / sqrt(3) (a shifted scale or a
# dropped key moves the mean by far more).  The fp32 kernel's log-sum-exp is a value of size
# up to ~40 with large-norm inputs, where one fp32 ulp is 3.8e-6 and its 128-term score sums
# add a few ulps; it is held to the fp32 outputs' 1e-4.
LSE_TOL = {"bf16": 4e-3, "f32": 1e-4}
LSE_RMS_ONE = {"bf16": 2.0 ** -8 / np.sqrt(3.0), "f32": 1e-6}


def _check_lse(got, ref, dtype, what):
    d = np.asarray(got, dtype=np.float64) - ref
    err = float(np.max(np.abs(d))) if ref.size else 0.0
    assert err <= LSE_TOL[dtype], f"{what}: lse max-abs {err:.3e} > {LSE_TOL[dtype]:.0e}"
    bias = float(np.mean(d)) if ref.size else 0.0
    bias_tol = 4.0 * LSE_RMS_ONE[dtype] / np.sqrt(max(ref.size, 1)) + 1e-5
    assert abs(bias) <= bias_tol, f"{what}: lse mean error {bias:+.3e} beyond {bias_tol:.1e}"
    print(f"[parity] {what} lse: max-abs {err:.3e} mean {bias:+.2e} (bound {bias_tol:.1e})",
          flush=True)


@pytest.fixture(scope="module")
def neo():
    _cuda()
    import pixel_space_flow_amd as P
    P.lib()  # raises if the library is missing
    return P


# --------------------------------------------------------------------------------------
# Euler step
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_euler_configs(neo, name):
    torch = _cuda()
    w = W.make(name)
    t, tn = w.t_grid[0], w.t_grid[1]
    z0 = w.z_start if w.z_start is not None else (np.float32(w.sigma_R) * w.eps_pixels)
    z0 = z0.astype(np.float32)
    _say(f"euler {name} n={z0.size} t={t}->{tn}")
    z = H.dev_f32(z0)
    x = H.dev_f32(w.x_hat)
    neo.fm_euler_step(z, x, t, tn, w.t_eps)
    torch.cuda.synchronize()
    ref = oracle.euler_step(z0, w.x_hat, t, tn, w.t_eps)
    H.assert_close(H.host(z), ref, "f32", f"euler {name}")


def test_euler_trajectory_small(neo):
    """8 steps with x0 fixed to the clean image stay on z_t = t x + (1-t) sigma eps."""
    torch = _cuda()
    w = W.make("small")
    z0 = (np.float32(w.sigma_R) * w.eps_pixels).astype(np.float32)
    z = H.dev_f32(z0)
    x = H.dev_f32(w.x_hat)
    zr = z0.astype(np.float64)
    for k in range(len(w.t_grid) - 1):
        t, tn = w.t_grid[k], w.t_grid[k + 1]
        _say(f"euler trajectory step {k}")
        neo.fm_euler_step(z, x, t, tn, w.t_eps)
        zr = oracle.euler_step(zr, w.x_hat, t, tn, w.t_eps)
        torch.cuda.synchronize()
        got = H.host(z)
        H.assert_close(got, zr, "f32", f"trajectory step {k}")
        closed = tn * w.x_hat.astype(np.float64) + (1 - tn) * w.sigma_R * w.eps_pixels
        assert np.max(np.abs(got - closed)) < 1e-4
    np.testing.assert_allclose(H.host(z), w.x_hat, atol=1e-5)


def test_euler_edges(neo):
    """Clamp branch, a length that is not a multiple of 4, an unaligned start, n = 0."""
    torch = _cuda()
    rng = np.random.default_rng(3)
    for n, off, t, tn in ((1003, 0, 0.99, 1.0), (4099, 1, 0.25, 0.3), (7, 3, 0.0, 0.05),
                          (1, 0, 0.5, 0.5)):
        _say(f"euler edge n={n} offset={off}")
        z0 = rng.standard_normal(n + off).astype(np.float32)
        x0 = rng.standard_normal(n + off).astype(np.float32)
        zb, xb = H.dev_f32(z0), H.dev_f32(x0)
        neo.fm_euler_step(zb[off:], xb[off:], t, tn, 0.02)
        torch.cuda.synchronize()
        ref = oracle.euler_step(z0[off:], x0[off:], t, tn, 0.02)
        got = H.host(zb)
        H.assert_close(got[off:], ref, "f32", f"euler edge n={n}")
        np.testing.assert_array_equal(got[:off], z0[:off])
    empty = torch.empty(0, device="cuda")
    neo.fm_euler_step(empty, empty, 0.1, 0.2)


# --------------------------------------------------------------------------------------
# Classifier-free guidance fused with the Euler step
# --------------------------------------------------------------------------------------

# (cfg_scale, img_cfg_scale, interval): paths 1 (guidance off by the interval), 2 (the
# pages' text-to-image defaults), 3 and 4
CFG_CASES = [(4.0, 1.0, (0.95, 1.0)), (4.0, 1.0, (0.0, 1.0)), (3.0, 3.0, (0.0, 1.0)),
             (4.0, 1.5, (0.0, 1.0))]


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_cfg_euler_configs(neo, name):
    torch = _cuda()
    w = W.make(name)
    x_tu, x_u = W.cfg_branches(w)
    t, tn = w.t_grid[0], w.t_grid[1]
    z0 = w.z_start if w.z_start is not None else (np.float32(w.sigma_R) * w.eps_pixels)
    z0 = z0.astype(np.float32)
    xc_d, xtu_d, xu_d = H.dev_f32(w.x_hat), H.dev_f32(x_tu), H.dev_f32(x_u)
    for g, gi, iv in CFG_CASES:
        path = neo.cfg_path(t, g, gi, iv)
        assert path == oracle.cfg_path(np.float32(t), g, gi, iv)
        _say(f"cfg euler {name} n={z0.size} t={t}->{tn} gamma={g} gamma_img={gi} path={path}")
        z = H.dev_f32(z0)
        neo.fm_euler_step_cfg(z, xc_d, xtu_d, xu_d, t=t, t_next=tn, t_eps=w.t_eps,
                              cfg_scale=g, img_cfg_scale=gi, cfg_interval=iv)
        torch.cuda.synchronize()
        ref = oracle.euler_step_cfg(z0, w.x_hat, x_tu, x_u, t=t, t_next=tn, t_eps=w.t_eps,
                                    cfg_scale=g, img_cfg_scale=gi, cfg_interval=iv)
        H.assert_close(H.host(z), ref, "f32", f"cfg euler {name} path {path}")


def test_cfg_euler_trajectory_mid(neo):
    """The mid workload's 20 steps with guidance on the pages' defaults (path 2) and on
    the full three-branch path, against the oracle after every step."""
    torch = _cuda()
    w = W.make("mid")
    x_tu, x_u = W.cfg_branches(w)
    z0 = (np.float32(w.sigma_R) * w.eps_pixels).astype(np.float32)
    xs = [H.dev_f32(a) for a in (w.x_hat, x_tu, x_u)]
    for g, gi in ((4.0, 1.0), (4.0, 1.5)):
        z = H.dev_f32(z0)
        zr = z0.astype(np.float64)
        for k in range(len(w.t_grid) - 1):
            t, tn = w.t_grid[k], w.t_grid[k + 1]
            _say(f"cfg trajectory gamma={g} gamma_img={gi} step {k}")
            neo.fm_euler_step_cfg(z, *xs, t=t, t_next=tn, t_eps=w.t_eps, cfg_scale=g,
                                  img_cfg_scale=gi)
            zr = oracle.euler_step_cfg(zr, w.x_hat, x_tu, x_u, t=t, t_next=tn, t_eps=w.t_eps,
                                       cfg_scale=g, img_cfg_scale=gi)
        torch.cuda.synchronize()
        H.assert_close(H.host(z), zr, "f32", f"cfg trajectory {g}/{gi}")


def test_cfg_euler_edges(neo):
    """Ragged lengths and unaligned starts (scalar path), branches the path does not read
    passed as None, z aliasing the conditional branch, the clamp at t near 1, and n = 0;
    path 1 matches the plain Euler kernel bit for bit."""
    torch = _cuda()
    rng = np.random.default_rng(9)
    for n, off, t, tn, (g, gi) in ((1003, 0, 0.99, 1.0, (4.0, 1.5)), (4099, 1, 0.25, 0.3, (4.0, 1.0)),
                                   (7, 3, 0.0, 0.05, (2.0, 2.0)), (64, 2, 0.5, 0.5, (4.0, 1.5))):
        _say(f"cfg edge n={n} offset={off} gamma={g} gamma_img={gi}")
        z0, xc, xtu, xu = (rng.standard_normal(n + off).astype(np.float32) for _ in range(4))
        path = neo.cfg_path(t, g, gi)
        d = [H.dev_f32(a) for a in (z0, xc, xtu, xu)]
        args = [d[1][off:], d[2][off:] if path in (2, 4) else None,
                d[3][off:] if path in (3, 4) else None]
        neo.fm_euler_step_cfg(d[0][off:], *args, t=t, t_next=tn, cfg_scale=g, img_cfg_scale=gi)
        torch.cuda.synchronize()
        ref = oracle.euler_step_cfg(z0[off:], xc[off:], xtu[off:], xu[off:], t=t, t_next=tn,
                                    cfg_scale=g, img_cfg_scale=gi)
        got = H.host(d[0])
        H.assert_close(got[off:], ref, "f32", f"cfg edge n={n} path {path}")
        np.testing.assert_array_equal(got[:off], z0[:off])
    # z is the conditional branch itself (read before written, element by element)
    z0, xtu = (rng.standard_normal(513).astype(np.float32) for _ in range(2))
    zd = H.dev_f32(z0)
    neo.fm_euler_step_cfg(zd, zd, H.dev_f32(xtu), None, t=0.3, t_next=0.4, cfg_scale=4.0,
                          img_cfg_scale=1.0)
    torch.cuda.synchronize()
    ref = oracle.euler_step_cfg(z0, z0, xtu, None, t=0.3, t_next=0.4, cfg_scale=4.0,
                                img_cfg_scale=1.0)
    H.assert_close(H.host(zd), ref, "f32", "cfg z aliases x0_cond")
    # path 1 is the plain step: same bits as neo_fm_euler_step
    z0, xc = (rng.standard_normal(4096 + 3).astype(np.float32) for _ in range(2))
    a, b, xd = H.dev_f32(z0), H.dev_f32(z0), H.dev_f32(xc)
    neo.fm_euler_step_cfg(a, xd, None, None, t=0.2, t_next=0.25, cfg_scale=1.0,
                          img_cfg_scale=1.0)
    neo.fm_euler_step(b, xd, 0.2, 0.25)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(H.host(a), H.host(b))
    empty = torch.empty(0, device="cuda")
    neo.fm_euler_step_cfg(empty, empty, empty, empty, t=0.1, t_next=0.2, cfg_scale=4.0,
                          img_cfg_scale=1.5)


# --------------------------------------------------------------------------------------
# Norm + rotary prologue
# --------------------------------------------------------------------------------------

def _prologue_ref(w):
    return oracle.qknorm_rope3(w.q, w.k, w.wq_t, w.wq_hw, w.wk_t, w.wk_hw, w.pos_img,
                               w.rope_theta, w.rope_theta_hw, w.eps)


def _prologue_gpu(neo, w, in_place=False):
    q, k = H.dev(w.q, w.dtype), H.dev(w.k, w.dtype)
    args = (H.dev_f32(w.wq_t), H.dev_f32(w.wq_hw), H.dev_f32(w.wk_t), H.dev_f32(w.wk_hw),
            H.dev_i32(w.pos_img), w.rope_theta, w.rope_theta_hw, w.eps)
    if in_place:
        return neo.qknorm_rope3(q, k, *args, q_out=q, k_out=k)
    return neo.qknorm_rope3(q, k, *args)


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_prologue_configs(neo, name):
    torch = _cuda()
    w = W.make(name, pixels=False)
    _say(f"prologue {name} T={w.Tq} Hq={w.Hq} Hkv={w.Hkv} {w.dtype}")
    qo, ko = _prologue_gpu(neo, w)
    torch.cuda.synchronize()
    qr, kr = _prologue_ref(w)
    H.assert_close(H.host(qo), qr, w.dtype, f"prologue q {name}")
    H.assert_close(H.host(ko), kr, w.dtype, f"prologue k {name}")
    if w.dtype == "bf16":
        # one rounding: every element is within half a bf16 ulp of the fp64 value (plus
        # the fp32 arithmetic error), i.e. at most 2^-8 relative
        got = H.host(qo).astype(np.float64)
        assert np.all(np.abs(got - qr) <= np.abs(qr) * 2.0 ** -8 + 1e-6)


def test_prologue_in_place(neo):
    torch = _cuda()
    w = W.make("small", pixels=False)
    _say("prologue in place")
    qo, ko = _prologue_gpu(neo, w, in_place=True)
    torch.cuda.synchronize()
    qr, kr = _prologue_ref(w)
    H.assert_close(H.host(qo), qr, "bf16", "in-place q")
    H.assert_close(H.host(ko), kr, "bf16", "in-place k")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,Hq,Hkv", [(1, 1, 1), (5, 3, 1), (33, 6, 2), (7, 32, 8), (3, 16, 16)])
def test_prologue_shapes(neo, dtype, T, Hq, Hkv):
    """Row counts that leave the last 4-row group partly empty; large positions."""
    torch = _cuda()
    rng = np.random.default_rng(T * 100 + Hq)
    q = H.round_to(rng.standard_normal((T, Hq, 128)) * 3, dtype)
    k = H.round_to(rng.standard_normal((T, Hkv, 128)) * 0.01, dtype)
    ws = [rng.uniform(0.5, 1.5, 64).astype(np.float32) for _ in range(4)]
    pos = np.stack([rng.integers(0, 20000, T), rng.integers(0, 256, T),
                    rng.integers(0, 256, T)]).astype(np.int32)
    _say(f"prologue shape T={T} Hq={Hq} Hkv={Hkv} {dtype}")
    qo, ko = neo.qknorm_rope3(H.dev(q, dtype), H.dev(k, dtype), *[H.dev_f32(x) for x in ws],
                              H.dev_i32(pos), 5e6, 1e4, 1e-6)
    torch.cuda.synchronize()
    qr, kr = oracle.qknorm_rope3(q, k, *ws, pos, 5e6, 1e4, 1e-6)
    H.assert_close(H.host(qo), qr, dtype, "q")
    H.assert_close(H.host(ko), kr, dtype, "k")


def test_prologue_empty(neo):
    torch = _cuda()
    e = torch.empty((0, 4, 128), device="cuda", dtype=torch.bfloat16)
    w = torch.ones(64, device="cuda")
    neo.qknorm_rope3(e, e[:, :1].contiguous(), w, w, w, w,
                     torch.empty((3, 0), dtype=torch.int32, device="cuda"))


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------

def _attn_inputs(w):
    """Identical inputs for both sides: rotated q/k (the oracle's, rounded), raw v."""
    qr, kr = _prologue_ref(w)
    q = H.round_to(qr, w.dtype)
    k = H.round_to(kr, w.dtype)
    kp, vp = H.frozen_prefix(w)
    return q, k, w.v, kp, vp


def _attn_gpu(neo, w, q, k, v, kp, vp, return_lse=True):
    d = w.dtype
    return neo.gen_attn_fwd(H.dev(q, d), H.dev(k, d), H.dev(v, d), H.dev(kp, d), H.dev(vp, d),
                            H.dev_i32(w.cu_q), H.dev_i32(w.cu_p), max(w.n_img), max(w.n_prefix),
                            return_lse=return_lse)


def _block_rows(n, rng):
    """One query row from every 32-row block of [0, n) (at a varying offset inside the
    block), plus both ends: every workgroup's rows are represented."""
    starts = np.arange(0, n, 32)
    rows = np.minimum(starts + rng.integers(0, 32, starts.size), n - 1)
    return np.unique(np.concatenate([rows, [0, n - 1]])).astype(np.int64)


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_attn_configs(neo, name):
    """Every workload in the benchmark's launch configuration, every query row and head
    (output and log-sum-exp) against the oracle's full evaluation."""
    torch = _cuda()
    w = W.make(name, pixels=False)
    q, k, v, kp, vp = _attn_inputs(w)
    _say(f"attention {name} Tq={w.Tq} Tp={w.Tp} {w.dtype}")
    out, lse = _attn_gpu(neo, w, q, k, v, kp, vp)
    torch.cuda.synchronize()
    ref, lse_ref = _timed(f"attention {name}", oracle.gen_attn, q, k, v, kp, vp, w.cu_q, w.cu_p,
                          with_lse=True)
    H.assert_close(H.host(out), ref, w.dtype, f"attention {name}")
    _check_lse(H.host(lse).T, lse_ref, w.dtype, f"attention {name}")


def _random_case(rng, n_img, n_pre, Hq, Hkv, dtype, wscale=1.0):
    Tq, Tp = sum(n_img), sum(n_pre)
    f = lambda *s: H.round_to(rng.standard_normal(s) * wscale, dtype)
    return dict(q=f(Tq, Hq, 128), k=f(Tq, Hkv, 128), v=H.round_to(rng.standard_normal((Tq, Hkv, 128)), dtype),
                kp=f(Tp, Hkv, 128), vp=H.round_to(rng.standard_normal((Tp, Hkv, 128)), dtype),
                cu_q=np.concatenate([[0], np.cumsum(n_img)]).astype(np.int32),
                cu_p=np.concatenate([[0], np.cumsum(n_pre)]).astype(np.int32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_img,n_pre,Hq,Hkv", [
    ([37], [0], 4, 1),            # no prefix, ragged query block
    ([1], [1], 8, 2),             # single query, two keys
    ([100, 3, 64], [65, 130, 0], 8, 2),   # ragged batch, tiles straddling the boundary
    ([50, 0, 29], [10, 7, 1], 4, 4),      # an empty sample, MHA
    ([40], [200], 6, 2),          # G = 3
    ([96], [33], 16, 2),          # G = 8: 4 waves x 2 heads per chunk group
    ([257], [511], 32, 8),        # odd lengths on the production head shape
    # a grid of more than 128 eight-wave workgroups (the launch above that size), with
    # ragged, tiny and empty samples; the cases above run the four-wave launch
    ([700, 3, 1000, 64, 0, 513], [100, 0, 37, 255, 12, 64], 32, 8),
])
def test_attn_edges(neo, dtype, n_img, n_pre, Hq, Hkv):
    torch = _cuda()
    rng = np.random.default_rng(sum(n_img) * 7 + sum(n_pre) + Hq)
    c = _random_case(rng, n_img, n_pre, Hq, Hkv, dtype, wscale=0.5)
    _say(f"attention edge n_img={n_img} n_pre={n_pre} Hq={Hq} Hkv={Hkv} {dtype}")
    d = dtype
    out, lse = neo.gen_attn_fwd(H.dev(c["q"], d), H.dev(c["k"], d), H.dev(c["v"], d),
                                H.dev(c["kp"], d), H.dev(c["vp"], d), H.dev_i32(c["cu_q"]),
                                H.dev_i32(c["cu_p"]), max(n_img), max(n_pre), return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"], c["cu_p"],
                                   with_lse=True)
    H.assert_close(H.host(out), ref, dtype, "attention edge")
    _check_lse(H.host(lse).T, lse_ref, dtype, "attention edge")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attn_many_samples_loose_bounds(neo, dtype):
    """24 small samples (some with no queries, some with no prefix) and max_seqlen bounds well
    above the true maxima.  The bounds only size the grid: the surplus workgroups find no rows
    and every sample's rows still match the oracle."""
    torch = _cuda()
    rng = np.random.default_rng(2024)
    n_img = [int(x) for x in rng.integers(0, 41, size=24)]
    n_img[5] = 0
    n_pre = [int(x) for x in rng.integers(0, 71, size=24)]
    n_pre[3] = 0
    n_pre[5] = 0
    c = _random_case(rng, n_img, n_pre, 8, 2, dtype, wscale=0.5)
    _say(f"attention 24 samples, loose bounds {max(n_img) + 50}/{max(n_pre) + 30} {dtype}")
    d = dtype
    out, lse = neo.gen_attn_fwd(H.dev(c["q"], d), H.dev(c["k"], d), H.dev(c["v"], d),
                                H.dev(c["kp"], d), H.dev(c["vp"], d), H.dev_i32(c["cu_q"]),
                                H.dev_i32(c["cu_p"]), max(n_img) + 50, max(n_pre) + 30,
                                return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"], c["cu_p"],
                                   with_lse=True)
    H.assert_close(H.host(out), ref, dtype, "attention, many samples")
    _check_lse(H.host(lse).T, lse_ref, dtype, "attention, many samples")


@pytest.mark.parametrize("n_img,n_pre,Hq,Hkv,wscale", [
    ([1], [0], 4, 1, 1.0),                  # one 32-key sub-tile: the second key half is empty
    ([33, 1, 20], [0, 0, 20], 8, 2, 1.0),   # two sub-tiles, one key each side; prefix + image
    ([100, 64], [65, 31], 32, 8, 1.0),      # odd sub-tile counts: the second half's last is empty
    ([70, 5, 129], [300, 1, 0], 8, 1, 3.0), # G = 8, peaky scores: the halves' maxima differ
    ([96], [33], 16, 16, 3.0),              # MHA, peaky
])
def test_attn_split_keys(neo, n_img, n_pre, Hq, Hkv, wscale):
    """Small launches run the split-key kernel (each workgroup's keys in two halves merged
    at the end): a half with no keys, halves ending in an empty sub-tile, and peaky scores
    whose maxima differ between the halves; output and log-sum-exp against the oracle."""
    torch = _cuda()
    rng = np.random.default_rng(sum(n_img) * 13 + sum(n_pre) + Hq)
    c = _random_case(rng, n_img, n_pre, Hq, Hkv, "bf16", wscale=wscale)
    _say(f"attention split keys n_img={n_img} n_pre={n_pre} Hq={Hq} Hkv={Hkv} scale={wscale}")
    out, lse = neo.gen_attn_fwd(H.dev(c["q"], "bf16"), H.dev(c["k"], "bf16"), H.dev(c["v"], "bf16"),
                                H.dev(c["kp"], "bf16"), H.dev(c["vp"], "bf16"), H.dev_i32(c["cu_q"]),
                                H.dev_i32(c["cu_p"]), max(n_img), max(n_pre), return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"], c["cu_p"],
                                   with_lse=True)
    H.assert_close(H.host(out), ref, "bf16", "attention split keys")
    _check_lse(H.host(lse).T, lse_ref, "bf16", "attention split keys")


@pytest.mark.parametrize("n_img,n_pre,seed", [
    ([300, 200], [700, 64], 77),                                  # the four-wave launch
    ([700, 3, 1000, 64, 0, 513], [100, 0, 37, 255, 12, 64], 5),   # the eight-wave launch
])
def test_attn_peaky_softmax(neo, n_img, n_pre, seed):
    """Large-norm queries and keys make the softmax peaky (the lazy rescale path is
    exercised on later tiles and score errors are not averaged away); one weight dominates
    most rows, so the log-sum-exp error approaches its one-rounding bound."""
    torch = _cuda()
    rng = np.random.default_rng(seed)
    c = _random_case(rng, n_img, n_pre, 32, 8, "bf16", wscale=3.0)
    _say(f"attention peaky n_img={n_img} n_pre={n_pre}")
    out = neo.gen_attn_fwd(H.dev(c["q"], "bf16"), H.dev(c["k"], "bf16"), H.dev(c["v"], "bf16"),
                           H.dev(c["kp"], "bf16"), H.dev(c["vp"], "bf16"), H.dev_i32(c["cu_q"]),
                           H.dev_i32(c["cu_p"]), max(n_img), max(n_pre), return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"], c["cu_p"],
                                   with_lse=True)
    H.assert_close(H.host(out[0]), ref, "bf16", "peaky")
    _check_lse(H.host(out[1]).T, lse_ref, "bf16", "peaky")


def test_attn_no_prefix_buffers(neo):
    """Tp = 0: the prefix tensors are empty and no prefix pointer is passed."""
    torch = _cuda()
    rng = np.random.default_rng(5)
    c = _random_case(rng, [70], [0], 4, 1, "bf16")
    e = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    out = neo.gen_attn_fwd(H.dev(c["q"], "bf16"), H.dev(c["k"], "bf16"), H.dev(c["v"], "bf16"),
                           e, e, H.dev_i32(c["cu_q"]), H.dev_i32(c["cu_p"]), 70, 0)
    torch.cuda.synchronize()
    ref = oracle.gen_attn(c["q"], c["k"], c["v"], c["kp"], c["vp"], c["cu_q"], c["cu_p"])
    H.assert_close(H.host(out), ref, "bf16", "no prefix")


def test_attn_long_sample(neo):
    """A maximum-size single sample: 16384 image tokens over a 2048-token prefix
    (the 4096x4096-pixel image); one row of every 32-row query block, all heads."""
    torch = _cuda()
    rng = np.random.default_rng(8)
    c = _random_case(rng, [16384], [2048], 32, 8, "bf16")
    _say("attention long sample 16384 + 2048")
    out = neo.gen_attn_fwd(H.dev(c["q"], "bf16"), H.dev(c["k"], "bf16"), H.dev(c["v"], "bf16"),
                           H.dev(c["kp"], "bf16"), H.dev(c["vp"], "bf16"), H.dev_i32(c["cu_q"]),
                           H.dev_i32(c["cu_p"]), 16384, 2048)
    torch.cuda.synchronize()
    rows = _block_rows(16384, np.random.default_rng(9))
    ref = _timed("attention long sample", oracle.gen_attn, c["q"], c["k"], c["v"], c["kp"],
                 c["vp"], c["cu_q"], c["cu_p"], tokens=rows)
    H.assert_close(H.host(out)[rows], ref, "bf16", "long sample")


# --------------------------------------------------------------------------------------
# The block: prologue -> attention, each workload, against the fp64 chain
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_block_end_to_end(neo, name):
    torch = _cuda()
    w = W.make(name, pixels=False)
    kp, vp = H.frozen_prefix(w)
    _say(f"block {name}")
    qo, ko = _prologue_gpu(neo, w)
    d = w.dtype
    out = neo.gen_attn_fwd(qo, ko, H.dev(w.v, d), H.dev(kp, d), H.dev(vp, d), H.dev_i32(w.cu_q),
                           H.dev_i32(w.cu_p), max(w.n_img), max(w.n_prefix))
    torch.cuda.synchronize()
    qr, kr = _prologue_ref(w)
    ref = _timed(f"block {name}", oracle.gen_attn, qr, kr, w.v, kp, vp, w.cu_q, w.cu_p)
    H.assert_close(H.host(out), ref, d, f"block {name}")


# --------------------------------------------------------------------------------------
# Understanding-pass attention with the block-causal mask
# --------------------------------------------------------------------------------------

def _prefill_case(neo, d, what, rows=None, lse=True):
    torch = _cuda()
    qb, kb, vb = (W.bf16_round(d[x]) for x in ("q", "k", "v"))
    _say(f"prefill {what}: T={qb.shape[0]} Hq={qb.shape[1]} Hkv={kb.shape[1]} "
         f"cu={list(d['cu'])[:6]}")
    out, lse_d = neo.prefill_attn_fwd(H.dev(qb, "bf16"), H.dev(kb, "bf16"), H.dev(vb, "bf16"),
                                      H.dev_i32(d["idx"]), H.dev_i32(d["cu"]), d["max_len"],
                                      return_lse=True)
    torch.cuda.synchronize()
    got = H.host(out)
    ref, ref_lse = _timed(f"prefill {what}", oracle.prefill_attn, qb, kb, vb, d["idx"], d["cu"],
                          tokens=rows, with_lse=True)
    if rows is not None:
        got = got[rows]
    H.assert_close(got, ref, "bf16", f"prefill {what}")
    if lse:
        gl = H.host(lse_d).T
        gl = gl[rows] if rows is not None else gl
        _check_lse(gl, ref_lse, "bf16", f"prefill {what}")


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_prefill_configs(neo, name):
    """Each workload's prefix through the prefill attention: pure text (causal) for all but
    the editing workload, whose four ragged prefixes hold a 1024-token reference image
    between text and suffix; every row of every workload is compared."""
    w = W.make(name, pixels=False)
    d = W.prefill_inputs(w)
    _prefill_case(neo, d, name)


PREFILL_LAYOUTS = {
    # a run crossing 32-token wave and 64-token workgroup boundaries
    "text20_img50_text30": [[("text", 20), ("image", 50), ("text", 30)]],
    # one sample that is one image block (bidirectional), one shorter than a wave
    "image_only_and_short": [[("image", 150)], [("text", 5)]],
    # a run ending exactly at a wave boundary and another starting at one
    "aligned_runs": [[("text", 32), ("image", 32), ("image", 64), ("text", 1)]],
    # ragged batch, single-token sample, text-only sample with a ragged tail
    "ragged": [[("text", 1)], [("text", 97)], [("text", 3), ("image", 200), ("text", 10)]],
    # an image run that starts in one workgroup's last wave and runs 300 tokens on
    "long_run": [[("text", 60), ("image", 300), ("text", 70)]],
}


@pytest.mark.parametrize("layout", sorted(PREFILL_LAYOUTS))
def test_prefill_layouts(neo, layout):
    d = W.prefill_layout(PREFILL_LAYOUTS[layout], 32, 8, seed=len(layout))
    _prefill_case(neo, d, layout)


def test_prefill_run_beyond_probe(neo):
    """An image run of 2300 tokens: the kernel finds a run's end 1024 positions per probe,
    so the workgroups whose last query lies early in the run need three probes.  Every row
    is compared."""
    d = W.prefill_layout([[("text", 70), ("image", 2300), ("text", 40)]], 8, 2, seed=2300)
    _prefill_case(neo, d, "run beyond one probe")


def test_prefill_loose_bound(neo):
    """max_len at its largest allowed value, the total row count (311 against a longest
    sample of 213), only sizes the grid: the surplus workgroups find no rows (under the
    heaviest-first order they are the first to start), and every row still matches the
    oracle."""
    d = dict(W.prefill_layout(PREFILL_LAYOUTS["ragged"], 8, 2, seed=77))
    assert int(d["max_len"]) < int(d["cu"][-1])
    d["max_len"] = int(d["cu"][-1])
    _prefill_case(neo, d, "loose max_len")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 4), (12, 4)])
def test_prefill_heads(neo, hq, hkv):
    d = W.prefill_layout([[("text", 40), ("image", 70), ("text", 9)], [("text", 33)]], hq, hkv,
                         seed=hq * 10 + hkv)
    _prefill_case(neo, d, f"Hq={hq} Hkv={hkv}")


# --------------------------------------------------------------------------------------
# Generation-branch q/k/v projection fused with the q/k prologue
# --------------------------------------------------------------------------------------

def _proj_case(neo, x, wq, Hq, Hkv, nw, pos, what, rows=None, theta=5.0e6, theta_hw=1.0e4,
               eps=1e-6):
    torch = _cuda()
    xb, wb = W.bf16_round(x), W.bf16_round(wq)
    _say(f"qkv proj {what}: N={x.shape[0]} hidden={x.shape[1]} Hq={Hq} Hkv={Hkv}")
    q, k, v = neo.qkv_proj_norm_rope(H.dev(xb, "bf16"), H.dev(wb, "bf16"), Hq, Hkv,
                                     *[H.dev_f32(a) for a in nw], H.dev_i32(pos), theta, theta_hw,
                                     eps)
    torch.cuda.synchronize()
    rq, rk, rv = _timed(f"qkv proj {what}", oracle.qkv_proj_norm_rope, xb, wb, Hq, Hkv, *nw, pos,
                        theta, theta_hw, eps, tokens=rows)
    sel = (lambda a: a[rows]) if rows is not None else (lambda a: a)
    H.assert_close(sel(H.host(q)), rq, "bf16", f"qkv proj {what} q")
    H.assert_close(sel(H.host(k)), rk, "bf16", f"qkv proj {what} k")
    H.assert_close(sel(H.host(v)), rv, "bf16", f"qkv proj {what} v")


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_proj_configs(neo, name):
    """Each workload's image tokens (hidden = Hq * 128), every output row."""
    w = W.make(name, pixels=False)
    d = W.proj_inputs(w)
    _proj_case(neo, d["x"], d["w_qkv"], w.Hq, w.Hkv, (w.wq_t, w.wq_hw, w.wk_t, w.wk_hw),
               w.pos_img, name, None, w.rope_theta, w.rope_theta_hw, w.eps)


@pytest.mark.parametrize("N,hidden,Hq,Hkv", [
    (1, 64, 1, 1),          # one token, one stage of 64 hidden dims
    (130, 192, 3, 1),       # ragged token tile, 5 heads (half-empty feature tile), 3 stages
    (257, 256, 2, 2),       # 4 stages (loop break after one), two ragged token tiles
    (96, 1024, 4, 1),       # 16 stages, tokens fewer than one tile
])
def test_proj_shapes(neo, N, hidden, Hq, Hkv):
    _proj_random(neo, N, hidden, Hq, Hkv)


def test_proj_half_tiles(neo):
    """More 256x256 tiles than whole rounds of CUs: the surplus runs as 128-token halves,
    one of which starts past the last token (4196 tokens, 48 heads); every row."""
    _proj_random(neo, 4196, 4096, 32, 8)


def _proj_random(neo, N, hidden, Hq, Hkv, rows=None):
    rng = np.random.default_rng(N + hidden)
    x = rng.standard_normal((N, hidden)).astype(np.float32)
    wq = (rng.standard_normal(((Hq + 2 * Hkv) * 128, hidden)) / np.sqrt(hidden)).astype(np.float32)
    nw = tuple(rng.uniform(0.5, 1.5, 64).astype(np.float32) for _ in range(4))
    pos = np.stack([np.full(N, 300 + N), rng.integers(0, 64, N), rng.integers(0, 64, N)]).astype(np.int32)
    _proj_case(neo, x, wq, Hq, Hkv, nw, pos, f"N={N} hidden={hidden} Hq={Hq} Hkv={Hkv}", rows)
