"""The generation step under HIP graph capture.

One step of the path (norm + rotary on the image queries and keys, the attention over
[prefix ; image block], one Euler step on the pixels) enqueues only the library's own
kernels on the caller's stream: no allocation, no synchronisation, no memset.  A caller can
therefore capture it once and replay it.  The step is captured on torch's capture stream
and replayed several times, each replay preceded by eager work on the same buffers (the
pixel state reset by a copy, an eager step on other buffers) and a synchronisation; every
replay must reproduce the eager step bit for bit (the kernels are deterministic: no
atomics, a fixed reduction order).
"""
import sys

import numpy as np
import pytest

import workloads as W
from tests import harness as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(torch, w, roll=0):
    kp, vp = H.frozen_prefix(w)
    z0 = (np.float32(w.sigma_R) * w.eps_pixels).astype(np.float32)
    d = dict(q=H.dev(np.roll(w.q, roll, 0), w.dtype), k=H.dev(np.roll(w.k, roll, 0), w.dtype),
             v=H.dev(w.v, w.dtype), kp=H.dev(kp, w.dtype), vp=H.dev(vp, w.dtype),
             cu_q=H.dev_i32(w.cu_q), cu_p=H.dev_i32(w.cu_p), wq_t=H.dev_f32(w.wq_t),
             wq_hw=H.dev_f32(w.wq_hw), wk_t=H.dev_f32(w.wk_t), wk_hw=H.dev_f32(w.wk_hw),
             pos=H.dev_i32(w.pos_img), z0=H.dev_f32(z0), x=H.dev_f32(w.x_hat))
    d["z"] = d["z0"].clone()
    d["qo"] = torch.empty_like(d["q"])
    d["ko"] = torch.empty_like(d["k"])
    d["out"] = torch.empty_like(d["q"])
    return d


def _step(neo, w, d):
    neo.qknorm_rope3(d["q"], d["k"], d["wq_t"], d["wq_hw"], d["wk_t"], d["wk_hw"], d["pos"],
                     w.rope_theta, w.rope_theta_hw, w.eps, q_out=d["qo"], k_out=d["ko"])
    neo.gen_attn_fwd(d["qo"], d["ko"], d["v"], d["kp"], d["vp"], d["cu_q"], d["cu_p"],
                     max(w.n_img), max(w.n_prefix), out=d["out"])
    neo.fm_euler_step(d["z"], d["x"], w.t_grid[0], w.t_grid[1], w.t_eps)


@pytest.fixture(scope="module")
def neo():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import pixel_space_flow_amd as P
    P.lib()  # raises if the library is missing
    return P


def _same_bits(torch, a, b):
    iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.reshape(-1).view(iv), b.reshape(-1).view(iv))


# the small workload takes the split-key attention launch, the 4096-token one the
# 64-token launch of the benchmark
@pytest.mark.parametrize("name", ["small", "large"])
def test_step_graph_replay(neo, name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    w = W.make(name)
    _say(f"{name}: {w.Tq} image tokens, prefix {w.n_prefix}, pixels {list(w.pixel_shape)}")
    d = _inputs(torch, w)
    other = _inputs(torch, w, roll=1)

    # the eager step
    d["z"].copy_(d["z0"])
    _step(neo, w, d)
    torch.cuda.synchronize()
    ref = {key: d[key].clone() for key in ("qo", "ko", "out", "z")}

    # capture (after a warm-up on the capture's side stream, as torch asks)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d["z"].copy_(d["z0"])
        _step(neo, w, d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(neo, w, d)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays: clear the outputs, reset the pixel state, run an
        # eager step on other buffers
        for key in ("qo", "ko", "out"):
            d[key].zero_()
        d["z"].copy_(d["z0"])
        other["z"].copy_(other["z0"])
        _step(neo, w, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, r in ref.items():
            assert _same_bits(torch, d[key], r), \
                f"{name}: replay {rep} differs from the eager step in {key}"
        _say(f"{name}: replay {rep} bit-identical to the eager step")

    # the eager path still gives the same result after the replays
    d["z"].copy_(d["z0"])
    _step(neo, w, d)
    torch.cuda.synchronize()
    for key, r in ref.items():
        assert _same_bits(torch, d[key], r), \
            f"{name}: eager step after the replays differs in {key}"
    del g
