"""Helpers shared by the tests, the smoke check and the benchmark's CPU leg.

Builds the frozen prefix cache where a workload specifies it by structure (the
understanding pass's norm + rotary applied to raw keys, computed by the oracle
and rounded to the workload dtype), moves workloads to the device, and holds
the parity tolerances.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

# Tolerances of the block's outputs against the fp64 oracle, per call:
#   fp32 outputs: max-abs <= 1e-4
#   bf16 outputs: max-abs <= 2e-2 and relative L2 <= 5e-3
TOL = {"f32": {"max_abs": 1e-4, "rel_l2": None}, "bf16": {"max_abs": 2e-2, "rel_l2": 5e-3}}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return W.bf16_round(x) if dtype == "bf16" else x


def frozen_prefix(w: W.Workload):
    """(k_prefix, v_prefix) as float32 arrays holding exact values of w.dtype."""
    if w.prefix_kind == "direct":
        return w.k_prefix, w.v_prefix
    k = oracle.norm_rope(w.k_prefix_pre, w.wk_und_t, w.wk_und_hw, w.pos_prefix, w.rope_theta,
                         w.rope_theta_hw, w.eps)
    return round_to(k, w.dtype), w.v_prefix


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str = ""):
    tol = TOL[dtype]
    max_abs, rel = errors(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']:.1e}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e} > {tol['rel_l2']:.1e}"
    print(f"[parity] {what}: max-abs {max_abs:.3e} rel-L2 {rel:.3e}", flush=True)
    return max_abs, rel


# Embedding front end (pixels and patch features enter the matrix cores in bf16): every
# element within 2^-5 (|ref| + rms(ref)) and relative L2 <= 5e-3.  Two bf16 roundings (the
# pixels, the patch features), each <= 2^-8 relative, reach an output through sums that
# scale like the output itself; a bf16 emulation of the chain in numpy measures
# max |err| / (|ref| + rms) ~ 1.0e-2 and rel-L2 ~ 2.4e-3 at noise scales 1 and 4, so the
# bound leaves a factor of three.
FRONT_END_REL = 2.0 ** -5


def assert_front_end(got, ref, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    worst = float(np.max(err / (np.abs(ref) + rms))) if ref.size else 0.0
    _, rel = errors(got, ref)
    assert worst <= FRONT_END_REL, f"{what}: max |err|/(|ref|+rms) {worst:.3e} > {FRONT_END_REL:.2e}"
    assert rel <= 5e-3, f"{what}: rel-L2 {rel:.3e} > 5e-3"
    max_abs = float(np.max(err)) if ref.size else 0.0
    print(f"[parity] {what}: max |err|/(|ref|+rms) {worst:.3e} rel-L2 {rel:.3e} "
          f"max-abs {max_abs:.3e} (max |ref| {float(np.max(np.abs(ref))) if ref.size else 0.0:.3g}, "
          f"rms {rms:.3g})", flush=True)
    return worst, rel


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype: str, device="cuda"):
    """float32 numpy (exact in dtype) -> device tensor of dtype."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(
        torch_dtype(dtype))


def dev_i32(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def dev_f32(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()
