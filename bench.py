"""Benchmark of the generation-pass attention block on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
split-half QK-RMSNorm + three-axis rotary on the image queries and keys, the
image queries' attention over [512-token frozen prefix ; 4096 image tokens],
and one x0 -> velocity Euler step on the 3x2048x2048 pixel tensor.  Inputs are
resident in HBM before the timed region; a few input sets are rotated so the
bandwidth-bound kernels are not served from the 256 MB Infinity Cache.

Prints one JSON line.  value = image tokens per second per step (4096 / wall-clock
time per step over exactly --steps steps after --warmup untimed ones).  Before that
loop, --calls steps (after a warm-up of at least 10 steps and 100 ms) time every
kernel between its own HIP events on the launch stream: roofline = the attention kernel's achieved bf16 MFMA
TFLOP/s (algorithmic 4*Hq*D*N*(P+N) flops over its mean per-call duration) against
the 2.5 PFLOP/s dense peak, and the per-kernel rates use the medians.  The same
per-call figures are given for the 1024-token workload (1024x1024 pixels).
cpu_baseline = the fp64 oracle on the host cores (and on one thread), on a bounded
sample of the same step, median of 3 runs after 1 warm-up.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gen-pass attention TFLOP/s + image-tokens/s per FM step at 4096 tokens (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# decoder layers of the generation branch, each with its own norm + rotary and attention
# ("SenseNova-U1.5 (NEO-unify) architecture", §Mixture of Transformers)
N_LAYERS = 42


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large", choices=["large", "mid", "small", "editing"])
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--proj-steps", type=int, default=50,
                    help="timed calls of the fused q/k/v projection + prologue on the workload's "
                         "image tokens, beside a library GEMM plus the separate prologue (0 skips)")
    ap.add_argument("--embed-steps", type=int, default=50,
                    help="calls per kernel of the embedding front end at the workload's pixels")
    ap.add_argument("--prefill-steps", type=int, default=100,
                    help="timed calls of the block-causal prefill attention on the editing "
                         "workload's prefixes (0 skips it)")
    ap.add_argument("--cfg-steps", type=int, default=100,
                    help="timed calls of the guided Euler step per guidance path (0 skips it)")
    ap.add_argument("--calls", type=int, default=300,
                    help="steps timed kernel by kernel (after the warm-up) for the per-call "
                         "durations the roofline and rates use (0: use the --steps loop)")
    ap.add_argument("--mid-calls", type=int, default=300,
                    help="steps of the 1024-token workload timed the same way (0 skips it)")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="query tokens in the oracle's attention sample with all host cores")
    ap.add_argument("--cpu-tokens-1t", type=int, default=16,
                    help="query tokens in the oracle's attention sample with one thread")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters, if present")
    ap.add_argument("--calib-mib", type=int, default=256,
                    help="size of the device-to-device copy run once before warm-up, the known-size "
                         "reference for the HBM byte counters")
    ap.add_argument("--derive-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, -f csv) into HBM bytes per launch and write --traffic-json")
    return ap.parse_args()


KERNELS = {"patch_gemm_kernel": "patch_gemm_kernel", "merge_gemm_kernel": "merge_gemm_kernel",
           "patch_px_gemm_kernel": "patch_px_gemm_kernel",
           "gen_attn_bf16_kernel": "gen_attn_bf16_kernel", "qknorm_rope3": "qknorm_rope3_kernel",
           "fm_euler_step": "euler_vec4_kernel", "prefill_attn_bf16_kernel": "prefill_attn_bf16_kernel",
           "fm_euler_step_cfg": "euler_cfg_vec4_kernel", "qkv_proj_bf16_kernel": "qkv_proj_bf16_kernel"}
KERNEL_SOURCES = {"patch_gemm_kernel": "front_end.hip", "merge_gemm_kernel": "front_end.hip",
                  "patch_px_gemm_kernel": "front_end.hip",
                  "gen_attn_bf16_kernel": "gen_attn.hip", "qknorm_rope3": "qknorm_rope3.hip",
                  "fm_euler_step": "euler_step.hip", "prefill_attn_bf16_kernel": "gen_attn.hip",
                  "fm_euler_step_cfg": "euler_step.hip", "qkv_proj_bf16_kernel": "qkv_proj.hip"}


def _counter_rows(d, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def _kernel_source_hash(key):
    """sha256 of the HIP source a kernel is built from, followed by every header of the
    library (the shared tile core and device helpers): byte counts taken from one build are
    not reported for another."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "pixel_space_flow_amd", "csrc")
    files = [os.path.join(csrc, KERNEL_SOURCES[key])]
    files += sorted(glob.glob(os.path.join(csrc, "*.h")))
    files += [os.path.join(ROOT, "include", "neo.h")]
    h = hashlib.sha256()
    for path in files:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def derive_traffic(a):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for the known-size calibration copy."""
    out = {"calibration_bytes": a.calib_mib << 20, "workload": a.workload}
    for counter, d in (("FETCH_SIZE", a.derive_traffic[0]), ("WRITE_SIZE", a.derive_traffic[1])):
        rows = _counter_rows(d, counter)
        calib_bytes = a.calib_mib << 20
        copies = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]]
        # the copy's counter reads within a small factor of its size (FETCH_SIZE about half
        # of it on this part); smaller copies (set-up) fall far below a quarter
        big = [c for c in copies if c > 0.25 * calib_bytes]
        if not big:
            raise SystemExit(f"{counter}: calibration copy not found in {d}")
        scale = calib_bytes / (sum(big) / len(big))
        out[f"{counter}_scale"] = scale
        for key, pat in KERNELS.items():
            vals = [float(r["Counter_Value"]) * 1024 for r in rows if pat in r["Kernel_Name"]]
            if vals:
                out.setdefault(key, {})[counter] = sum(vals) / len(vals) * scale
    for key in KERNELS:
        if key in out and {"FETCH_SIZE", "WRITE_SIZE"} <= set(out[key]):
            out[key]["bytes"] = out[key]["FETCH_SIZE"] + out[key]["WRITE_SIZE"]
            out[key]["source_sha256"] = _kernel_source_hash(key)
    os.makedirs(os.path.dirname(a.traffic_json), exist_ok=True)
    with open(a.traffic_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def stats_us(ms_values):
    """Summary of per-call durations given in ms: median, mean, min, p90, count (in us)."""
    v = np.asarray(ms_values, dtype=np.float64) * 1e3
    return {"median": float(np.median(v)), "mean": float(v.mean()), "min": float(v.min()),
            "p90": float(np.percentile(v, 90)), "calls": int(v.size)}


# Untimed work before every per-call measurement.  Under sustained load the part's clock
# settles only after a transient: in a kernel trace the 4096-token attention starts near
# 280 us, climbs to 320-345 us within a few ms and settles at ~264 us after about 80
# back-to-back calls (~25 ms); a pause of a few ms restarts the transient.  Warming up
# for WARM_MS (and at least 10 calls) puts the timed calls in the settled state.
WARM_MS = 100.0


def warm_up(fn, min_calls=10, ms=WARM_MS):
    """Call fn() (fn(i) with a counter when it takes one) until at least min_calls calls
    and `ms` milliseconds of device time have passed; returns the calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if n >= min_calls and (time.perf_counter() - t0) * 1e3 >= ms:
            return n


def timed_calls(fn, n):
    """Per-call durations (us) of n calls of fn after the warm-up, each call bracketed by
    its own pair of events on the current stream (the stream the library launches on):
    the summary of stats_us."""
    import torch
    warm_up(lambda i: fn())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return stats_us([e0.elapsed_time(e1) for e0, e1 in evs])


def measured_bytes(a, key):
    """HBM bytes per launch of kernel `key` from the stored counter runs, or None when they
    were taken on another workload or before the kernel's source last changed."""
    if not os.path.exists(a.traffic_json):
        return None
    with open(a.traffic_json) as f:
        tj = json.load(f)
    k = tj.get(key, {})
    if tj.get("workload") != a.workload or k.get("source_sha256") != _kernel_source_hash(key):
        return None
    return k.get("bytes")


def algorithmic(w):
    D = 128
    flops = 4.0 * w.Hq * D * sum(n * (p + n) for n, p in zip(w.n_img, w.n_prefix))
    pro_bytes = w.Tq * ((w.Hq + w.Hkv) * D * 2 * 2 + 3 * 4)   # bf16 read + write, positions
    npx = int(np.prod(w.pixel_shape))
    euler_bytes = npx * 12                                     # fp32 z, x0 read; z written
    attn_bytes = (w.Tq * (w.Hq * 2 + w.Hkv * 2) + w.Tp * w.Hkv * 2) * D * 2
    return flops, pro_bytes, euler_bytes, attn_bytes


def cpu_baseline(w, kp, vp, tokens_all, tokens_one):
    """The fp64 oracle on the host, on a bounded sample of one step of workload w: norm +
    rotary on every token, the Euler step on every pixel, and attention on a spread of query
    tokens (all heads, all keys) whose time is scaled to all Tq tokens.  Timed with all
    host cores and with one thread; each figure is the median of 3 runs after 1 warm-up."""
    import oracle
    z0 = np.float32(w.sigma_R) * w.eps_pixels

    def one_run(n_tokens):
        rows = np.linspace(0, w.Tq - 1, n_tokens).astype(np.int64)
        t0 = time.perf_counter()
        qr, kr = oracle.qknorm_rope3(w.q, w.k, w.wq_t, w.wq_hw, w.wk_t, w.wk_hw, w.pos_img,
                                     w.rope_theta, w.rope_theta_hw, w.eps)
        t1 = time.perf_counter()
        oracle.gen_attn(qr, kr, w.v, kp, vp, w.cu_q, w.cu_p, tokens=rows)
        t2 = time.perf_counter()
        oracle.euler_step(z0, w.x_hat, w.t_grid[0], w.t_grid[1], w.t_eps)
        t3 = time.perf_counter()
        attn = (t2 - t1) * (w.Tq / n_tokens)
        return {"prologue": t1 - t0, "attention_scaled": attn, "euler": t3 - t2,
                "step": (t1 - t0) + attn + (t3 - t2)}

    def median_of_3(n_tokens, threads):
        oracle.set_num_threads(threads)
        one_run(n_tokens)                                     # warm-up
        runs = sorted((one_run(n_tokens) for _ in range(3)), key=lambda r: r["step"])
        return runs[1], oracle.num_threads()   # the run with the median step time

    all_threads = os.cpu_count() or 1
    med_all, cores = median_of_3(tokens_all, all_threads)
    med_one, _ = median_of_3(tokens_one, 1)
    oracle.set_num_threads(all_threads)
    flops = 4.0 * w.Hq * 128 * sum(n * (p + n) for n, p in zip(w.n_img, w.n_prefix))
    return {
        "value": w.Tq / med_all["step"], "unit": "image-tokens/s", "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 oracle, one step of the {w.name} workload: norm+rotary on all {w.Tq} "
                   f"tokens, the Euler step on all {int(np.prod(w.pixel_shape))} pixels, attention "
                   f"on {tokens_all} of {w.Tq} query tokens spread over the image (all {w.Hq} "
                   f"heads, all keys) with its time scaled by {w.Tq / tokens_all:g}; median of 3 "
                   f"runs after 1 warm-up"),
        "seconds": med_all,
        "attention_gflops": flops / med_all["attention_scaled"] / 1e9,
        "one_thread": {"value": w.Tq / med_one["step"], "cores": 1, "seconds": med_one,
                       "sample": (f"as above with {tokens_one} attention query tokens, time "
                                  f"scaled by {w.Tq / tokens_one:g}")},
    }


def resident_sets(w, n_sets):
    """Input sets of workload w resident in HBM (each set rolls the seeded inputs so the
    buffers differ), plus the tensors every step shares."""
    import torch
    from tests import harness as H
    if w.prefix_kind == "direct":
        kp, vp = w.k_prefix, w.v_prefix
    else:
        kp, vp = H.frozen_prefix(w)
    z0 = (np.float32(w.sigma_R) * w.eps_pixels).astype(np.float32)
    base = dict(q=H.dev(w.q, "bf16"), k=H.dev(w.k, "bf16"), v=H.dev(w.v, "bf16"),
                z=H.dev_f32(z0), x=H.dev_f32(w.x_hat))
    sets = []
    for s in range(n_sets):
        sets.append({
            "q": base["q"].roll(s, 0).contiguous(), "k": base["k"].roll(s, 0).contiguous(),
            "v": base["v"].roll(s, 0).contiguous(), "z": base["z"].roll(s).contiguous(),
            "x": base["x"].roll(s).contiguous(),
            "qo": torch.empty_like(base["q"]), "ko": torch.empty_like(base["k"]),
            "out": torch.empty_like(base["q"]),
        })
    del base
    shared = dict(kp=H.dev(kp, "bf16"), vp=H.dev(vp, "bf16"), cu_q=H.dev_i32(w.cu_q),
                  cu_p=H.dev_i32(w.cu_p), wq_t=H.dev_f32(w.wq_t), wq_hw=H.dev_f32(w.wq_hw),
                  wk_t=H.dev_f32(w.wk_t), wk_hw=H.dev_f32(w.wk_hw), pos=H.dev_i32(w.pos_img))
    return sets, shared, kp, vp


def step_fn(neo, w, sets, shared):
    """One step of the path on input set i % len(sets): norm + rotary, attention, Euler.
    With ev (4 events) the kernel boundaries are recorded on the launch stream."""
    max_q, max_p = max(w.n_img), max(w.n_prefix)
    t, tn = w.t_grid[0], w.t_grid[1]

    def step(i, ev=None):
        s = sets[i % len(sets)]
        if ev is not None:
            ev[0].record()
        neo.qknorm_rope3(s["q"], s["k"], shared["wq_t"], shared["wq_hw"], shared["wk_t"],
                         shared["wk_hw"], shared["pos"], w.rope_theta, w.rope_theta_hw, w.eps,
                         q_out=s["qo"], k_out=s["ko"])
        if ev is not None:
            ev[1].record()
        neo.gen_attn_fwd(s["qo"], s["ko"], s["v"], shared["kp"], shared["vp"], shared["cu_q"],
                         shared["cu_p"], max_q, max_p, out=s["out"])
        if ev is not None:
            ev[2].record()
        neo.fm_euler_step(s["z"], s["x"], t, tn, w.t_eps)
        if ev is not None:
            ev[3].record()
    return step


def per_call_enqueue(step, calls):
    """Warm up, then enqueue `calls` steps with each kernel between its own pair of events.
    Returns the events; nothing waits for them, so work enqueued next follows without a
    pause on the device."""
    import torch
    warm_up(step)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(calls)]
    for i in range(calls):
        step(i, evs[i])
    return evs


def per_call_stats(evs):
    """stats_us per kernel from per_call_enqueue's events (after the stream has drained)."""
    return {"qknorm_rope3": stats_us([e[0].elapsed_time(e[1]) for e in evs]),
            "gen_attn": stats_us([e[1].elapsed_time(e[2]) for e in evs]),
            "fm_euler_step": stats_us([e[2].elapsed_time(e[3]) for e in evs])}


def per_call(step, calls):
    """Per-kernel durations of `calls` steps after the warm-up (stats_us per kernel)."""
    import torch
    evs = per_call_enqueue(step, calls)
    torch.cuda.synchronize()
    return per_call_stats(evs)


def path_figures(w, k_us, stat):
    """Rates of one step of workload w from per-kernel durations k_us[kernel][stat] (us)."""
    flops, pro_bytes, euler_bytes, _ = algorithmic(w)
    att_s = k_us["gen_attn"][stat] * 1e-6
    pro_s = k_us["qknorm_rope3"][stat] * 1e-6
    eul_s = k_us["fm_euler_step"][stat] * 1e-6
    step_s = att_s + pro_s + eul_s
    roof_step_s = flops / (PEAK_BF16_TFLOPS * 1e12) + (pro_bytes + euler_bytes) / (PEAK_HBM_GBS * 1e9)
    return {
        "attention_tflops": flops / att_s / 1e12,
        "attention_frac": flops / att_s / 1e12 / PEAK_BF16_TFLOPS,
        "prologue_gbs": pro_bytes / pro_s / 1e9, "euler_gbs": euler_bytes / eul_s / 1e9,
        "image_tokens_per_s": w.Tq / step_s,
        "image_tokens_per_s_at_roofline": w.Tq / roof_step_s,
        "step_frac": roof_step_s / step_s,
    }


def main():
    a = parse()
    if a.derive_traffic:
        derive_traffic(a)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the block shards by KV head or by CFG branch with no exchange inside it). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import pixel_space_flow_amd as neo
    import workloads as W
    from tests import harness as H

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    neo.lib()

    w = W.make(a.workload)
    sets, shared, kp, vp = resident_sets(w, a.sets)
    flops, pro_bytes, euler_bytes, attn_bytes = algorithmic(w)
    step = step_fn(neo, w, sets, shared)
    t, tn = w.t_grid[0], w.t_grid[1]

    # known-size plain copy: the reference the HBM byte counters are scaled by
    if a.calib_mib > 0:
        src = torch.empty(a.calib_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # per-call durations: warm-up (at least WARM_MS of steps), then `calls` steps with every
    # kernel between its own events; the roofline and the per-kernel rates come from these.
    # The W warm-up steps of the benchmark proper are enqueued right behind them and the
    # events are read only after the timed steps, so the device runs without a pause from
    # the warm-up to the end of the timed steps (a pause of a few ms restarts the clock
    # transient described at WARM_MS).
    pc_events = per_call_enqueue(step, a.calls) if a.calls > 0 else None
    for i in range(a.warmup):
        step(i)

    # the benchmark proper: W untimed steps (above), then exactly K steps between two
    # synchronisations.  No event is recorded inside them: an event record between two
    # kernels adds its own dispatch to the stream (about 4% of a step in same-box runs).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / a.steps
    # the same K steps once more, each kernel between its own events, for the per-kernel
    # durations of the steps as timed (queued back to back, read after the stream drains)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    for i in range(a.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    steps_us = {"qknorm_rope3": stats_us([e[0].elapsed_time(e[1]) for e in events]),
                "gen_attn": stats_us([e[1].elapsed_time(e[2]) for e in events]),
                "fm_euler_step": stats_us([e[2].elapsed_time(e[3]) for e in events])}
    print(f"[bench] warm-up ({a.warmup} steps) and {a.steps} timed steps: {ms_step:.4f} ms/step",
          file=sys.stderr, flush=True)
    kus = per_call_stats(pc_events) if pc_events is not None else steps_us
    if pc_events is not None:
        print(f"[bench] per-call timing: {a.calls} steps after a {WARM_MS:g} ms warm-up; "
              f"attention median {kus['gen_attn']['median']:.1f} us", file=sys.stderr, flush=True)

    attn_mean_s = kus["gen_attn"]["mean"] * 1e-6
    achieved = flops / attn_mean_s / 1e12
    traffic = measured_bytes(a, "gen_attn_bf16_kernel")
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic}
    fig = path_figures(w, kus, "median")
    del sets, shared

    # the pages' other resolution: 1024x1024 pixels -> 1024 image tokens (256-token prefix),
    # the same step path at that size, timed the same way
    mid = {}
    if a.mid_calls > 0 and a.workload != "mid":
        wm = W.make("mid")
        m_sets, m_shared, m_kp, m_vp = resident_sets(wm, a.sets)
        m_kus = per_call(step_fn(neo, wm, m_sets, m_shared), a.mid_calls)
        del m_sets, m_shared
        m_fig = path_figures(wm, m_kus, "median")
        m_flops = algorithmic(wm)[0]
        mid = {
            "workload": (f"mid: {wm.B} sample, {wm.Tq} image tokens (1024x1024 px), prefix "
                         f"{wm.n_prefix}, Hq={wm.Hq}, Hkv={wm.Hkv}, head_dim=128"),
            "attention_gflop": m_flops / 1e9,
            "kernels_us": m_kus,
            "roofline": {"bound": "mfma",
                         "achieved": m_flops / (m_kus["gen_attn"]["mean"] * 1e-6) / 1e12,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": m_flops / (m_kus["gen_attn"]["mean"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS},
            **m_fig,
        }
        print(f"[bench] 1024-token workload timed ({a.mid_calls} steps): attention median "
              f"{m_kus['gen_attn']['median']:.1f} us", file=sys.stderr, flush=True)

    # the guided step of the next row: guidance over the branches' x0 fused with the
    # Euler update, on the pages' text-to-image path (2 branches) and the full 3-branch path
    cfg = {}
    if a.cfg_steps > 0:
        x_tu, x_u = W.cfg_branches(w)
        z0 = (np.float32(w.sigma_R) * w.eps_pixels).astype(np.float32)
        npx = int(np.prod(w.pixel_shape))
        zs = [H.dev_f32(np.roll(z0, k_)) for k_ in range(a.sets)]
        xs = [[H.dev_f32(np.roll(x_, k_)) for x_ in (w.x_hat, x_tu, x_u)] for k_ in range(a.sets)]
        for label, g, gi, nbr in (("path2_text_to_image", 4.0, 1.0, 2), ("path4_three_branch", 4.0, 1.5, 3)):
            assert neo.cfg_path(t, g, gi) == (2 if nbr == 2 else 4)
            ctr = [0]

            def cfg_step():
                k_ = ctr[0] % a.sets
                ctr[0] += 1
                neo.fm_euler_step_cfg(zs[k_], *xs[k_], t=t, t_next=tn, t_eps=w.t_eps,
                                      cfg_scale=g, img_cfg_scale=gi)
            st = timed_calls(cfg_step, a.cfg_steps)
            nbytes = npx * 4 * (nbr + 2)
            cfg[label] = {"us": st, "bytes": nbytes,
                          "gbs": nbytes / (st["median"] * 1e-6) / 1e9,
                          "hbm_frac": nbytes / (st["median"] * 1e-6) / 1e9 / PEAK_HBM_GBS}
        del zs, xs
        print(f"[bench] guided Euler step timed ({a.cfg_steps} calls per path)", file=sys.stderr,
              flush=True)

    # the generation branch's q/k/v projection fused with the prologue, beside the unfused
    # route (library bf16 GEMM, then the stand-alone norm + rotary pass)
    proj = {}
    if a.proj_steps > 0:
        d = W.proj_inputs(w)
        px = H.dev(W.bf16_round(d["x"]), "bf16")
        pw = H.dev(W.bf16_round(d["w_qkv"]), "bf16")
        hid = d["hidden"]
        nq, nk = w.Hq * 128, w.Hkv * 128
        pq = torch.empty((w.Tq, w.Hq, 128), dtype=torch.bfloat16, device=dev)
        pk = torch.empty((w.Tq, w.Hkv, 128), dtype=torch.bfloat16, device=dev)
        pv = torch.empty_like(pk)
        nws = [H.dev_f32(x_) for x_ in (w.wq_t, w.wq_hw, w.wk_t, w.wk_hw)]
        pos = H.dev_i32(w.pos_img)
        pflops = 2.0 * w.Tq * hid * (nq + 2 * nk)

        def fused():
            neo.qkv_proj_norm_rope(px, pw, w.Hq, w.Hkv, *nws, pos, w.rope_theta,
                                   w.rope_theta_hw, w.eps, q_out=pq, k_out=pk, v_out=pv)
        y = torch.empty((w.Tq, nq + 2 * nk), dtype=torch.bfloat16, device=dev)

        def unfused():
            torch.matmul(px, pw.t(), out=y)
            neo.qknorm_rope3(y[:, :nq].view(w.Tq, w.Hq, 128).contiguous(),
                             y[:, nq:nq + nk].view(w.Tq, w.Hkv, 128).contiguous(), *nws,
                             pos, w.rope_theta, w.rope_theta_hw, w.eps)

        st = timed_calls(fused, a.proj_steps)
        st_lib = timed_calls(unfused, a.proj_steps)
        us = st["median"]
        proj = {"workload": f"{w.Tq} tokens x hidden {hid} -> {w.Hq}+{w.Hkv}+{w.Hkv} heads",
                "gflop": pflops / 1e9, "us": st, "tflops": pflops / (us * 1e-6) / 1e12,
                "frac": pflops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                "unfused_library_gemm_plus_prologue_us": st_lib,
                "hbm_bytes_measured": measured_bytes(a, "qkv_proj_bf16_kernel")}
        del px, pw, pq, pk, pv, y
        print(f"[bench] fused projection timed ({a.proj_steps} calls)", file=sys.stderr, flush=True)

    # the generation branch's embedding front end at the workload's pixel shape: patchify,
    # patch convolution (+ GELU + rotary), the two embedders, the merge convolution
    embed = {}
    if a.embed_steps > 0:
        d = W.embed_inputs(w)
        r = W.bf16_round
        Bz, _, Hz, Wz = d["z"].shape
        C1, D = d["w1"].shape[0], d["w2"].shape[0]
        ez = H.dev_f32(d["z"])
        ew1 = H.dev(r(d["w1"]).reshape(C1, -1), "bf16")
        eb1, eb2 = H.dev_f32(d["b1"]), H.dev_f32(d["b2"])
        ew2 = H.dev(np.ascontiguousarray(r(d["w2"]).transpose(0, 2, 3, 1)), "bf16")
        embs = [(H.dev(r(e[0]), "bf16"), H.dev_f32(e[1]), H.dev(r(e[2]), "bf16"), H.dev_f32(e[3]))
                for e in (d["emb_t"], d["emb_s"])]
        del d["w2"], d["emb_t"], d["emb_s"]
        npix, P = Bz * 3 * Hz * Wz, Bz * (Hz // 16) * (Wz // 16)
        ntok = Bz * (Hz // 32) * (Wz // 32)
        pbuf = torch.empty((P, 768), dtype=torch.bfloat16, device=dev)
        hbuf = torch.empty((P, C1), dtype=torch.bfloat16, device=dev)
        hid = torch.empty((2, D), dtype=torch.float32, device=dev)
        cbuf = torch.empty((D,), dtype=torch.float32, device=dev)
        tbuf = torch.empty((ntok, D), dtype=torch.float32, device=dev)
        st_x = timed_calls(lambda: neo.gen_patch_embed_px(ez, ew1, eb1, h_out=hbuf), a.embed_steps)
        st_p = timed_calls(lambda: neo.gen_patchify(ez, patches=pbuf), a.embed_steps)
        st_c = timed_calls(lambda: neo.gen_patch_embed(pbuf, Bz, Hz, Wz, ew1, eb1, h_out=hbuf),
                           a.embed_steps)
        st_e = timed_calls(lambda: neo.gen_cond_embed(d["t"], d["noise_scale"], d["noise_scale_max"],
                                                      embs[0], embs[1], hidden=hid, cond=cbuf),
                           a.embed_steps)
        st_m = timed_calls(lambda: neo.gen_merge_embed(hbuf, Bz, Hz, Wz, ew2, eb2, cbuf, tokens=tbuf),
                           a.embed_steps)
        # a library matrix product of the merge's shape (contiguous operands), for scale
        ga = torch.empty((ntok, 4 * C1), dtype=torch.bfloat16, device=dev).normal_()
        gy = torch.empty((ntok, D), dtype=torch.bfloat16, device=dev)
        st_lib = timed_calls(lambda: torch.matmul(ga, ew2.view(D, -1).t(), out=gy), a.embed_steps)
        us_x, us_p, us_c, us_e, us_m = (x_["median"] for x_ in (st_x, st_p, st_c, st_e, st_m))
        p_bytes = npix * 6                                   # fp32 read + bf16 written
        c_flop = 2.0 * P * C1 * 768
        e_bytes = 2 * D * 256 * 2 + 2 * D * D * 2           # both layers' bf16 weights
        m_flop = 2.0 * ntok * D * 4 * C1
        embed = {
            "workload": f"{Bz}x3x{Hz}x{Wz} px -> {ntok} tokens, C1={C1}, D={D}",
            "patch_conv_from_pixels": {"us": st_x, "gflop": c_flop / 1e9,
                                       "tflops": c_flop / (us_x * 1e-6) / 1e12,
                                       "frac": c_flop / (us_x * 1e-6) / 1e12 / PEAK_BF16_TFLOPS},
            "two_launch_route": {
                "patchify": {"us": st_p, "bytes": p_bytes, "gbs": p_bytes / (us_p * 1e-6) / 1e9},
                "patch_conv_gelu_rope": {"us": st_c, "gflop": c_flop / 1e9,
                                         "tflops": c_flop / (us_c * 1e-6) / 1e12,
                                         "frac": c_flop / (us_c * 1e-6) / 1e12 / PEAK_BF16_TFLOPS},
                "us_median": us_p + us_c},
            "cond_embedders": {"us": st_e, "bytes": e_bytes, "gbs": e_bytes / (us_e * 1e-6) / 1e9},
            "merge_conv": {"us": st_m, "gflop": m_flop / 1e9, "tflops": m_flop / (us_m * 1e-6) / 1e12,
                           "frac": m_flop / (us_m * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                           "library_gemm_same_shape_us": st_lib},
            "total_us_median": us_x + us_e + us_m,
        }
        del ez, ew1, ew2, embs, pbuf, hbuf, tbuf, ga, gy
        print(f"[bench] embedding front end timed ({a.embed_steps} calls per kernel)",
              file=sys.stderr, flush=True)

    # the understanding-pass (prefill) attention of the next row, on the editing workload's
    # four ragged prefixes (text, a 1024-token reference image, suffix)
    prefill = {}
    if a.prefill_steps > 0:
        we = W.make("editing", pixels=False)
        d = W.prefill_inputs(we)
        pq, pk, pv = (H.dev(W.bf16_round(d[x]), "bf16") for x in ("q", "k", "v"))
        pidx, pcu = H.dev_i32(d["idx"]), H.dev_i32(d["cu"])
        pout = torch.empty_like(pq)
        # algorithmic work: 4*Hq*128 flops per allowed (query, key) pair
        pairs = 0
        for b in range(len(d["cu"]) - 1):
            ix = d["idx"][d["cu"][b]:d["cu"][b + 1]]
            last = np.searchsorted(ix, ix, side="right") - 1   # end of each query's index run
            pairs += int(np.sum(np.maximum(np.arange(ix.size), last) + 1))
        pflops = 4.0 * we.Hq * 128 * pairs
        st = timed_calls(lambda: neo.prefill_attn_fwd(pq, pk, pv, pidx, pcu, d["max_len"], out=pout),
                         a.prefill_steps)
        us = st["median"]
        prefill = {"workload": (f"editing prefixes: {len(d['cu']) - 1} samples, "
                                f"{[int(x_) for x_ in np.diff(d['cu'])]} tokens, Hq={we.Hq}, "
                                f"Hkv={we.Hkv}"),
                   "allowed_pairs": pairs, "gflop": pflops / 1e9, "us": st,
                   "tflops": pflops / (us * 1e-6) / 1e12,
                   "frac": pflops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
        del pq, pk, pv, pout
        print(f"[bench] prefill attention timed ({a.prefill_steps} calls)", file=sys.stderr,
              flush=True)

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, kp, vp, a.cpu_tokens, a.cpu_tokens_1t)
        if mid:
            wm = W.make("mid")
            mid["cpu_baseline"] = cpu_baseline(wm, wm.k_prefix, wm.v_prefix, a.cpu_tokens,
                                               a.cpu_tokens_1t)
        print("[bench] oracle timed", file=sys.stderr, flush=True)

    ntok = w.Tq
    pro_us, att_us, eul_us = (kus[k_]["median"] for k_ in ("qknorm_rope3", "gen_attn", "fm_euler_step"))
    result = {
        "metric": METRIC,
        "value": ntok / (ms_step * 1e-3),
        "unit": "image-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{a.workload}: {w.B} sample(s), {ntok} image tokens "
                         f"({w.pixel_shape[2]}x{w.pixel_shape[3]} px), prefix {w.n_prefix}, "
                         f"Hq={w.Hq}, Hkv={w.Hkv}, head_dim=128; one norm+rotary, one "
                         f"attention and one Euler step per step"),
            "batch": w.B, "image_tokens": ntok, "prefix_tokens": w.Tp,
            "pixels": list(w.pixel_shape), "input_sets": a.sets,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "attention_tflops": achieved,
        "per_call": {"protocol": (f"{a.calls} steps after a warm-up of at least 10 steps and "
                                  f"{WARM_MS:g} ms, each kernel between its own HIP events on the "
                                  f"launch stream; roofline.achieved uses the attention's mean, "
                                  f"the rates the medians"),
                     "kernels_us": kus},
        # K more steps right after the timed ones, each kernel between its own events
        "timed_steps_kernels_us": steps_us,
        "kernels_us": {"qknorm_rope3": pro_us, "gen_attn": att_us, "fm_euler_step": eul_us},
        "hbm_gbs": {"qknorm_rope3": fig["prologue_gbs"], "fm_euler_step": fig["euler_gbs"]},
        "hbm_frac": {"qknorm_rope3": fig["prologue_gbs"] / PEAK_HBM_GBS,
                     "fm_euler_step": fig["euler_gbs"] / PEAK_HBM_GBS},
        "step_roofline": {"image_tokens_per_s": fig["image_tokens_per_s"],
                          "tokens_per_s_at_roofline": fig["image_tokens_per_s_at_roofline"],
                          "frac": fig["step_frac"]},
        "mid_1024_tokens": mid,
        # the whole denoiser's share of this path: every layer's norm + rotary and attention
        # (the layers' projections and MLPs are not part of it), then one Euler step
        "model_shaped_step": {
            "layers": N_LAYERS,
            "us": N_LAYERS * (pro_us + att_us) + eul_us,
            "image_tokens_per_s": ntok / ((N_LAYERS * (pro_us + att_us) + eul_us) * 1e-6)},
        "cfg_euler": cfg,
        "prefill_attention": prefill,
        "qkv_projection": proj,
        "embedding_front_end": embed,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
