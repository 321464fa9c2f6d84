"""The C-ABI library on the CPU: it loads, exports every call include/neo.h declares,
and rejects invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import pixel_space_flow_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "neo.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(neo_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(P.LIB_PATH):
        import pixel_space_flow_amd.build as b
        b.build()
    return P.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(P.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_status_strings(L):
    for code, text in enumerate(["ok", "null pointer", "bad shape", "bad value", "unsupported",
                                 "HIP error"]):
        assert L.neo_status_string(code).decode() == text
    assert L.neo_status_string(99).decode() == "unknown status"


# a fake, 256-aligned "device" address: never dereferenced, because every call below
# fails validation before any HIP call
FAKE = 1 << 40
W = FAKE + 4096


def _rope(L, **kw):
    a = dict(q_in=FAKE, k_in=FAKE + (1 << 30), q_out=FAKE + (2 << 30), k_out=FAKE + (3 << 30),
             T=16, Hq=4, Hkv=1, D=128, w0=W, w1=W, w2=W, w3=W, pos=W, th=5e6, thw=1e4, eps=1e-6,
             dtype=P.NEO_BF16)
    a.update(kw)
    return L.neo_qknorm_rope3(a["q_in"], a["k_in"], a["q_out"], a["k_out"], a["T"], a["Hq"],
                              a["Hkv"], a["D"], a["w0"], a["w1"], a["w2"], a["w3"], a["pos"],
                              a["th"], a["thw"], a["eps"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), P.NEO_ERR_UNSUPPORTED),
    (dict(D=64), P.NEO_ERR_SHAPE),
    (dict(Hq=0), P.NEO_ERR_SHAPE),
    (dict(T=-1), P.NEO_ERR_SHAPE),
    (dict(th=0.0), P.NEO_ERR_VALUE),
    (dict(thw=math.inf), P.NEO_ERR_VALUE),
    (dict(eps=-1.0), P.NEO_ERR_VALUE),
    (dict(eps=math.nan), P.NEO_ERR_VALUE),
    (dict(q_in=None), P.NEO_ERR_NULL),
    (dict(pos=None), P.NEO_ERR_NULL),
    (dict(q_in=FAKE + 8), P.NEO_ERR_VALUE),                    # misaligned
    (dict(q_out=FAKE + 512), P.NEO_ERR_VALUE),                 # partial overlap with q_in
    (dict(k_out=FAKE + 256), P.NEO_ERR_VALUE),                 # k_out overlaps q_in
])
def test_rope_validation(L, kw, status):
    assert _rope(L, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_qknorm_rope3")


def test_rope_empty_is_ok(L):
    assert _rope(L, T=0, q_in=None, k_in=None, q_out=None, k_out=None) == P.NEO_OK
    assert L.neo_last_error().decode() == ""


def _attn(L, **kw):
    a = dict(q=FAKE, ki=FAKE + (1 << 30), vi=FAKE + (2 << 30), kp=FAKE + (3 << 30),
             vp=FAKE + (4 << 30), cuq=W, cup=W + 256, B=1, Hq=32, Hkv=8, D=128, Tq=4096, Tp=512,
             mq=4096, mp=512, scale=0.0, out=FAKE + (5 << 30), lse=None, dtype=P.NEO_BF16)
    a.update(kw)
    return L.neo_gen_attn_fwd(a["q"], a["ki"], a["vi"], a["kp"], a["vp"], a["cuq"], a["cup"],
                              a["B"], a["Hq"], a["Hkv"], a["D"], a["Tq"], a["Tp"], a["mq"],
                              a["mp"], a["scale"], a["out"], a["lse"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), P.NEO_ERR_UNSUPPORTED),
    (dict(D=256), P.NEO_ERR_SHAPE),
    (dict(B=0), P.NEO_ERR_SHAPE),
    (dict(Hkv=7), P.NEO_ERR_SHAPE),                            # Hq % Hkv != 0
    (dict(mq=-1), P.NEO_ERR_SHAPE),
    (dict(mq=5000), P.NEO_ERR_SHAPE),                          # above the tensor's rows
    (dict(Tq=-5), P.NEO_ERR_SHAPE),
    (dict(scale=math.inf), P.NEO_ERR_VALUE),
    (dict(q=None), P.NEO_ERR_NULL),
    (dict(cuq=None), P.NEO_ERR_NULL),
    (dict(kp=None), P.NEO_ERR_NULL),                           # prefix rows but no pointer
    (dict(out=FAKE + (1 << 30)), P.NEO_ERR_VALUE),             # out aliases k_img
    (dict(lse=FAKE + (5 << 30)), P.NEO_ERR_VALUE),             # lse overlaps out
    (dict(vi=FAKE + (2 << 30) + 4), P.NEO_ERR_VALUE),          # misaligned
    (dict(B=1 << 30, Hkv=8, mq=4096), P.NEO_ERR_SHAPE),        # grid beyond 2^31 workgroups
    (dict(B=16384, Hkv=8, mq=4096), P.NEO_ERR_SHAPE),          # 2^23 workgroups of 512: > 2^32 - 1 work-items
    (dict(Tq=1 << 21, mq=1 << 21), P.NEO_ERR_SHAPE),            # one sample's K/V beyond 2 GiB
])
def test_attn_validation(L, kw, status):
    assert _attn(L, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_gen_attn_fwd")


def test_attn_empty_is_ok(L):
    assert _attn(L, mq=0, q=None) == P.NEO_OK
    assert _attn(L, Tq=0, mq=0) == P.NEO_OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE + 4096, -1, 0.1, 0.2, 0.02), P.NEO_ERR_SHAPE),
    ((FAKE, FAKE + 4096, 10, 0.3, 0.2, 0.02), P.NEO_ERR_VALUE),    # t_next < t
    ((FAKE, FAKE + 4096, 10, 0.1, 0.2, 0.0), P.NEO_ERR_VALUE),     # t_eps <= 0
    ((FAKE, FAKE + 4096, 10, math.nan, 0.2, 0.02), P.NEO_ERR_VALUE),
    ((None, FAKE, 10, 0.1, 0.2, 0.02), P.NEO_ERR_NULL),
    ((FAKE, FAKE + 8, 10, 0.1, 0.2, 0.02), P.NEO_ERR_VALUE),       # partial overlap
    ((FAKE + 2, FAKE + 4096, 10, 0.1, 0.2, 0.02), P.NEO_ERR_VALUE),  # misaligned
])
def test_euler_validation(L, args, status):
    assert L.neo_fm_euler_step(*args, None) == status
    assert L.neo_last_error().decode().startswith("neo_fm_euler_step")


def test_euler_empty_is_ok(L):
    assert L.neo_fm_euler_step(None, None, 0, 0.1, 0.2, 0.02, None) == P.NEO_OK


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((4, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        P.gen_attn_fwd(q, q[:, :1], q[:, :1], q[:0, :1], q[:0, :1], torch.zeros(2, dtype=torch.int32),
                       torch.zeros(2, dtype=torch.int32), 4, 0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(P, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(P, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        P.lib()


def _cfg(L, **kw):
    a = dict(z=FAKE, xc=FAKE + (1 << 30), xtu=FAKE + (2 << 30), xu=FAKE + (3 << 30), n=1000,
             t=0.5, tn=0.55, eps=0.02, g=4.0, gi=1.5, lo=0.0, hi=1.0)
    a.update(kw)
    return L.neo_fm_euler_step_cfg(a["z"], a["xc"], a["xtu"], a["xu"], a["n"], a["t"], a["tn"],
                                   a["eps"], a["g"], a["gi"], a["lo"], a["hi"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), P.NEO_ERR_SHAPE),
    (dict(tn=0.4), P.NEO_ERR_VALUE),                             # t_next < t
    (dict(eps=0.0), P.NEO_ERR_VALUE),
    (dict(g=math.nan), P.NEO_ERR_VALUE),
    (dict(hi=math.inf), P.NEO_ERR_VALUE),
    (dict(z=None), P.NEO_ERR_NULL),
    (dict(xc=None), P.NEO_ERR_NULL),
    (dict(xtu=None), P.NEO_ERR_NULL),                           # path 4 reads text-uncond
    (dict(xu=None), P.NEO_ERR_NULL),                            # path 4 reads uncond
    (dict(gi=1.0, xu=None, xtu=None), P.NEO_ERR_NULL),          # path 2 reads text-uncond
    (dict(g=2.0, gi=2.0, xu=None), P.NEO_ERR_NULL),             # path 3 reads uncond
    (dict(xtu=FAKE + 64), P.NEO_ERR_VALUE),                     # partial overlap with z
    (dict(xc=FAKE + (1 << 30) + 2), P.NEO_ERR_VALUE),           # misaligned
])
def test_cfg_validation(L, kw, status):
    assert _cfg(L, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_fm_euler_step_cfg")


def test_cfg_unread_branches_may_be_null(L):
    # each path leaves the branches it does not read unchecked; n = 0 launches nothing
    assert _cfg(L, n=0, g=1.0, gi=1.0, xtu=None, xu=None) == P.NEO_OK
    assert _cfg(L, n=0, gi=1.0, xu=None) == P.NEO_OK
    assert _cfg(L, n=0, g=2.0, gi=2.0, xtu=None) == P.NEO_OK


def test_cfg_path_matches_the_oracle_rule():
    """The library's host-side path choice against the oracle's, on the pages' cases,
    the interval rules and a sweep of scales."""
    import oracle
    cases = [(0.5, 1, 1, 0, 1), (0.5, 4, 1, 0, 1), (0.5, 3, 3, 0, 1), (0.5, 4, 1.5, 0, 1),
             (0.5, 4, 1, 0.7, 1), (0.5, 4, 1, 0, 0.3), (0.5, 4, 1, 0.5, 1), (0.5, 4, 1, 0.2, 0.5),
             (0.9, 4, 2, 0.1, 0.95), (0.05, 7, 7, 0.1, 0.95)]
    rng = np.random.default_rng(5)
    for _ in range(200):
        cases.append((float(rng.uniform()), float(rng.choice([1.0, 2.0, 4.0])),
                      float(rng.choice([1.0, 2.0, 1.5])), float(rng.choice([0.0, 0.25])),
                      float(rng.choice([1.0, 0.75]))))
    for t, g, gi, lo, hi in cases:
        assert P.cfg_path(t, g, gi, (lo, hi)) == oracle.cfg_path(np.float32(t), g, gi, (lo, hi))


def _pre(L, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), ti=W, cu=W + 256, B=1, Hq=32, Hkv=8,
             D=128, T=1500, mx=1500, scale=0.0, out=FAKE + (3 << 30), lse=None,
             dtype=P.NEO_BF16)
    a.update(kw)
    return L.neo_prefill_attn_fwd(a["q"], a["k"], a["v"], a["ti"], a["cu"], a["B"], a["Hq"],
                                  a["Hkv"], a["D"], a["T"], a["mx"], a["scale"], a["out"],
                                  a["lse"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=P.NEO_F32), P.NEO_ERR_UNSUPPORTED),             # the understanding pass is bf16
    (dict(dtype=5), P.NEO_ERR_UNSUPPORTED),
    (dict(D=64), P.NEO_ERR_SHAPE),
    (dict(Hkv=5), P.NEO_ERR_SHAPE),
    (dict(mx=1501), P.NEO_ERR_SHAPE),
    (dict(B=0), P.NEO_ERR_SHAPE),
    (dict(scale=math.nan), P.NEO_ERR_VALUE),
    (dict(ti=None), P.NEO_ERR_NULL),
    (dict(cu=None), P.NEO_ERR_NULL),
    (dict(k=FAKE + (1 << 30) + 8), P.NEO_ERR_VALUE),             # misaligned
    (dict(ti=W + 2), P.NEO_ERR_VALUE),                           # misaligned indices
    (dict(out=FAKE + (2 << 30)), P.NEO_ERR_VALUE),              # out aliases v
    (dict(lse=FAKE + (3 << 30) + 4096), P.NEO_ERR_VALUE),       # lse inside out
    (dict(T=1 << 21, mx=1 << 21), P.NEO_ERR_SHAPE),             # one sample's K/V beyond 2 GiB
    (dict(B=1 << 16), P.NEO_ERR_SHAPE),                          # grid beyond 2^32 work-items
])
def test_prefill_validation(L, kw, status):
    assert _pre(L, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_prefill_attn_fwd")


def test_prefill_empty_is_ok(L):
    assert _pre(L, mx=0, q=None) == P.NEO_OK
    assert _pre(L, T=0, mx=0) == P.NEO_OK


def _proj(L, **kw):
    a = dict(x=FAKE, w=FAKE + (1 << 30), N=4096, hidden=4096, Hq=32, Hkv=8, D=128, w0=W, w1=W,
             w2=W, w3=W, pos=W + 4096, th=5e6, thw=1e4, eps=1e-6, q=FAKE + (2 << 30),
             k=FAKE + (3 << 30), v=FAKE + (4 << 30), dtype=P.NEO_BF16)
    a.update(kw)
    return L.neo_qkv_proj_norm_rope(a["x"], a["w"], a["N"], a["hidden"], a["Hq"], a["Hkv"], a["D"],
                                    a["w0"], a["w1"], a["w2"], a["w3"], a["pos"], a["th"],
                                    a["thw"], a["eps"], a["q"], a["k"], a["v"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=P.NEO_F32), P.NEO_ERR_UNSUPPORTED),
    (dict(D=64), P.NEO_ERR_SHAPE),
    (dict(hidden=100), P.NEO_ERR_SHAPE),                         # not a multiple of 64
    (dict(hidden=0), P.NEO_ERR_SHAPE),
    (dict(Hkv=0), P.NEO_ERR_SHAPE),
    (dict(N=-1), P.NEO_ERR_SHAPE),
    (dict(th=-1.0), P.NEO_ERR_VALUE),
    (dict(eps=math.inf), P.NEO_ERR_VALUE),
    (dict(w=None), P.NEO_ERR_NULL),
    (dict(pos=None), P.NEO_ERR_NULL),
    (dict(v=None), P.NEO_ERR_NULL),
    (dict(x=FAKE + 8), P.NEO_ERR_VALUE),                         # misaligned
    (dict(k=FAKE + (2 << 30) + 4096), P.NEO_ERR_VALUE),          # k_out inside q_out
    (dict(q=FAKE + 1024), P.NEO_ERR_VALUE),                      # q_out overlaps x
    (dict(N=1 << 26), P.NEO_ERR_SHAPE),                          # grid beyond 2^32 work-items
])
def test_proj_validation(L, kw, status):
    assert _proj(L, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_qkv_proj_norm_rope")


def test_proj_empty_is_ok(L):
    assert _proj(L, N=0, x=None) == P.NEO_OK


# ---- embedding front end: host-side validation (nothing is launched) ------------------------

def _fe(L, fn, **kw):
    d = dict(z=FAKE, B=1, H=512, Wd=512, p=FAKE + (1 << 30), w1=FAKE + (2 << 30),
             b1=FAKE + (3 << 30), C1=1024, th=1e4, h=FAKE + (4 << 30), t=0.5, ns=2.0, nsm=16.0,
             D=4096, wa_t=FAKE + (5 << 30), ba_t=FAKE + (6 << 30), wa_s=FAKE + (7 << 30),
             ba_s=FAKE + (8 << 30), hid=FAKE + (9 << 30), wb_t=FAKE + (10 << 30),
             bb_t=FAKE + (11 << 30), wb_s=FAKE + (12 << 30), bb_s=FAKE + (13 << 30),
             cond=FAKE + (14 << 30), w2=FAKE + (15 << 30), b2=FAKE + (16 << 30),
             tok=FAKE + (17 << 30))
    d.update(kw)
    if fn == "patchify":
        return L.neo_gen_patchify(d["z"], d["B"], d["H"], d["Wd"], d["p"], None)
    if fn == "patch":
        return L.neo_gen_patch_embed(d["p"], d["B"], d["H"], d["Wd"], d["w1"], d["b1"], d["C1"],
                                     d["th"], d["h"], None)
    if fn == "patchpx":
        return L.neo_gen_patch_embed_px(d["z"], d["B"], d["H"], d["Wd"], d["w1"], d["b1"], d["C1"],
                                        d["th"], d["h"], None)
    if fn == "hidden":
        return L.neo_gen_cond_hidden(d["t"], d["ns"], d["nsm"], d["D"], d["wa_t"], d["ba_t"],
                                     d["wa_s"], d["ba_s"], d["hid"], None)
    if fn == "out":
        return L.neo_gen_cond_out(d["D"], d["hid"], d["wb_t"], d["bb_t"], d["wb_s"], d["bb_s"],
                                  d["cond"], None)
    return L.neo_gen_merge_embed(d["h"], d["B"], d["H"], d["Wd"], d["C1"], d["w2"], d["b2"],
                                 d["cond"], d["D"], d["tok"], None)


@pytest.mark.parametrize("fn,kw,status", [
    ("patchify", dict(H=520), P.NEO_ERR_SHAPE),                 # not a multiple of 16
    ("patchify", dict(Wd=0), P.NEO_ERR_SHAPE),
    ("patchify", dict(B=-1), P.NEO_ERR_SHAPE),
    ("patchify", dict(H=1 << 16), P.NEO_ERR_SHAPE),
    ("patchify", dict(z=None), P.NEO_ERR_NULL),
    ("patchify", dict(p=FAKE + 8), P.NEO_ERR_VALUE),              # misaligned
    ("patchify", dict(p=FAKE + 4096), P.NEO_ERR_VALUE),           # patches overlap z
    ("patch", dict(C1=100), P.NEO_ERR_SHAPE),                   # not a multiple of 64
    ("patch", dict(C1=0), P.NEO_ERR_SHAPE),
    ("patch", dict(H=40), P.NEO_ERR_SHAPE),
    ("patch", dict(th=1.0), P.NEO_ERR_VALUE),
    ("patch", dict(th=math.inf), P.NEO_ERR_VALUE),
    ("patch", dict(b1=None), P.NEO_ERR_NULL),
    ("patch", dict(h=FAKE + (1 << 30) + 64), P.NEO_ERR_VALUE),   # h overlaps the patches
    ("patch", dict(B=1 << 16, H=1 << 15, Wd=1 << 15), P.NEO_ERR_SHAPE),  # grid too large
    ("patchpx", dict(H=40), P.NEO_ERR_SHAPE),                   # not a multiple of 16
    ("patchpx", dict(C1=100), P.NEO_ERR_SHAPE),
    ("patchpx", dict(B=4, H=8192, Wd=8192), P.NEO_ERR_SHAPE),   # z reaches 2 GiB
    ("patchpx", dict(th=0.5), P.NEO_ERR_VALUE),
    ("patchpx", dict(z=None), P.NEO_ERR_NULL),
    ("patchpx", dict(w1=FAKE + (2 << 30) + 8), P.NEO_ERR_VALUE),  # misaligned
    ("patchpx", dict(h=FAKE + 4096), P.NEO_ERR_VALUE),          # h overlaps z
    ("hidden", dict(D=100), P.NEO_ERR_SHAPE),                   # not a multiple of 8
    ("hidden", dict(nsm=0.0), P.NEO_ERR_VALUE),
    ("hidden", dict(t=math.nan), P.NEO_ERR_VALUE),
    ("hidden", dict(wa_s=None), P.NEO_ERR_NULL),
    ("hidden", dict(hid=FAKE + (5 << 30) + 128), P.NEO_ERR_VALUE),  # hidden inside wa_t
    ("out", dict(D=0), P.NEO_ERR_SHAPE),
    ("out", dict(bb_s=None), P.NEO_ERR_NULL),
    ("out", dict(cond=FAKE + (9 << 30)), P.NEO_ERR_VALUE),      # cond overlaps hidden
    ("out", dict(wb_t=FAKE + (10 << 30) + 4), P.NEO_ERR_VALUE),  # misaligned
    ("merge", dict(H=48), P.NEO_ERR_SHAPE),                     # not a multiple of 32
    ("merge", dict(D=48), P.NEO_ERR_SHAPE),                     # not a multiple of 32
    ("merge", dict(C1=96), P.NEO_ERR_SHAPE),
    ("merge", dict(B=4, H=8192, Wd=8192), P.NEO_ERR_SHAPE),      # features reach 2 GiB
    ("merge", dict(cond=None), P.NEO_ERR_NULL),
    ("merge", dict(tok=FAKE + (16 << 30)), P.NEO_ERR_VALUE),     # tokens overlap b2
])
def test_front_end_validation(L, fn, kw, status):
    assert _fe(L, fn, **kw) == status
    assert L.neo_last_error().decode().startswith("neo_gen_")


def test_front_end_empty_is_ok(L):
    assert _fe(L, "patchify", B=0, z=None) == P.NEO_OK
    assert _fe(L, "patch", B=0, p=None) == P.NEO_OK
    assert _fe(L, "patchpx", B=0, z=None) == P.NEO_OK
    assert _fe(L, "merge", B=0, h=None) == P.NEO_OK


def test_shift_time_matches_oracle(L):
    from oracle import front_end as fe
    for t in np.linspace(0.0, 1.0, 17):
        for s in (0.5, 1.0, 3.0, 6.0):
            assert P.shift_time(t, s) == pytest.approx(fe.shift_time(t, s), abs=1e-15)
