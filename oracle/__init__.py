"""fp64 CPU oracle for the NEO-unify generation-pass attention block.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the HIP library never imports, links or calls it, and
it never imports the library.  The arithmetic of the attention block lives in
``neo_oracle.c`` (plain fp64 loops, cited there against the pages) and this module
marshals numpy arrays through ctypes to it; the q/k/v projection below is an fp64
library matmul ahead of that code, and the generation branch's embedding front end
is the numpy module ``front_end.py`` (fp64, each step from its definition).

Pages cited:
  [A] "SenseNova-U1.5 (NEO-unify) architecture" (Mobius design note)
  [B] "SenseNova-U1: Unifying Multimodal Understanding and Generation with
      NEO-unify Architecture" (paper notes)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "neo_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile neo_oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
               "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_split_rmsnorm.argtypes = [_dp, _dp, ctypes.c_int64, _dp, _dp, ctypes.c_double]
        lib.oracle_rope3.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _ip,
                                     ctypes.c_double, ctypes.c_double]
        lib.oracle_norm_rope.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int64, _dp, _dp, _ip,
                                         ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.oracle_gen_attn.argtypes = [_dp, _dp, _dp, _dp, _dp, _ip, _ip, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_double, _lp, ctypes.c_int64, _dp, _dp]
        lib.oracle_euler_step.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double]
        lib.oracle_prefill_attn.argtypes = [_dp, _dp, _dp, _ip, _ip, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_double, _lp, ctypes.c_int64, _dp, _dp]
        lib.oracle_cfg_path.restype = ctypes.c_int
        lib.oracle_cfg_path.argtypes = [ctypes.c_double] * 5
        lib.oracle_euler_step_cfg.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64] + [ctypes.c_double] * 7
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops from now on (for timing runs)."""
    _load().oracle_set_num_threads(int(n))


def split_rmsnorm(x, w_t, w_hw, eps=1e-6) -> np.ndarray:
    """Split-half RMSNorm of head rows [..., 128]; [A] §Three rotary axes."""
    x = _f64(x)
    assert x.shape[-1] == 128
    y = np.empty_like(x)
    rows = x.size // 128
    _load().oracle_split_rmsnorm(_ptr(x, _dp), _ptr(y, _dp), rows, _ptr(_f64(w_t), _dp),
                                 _ptr(_f64(w_hw), _dp), float(eps))
    return y


def rope3(x, pos, theta=5.0e6, theta_hw=1.0e4) -> np.ndarray:
    """Three-axis half-split rotary of [T, H, 128] at positions [3, T]; [A] §Three rotary axes."""
    y = _f64(x).copy()
    T, H, D = y.shape
    assert D == 128
    pos = _i32(pos)
    assert pos.shape == (3, T)
    _load().oracle_rope3(_ptr(y, _dp), T, H, _ptr(pos, _ip), float(theta), float(theta_hw))
    return y


def norm_rope(x, w_t, w_hw, pos, theta=5.0e6, theta_hw=1.0e4, eps=1e-6) -> np.ndarray:
    """Split-half RMSNorm followed by three-axis rotary, [T, H, 128]."""
    x = _f64(x)
    T, H, D = x.shape
    assert D == 128
    pos = _i32(pos)
    assert pos.shape == (3, T)
    y = np.empty_like(x)
    _load().oracle_norm_rope(_ptr(x, _dp), _ptr(y, _dp), T, H, _ptr(_f64(w_t), _dp),
                             _ptr(_f64(w_hw), _dp), _ptr(pos, _ip), float(theta),
                             float(theta_hw), float(eps))
    return y


def qknorm_rope3(q, k, wq_t, wq_hw, wk_t, wk_hw, pos, theta=5.0e6, theta_hw=1.0e4,
                 eps=1e-6):
    """The generation-pass prologue on queries and the image block's keys."""
    return (norm_rope(q, wq_t, wq_hw, pos, theta, theta_hw, eps),
            norm_rope(k, wk_t, wk_hw, pos, theta, theta_hw, eps))


def gen_attn(q, k_img, v_img, k_pre, v_pre, cu_q, cu_p, scale=None, tokens=None,
             with_lse=False):
    """Generation-pass attention over [prefix_b ; image_b]; [A] §Mixture of Transformers.

    q: [Tq, Hq, D]; k_img/v_img: [Tq, Hkv, D]; k_pre/v_pre: [Tp, Hkv, D];
    cu_q/cu_p: [B+1].  tokens: optional global query rows to evaluate.
    Returns out [n, Hq, D] (and lse [n, Hq] when with_lse).
    """
    q, k_img, v_img = _f64(q), _f64(k_img), _f64(v_img)
    k_pre, v_pre = _f64(k_pre), _f64(v_pre)
    cu_q, cu_p = _i32(cu_q), _i32(cu_p)
    Tq, Hq, D = q.shape
    Hkv = k_img.shape[1]
    B = cu_q.shape[0] - 1
    if k_pre.size == 0:  # keep valid pointers for an empty prefix
        k_pre = np.zeros((1, Hkv, D))
        v_pre = np.zeros((1, Hkv, D))
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if tokens is None:
        tok_arr, n, tok_ptr = None, Tq, None
    else:
        tok_arr = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tok_arr.shape[0]
        tok_ptr = _ptr(tok_arr, _lp)
    out = np.zeros((max(n, 1), Hq, D))
    lse = np.zeros((max(n, 1), Hq))
    _load().oracle_gen_attn(_ptr(q, _dp), _ptr(k_img, _dp), _ptr(v_img, _dp), _ptr(k_pre, _dp),
                            _ptr(v_pre, _dp), _ptr(cu_q, _ip), _ptr(cu_p, _ip), B, Hq, Hkv, D,
                            float(scale), tok_ptr, n, _ptr(out, _dp), _ptr(lse, _dp))
    out, lse = out[:n], lse[:n]
    return (out, lse) if with_lse else out


def euler_step(z, x0, t, t_next, t_eps=0.02) -> np.ndarray:
    """One x0->velocity Euler update; [A] §Flow matching without a VAE."""
    z = _f64(z).copy()
    x0 = _f64(x0)
    assert z.shape == x0.shape
    _load().oracle_euler_step(_ptr(z, _dp), _ptr(x0, _dp), z.size, float(t), float(t_next),
                              float(t_eps))
    return z


def cfg_path(t, cfg_scale, img_cfg_scale, cfg_interval=(0.0, 1.0)) -> int:
    """Guidance path 1..4 of a step; [B] §2.7 (the four code paths)."""
    return int(_load().oracle_cfg_path(float(t), float(cfg_scale), float(img_cfg_scale),
                                       float(cfg_interval[0]), float(cfg_interval[1])))


def euler_step_cfg(z, x0_cond, x0_text_uncond=None, x0_uncond=None, *, t, t_next, t_eps=0.02,
                   cfg_scale=4.0, img_cfg_scale=1.0, cfg_interval=(0.0, 1.0)) -> np.ndarray:
    """Three-branch classifier-free guidance, then one Euler step; [B] §2.7.

    Branch predictions the selected path does not read may be None."""
    z = _f64(z).copy()
    xc = _f64(x0_cond)
    path = cfg_path(t, cfg_scale, img_cfg_scale, cfg_interval)
    need_tu, need_u = path in (2, 4), path in (3, 4)
    if (need_tu and x0_text_uncond is None) or (need_u and x0_uncond is None):
        raise ValueError(f"guidance path {path} needs the missing branch prediction")
    xtu = _f64(x0_text_uncond) if x0_text_uncond is not None else None
    xu = _f64(x0_uncond) if x0_uncond is not None else None
    for x in (xc, xtu, xu):
        assert x is None or x.shape == z.shape
    _load().oracle_euler_step_cfg(
        _ptr(z, _dp), _ptr(xc, _dp), _ptr(xtu, _dp) if xtu is not None else None,
        _ptr(xu, _dp) if xu is not None else None, z.size, float(t), float(t_next), float(t_eps),
        float(cfg_scale), float(img_cfg_scale), float(cfg_interval[0]), float(cfg_interval[1]))
    return z


def prefill_attn(q, k, v, idx, cu, scale=None, tokens=None, with_lse=False):
    """Understanding-pass attention with the block-causal mask; [A] §Block-causal
    attention: key j is allowed for query i when idx[j] == idx[i] or j <= i.

    q: [T, Hq, D]; k/v: [T, Hkv, D]; idx: [T] temporal index; cu: [B+1].
    tokens: optional global query rows to evaluate.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    idx, cu = _i32(idx), _i32(cu)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = cu.shape[0] - 1
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if tokens is None:
        n, tok_ptr = T, None
    else:
        tok_arr = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tok_arr.shape[0]
        tok_ptr = _ptr(tok_arr, _lp)
    out = np.zeros((max(n, 1), Hq, D))
    lse = np.zeros((max(n, 1), Hq))
    _load().oracle_prefill_attn(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(idx, _ip),
                                _ptr(cu, _ip), B, Hq, Hkv, D, float(scale), tok_ptr, n,
                                _ptr(out, _dp), _ptr(lse, _dp))
    out, lse = out[:n], lse[:n]
    return (out, lse) if with_lse else out


def qkv_proj_norm_rope(x, w_qkv, Hq, Hkv, wq_t, wq_hw, wk_t, wk_hw, pos, theta=5.0e6,
                       theta_hw=1.0e4, eps=1e-6, tokens=None):
    """The generation branch's q/k/v projection followed by the q/k prologue; [A] §Mixture
    of Transformers (the `_mot_gen` q/k/v projections and q/k norms) and §Three rotary axes.

    x [N, hidden]; w_qkv [(Hq + 2 Hkv) * 128, hidden], rows: the Hq query heads, then the Hkv
    key heads, then the Hkv value heads (y = x w_qkv^T).  pos [3, N].  The projection is an
    fp64 library matmul; q and k then go through norm_rope (split-half RMSNorm + three-axis
    rotary); v is the projection itself.  tokens: optional rows to evaluate.
    Returns (q [n, Hq, 128], k [n, Hkv, 128], v [n, Hkv, 128]).
    """
    x, w = _f64(x), _f64(w_qkv)
    pos = _i32(pos)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x, pos = x[tokens], np.ascontiguousarray(pos[:, tokens])
    n = x.shape[0]
    assert w.shape == ((Hq + 2 * Hkv) * 128, x.shape[1])
    y = x @ w.T
    q = np.ascontiguousarray(y[:, :Hq * 128]).reshape(n, Hq, 128)
    k = np.ascontiguousarray(y[:, Hq * 128:(Hq + Hkv) * 128]).reshape(n, Hkv, 128)
    v = np.ascontiguousarray(y[:, (Hq + Hkv) * 128:]).reshape(n, Hkv, 128)
    return (norm_rope(q, wq_t, wq_hw, pos, theta, theta_hw, eps),
            norm_rope(k, wk_t, wk_hw, pos, theta, theta_hw, eps), v)
