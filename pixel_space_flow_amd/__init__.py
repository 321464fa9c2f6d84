"""Python binding of libneo, the MI355X generation-pass attention block.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/neo.h.  torch supplies device memory and the current stream.
There is no fallback: if libneo.so is missing or fails to load, every call
raises.

Pages cited:
  [A] "SenseNova-U1.5 (NEO-unify) architecture" (Mobius design note)
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["qknorm_rope3", "qkv_proj_norm_rope", "gen_attn_fwd", "prefill_attn_fwd",
           "fm_euler_step",
           "fm_euler_step_cfg", "cfg_path", "gen_patchify", "gen_patch_embed", "gen_patch_embed_px",
           "gen_cond_embed", "gen_merge_embed", "gen_embed", "shift_time",
           "NeoError", "lib", "LIB_PATH", "EXPORTED_SYMBOLS", "NEO_OK", "NEO_ERR_NULL", "NEO_ERR_SHAPE", "NEO_ERR_VALUE",
           "NEO_ERR_UNSUPPORTED", "NEO_ERR_HIP", "NEO_F32", "NEO_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libneo.so")

NEO_OK, NEO_ERR_NULL, NEO_ERR_SHAPE, NEO_ERR_VALUE, NEO_ERR_UNSUPPORTED, NEO_ERR_HIP = range(6)
NEO_F32, NEO_BF16 = 0, 1

EXPORTED_SYMBOLS = ("neo_qknorm_rope3", "neo_gen_attn_fwd", "neo_fm_euler_step",
                    "neo_cfg_path", "neo_fm_euler_step_cfg", "neo_prefill_attn_fwd",
                    "neo_qkv_proj_norm_rope", "neo_gen_patchify", "neo_gen_patch_embed",
                    "neo_gen_patch_embed_px",
                    "neo_gen_cond_hidden", "neo_gen_cond_out", "neo_gen_merge_embed",
                    "neo_shift_time", "neo_status_string", "neo_last_error")

_vp = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class NeoError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libneo.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m pixel_space_flow_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.neo_qknorm_rope3.restype = ctypes.c_int
        L.neo_qknorm_rope3.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp,
                                       _vp, _vp, _f32, _f32, _f32, ctypes.c_int, _vp]
        L.neo_gen_attn_fwd.restype = ctypes.c_int
        L.neo_gen_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _i64, _i64, _i32, _i32, _f32, _vp, _vp, ctypes.c_int, _vp]
        L.neo_fm_euler_step.restype = ctypes.c_int
        L.neo_fm_euler_step.argtypes = [_vp, _vp, _i64, _f32, _f32, _f32, _vp]
        L.neo_qkv_proj_norm_rope.restype = ctypes.c_int
        L.neo_qkv_proj_norm_rope.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                             _vp, _vp, _f32, _f32, _f32, _vp, _vp, _vp,
                                             ctypes.c_int, _vp]
        L.neo_prefill_attn_fwd.restype = ctypes.c_int
        L.neo_prefill_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64,
                                           _i32, _f32, _vp, _vp, ctypes.c_int, _vp]
        L.neo_cfg_path.restype = ctypes.c_int
        L.neo_cfg_path.argtypes = [_f32] * 5
        L.neo_fm_euler_step_cfg.restype = ctypes.c_int
        L.neo_fm_euler_step_cfg.argtypes = [_vp, _vp, _vp, _vp, _i64] + [_f32] * 7 + [_vp]
        L.neo_gen_patchify.restype = ctypes.c_int
        L.neo_gen_patchify.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp]
        L.neo_gen_patch_embed.restype = ctypes.c_int
        L.neo_gen_patch_embed.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _f32, _vp, _vp]
        L.neo_gen_patch_embed_px.restype = ctypes.c_int
        L.neo_gen_patch_embed_px.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _f32, _vp, _vp]
        L.neo_gen_cond_hidden.restype = ctypes.c_int
        L.neo_gen_cond_hidden.argtypes = [_f32, _f32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.neo_gen_cond_out.restype = ctypes.c_int
        L.neo_gen_cond_out.argtypes = [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.neo_gen_merge_embed.restype = ctypes.c_int
        L.neo_gen_merge_embed.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp,
                                          _vp]
        L.neo_shift_time.restype = ctypes.c_double
        L.neo_shift_time.argtypes = [ctypes.c_double, ctypes.c_double]
        L.neo_status_string.restype = ctypes.c_char_p
        L.neo_status_string.argtypes = [ctypes.c_int]
        L.neo_last_error.restype = ctypes.c_char_p
        L.neo_last_error.argtypes = []
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != NEO_OK:
        detail = lib().neo_last_error().decode(errors="replace")
        raise NeoError(fn, status, detail)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return NEO_BF16
    if t.dtype == torch.float32:
        return NEO_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def qknorm_rope3(q, k, q_norm_w, q_norm_hw_w, k_norm_w, k_norm_hw_w, pos_thw,
                 rope_theta=5.0e6, rope_theta_hw=1.0e4, eps=1e-6, q_out=None, k_out=None):
    """Split-half QK-RMSNorm + three-axis rotary ([A] §Three rotary axes).

    q [T, Hq, 128], k [T, Hkv, 128] (bf16 or fp32), norm weights [64] fp32,
    pos_thw [3, T] int32.  Writes q_out/k_out (new tensors unless given; pass
    q_out=q, k_out=k for in place) and returns them.
    """
    torch = _torch()
    _dev(q, "q")
    T, Hq, D = q.shape
    _dev(k, "k", q.dtype)
    Hkv = k.shape[1]
    if k.shape[0] != T or k.shape[2] != D:
        raise ValueError("k must be [T, Hkv, 128] with q's T")
    for nm, w in (("q_norm_w", q_norm_w), ("q_norm_hw_w", q_norm_hw_w), ("k_norm_w", k_norm_w),
                  ("k_norm_hw_w", k_norm_hw_w)):
        _dev(w, nm, torch.float32, (64,))
    _dev(pos_thw, "pos_thw", torch.int32, (3, T))
    q_out = torch.empty_like(q) if q_out is None else _dev(q_out, "q_out", q.dtype, q.shape)
    k_out = torch.empty_like(k) if k_out is None else _dev(k_out, "k_out", k.dtype, k.shape)
    st = lib().neo_qknorm_rope3(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), T,
                                Hq, Hkv, D, q_norm_w.data_ptr(), q_norm_hw_w.data_ptr(),
                                k_norm_w.data_ptr(), k_norm_hw_w.data_ptr(), pos_thw.data_ptr(),
                                rope_theta, rope_theta_hw, eps, _dtype_code(q), _stream(q))
    _check("neo_qknorm_rope3", st)
    return q_out, k_out


def gen_attn_fwd(q, k_img, v_img, k_prefix, v_prefix, cu_seqlens_q, cu_seqlens_prefix,
                 max_seqlen_q, max_seqlen_prefix, softmax_scale=0.0, out=None,
                 return_lse=False):
    """Generation-pass attention over [frozen prefix ; image block] ([A] §Mixture of
    Transformers; §GQA fusion does not apply).

    q [Tq, Hq, 128]; k_img/v_img [Tq, Hkv, 128]; k_prefix/v_prefix [Tp, Hkv, 128]
    (Tp may be 0); cu_seqlens_* int32 [B+1] on the device; max_seqlen_* host ints.
    Returns out [Tq, Hq, 128] (and lse [Hq, Tq] fp32 if return_lse).
    """
    torch = _torch()
    _dev(q, "q")
    Tq, Hq, D = q.shape
    _dev(k_img, "k_img", q.dtype)
    _dev(v_img, "v_img", q.dtype, k_img.shape)
    Hkv = k_img.shape[1]
    _dev(k_prefix, "k_prefix", q.dtype)
    _dev(v_prefix, "v_prefix", q.dtype, k_prefix.shape)
    if k_prefix.dim() != 3 or (k_prefix.shape[0] > 0 and tuple(k_prefix.shape[1:]) != (Hkv, D)):
        raise ValueError("k_prefix must be [Tp, Hkv, 128]")
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_prefix, "cu_seqlens_prefix", torch.int32, cu_seqlens_q.shape)
    B = cu_seqlens_q.shape[0] - 1
    Tp = k_prefix.shape[0]
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype, q.shape)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device) if return_lse else None
    pre_k = k_prefix.data_ptr() if Tp > 0 else None
    pre_v = v_prefix.data_ptr() if Tp > 0 else None
    st = lib().neo_gen_attn_fwd(q.data_ptr(), k_img.data_ptr(), v_img.data_ptr(), pre_k, pre_v,
                                cu_seqlens_q.data_ptr(), cu_seqlens_prefix.data_ptr(), B, Hq, Hkv,
                                D, Tq, Tp, int(max_seqlen_q), int(max_seqlen_prefix),
                                float(softmax_scale), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, _dtype_code(q),
                                _stream(q))
    _check("neo_gen_attn_fwd", st)
    return (out, lse) if return_lse else out


def qkv_proj_norm_rope(x, w_qkv, Hq, Hkv, q_norm_w, q_norm_hw_w, k_norm_w, k_norm_hw_w, pos_thw,
                       rope_theta=5.0e6, rope_theta_hw=1.0e4, eps=1e-6, q_out=None, k_out=None,
                       v_out=None):
    """The generation branch's q/k/v projection fused with the q/k prologue ([A] §Mixture of
    Transformers, §Three rotary axes).  x [N, hidden] bf16; w_qkv [(Hq + 2 Hkv) * 128,
    hidden] bf16 (q heads, then k heads, then v heads); norm weights [64] fp32; pos_thw
    int32 [3, N].  Returns (q [N, Hq, 128], k [N, Hkv, 128], v [N, Hkv, 128]) bf16."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    N, hidden = x.shape
    _dev(w_qkv, "w_qkv", torch.bfloat16, ((Hq + 2 * Hkv) * 128, hidden))
    for name, t in (("q_norm_w", q_norm_w), ("q_norm_hw_w", q_norm_hw_w),
                    ("k_norm_w", k_norm_w), ("k_norm_hw_w", k_norm_hw_w)):
        _dev(t, name, torch.float32, (64,))
    _dev(pos_thw, "pos_thw", torch.int32, (3, N))
    mk = lambda h: torch.empty((N, h, 128), dtype=torch.bfloat16, device=x.device)
    q_out = mk(Hq) if q_out is None else _dev(q_out, "q_out", torch.bfloat16, (N, Hq, 128))
    k_out = mk(Hkv) if k_out is None else _dev(k_out, "k_out", torch.bfloat16, (N, Hkv, 128))
    v_out = mk(Hkv) if v_out is None else _dev(v_out, "v_out", torch.bfloat16, (N, Hkv, 128))
    st = lib().neo_qkv_proj_norm_rope(x.data_ptr(), w_qkv.data_ptr(), N, hidden, Hq, Hkv, 128,
                                      q_norm_w.data_ptr(), q_norm_hw_w.data_ptr(),
                                      k_norm_w.data_ptr(), k_norm_hw_w.data_ptr(),
                                      pos_thw.data_ptr(), float(rope_theta), float(rope_theta_hw),
                                      float(eps), q_out.data_ptr(), k_out.data_ptr(),
                                      v_out.data_ptr(), NEO_BF16, _stream(x))
    _check("neo_qkv_proj_norm_rope", st)
    return q_out, k_out, v_out


def prefill_attn_fwd(q, k, v, temporal_idx, cu_seqlens, max_seqlen, softmax_scale=0.0, out=None,
                     return_lse=False):
    """Understanding-pass attention with the block-causal mask ([A] §Block-causal
    attention): key j is open to query i when their temporal indices are equal or j <= i.

    q [T, Hq, 128] bf16; k/v [T, Hkv, 128] bf16; temporal_idx int32 [T] and cu_seqlens
    int32 [B+1] on the device (indices non-decreasing within a sample, equal ones
    contiguous); max_seqlen a host int.  Returns out (and lse [Hq, T] if return_lse).
    """
    torch = _torch()
    _dev(q, "q")
    T, Hq, D = q.shape
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype, k.shape)
    if k.dim() != 3 or k.shape[0] != T:
        raise ValueError("k must be [T, Hkv, 128]")
    Hkv = k.shape[1]
    _dev(temporal_idx, "temporal_idx", torch.int32, (T,))
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    B = cu_seqlens.shape[0] - 1
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype, q.shape)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib().neo_prefill_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    temporal_idx.data_ptr(), cu_seqlens.data_ptr(), B, Hq, Hkv,
                                    D, T, int(max_seqlen), float(softmax_scale), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, _dtype_code(q),
                                    _stream(q))
    _check("neo_prefill_attn_fwd", st)
    return (out, lse) if return_lse else out


def fm_euler_step(z, x0_pred, t, t_next, t_eps=0.02):
    """In place: z <- z + (t_next - t) * (x0_pred - z) / max(1 - t, t_eps)
    ([A] §Flow matching without a VAE).  z and x0_pred are fp32 device tensors."""
    torch = _torch()
    _dev(z, "z", torch.float32)
    _dev(x0_pred, "x0_pred", torch.float32, z.shape)
    st = lib().neo_fm_euler_step(z.data_ptr(), x0_pred.data_ptr(), z.numel(), float(t),
                                 float(t_next), float(t_eps), _stream(z))
    _check("neo_fm_euler_step", st)
    return z


def cfg_path(t, cfg_scale=4.0, img_cfg_scale=1.0, cfg_interval=(0.0, 1.0)) -> int:
    """Guidance path 1..4 of a flow step ([B] §2.7): 1 = cond only, 2 = cond and
    text-uncond, 3 = cond and full uncond, 4 = all three branches."""
    return int(lib().neo_cfg_path(float(t), float(cfg_scale), float(img_cfg_scale),
                                  float(cfg_interval[0]), float(cfg_interval[1])))


def fm_euler_step_cfg(z, x0_cond, x0_text_uncond=None, x0_uncond=None, *, t, t_next,
                      t_eps=0.02, cfg_scale=4.0, img_cfg_scale=1.0, cfg_interval=(0.0, 1.0)):
    """In place: three-branch classifier-free guidance over the branches' x0
    predictions fused with the Euler step ([B] §2.7).  Branches the guidance path
    does not read (see cfg_path) may be None.  All tensors fp32 on the HIP device."""
    torch = _torch()
    _dev(z, "z", torch.float32)
    xs = []
    for name, x in (("x0_cond", x0_cond), ("x0_text_uncond", x0_text_uncond),
                    ("x0_uncond", x0_uncond)):
        if x is not None:
            _dev(x, name, torch.float32, z.shape)
        xs.append(x.data_ptr() if x is not None else None)
    st = lib().neo_fm_euler_step_cfg(z.data_ptr(), xs[0], xs[1], xs[2], z.numel(), float(t),
                                     float(t_next), float(t_eps), float(cfg_scale),
                                     float(img_cfg_scale), float(cfg_interval[0]),
                                     float(cfg_interval[1]), _stream(z))
    _check("neo_fm_euler_step_cfg", st)
    return z


# ---- generation-branch embedding front end ([A] §Vision tower; §Timestep and noise-scale
# conditioning; [B] §2.1) ------------------------------------------------------------------

def gen_patchify(z, patches=None):
    """z [B, 3, H, W] fp32 -> patch rows [B*P, 768] bf16 (channel, ky, kx order)."""
    torch = _torch()
    _dev(z, "z", torch.float32)
    if z.dim() != 4 or z.shape[1] != 3:
        raise ValueError(f"z must be [B, 3, H, W], got {tuple(z.shape)}")
    B, _, H, W = z.shape
    shape = (B * (H // 16) * (W // 16), 768)
    patches = (torch.empty(shape, dtype=torch.bfloat16, device=z.device) if patches is None
               else _dev(patches, "patches", torch.bfloat16, shape))
    _check("neo_gen_patchify", lib().neo_gen_patchify(z.data_ptr(), B, H, W, patches.data_ptr(),
                                                      _stream(z)))
    return patches


def gen_patch_embed(patches, B, H, W, w1, b1, rope_theta=1.0e4, h_out=None):
    """Patch convolution + bias, GELU, interleaved two-axis rotary -> [B*P, C1] bf16.
    w1: [C1, 768] bf16 (the [C1, 3, 16, 16] weight flattened), b1 [C1] fp32."""
    torch = _torch()
    P = (H // 16) * (W // 16)
    _dev(patches, "patches", torch.bfloat16, (B * P, 768))
    _dev(w1, "w1", torch.bfloat16)
    C1 = w1.shape[0]
    _dev(w1, "w1", torch.bfloat16, (C1, 768))
    _dev(b1, "b1", torch.float32, (C1,))
    h_out = (torch.empty((B * P, C1), dtype=torch.bfloat16, device=patches.device) if h_out is None
             else _dev(h_out, "h_out", torch.bfloat16, (B * P, C1)))
    st = lib().neo_gen_patch_embed(patches.data_ptr(), B, H, W, w1.data_ptr(), b1.data_ptr(), C1,
                                   float(rope_theta), h_out.data_ptr(), _stream(patches))
    _check("neo_gen_patch_embed", st)
    return h_out


def gen_patch_embed_px(z, w1, b1, rope_theta=1.0e4, h_out=None):
    """Patchify and the patch convolution + GELU + rotary in one launch, from the pixels:
    z [B, 3, H, W] fp32 -> [B*P, C1] bf16 (bit-identical to gen_patchify + gen_patch_embed)."""
    torch = _torch()
    _dev(z, "z", torch.float32)
    if z.dim() != 4 or z.shape[1] != 3:
        raise ValueError(f"z must be [B, 3, H, W], got {tuple(z.shape)}")
    B, _, H, W = z.shape
    P = (H // 16) * (W // 16)
    _dev(w1, "w1", torch.bfloat16)
    C1 = w1.shape[0]
    _dev(w1, "w1", torch.bfloat16, (C1, 768))
    _dev(b1, "b1", torch.float32, (C1,))
    h_out = (torch.empty((B * P, C1), dtype=torch.bfloat16, device=z.device) if h_out is None
             else _dev(h_out, "h_out", torch.bfloat16, (B * P, C1)))
    st = lib().neo_gen_patch_embed_px(z.data_ptr(), B, H, W, w1.data_ptr(), b1.data_ptr(), C1,
                                      float(rope_theta), h_out.data_ptr(), _stream(z))
    _check("neo_gen_patch_embed_px", st)
    return h_out


def gen_cond_embed(t, noise_scale, noise_scale_max, emb_t, emb_s, hidden=None, cond=None):
    """Time + noise-scale embedders summed -> cond [D] fp32.  emb_t, emb_s: (wa [D, 256] bf16,
    ba [D] fp32, wb [D, D] bf16, bb [D] fp32).  Two calls; hidden [2, D] fp32 holds the
    first layer's output.  Returns (cond, hidden)."""
    torch = _torch()
    D = emb_t[0].shape[0]
    for tag, (wa, ba, wb, bb) in (("t", emb_t), ("s", emb_s)):
        _dev(wa, f"wa_{tag}", torch.bfloat16, (D, 256))
        _dev(ba, f"ba_{tag}", torch.float32, (D,))
        _dev(wb, f"wb_{tag}", torch.bfloat16, (D, D))
        _dev(bb, f"bb_{tag}", torch.float32, (D,))
    dev = emb_t[0].device
    hidden = (torch.empty((2, D), dtype=torch.float32, device=dev) if hidden is None
              else _dev(hidden, "hidden", torch.float32, (2, D)))
    cond = (torch.empty((D,), dtype=torch.float32, device=dev) if cond is None
            else _dev(cond, "cond", torch.float32, (D,)))
    s = _stream(emb_t[0])
    st = lib().neo_gen_cond_hidden(float(t), float(noise_scale), float(noise_scale_max), D,
                                   emb_t[0].data_ptr(), emb_t[1].data_ptr(), emb_s[0].data_ptr(),
                                   emb_s[1].data_ptr(), hidden.data_ptr(), s)
    _check("neo_gen_cond_hidden", st)
    st = lib().neo_gen_cond_out(D, hidden.data_ptr(), emb_t[2].data_ptr(), emb_t[3].data_ptr(),
                                emb_s[2].data_ptr(), emb_s[3].data_ptr(), cond.data_ptr(), s)
    _check("neo_gen_cond_out", st)
    return cond, hidden


def gen_merge_embed(h, B, H, W, w2, b2, cond, tokens=None):
    """2x2 stride-2 convolution + bias + cond -> tokens [B*(H/32)*(W/32), D] fp32.
    h [B*P, C1] bf16; w2 [D, 2, 2, C1] bf16 (out, ky, kx, in); b2, cond [D] fp32."""
    torch = _torch()
    P = (H // 16) * (W // 16)
    _dev(h, "h", torch.bfloat16)
    C1 = h.shape[1]
    _dev(h, "h", torch.bfloat16, (B * P, C1))
    D = w2.shape[0]
    _dev(w2, "w2", torch.bfloat16, (D, 2, 2, C1))
    _dev(b2, "b2", torch.float32, (D,))
    _dev(cond, "cond", torch.float32, (D,))
    n = B * (H // 32) * (W // 32)
    tokens = (torch.empty((n, D), dtype=torch.float32, device=h.device) if tokens is None
              else _dev(tokens, "tokens", torch.float32, (n, D)))
    st = lib().neo_gen_merge_embed(h.data_ptr(), B, H, W, C1, w2.data_ptr(), b2.data_ptr(),
                                   cond.data_ptr(), D, tokens.data_ptr(), _stream(h))
    _check("neo_gen_merge_embed", st)
    return tokens


def gen_embed(z, w1, b1, w2, b2, emb_t, emb_s, t, noise_scale, noise_scale_max,
              rope_theta=1.0e4):
    """The whole front end, z [B, 3, H, W] fp32 -> tokens [B*N, D] fp32 (four launches)."""
    B, _, H, W = z.shape
    h = gen_patch_embed_px(z, w1, b1, rope_theta)
    cond, _ = gen_cond_embed(t, noise_scale, noise_scale_max, emb_t, emb_s)
    return gen_merge_embed(h, B, H, W, w2, b2, cond)


def shift_time(t, shift) -> float:
    """The shifted time grid point of [A] §Timestep schedule (host only)."""
    return float(lib().neo_shift_time(float(t), float(shift)))
