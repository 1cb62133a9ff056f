"""fp64 CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The HIP library never loads it and it never
loads the HIP library; the two share no code.  ``oracle.c`` holds the
arithmetic; this module only compiles it with gcc and marshals numpy arrays.

Functions with a pin in ``tests/test_oracle_pins.py``: every function here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3, F64 = 0, 1, 2, 3

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I, D, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
        L.oracle_sdpa.argtypes = [P, I, P, I, P, I, P, I, I, I, I, I, I, D, P, P]
        L.oracle_layernorm.argtypes = [P, I64, I, P, P, D, P, P, P]
        L.oracle_encoder_block.argtypes = [P, P, P, I, P, I, I, I, I, I, D, P, P, P, D, P, P, P, P, P]
        L.oracle_prefill_paged.argtypes = [P, I, P, P, D, D, P, I, I, I, I, D, I, I, I, I, P, I, P, P]
        L.oracle_prefill_causal.argtypes = [P, I, P, P, D, D, P, I, I, I, I, P, P, I, D, I, I, I, I, P, I, P, P]
        L.oracle_decode.argtypes = [P, I, I64, P]
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = D
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = D
        _lib = L
    return _lib


def _raw(x):
    """Return (contiguous numpy array of the raw storage, dtype code)."""
    import torch

    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), BF16
        if x.dtype == torch.float8_e4m3fn:
            return x.view(torch.uint8).numpy(), E4M3
        if x.dtype == torch.float32:
            return x.numpy(), F32
        if x.dtype == torch.float64:
            return x.numpy(), F64
        raise TypeError(f"oracle: unsupported dtype {x.dtype}")
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError(f"oracle: unsupported dtype {x.dtype}")


def _f64(x):
    if x is None:
        return None
    import torch

    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(x) -> np.ndarray:
    """Widen raw bf16 / e4m3fn / fp32 storage to fp64 with the oracle's own decoders."""
    raw, dt = _raw(x)
    out = np.empty(raw.size, dtype=np.float64)
    lib().oracle_decode(_ptr(raw), dt, raw.size, _ptr(out))
    return out.reshape(raw.shape)


def sdpa(q, k, v, scale: float, mask=None, return_lse: bool = False):
    """q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]; mask additive [B,1,1,Skv] or [B,Skv] (nullable)."""
    qr, qt = _raw(q)
    kr, kt = _raw(k)
    vr, vt = _raw(v)
    B, Hq, Sq, D = qr.shape
    _, Hkv, Skv, _ = kr.shape
    m = None if mask is None else _f64(mask).reshape(B, Skv)
    out = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)
    rc = lib().oracle_sdpa(_ptr(qr), qt, _ptr(kr), kt, _ptr(vr), vt, _ptr(m), B, Hq, Hkv, Sq, Skv, D,
                           float(scale), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_sdpa rc={rc}")
    return (out, lse) if return_lse else out


def window_range(S_ctx: int, B: int, key_begin=None, key_end=None, max_keys=None):
    """Per-sequence key range [s_b, e_b) of a windowed decode.

    head_dim>128 (256/512) GQA Flash-Decode NKI Kernel for AWS Trainium,
    "Future performance follow-on": a sliding-window layer needs only the
    most recent window of keys.  Reading taken here: the caller's range is
    clamped to the cache, e_b = clamp(end_b, 0, S_ctx), s_b = clamp(begin_b,
    0, e_b), and then cut to its last max_keys keys, s_b = max(s_b, e_b -
    max_keys).  Missing bounds mean 0 and S_ctx.
    """
    W = S_ctx if max_keys is None else int(max_keys)
    beg = [0] * B if key_begin is None else [int(x) for x in np.asarray(key_begin).reshape(-1)]
    end = [S_ctx] * B if key_end is None else [int(x) for x in np.asarray(key_end).reshape(-1)]
    out = []
    for b in range(B):
        e = min(max(end[b], 0), S_ctx)
        s = min(max(beg[b], 0), e)
        out.append((max(s, e - W), e))
    return out


def decode_window(q, k, v, scale: float, mask=None, key_begin=None, key_end=None, max_keys=None):
    """Single-token GQA decode over per-sequence key ranges (``window_range``).

    The range is one more additive mask: keys outside [s_b, e_b) get -inf,
    added to the caller's mask; then plain attention (``sdpa``).  A sequence
    with no key left gets o = 0, as every fully masked row does.
    """
    import torch

    B, Skv = q.shape[0], k.shape[2]
    add = np.full((B, Skv), -np.inf)
    for b, (s, e) in enumerate(window_range(Skv, B, key_begin, key_end, max_keys)):
        add[b, s:e] = 0.0
    if mask is not None:
        add = add + _f64(mask).reshape(B, Skv)
    return sdpa(q, k, v, scale, torch.from_numpy(add))


def rope(x, cos, sin, pairing: str):
    """Rotary position embedding of x [..., S, D] with per-token tables
    cos/sin [S, D/2] (pair k of token s turns by the angle whose cosine and
    sine are cos[s, k], sin[s, k]).  Returns fp64.

    vit-encoder-neuron-kernels, "Kernels": the two pairings of lanes,
    "half" (lane k with lane k + D/2, rotate-half) and "interleaved" (lane 2k
    with lane 2k + 1).  For a pair (a, b) the rotation is
    a' = a cos - b sin,  b' = b cos + a sin.
    """
    x = _f64(x).copy()
    c = _f64(cos)
    s_ = _f64(sin)
    D = x.shape[-1]
    if pairing == "half":
        a, b = x[..., : D // 2].copy(), x[..., D // 2:].copy()
        x[..., : D // 2] = a * c - b * s_
        x[..., D // 2:] = b * c + a * s_
    elif pairing == "interleaved":
        a, b = x[..., 0::2].copy(), x[..., 1::2].copy()
        x[..., 0::2] = a * c - b * s_
        x[..., 1::2] = b * c + a * s_
    else:
        raise ValueError(f"rope: unknown pairing {pairing!r}")
    return x


def encoder_block_rope(q, k, v, scale, residual, gamma, beta, eps, mask, cos, sin, pairing: str):
    """The encoder block with RoPE applied to q and k first (token i of the
    queries and token j of the keys use table rows i and j)."""
    import torch

    Sq, Skv = q.shape[2], k.shape[2]
    qr = torch.from_numpy(rope(q, _f64(cos)[:Sq], _f64(sin)[:Sq], pairing))
    kr = torch.from_numpy(rope(k, _f64(cos)[:Skv], _f64(sin)[:Skv], pairing))
    return encoder_block(qr, kr, torch.from_numpy(_f64(v)), scale, residual, gamma, beta, eps, mask)


def layernorm(x, gamma=None, beta=None, eps: float = 1e-6):
    """LayerNorm over the last dim; returns (y, mean, rstd) in fp64."""
    xs = _f64(x)
    N = xs.shape[-1]
    rows = xs.size // N
    xs = xs.reshape(rows, N)
    g, b = _f64(gamma), _f64(beta)
    y = np.empty_like(xs)
    mean = np.empty(rows)
    rstd = np.empty(rows)
    rc = lib().oracle_layernorm(_ptr(xs), rows, N, _ptr(g), _ptr(b), float(eps), _ptr(y), _ptr(mean),
                                _ptr(rstd))
    if rc:
        raise ValueError(f"oracle_layernorm rc={rc}")
    return y.reshape(np.shape(x)), mean, rstd


def encoder_block(q, k, v, scale, residual, gamma=None, beta=None, eps=1e-6, mask=None):
    """Attention -> token-major [B,S_q,H*D] -> + fp32 residual -> LayerNorm.

    q [B,H,S_q,D], k/v [B,H,S_kv,D], mask additive [B,1,1,S_kv] (nullable),
    residual [B,S_q,H*D].  Returns dict with attn [B,H,S_q,D], res_out
    [B,S_q,H*D], ln_out, mean, rstd (fp64).
    """
    import torch

    qr, qt = _raw(q)
    kr, kt = _raw(k)
    vr, vt = _raw(v)
    if not (qt == kt == vt):
        raise TypeError("encoder_block: q/k/v must share a dtype")
    B, H, Sq, D = qr.shape
    Skv = kr.shape[2]
    if kr.shape != (B, H, Skv, D) or vr.shape != kr.shape:
        raise ValueError("encoder_block: k and v must be [B, H, S_kv, D] with q's B, H and D")
    res = residual.detach().cpu().contiguous().to(torch.float32).numpy() \
        if isinstance(residual, torch.Tensor) else np.ascontiguousarray(residual, dtype=np.float32)
    if res.size != B * Sq * H * D:
        raise ValueError("encoder_block: residual must be [B, S_q, H*D]")
    m = None if mask is None else _f64(mask).reshape(B, Skv)
    attn = np.empty((B, H, Sq, D))
    res_out = np.empty((B, Sq, H * D))
    ln = np.empty((B, Sq, H * D))
    mean = np.empty(B * Sq)
    rstd = np.empty(B * Sq)
    rc = lib().oracle_encoder_block(_ptr(qr), _ptr(kr), _ptr(vr), qt, _ptr(m), B, H, Sq, Skv, D, float(scale),
                                    _ptr(res), _ptr(_f64(gamma)), _ptr(_f64(beta)), float(eps), _ptr(attn),
                                    _ptr(res_out), _ptr(ln), _ptr(mean), _ptr(rstd))
    if rc:
        raise ValueError(f"oracle_encoder_block rc={rc}")
    return {"attn": attn, "res_out": res_out, "ln_out": ln, "mean": mean, "rstd": rstd}


def prefill_paged(q, k_cache, v_cache, k_scale, v_scale, block_table, L_act, scale, rows,
                  return_lse: bool = False):
    """History-only paged prefill for token indices ``rows`` and all query heads.

    q [Hq,Lq,D]; caches [num_blocks,Hkv,bs,D] e4m3fn; returns out [Hq,len(rows),D] fp64.
    """
    import torch

    qr, qt = _raw(q)
    kc = k_cache.detach().cpu().contiguous().view(torch.uint8).numpy()
    vc = v_cache.detach().cpu().contiguous().view(torch.uint8).numpy()
    bt = np.ascontiguousarray(np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table),
                              dtype=np.int32)
    r = np.ascontiguousarray(np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows), dtype=np.int64)
    Hq, Lq, D = qr.shape
    nb, Hkv, bs, _ = kc.shape
    out = np.empty((Hq, r.size, D))
    lse = np.empty((Hq, r.size))
    rc = lib().oracle_prefill_paged(_ptr(qr), qt, _ptr(kc), _ptr(vc), float(k_scale), float(v_scale), _ptr(bt),
                                    bt.size, nb, bs, int(L_act), float(scale), Hq, Hkv, Lq, D, _ptr(r), r.size,
                                    _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_prefill_paged rc={rc}")
    return (out, lse) if return_lse else out


def prefill_causal(q, k_cache, v_cache, k_scale, v_scale, block_table, L_act, k_cur, v_cur, scale, rows,
                   return_lse: bool = False):
    """Paged history plus causal current-token prefill for token indices
    ``rows`` and all query heads: token t attends history keys 0..L_act-1 and
    current keys 0..t.  q [Hq,Lq,D]; caches [num_blocks,Hkv,bs,D] e4m3fn;
    k_cur/v_cur [Hkv,Lq,D]; returns out [Hq,len(rows),D] fp64 (and lse)."""
    import torch

    qr, qt = _raw(q)
    kr, kt = _raw(k_cur)
    vr, vt = _raw(v_cur)
    if kt != vt:
        raise TypeError("prefill_causal: k_cur and v_cur must share a dtype")
    kc = k_cache.detach().cpu().contiguous().view(torch.uint8).numpy()
    vc = v_cache.detach().cpu().contiguous().view(torch.uint8).numpy()
    bt = np.ascontiguousarray(np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table),
                              dtype=np.int32)
    r = np.ascontiguousarray(np.asarray(rows.cpu() if hasattr(rows, "cpu") else rows), dtype=np.int64)
    Hq, Lq, D = qr.shape
    nb, Hkv, bs, _ = kc.shape
    out = np.empty((Hq, r.size, D))
    lse = np.empty((Hq, r.size))
    rc = lib().oracle_prefill_causal(_ptr(qr), qt, _ptr(kc), _ptr(vc), float(k_scale), float(v_scale), _ptr(bt),
                                     bt.size, nb, bs, int(L_act), _ptr(kr), _ptr(vr), kt, float(scale), Hq, Hkv, Lq,
                                     D, _ptr(r), r.size, _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_prefill_causal rc={rc}")
    return (out, lse) if return_lse else out
