"""Python binding of libmi355attn.so (gfx950 flash attention + residual LayerNorm).

Argument marshalling only: every step of every call runs in the HIP kernels of
the shared library.  torch supplies device memory (outputs are allocated here
when the caller passes none) and the current HIP stream.  There is no CPU or
PyTorch fallback: if the library is missing or a call is rejected, an exception
is raised.

Entry points (same names as the C ABI in include/mi355attn.h):
  attn_encoder_fwd, attn_decode_gqa, attn_decode_gqa_workspace_size,
  attn_decode_gqa_window, attn_decode_gqa_window_workspace_size,
  attn_prefill_paged, attn_prefill_paged_expanded, attn_prefill_paged_expanded_workspace_size,
  attn_prefill_paged_causal, attn_prefill_paged_causal_expanded, res_ln, attn_status_string, attn_version.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355attn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3FN = 0, 1, 2
ATTN_ROPE_NONE, ATTN_ROPE_HALF, ATTN_ROPE_INTERLEAVED = 0, 1, 2
_ROPE = {None: ATTN_ROPE_NONE, "half": ATTN_ROPE_HALF, "interleaved": ATTN_ROPE_INTERLEAVED}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {attn_status_string(status)}")


class EncoderArgs(ctypes.Structure):
    """Mirror of attn_encoder_args_t."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("S_q", ctypes.c_int), ("S_kv", ctypes.c_int),
        ("D", ctypes.c_int),
        ("q_stride", ctypes.c_int64 * 4), ("k_stride", ctypes.c_int64 * 4), ("v_stride", ctypes.c_int64 * 4),
        ("mask", ctypes.c_void_p), ("mask_stride_b", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int), ("out_stride", ctypes.c_int64 * 4),
        ("lse", ctypes.c_void_p),
        ("residual", ctypes.c_void_p), ("residual_out", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("eps", ctypes.c_float),
        ("ln_out", ctypes.c_void_p), ("ln_dtype", ctypes.c_int),
        ("ln_mean", ctypes.c_void_p), ("ln_rstd", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p), ("rope_stride_b", ctypes.c_int64),
        ("rope", ctypes.c_int),
        ("rope_workspace", ctypes.c_void_p), ("rope_workspace_bytes", ctypes.c_size_t),
        ("key_len", ctypes.c_void_p),
    ]


def load(path: str | None = None):
    """Load the HIP library (torch is imported first so that the process maps
    a single HIP runtime: the library binds to the one torch loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m transformer_attention_attn_amd.build`")
    L = ctypes.CDLL(p)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_status_string.argtypes = [I]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.restype = I
    L.attn_encoder_fwd.argtypes = [ctypes.POINTER(EncoderArgs), P]
    L.attn_encoder_fwd.restype = I
    L.attn_encoder_rope_workspace_size.argtypes = [I, I, I, I, I]
    L.attn_encoder_rope_workspace_size.restype = Z
    L.attn_decode_gqa_workspace_size.argtypes = [I, I, I, I]
    L.attn_decode_gqa_workspace_size.restype = Z
    L.attn_decode_gqa.argtypes = [P, P, P, P, F, I, I, I, I, I, I, P, P, Z, P]
    L.attn_decode_gqa.restype = I
    L.attn_decode_gqa_noalloc.argtypes = [P, P, P, P, F, I, I, I, I, I, I, P, P]
    L.attn_decode_gqa_noalloc.restype = I
    L.attn_decode_gqa_window_workspace_size.argtypes = [I, I, I, I, I]
    L.attn_decode_gqa_window_workspace_size.restype = Z
    L.attn_decode_gqa_window.argtypes = [P, P, P, P, P, P, I, F, I, I, I, I, I, I, P, P, Z, P]
    L.attn_decode_gqa_window.restype = I
    L.attn_prefill_paged.argtypes = [P, P, P, F, F, P, I, I, I, I, F, I, I, I, I, I, P, P, P]
    L.attn_prefill_paged.restype = I
    L.attn_prefill_paged_expanded.argtypes = [P, P, P, F, F, P, I, I, I, I, F, I, I, I, I, I, P, P, P, Z, P]
    L.attn_prefill_paged_expanded.restype = I
    L.attn_prefill_paged_expanded_workspace_size.argtypes = [I, I, I]
    L.attn_prefill_paged_expanded_workspace_size.restype = Z
    L.attn_prefill_paged_causal.argtypes = [P, P, P, F, F, P, I, I, I, I, P, P, F, I, I, I, I, I, P, P, P, Z, P]
    L.attn_prefill_paged_causal_expanded.argtypes = [P, P, P, F, F, P, I, I, I, I, P, P, F, I, I, I, I, I, P, P, P, Z,
                                                     P]
    L.attn_prefill_paged_causal_expanded.restype = I
    L.attn_prefill_paged_causal_expanded_workspace_size.argtypes = [I, I, I, I, I]
    L.attn_prefill_paged_causal_expanded_workspace_size.restype = Z
    L.attn_prefill_paged_causal_workspace_size.argtypes = [I, I, I, I]
    L.attn_prefill_paged_causal_workspace_size.restype = Z
    L.attn_prefill_paged_causal.restype = I
    L.res_ln.argtypes = [P, P, I, P, P, F, I, I, P, P, I, P, P, P]
    L.res_ln.restype = I
    _lib = L
    return L


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return load().attn_version()


# ----------------------------------------------------------------------------- helpers

_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float8_e4m3fn: ATTN_FP8_E4M3FN}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != ATTN_OK:
        raise AttnError(rc, what)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _expect(t, name: str, shape=None, dtype=None, contiguous: bool = False, numel=None):
    """Raise ValueError unless tensor `t` (skipped when None) has the given
    shape, dtype, element count and contiguity: the kernels write and read
    exactly these extents."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            raise ValueError(f"{name} must be {' or '.join(str(d) for d in ok)}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _alloc_ctx(stream):
    """Allocation context of a call: tensors this binding allocates (outputs,
    workspaces) come from the pool of the stream the kernels run on, so the
    caching allocator never hands their memory to other work while the
    kernels may still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


# ----------------------------------------------------------------------------- entry points


def attn_encoder_rope_workspace_size(B: int, H: int, S_kv: int, D: int, dtype=torch.bfloat16) -> int:
    return int(load().attn_encoder_rope_workspace_size(B, H, S_kv, D, _DT.get(dtype, -1)))


def attn_encoder_fwd(q, k, v, softmax_scale: float, mask=None, *, out=None, out_dtype=torch.bfloat16,
                     want_out: bool = True, lse=None, residual=None, residual_out=None, gamma=None, beta=None,
                     eps: float = 1e-6, ln_out=None, ln_dtype=torch.bfloat16, want_ln: bool | None = None,
                     ln_mean=None, ln_rstd=None, rope=None, rope_cos=None, rope_sin=None, rope_workspace=None,
                     key_len=None, stream=None):
    """Non-causal SDPA over q/k/v [B,H,S,D] (bf16 or fp32, any strides with a
    unit d stride), optional additive key mask [B,1,1,S_kv] fp32 (or
    [1,1,1,S_kv], one row for the whole batch) or, instead of a mask, right
    padding as key lengths (key_len: int32 [B]; batch row b attends keys
    0 .. key_len[b]-1 and the rest are never read), optional fused residual add
    (+ LayerNorm) into the fp32 residual stream [B,S,H*D].
    rope: None, "half" or "interleaved", with fp32 tables rope_cos/rope_sin
    [rows, D/2] (shared by the batch) or [B, rows, D/2]; rope_workspace
    (uint8, allocated here when None) receives the rotated keys.

    Returns a dict of the produced tensors (out, lse, residual_out, ln_out,
    ln_mean, ln_rstd as requested).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    _expect(k, "k", shape=(B, H, Skv, D))
    _expect(v, "v", shape=(B, H, Skv, D))
    hidden = H * D
    _expect(out, "out", shape=(B, H, Sq, D), dtype=(torch.bfloat16, torch.float32))
    _expect(lse, "lse", shape=(B, H, Sq), dtype=torch.float32, contiguous=True)
    _expect(residual, "residual", dtype=torch.float32, contiguous=True, numel=B * Sq * hidden)
    _expect(residual_out, "residual_out", dtype=torch.float32, contiguous=True, numel=B * Sq * hidden)
    _expect(gamma, "gamma", dtype=torch.float32, contiguous=True, numel=hidden)
    _expect(beta, "beta", dtype=torch.float32, contiguous=True, numel=hidden)
    _expect(ln_out, "ln_out", dtype=(torch.bfloat16, torch.float32), contiguous=True, numel=B * Sq * hidden)
    _expect(ln_mean, "ln_mean", dtype=torch.float32, contiguous=True, numel=B * Sq)
    _expect(ln_rstd, "ln_rstd", dtype=torch.float32, contiguous=True, numel=B * Sq)
    if residual_out is not None and residual is None:
        raise ValueError("residual_out needs residual")
    if mask is not None and (mask.dtype != torch.float32 or mask.dim() != 4 or tuple(mask.shape[1:]) != (1, 1, Skv)
                             or mask.shape[0] not in (1, B) or mask.stride(-1) != 1):
        raise ValueError("mask must be fp32 [B,1,1,S_kv] or [1,1,1,S_kv] with a unit last stride")
    if key_len is not None:
        if mask is not None:
            raise ValueError("key_len replaces the mask: pass one of them")
        if key_len.dtype != torch.int32 or tuple(key_len.shape) != (B,) or not key_len.is_contiguous():
            raise ValueError("key_len must be a contiguous int32 [B] tensor")
    if rope not in _ROPE:
        raise ValueError(f"rope must be one of {list(_ROPE)}")
    if rope is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous() or t.shape[-1] != D // 2 \
                    or t.dim() not in (2, 3) or (t.dim() == 3 and t.shape[0] != B):
                raise ValueError(f"{name} must be a contiguous fp32 [rows, D/2] or [B, rows, D/2] tensor")
            if t.shape[-2] < max(Sq, Skv):
                raise ValueError(f"{name} needs at least max(S_q, S_kv) rows")
        if rope_cos.shape != rope_sin.shape:
            raise ValueError("rope_cos and rope_sin must have one shape")
    _need_cuda(q, k, v, mask, out, lse, residual, residual_out, gamma, beta, ln_out, ln_mean, ln_rstd,
               rope_cos, rope_sin, rope_workspace, key_len)
    res = {}
    with _alloc_ctx(stream):
        if want_out and out is None:
            out = torch.empty(B, H, Sq, D, dtype=out_dtype, device=q.device)
        if residual is not None and residual_out is None:
            residual_out = torch.empty_like(residual)
        if want_ln is None:
            want_ln = residual is not None
        if want_ln and ln_out is None:
            ln_out = torch.empty(B, Sq, H * D, dtype=ln_dtype, device=q.device)
            ln_mean = torch.empty(B * Sq, dtype=torch.float32, device=q.device) if ln_mean is None else ln_mean
            ln_rstd = torch.empty(B * Sq, dtype=torch.float32, device=q.device) if ln_rstd is None else ln_rstd
        a = EncoderArgs()
        a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
        a.in_dtype = _DT.get(q.dtype, -1)
        a.B, a.H, a.S_q, a.S_kv, a.D = B, H, Sq, Skv, D
        for i in range(4):
            a.q_stride[i], a.k_stride[i], a.v_stride[i] = q.stride(i), k.stride(i), v.stride(i)
        if mask is not None:
            a.mask = mask.data_ptr()
            # one row shared by the whole batch: batch stride 0
            a.mask_stride_b = mask.stride(0) if mask.shape[0] == B and B > 1 else (0 if B > 1 else Skv)
        a.softmax_scale = float(softmax_scale)
        if out is not None:
            a.out = out.data_ptr()
            a.out_dtype = _DT.get(out.dtype, -1)
            for i in range(4):
                a.out_stride[i] = out.stride(i)
        a.lse = None if lse is None else lse.data_ptr()
        a.residual = None if residual is None else residual.data_ptr()
        a.residual_out = None if residual_out is None else residual_out.data_ptr()
        a.gamma = None if gamma is None else gamma.data_ptr()
        a.beta = None if beta is None else beta.data_ptr()
        a.eps = float(eps)
        if ln_out is not None:
            a.ln_out = ln_out.data_ptr()
            a.ln_dtype = _DT.get(ln_out.dtype, -1)
        a.ln_mean = None if ln_mean is None else ln_mean.data_ptr()
        a.ln_rstd = None if ln_rstd is None else ln_rstd.data_ptr()
        a.key_len = None if key_len is None else key_len.data_ptr()
        a.rope = _ROPE[rope]
        if rope is not None:
            a.rope_cos, a.rope_sin = rope_cos.data_ptr(), rope_sin.data_ptr()
            a.rope_stride_b = rope_cos.stride(0) if rope_cos.dim() == 3 else 0
            if rope_workspace is None:
                need = attn_encoder_rope_workspace_size(B, H, Skv, D, q.dtype)
                rope_workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            a.rope_workspace, a.rope_workspace_bytes = rope_workspace.data_ptr(), rope_workspace.numel()
        _check(load().attn_encoder_fwd(ctypes.byref(a), _stream(stream)), "attn_encoder_fwd")
    for name, t in (("out", out), ("lse", lse), ("residual_out", residual_out), ("ln_out", ln_out),
                    ("ln_mean", ln_mean), ("ln_rstd", ln_rstd)):
        if t is not None:
            res[name] = t
    return res


def _decode_shapes(q, k, v, attn_mask, out, workspace):
    """Shape and dtype checks shared by the two decode entry points."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-dimensional")
        _expect(t, name, dtype=torch.bfloat16, contiguous=True)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, Hq, 1, D]")
    Hkv, S_ctx = k.shape[1], k.shape[2]
    _expect(k, "k", shape=(B, Hkv, S_ctx, D))
    _expect(v, "v", shape=(B, Hkv, S_ctx, D))
    _expect(attn_mask, "attn_mask", shape=(B, 1, 1, S_ctx), dtype=torch.float32, contiguous=True)
    _expect(out, "out", shape=(B, Hq, 1, D), dtype=torch.bfloat16, contiguous=True)
    _expect(workspace, "workspace", dtype=torch.uint8, contiguous=True)
    return B, Hq, Hkv, S_ctx, D


def attn_decode_gqa_workspace_size(B: int, Hq: int, S_ctx: int, D: int) -> int:
    return int(load().attn_decode_gqa_workspace_size(B, Hq, S_ctx, D))


def attn_decode_gqa(q, k, v, attn_mask, softmax_scale: float, num_kv_groups: int, *, out=None, workspace=None,
                    stream=None):
    """GQA single-token decode: q [B,Hq,1,D], k/v [B,Hkv,S_ctx,D] bf16, additive
    mask [B,1,1,S_ctx] fp32 (or None).  Returns out [B,Hq,1,D] bf16."""
    B, Hq, Hkv, S_ctx, D = _decode_shapes(q, k, v, attn_mask, out, workspace)
    _need_cuda(q, k, v, attn_mask, out, workspace)
    with _alloc_ctx(stream):
        if out is None:
            out = torch.empty(B, Hq, 1, D, dtype=torch.bfloat16, device=q.device)
        need = attn_decode_gqa_workspace_size(B, Hq, S_ctx, D)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        rc = load().attn_decode_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(attn_mask), float(softmax_scale),
                                    int(num_kv_groups), B, Hq, Hkv, S_ctx, D, _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream(stream))
    _check(rc, "attn_decode_gqa")
    return out


# bytes of the library's device scratch behind attn_decode_gqa_noalloc
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_decode_gqa_noalloc(q, k, v, attn_mask, softmax_scale: float, num_kv_groups: int, *, out, stream=None):
    """attn_decode_gqa without a workspace: the partials go to the library's
    own device scratch (DECODE_NOALLOC_SCRATCH_BYTES per GPU; calls that can
    overlap on one GPU race on it).  `out` [B,Hq,1,D] bf16 is required: this
    call allocates nothing."""
    if out is None:
        raise ValueError("out is required: attn_decode_gqa_noalloc allocates nothing")
    B, Hq, Hkv, S_ctx, D = _decode_shapes(q, k, v, attn_mask, out, None)
    _need_cuda(q, k, v, attn_mask, out)
    rc = load().attn_decode_gqa_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(attn_mask), float(softmax_scale),
                                        int(num_kv_groups), B, Hq, Hkv, S_ctx, D, _ptr(out), _stream(stream))
    _check(rc, "attn_decode_gqa_noalloc")
    return out


def attn_decode_gqa_window_workspace_size(B: int, Hq: int, S_ctx: int, max_keys: int, D: int) -> int:
    return int(load().attn_decode_gqa_window_workspace_size(B, Hq, S_ctx, max_keys, D))


def attn_decode_gqa_window(q, k, v, attn_mask, key_begin, key_end, max_keys: int, softmax_scale: float,
                           num_kv_groups: int, *, out=None, workspace=None, stream=None):
    """GQA single-token decode over per-sequence key ranges: as attn_decode_gqa,
    plus key_begin/key_end int32 [B] device tensors (or None) and the window
    bound max_keys.  Returns out [B,Hq,1,D] bf16."""
    B, Hq, Hkv, S_ctx, D = _decode_shapes(q, k, v, attn_mask, out, workspace)
    for name, t in (("key_begin", key_begin), ("key_end", key_end)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B):
            raise ValueError(f"{name} must be a contiguous int32 tensor of B entries")
    _need_cuda(q, k, v, attn_mask, key_begin, key_end, out, workspace)
    with _alloc_ctx(stream):
        if out is None:
            out = torch.empty(B, Hq, 1, D, dtype=torch.bfloat16, device=q.device)
        need = attn_decode_gqa_window_workspace_size(B, Hq, S_ctx, max_keys, D)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        rc = load().attn_decode_gqa_window(_ptr(q), _ptr(k), _ptr(v), _ptr(attn_mask), _ptr(key_begin),
                                           _ptr(key_end), int(max_keys), float(softmax_scale), int(num_kv_groups),
                                           B, Hq, Hkv, S_ctx, D, _ptr(out), _ptr(workspace), workspace.numel(),
                                           _stream(stream))
    _check(rc, "attn_decode_gqa_window")
    return out


def _prefill_shapes(q, k_cache, v_cache, block_table, out, lse, workspace):
    """Shape and dtype checks shared by the prefill entry points."""
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table)):
        _expect(t, name, contiguous=True)
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 1:
        raise ValueError("q must be [Hq, Lq, D], the caches [num_blocks, Hkv, block_size, D], block_table 1-D")
    _expect(q, "q", dtype=torch.bfloat16)
    _expect(k_cache, "k_cache", dtype=torch.float8_e4m3fn)
    _expect(v_cache, "v_cache", shape=tuple(k_cache.shape), dtype=torch.float8_e4m3fn)
    _expect(block_table, "block_table", dtype=torch.int32)
    Hq, Lq, D = q.shape
    nb, Hkv, bs, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("q and the caches must share head_dim")
    _expect(out, "out", shape=(Hq, Lq, D), dtype=torch.bfloat16, contiguous=True)
    _expect(lse, "lse", shape=(Hq, Lq), dtype=torch.float32, contiguous=True)
    _expect(workspace, "workspace", dtype=torch.uint8, contiguous=True)
    return Hq, Lq, D, nb, Hkv, bs


def attn_prefill_paged(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table, actual_history_len: int,
                       softmax_scale: float, num_kv_groups: int, *, out=None, lse=None, want_lse: bool = False,
                       stream=None):
    """History-only GQA prefill: q [Hq,Lq,D] bf16, caches [num_blocks,Hkv,bs,D]
    e4m3fn, block_table int32 [max_blocks].  Returns out [Hq,Lq,D] bf16 (and lse)."""
    Hq, Lq, D, nb, Hkv, bs = _prefill_shapes(q, k_cache, v_cache, block_table, out, lse, None)
    _need_cuda(q, k_cache, v_cache, block_table, out, lse)
    with _alloc_ctx(stream):
        if out is None:
            out = torch.empty(Hq, Lq, D, dtype=torch.bfloat16, device=q.device)
        if want_lse and lse is None:
            lse = torch.empty(Hq, Lq, dtype=torch.float32, device=q.device)
        rc = load().attn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale),
                                       _ptr(block_table), block_table.numel(), nb, bs, int(actual_history_len),
                                       float(softmax_scale), int(num_kv_groups), Hq, Hkv, Lq, D, _ptr(out),
                                       _ptr(lse), _stream(stream))
    _check(rc, "attn_prefill_paged")
    return (out, lse) if lse is not None else out


def attn_prefill_paged_expanded_workspace_size(Hkv: int, actual_history_len: int, D: int) -> int:
    return int(load().attn_prefill_paged_expanded_workspace_size(Hkv, actual_history_len, D))


def attn_prefill_paged_expanded(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table,
                                actual_history_len: int, softmax_scale: float, num_kv_groups: int, *, out=None,
                                lse=None, want_lse: bool = False, workspace=None, stream=None):
    """attn_prefill_paged through a workspace of bf16 tile images of the live
    history (allocated here when not given).  Same arguments and result."""
    Hq, Lq, D, nb, Hkv, bs = _prefill_shapes(q, k_cache, v_cache, block_table, out, lse, workspace)
    _need_cuda(q, k_cache, v_cache, block_table, out, lse, workspace)
    with _alloc_ctx(stream):
        if out is None:
            out = torch.empty(Hq, Lq, D, dtype=torch.bfloat16, device=q.device)
        if want_lse and lse is None:
            lse = torch.empty(Hq, Lq, dtype=torch.float32, device=q.device)
        if workspace is None:
            n = attn_prefill_paged_expanded_workspace_size(Hkv, int(actual_history_len), D)
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
        rc = load().attn_prefill_paged_expanded(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                                float(v_scale), _ptr(block_table), block_table.numel(), nb, bs,
                                                int(actual_history_len), float(softmax_scale), int(num_kv_groups),
                                                Hq, Hkv, Lq, D, _ptr(out), _ptr(lse), _ptr(workspace),
                                                workspace.numel(), _stream(stream))
    _check(rc, "attn_prefill_paged_expanded")
    return (out, lse) if lse is not None else out


def attn_prefill_paged_causal_workspace_size(Hq: int, Hkv: int, Lq: int, D: int) -> int:
    return int(load().attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D))


def attn_prefill_paged_causal(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table,
                              actual_history_len: int, k_cur, v_cur, softmax_scale: float, num_kv_groups: int, *,
                              out=None, lse=None, want_lse: bool = False, workspace=None, stream=None,
                              expanded: bool = False):
    """Paged history plus causal current-token GQA prefill: as
    attn_prefill_paged, plus the current tokens' K/V k_cur/v_cur [Hkv,Lq,D]
    bf16.  Returns out [Hq,Lq,D] bf16 (and the joined lse).  expanded=True
    calls attn_prefill_paged_causal_expanded (history through tile images)."""
    Hq, Lq, D, nb, Hkv, bs = _prefill_shapes(q, k_cache, v_cache, block_table, out, lse, workspace)
    if k_cur is None or v_cur is None:
        raise ValueError("k_cur and v_cur are required")
    _expect(k_cur, "k_cur", shape=(Hkv, Lq, D), dtype=torch.bfloat16, contiguous=True)
    _expect(v_cur, "v_cur", shape=(Hkv, Lq, D), dtype=torch.bfloat16, contiguous=True)
    _need_cuda(q, k_cache, v_cache, block_table, k_cur, v_cur, out, lse, workspace)
    with _alloc_ctx(stream):
        if out is None:
            out = torch.empty(Hq, Lq, D, dtype=torch.bfloat16, device=q.device)
        if want_lse and lse is None:
            lse = torch.empty(Hq, Lq, dtype=torch.float32, device=q.device)
        if workspace is None:
            need = (attn_prefill_paged_causal_expanded_workspace_size(Hq, Hkv, Lq, int(actual_history_len), D)
                    if expanded else attn_prefill_paged_causal_workspace_size(Hq, Hkv, Lq, D))
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        fn = load().attn_prefill_paged_causal_expanded if expanded else load().attn_prefill_paged_causal
        rc = fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale), _ptr(block_table),
                block_table.numel(), nb, bs, int(actual_history_len), _ptr(k_cur), _ptr(v_cur), float(softmax_scale),
                int(num_kv_groups), Hq, Hkv, Lq, D, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                _stream(stream))
    _check(rc, "attn_prefill_paged_causal_expanded" if expanded else "attn_prefill_paged_causal")
    return (out, lse) if lse is not None else out


def attn_prefill_paged_causal_expanded_workspace_size(Hq: int, Hkv: int, Lq: int, actual_history_len: int,
                                                      D: int) -> int:
    return int(load().attn_prefill_paged_causal_expanded_workspace_size(Hq, Hkv, Lq, actual_history_len, D))


def attn_prefill_paged_causal_expanded(*args, **kw):
    """attn_prefill_paged_causal with the history through expanded tile images
    (C-ABI attn_prefill_paged_causal_expanded); same arguments and result."""
    return attn_prefill_paged_causal(*args, expanded=True, **kw)


def res_ln(residual, x=None, gamma=None, beta=None, eps: float = 1e-6, *, residual_out=None, y=None,
           y_dtype=torch.bfloat16, mean=None, rstd=None, stream=None):
    """(Residual +) LayerNorm over the last dim of the fp32 residual [rows, hidden]."""
    _expect(residual, "residual", dtype=torch.float32, contiguous=True)
    hidden = residual.shape[-1]
    rows = residual.numel() // hidden
    _expect(x, "x", shape=tuple(residual.shape), dtype=(torch.bfloat16, torch.float32), contiguous=True)
    _expect(gamma, "gamma", dtype=torch.float32, contiguous=True, numel=hidden)
    _expect(beta, "beta", dtype=torch.float32, contiguous=True, numel=hidden)
    _expect(residual_out, "residual_out", dtype=torch.float32, contiguous=True, numel=rows * hidden)
    _expect(y, "y", dtype=(torch.bfloat16, torch.float32), contiguous=True, numel=rows * hidden)
    _expect(mean, "mean", dtype=torch.float32, contiguous=True, numel=rows)
    _expect(rstd, "rstd", dtype=torch.float32, contiguous=True, numel=rows)
    _need_cuda(residual, x, gamma, beta, residual_out, y, mean, rstd)
    with _alloc_ctx(stream):
        if y is None:
            y = torch.empty(residual.shape, dtype=y_dtype, device=residual.device)
        rc = load().res_ln(_ptr(residual), _ptr(x), _DT.get(x.dtype, -1) if x is not None else ATTN_F32,
                           _ptr(gamma), _ptr(beta), float(eps), rows, hidden, _ptr(residual_out), _ptr(y),
                           _DT.get(y.dtype, -1), _ptr(mean), _ptr(rstd), _stream(stream))
    _check(rc, "res_ln")
    return y
