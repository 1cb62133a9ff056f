"""Seeded synthetic inputs for the five attention workloads.

This module only draws random tensors, rounds them to the storage dtype the
workload names, and returns them on the CPU.  It holds none of the attention or
LayerNorm arithmetic: both the HIP path and the fp64 oracle consume the bytes
it returns, and neither imports the other.

Shapes follow the pages' input contracts:
  * encoder q/k/v ``[B, H, S, D]`` and the fp32 residual stream ``[B, S, H*D]``
    (vit-encoder-neuron-kernels, "Supported shapes and limits"; V-JEPA2 ViT-L
    Encoder NKI Kernels, "Quick start" output shape);
  * decode q ``[B, Hq, 1, D]``, k/v ``[B, Hkv, S_ctx, D]``, additive mask
    ``[B, 1, 1, S_ctx]`` (head_dim>128 GQA Flash-Decode kernel, "Input contract");
  * prefill q ``[Hq, Lq, D]``, paged k/v ``[num_blocks, Hkv, block_size, D]``
    (Prefill Context-Parallel Attention POC, "Layout").

Every generator is a ``torch.Generator('cpu')`` seeded with 1000 + the workload
number, and tensors are drawn in the order listed in each function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0  # largest finite OCP e4m3fn magnitude


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    return g


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 -> bf16 (round-to-nearest-even, torch's cast)."""
    return x.to(torch.bfloat16)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor OCP e4m3fn quantisation: scale = amax/448, RNE cast.

    Returns (uint8 codes viewed as torch.float8_e4m3fn, fp32 scale).
    """
    amax = float(x.abs().max())
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    scale = float(torch.tensor(scale, dtype=torch.float32))
    q = (x / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, scale


# --------------------------------------------------------------------------- encoder


@dataclass
class EncoderCase:
    name: str
    B: int
    H: int
    S: int
    D: int
    scale: float
    eps: float
    q: torch.Tensor  # [B,H,S,D] fp32 or bf16
    k: torch.Tensor
    v: torch.Tensor
    residual: torch.Tensor  # [B,S,H*D] fp32
    gamma: torch.Tensor | None  # [H*D] fp32
    beta: torch.Tensor | None
    mask: torch.Tensor | None = None  # [B,1,1,S] fp32 additive
    extra: dict = field(default_factory=dict)


def encoder_tiny(seed: int = 1001) -> EncoderCase:
    """Tiny non-causal SDPA: B=1, 2 heads, S=128, D=64, fp32 N(0,1) q/k/v,
    N(0,1) [128,128] residual, LayerNorm gamma=1, beta=0, eps 1e-6."""
    g = _gen(seed)
    B, H, S, D = 1, 2, 128, 64
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    v = torch.randn(B, H, S, D, generator=g)
    res = torch.randn(B, S, H * D, generator=g)
    gamma = torch.ones(H * D)
    beta = torch.zeros(H * D)
    return EncoderCase("tiny_sdpa_s128", B, H, S, D, 1.0 / 8.0, 1e-6, q, k, v, res, gamma, beta)


def _vit_block(name: str, seed: int, B: int, S: int, H: int = 16, D: int = 64) -> EncoderCase:
    g = _gen(seed)
    q = to_bf16(torch.randn(B, H, S, D, generator=g))
    k = to_bf16(torch.randn(B, H, S, D, generator=g))
    v = to_bf16(torch.randn(B, H, S, D, generator=g))
    res = torch.randn(B, S, H * D, generator=g)
    gamma = torch.rand(H * D, generator=g) + 0.5  # U(0.5, 1.5)
    beta = torch.randn(H * D, generator=g) * math.sqrt(0.1)  # N(0, var 0.1)
    return EncoderCase(name, B, H, S, D, 1.0 / 8.0, 1e-6, q, k, v, res, gamma, beta)


def encoder_vjepa2(seed: int = 1002) -> EncoderCase:
    """V-JEPA2 ViT-L block: B=1, 16 heads, 2048 tokens (16 frames, tubelet
    2x16x16 at 256 px), D=64, bf16 q/k/v, fp32 [2048,1024] residual."""
    return _vit_block("vjepa2_vitl_s2048", seed, B=1, S=2048)


def encoder_dinov3(seed: int = 1003) -> EncoderCase:
    """DINOv3 ViT-L/16 at 448 px: B=2, 789 tokens (CLS + 4 registers + 28x28
    patches), 16 heads, D=64."""
    return _vit_block("dinov3_vitl16_448_s789", seed, B=2, S=789)


def encoder_custom(seed: int, B: int, H: int, S: int, D: int = 64, masked_lens=None,
                   fp32_inputs: bool = False, scale: float | None = None) -> EncoderCase:
    """Smaller encoder cases for parity sweeps (ragged tiles, optional
    right-padding key mask built from per-batch lengths)."""
    g = _gen(seed)
    draw = (lambda *s: torch.randn(*s, generator=g)) if fp32_inputs else \
        (lambda *s: to_bf16(torch.randn(*s, generator=g)))
    q, k, v = draw(B, H, S, D), draw(B, H, S, D), draw(B, H, S, D)
    res = torch.randn(B, S, H * D, generator=g)
    gamma = torch.rand(H * D, generator=g) + 0.5
    beta = torch.randn(H * D, generator=g) * math.sqrt(0.1)
    mask = None
    if masked_lens is not None:
        mask = torch.zeros(B, 1, 1, S)
        for b, n in enumerate(masked_lens):
            mask[b, 0, 0, n:] = float("-inf")
    return EncoderCase(f"custom_b{B}h{H}s{S}d{D}", B, H, S, D,
                       scale if scale is not None else 1.0 / math.sqrt(D), 1e-6,
                       q, k, v, res, gamma, beta, mask)


# --------------------------------------------------------------------------- decode


@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    S_ctx: int
    D: int
    scale: float
    q: torch.Tensor  # [B,Hq,1,D] bf16
    k: torch.Tensor  # [B,Hkv,S_ctx,D] bf16
    v: torch.Tensor
    lens: torch.Tensor  # [B] int64
    mask: torch.Tensor  # [B,1,1,S_ctx] fp32 additive 0 / -inf

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def length_mask(lens: torch.Tensor, S_ctx: int) -> torch.Tensor:
    """Additive key mask [B,1,1,S_ctx]: 0 where j < len_b, -inf beyond."""
    j = torch.arange(S_ctx)
    m = torch.where(j[None, :] < lens[:, None], 0.0, float("-inf")).to(torch.float32)
    return m.view(len(lens), 1, 1, S_ctx)


def decode_gemma(seed: int = 1004, B: int = 8, Hq: int = 16, Hkv: int = 8, S_ctx: int = 4096,
                 D: int = 256, lens=None) -> DecodeCase:
    """Gemma-style GQA single-token decode at head_dim D (256: sliding-window
    layers, 512: global layers): bf16 entries N(0, 0.25^2), softmax_scale 1.0,
    len_b ~ U{1..S_ctx}."""
    g = _gen(seed)
    q = to_bf16(torch.randn(B, Hq, 1, D, generator=g) * 0.25)
    k = to_bf16(torch.randn(B, Hkv, S_ctx, D, generator=g) * 0.25)
    v = to_bf16(torch.randn(B, Hkv, S_ctx, D, generator=g) * 0.25)
    drawn = torch.randint(1, S_ctx + 1, (B,), generator=g)
    lens_t = drawn if lens is None else torch.as_tensor(lens, dtype=torch.int64)
    return DecodeCase(f"gqa_decode_b{B}_hq{Hq}_hkv{Hkv}_ctx{S_ctx}_d{D}", B, Hq, Hkv, S_ctx, D, 1.0,
                      q, k, v, lens_t, length_mask(lens_t, S_ctx))


# --------------------------------------------------------------------------- prefill


@dataclass
class PrefillCase:
    name: str
    Hq: int
    Hkv: int
    Lq: int
    D: int
    num_blocks: int
    block_size: int
    L_act: int
    scale: float
    q: torch.Tensor  # [Hq,Lq,D] bf16
    k_cache: torch.Tensor  # [num_blocks,Hkv,bs,D] float8_e4m3fn
    v_cache: torch.Tensor
    k_scale: float
    v_scale: float
    block_table: torch.Tensor  # [max_blocks] int32
    rows: torch.Tensor  # token indices the oracle checks

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def prefill_paged(seed: int = 1005, Hq: int = 32, Hkv: int = 2, Lq: int = 4096, D: int = 256,
                  num_blocks: int = 256, block_size: int = 512, L_act: int = 120000,
                  n_rows: int = 256, scale: float = 1.0 / 16.0) -> PrefillCase:
    """History-only GQA prefill over a paged FP8 cache: 4096 query tokens,
    131072 history tokens in 512-token blocks under a random-permutation block
    table, 32 Q heads / 2 KV heads, D=256, actual_history_len=120000."""
    g = _gen(seed)
    q = to_bf16(torch.randn(Hq, Lq, D, generator=g))
    kf = torch.randn(num_blocks, Hkv, block_size, D, generator=g)
    k8, ks = quantize_e4m3(kf)
    del kf
    vf = torch.randn(num_blocks, Hkv, block_size, D, generator=g)
    v8, vs = quantize_e4m3(vf)
    del vf
    bt = torch.randperm(num_blocks, generator=g).to(torch.int32)
    rows = torch.randperm(Lq, generator=g)[: min(n_rows, Lq)]
    return PrefillCase(f"paged_fp8_prefill_lq{Lq}_hq{Hq}_hkv{Hkv}_d{D}_hist{L_act}", Hq, Hkv, Lq, D,
                       num_blocks, block_size, L_act, scale, q, k8, v8, ks, vs, bt, rows)


def prefill_current_kv(seed: int, Hkv: int, Lq: int, D: int = 256):
    """The current tokens' K/V [Hkv, Lq, D] for causal prefill: bf16 entries
    N(0, 1), the magnitude of the dequantised history K/V."""
    g = _gen(seed)
    k = to_bf16(torch.randn(Hkv, Lq, D, generator=g))
    v = to_bf16(torch.randn(Hkv, Lq, D, generator=g))
    return k, v


CONFIGS = {
    1: encoder_tiny,
    2: encoder_vjepa2,
    3: encoder_dinov3,
    4: decode_gemma,
    5: prefill_paged,
}
