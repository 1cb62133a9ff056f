"""Algorithmic work per call, the denominators of every roofline figure.

Attention counts the two contractions only (QK^T and PV, 2 FLOPs per MAC);
softmax and normalisation are excluded, which is the convention the prefill
POC uses for its model-MFU column (Prefill Context-Parallel Attention POC,
"Profiling-optimized 4-chip case": QK and PV model FLOPs only).  Decode counts
bytes: the unmasked K/V rows it must read plus the mask, q and out.
"""
from __future__ import annotations

# MI355X published dense peaks and bandwidth (AMD public specifications).
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0


def attn_flops(n_q_rows: int, n_keys: int, D: int) -> int:
    """QK^T + PV FLOPs for n_q_rows query rows (all heads) each over n_keys keys."""
    return 4 * n_q_rows * n_keys * D


def encoder_flops(B: int, H: int, S_q: int, S_kv: int, D: int) -> int:
    return attn_flops(B * H * S_q, S_kv, D)


def prefill_flops(Lq: int, Hq: int, n_keys: int, D: int) -> int:
    return attn_flops(Lq * Hq, n_keys, D)


def decode_bytes(lens, Hkv: int, Hq: int, S_ctx: int, D: int, elem: int = 2, mask_elem: int = 4) -> int:
    """K+V rows actually attended (sum_b len_b per KV head), the fp32 mask, q and out."""
    B = len(lens)
    kv = sum(int(n) for n in lens) * Hkv * D * elem * 2
    return kv + B * S_ctx * mask_elem + 2 * B * Hq * D * elem


def causal_flops(Lq: int, Hq: int, D: int) -> int:
    """QK^T + PV FLOPs of causal attention among Lq tokens: token t sees t+1 keys."""
    return 4 * Hq * D * (Lq * (Lq + 1) // 2)


def decode_window_bytes(n_keys, Hkv: int, Hq: int, D: int, elem: int = 2) -> int:
    """K+V rows inside each sequence's key range (no mask read), q and out."""
    B = len(n_keys)
    return sum(int(n) for n in n_keys) * Hkv * D * elem * 2 + 2 * B * Hq * D * elem


def decode_dense_bytes(B: int, Hkv: int, Hq: int, S_ctx: int, D: int, elem: int = 2) -> int:
    return B * Hkv * S_ctx * D * elem * 2 + B * S_ctx * 4 + 2 * B * Hq * D * elem


def res_ln_bytes(rows: int, hidden: int, x_bytes: int = 0, y_bytes: int = 2, res_out: bool = True,
                 stats: bool = True) -> int:
    """Residual read + optional x read + optional residual_out write + y write + mean/rstd."""
    per_row = hidden * (4 + x_bytes + (4 if res_out else 0) + y_bytes) + (8 if stats else 0)
    return rows * per_row


def vit_encoder_flops(layers: int, tokens: int, hidden: int, mlp: int, patch_in: int) -> int:
    """Closed-form forward FLOPs of a ViT encoder: QKV + out-projection + MLP +
    attention (QK + PV) per layer, plus the patch embedding."""
    per_layer = (2 * tokens * hidden * 3 * hidden + 2 * tokens * hidden * hidden
                 + 2 * 2 * tokens * hidden * mlp + 4 * tokens * tokens * hidden)
    return layers * per_layer + 2 * tokens * patch_in * hidden


# The softmax's VALU work, the encoder's second roofline at head_dim 64.
# 256 CUs x 4 SIMDs issue at 2.4 GHz; a wave64 VALU instruction occupies its
# SIMD's VALU 4 cycles at full rate and 16 cycles for a transcendental
# (v_exp_f32 runs at a quarter of the rate).
SIMDS = 256 * 4
CLOCK_GHZ = 2.4
# Per score, at the least: one exp2 and, at full rate, the scale-and-subtract
# FMA (1), the row max (half an op: a max3 folds two scores), the bf16 pack of
# P (half: two scores per pack) and the row sum (half: a dot2 of two packed
# scores).
SOFTMAX_EXP_PER_SCORE = 1.0
SOFTMAX_FULL_RATE_PER_SCORE = 2.5


def softmax_valu_cycles(n_scores: int, exp_per_score: float = SOFTMAX_EXP_PER_SCORE,
                        full_rate_per_score: float = SOFTMAX_FULL_RATE_PER_SCORE) -> float:
    """SIMD-cycles of VALU issue the online softmax needs for n_scores scores."""
    return n_scores / 64 * (16 * exp_per_score + 4 * full_rate_per_score)


def softmax_valu_bound_us(n_scores: int, **kw) -> float:
    """Shortest time the whole chip's VALUs need for that softmax work (us)."""
    return softmax_valu_cycles(n_scores, **kw) / SIMDS / (CLOCK_GHZ * 1e3)
