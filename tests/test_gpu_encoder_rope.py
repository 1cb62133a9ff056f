"""Encoder attention with the fused RoPE prologue, HIP path vs the fp64
oracle (``oracle.encoder_block_rope``: q and k rotated in fp64, then the
block) through the C ABI.

The rotated q/k are rounded to bf16 before the contraction on the GPU (the
oracle keeps them exact); the tolerances are the encoder's.  Tables come from
the package's host builder: V-JEPA2's 8 x 16 x 16 token grid (3D,
interleaved pairing) and DINOv3's 28 x 28 patches after 5 unrotated tokens
(2D, rotate-half) - vit-encoder-neuron-kernels, "Kernels" names the two
pairings and the models that use them.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_close, assert_ln_stats
from transformer_attention_attn_amd.rope import grid_positions, rope_tables

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tables(pos, D, rotate=None, **kw):
    c, s = rope_tables(pos, D, rotate=rotate, **kw)
    return torch.from_numpy(c), torch.from_numpy(s)


def _run(taa, case, pairing, c, s, with_res=True, mask=True):
    d = lambda t: None if t is None else t.to(DEV)
    kw = dict(residual=d(case.residual), gamma=d(case.gamma), beta=d(case.beta), eps=case.eps) if with_res else {}
    r = taa.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(case.mask) if mask else None,
                             want_ln=with_res, rope=pairing, rope_cos=d(c), rope_sin=d(s), **kw)
    torch.cuda.synchronize()
    return r


def _check(taa, case, pairing, c, s, what):
    r = _run(taa, case, pairing, c, s)
    ref = oracle.encoder_block_rope(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta,
                                    case.eps, case.mask, c, s, pairing)
    assert_close(r["out"], ref["attn"], f"{what} attention")
    assert_close(r["residual_out"], ref["res_out"], f"{what} residual_out")
    assert_close(r["ln_out"], ref["ln_out"], f"{what} ln_out")
    assert_ln_stats(r["residual_out"], r["ln_mean"], r["ln_rstd"], case.gamma, case.beta, case.eps, what)


def test_vjepa2_block_3d_interleaved(gpu_lib):
    case = W.encoder_vjepa2()
    pos, _ = grid_positions(8, 16, 16)
    c, s = _tables(pos, 64)
    _say("[encoder-rope] V-JEPA2 B=1 H=16 S=2048, 3D tables, interleaved")
    _check(gpu_lib, case, "interleaved", c, s, "vjepa2 rope")


def test_dinov3_block_2d_half_with_prefix_tokens(gpu_lib):
    case = W.encoder_dinov3()
    pos, rot = grid_positions(28, 28, prefix_tokens=5)
    c, s = _tables(pos, 64, rotate=rot)
    _say("[encoder-rope] DINOv3 B=2 H=16 S=789, 2D tables + 5 unrotated tokens, rotate-half")
    _check(gpu_lib, case, "half", c, s, "dinov3 rope")


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
@pytest.mark.parametrize("B,H,S,lens,fp32", [
    (2, 3, 300, [300, 77], False),   # additive key mask, ragged tail
    (1, 2, 129, None, True),         # fp32 inputs: rotated in fp32 before the bf16 rounding
    (3, 2, 64, [1, 64, 33], True),   # mask and fp32 together
])
def test_rope_small_cases(gpu_lib, pairing, B, H, S, lens, fp32):
    case = W.encoder_custom(900 + S, B, H, S, masked_lens=lens, fp32_inputs=fp32)
    c, s = _tables(np.arange(S) * 1.5, 64, ntk_factor=2.0)
    _say(f"[encoder-rope] {pairing} B={B} H={H} S={S} lens={lens} fp32={fp32}")
    _check(gpu_lib, case, pairing, c, s, f"rope {pairing} small")


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_per_batch_tables(gpu_lib, pairing):
    """[B, rows, D/2] tables: each batch entry rotates with its own."""
    case = W.encoder_custom(950, 2, 2, 200)
    pos, _ = grid_positions(10, 20)
    c0, s0 = _tables(pos, 64)
    c1, s1 = _tables(np.arange(200) * 3.0, 64)
    c, s = torch.stack([c0, c1]), torch.stack([s0, s1])
    r = _run(gpu_lib, case, pairing, c, s, with_res=False)
    for b, (cb, sb) in enumerate(((c0, s0), (c1, s1))):
        ref = oracle.encoder_block_rope(case.q[b:b + 1], case.k[b:b + 1], case.v[b:b + 1], case.scale,
                                        case.residual[b:b + 1], None, None, case.eps, None, cb, sb, pairing)
        assert_close(r["out"][b:b + 1], ref["attn"], f"per-batch tables b={b}")


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_identity_tables_give_the_unrotated_bits(gpu_lib, pairing):
    case = W.encoder_custom(960, 2, 4, 333, masked_lens=[333, 100])
    c, s = torch.ones(333, 32), torch.zeros(333, 32)
    a = _run(gpu_lib, case, pairing, c, s)
    d = lambda t: t.to(DEV)
    b = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(case.mask),
                                 residual=d(case.residual), gamma=d(case.gamma), beta=d(case.beta), eps=case.eps)
    torch.cuda.synchronize()
    for key in ("out", "residual_out", "ln_out"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_with_key_lengths(gpu_lib, pairing):
    """RoPE with the right padding as key lengths (the direct-copy path over
    the rotated K): the oracle with the equivalent additive mask."""
    lens = [300, 77]
    case = W.encoder_custom(970, 2, 3, 300, masked_lens=lens)
    c, s = _tables(np.arange(300) * 1.5, 64, ntk_factor=2.0)
    d = lambda t: None if t is None else t.to(DEV)
    _say(f"[encoder-rope] {pairing} with key lengths {lens}")
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None,
                                 key_len=torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 residual=d(case.residual), gamma=d(case.gamma), beta=d(case.beta), eps=case.eps,
                                 rope=pairing, rope_cos=d(c), rope_sin=d(s))
    torch.cuda.synchronize()
    ref = oracle.encoder_block_rope(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta,
                                    case.eps, case.mask, c, s, pairing)
    assert_close(r["out"], ref["attn"], f"rope {pairing} key lengths attention")
    assert_close(r["residual_out"], ref["res_out"], f"rope {pairing} key lengths residual_out")
    assert_close(r["ln_out"], ref["ln_out"], f"rope {pairing} key lengths ln_out")
