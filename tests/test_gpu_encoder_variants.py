"""Encoder workload variants against the fp64 oracle (through the C ABI).

- gte-style right-padded batches: the fused attention block of the GTE encoder
  page ("Constraints": head_dim 64, right padding with a 0/1 attention mask;
  its supported L in {128, ..., 1024}), here as an additive -inf key mask;
- padding exactness: the rows of a sequence do not change when the batch is
  padded to a longer length or the padding holds other values;
- the long V-JEPA 2 clip (64 frames, 8192 tokens) of the ViT page's
  "Attention shapes", checked on sampled query rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_close, assert_ln_stats

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_block(taa, case, with_ln=True):
    d = lambda t: None if t is None else t.to(DEV)
    r = taa.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(case.mask), residual=d(case.residual),
                             gamma=d(case.gamma), beta=d(case.beta), eps=case.eps, want_ln=with_ln)
    torch.cuda.synchronize()
    return r


def _ragged_lengths(seed: int, B: int, L: int):
    """Per-sequence real lengths from 6 tokens up to L (the page's ragged inputs)."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(6, L + 1, (B,), generator=g).tolist()
    lens[0], lens[-1] = 6, L  # shortest and unpadded sequences always present
    return lens


@pytest.mark.parametrize("L", [128, 384, 1024])
def test_gte_right_padded_batch(gpu_lib, L):
    lens = _ragged_lengths(700 + L, 4, L)
    case = W.encoder_custom(700 + L, 4, 12, L, masked_lens=lens)  # gte-base: 12 heads x 64 = 768
    _say(f"[encoder-variant] gte padded L={L} lens={lens}")
    r = _run_block(gpu_lib, case)
    ref = oracle.encoder_block(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta, case.eps,
                               case.mask)
    assert_close(r["out"], ref["attn"], f"gte L={L} attention")
    assert_close(r["residual_out"], ref["res_out"], f"gte L={L} residual_out")
    assert_close(r["ln_out"], ref["ln_out"], f"gte L={L} ln_out")
    assert_ln_stats(r["residual_out"], r["ln_mean"], r["ln_rstd"], case.gamma, case.beta, case.eps, f"gte L={L}")


def test_padding_exactness(gpu_lib):
    """The rows of a sequence of n real tokens are bit-identical whether the
    batch is padded to 128 or 256 and whatever the padding holds."""
    n, H, D = 77, 12, 64
    short = W.encoder_custom(801, 1, H, 128, masked_lens=[n])
    long = W.encoder_custom(802, 1, H, 256, masked_lens=[n])  # different padding contents
    for name in ("q", "k", "v"):
        getattr(long, name)[:, :, :n] = getattr(short, name)[:, :, :n]
    long.residual[:, :n] = short.residual[:, :n]
    long.gamma.copy_(short.gamma)
    long.beta.copy_(short.beta)
    _say(f"[encoder-variant] padding exactness n={n}: L=128 vs L=256")
    a = _run_block(gpu_lib, short)
    b = _run_block(gpu_lib, long)
    for key in ("out", "residual_out", "ln_out"):
        x, y = a[key], b[key]
        x = x[:, :, :n] if key == "out" else x[:, :n]
        y = y[:, :, :n] if key == "out" else y[:, :n]
        assert torch.equal(x, y), f"{key}: rows of the real tokens depend on the padding"
    assert torch.equal(a["ln_mean"][:n], b["ln_mean"][:n]) and torch.equal(a["ln_rstd"][:n], b["ln_rstd"][:n])
    ref = oracle.encoder_block(short.q, short.k, short.v, short.scale, short.residual, short.gamma, short.beta,
                               short.eps, short.mask)
    assert_close(a["out"][:, :, :n], ref["attn"][:, :, :n], "padding exactness: attention vs oracle")


def test_vjepa2_long_clip_8192(gpu_lib):
    case = W.encoder_custom(803, 1, 16, 8192)
    _say(f"[encoder-variant] V-JEPA2 64-frame clip: B=1 H=16 S=8192 D=64")
    d = lambda t: t.to(DEV)
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None, want_ln=False)
    torch.cuda.synchronize()
    rows = torch.randperm(8192, generator=torch.Generator().manual_seed(803))[:48].sort().values
    rows = torch.cat([rows, torch.tensor([0, 8191])])
    ref = oracle.sdpa(case.q[:, :, rows], case.k, case.v, case.scale)
    assert_close(r["out"][:, :, rows.to(DEV)], ref, "V-JEPA2 8192 sampled rows")
    assert np.isfinite(r["out"].float().cpu().numpy()).all()


def test_rows_independent_of_other_rows(gpu_lib):
    """Replacing the queries of the odd rows leaves every even row's output
    bit-identical: each row's online softmax takes its own decisions."""
    case = W.encoder_custom(804, 2, 4, 333)
    d = lambda t: t.to(DEV)
    a = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None, want_ln=False)["out"]
    q2 = case.q.clone()
    q2[:, :, 1::2] *= 4.0  # sharper rows: their maxima move far more often
    b = gpu_lib.attn_encoder_fwd(d(q2), d(case.k), d(case.v), case.scale, None, want_ln=False)["out"]
    torch.cuda.synchronize()
    assert torch.equal(a[:, :, 0::2], b[:, :, 0::2])


def test_key_row_strides_give_identical_bits(gpu_lib):
    """bf16 K/V rows are copied global -> LDS by direct loads, one 16-byte
    piece per lane at an offset built from the key's row stride (K
    chunk-major, V rows with their halves swapped on key bit 1).  The same
    values in rows of another stride (head-major, padded 72-wide rows,
    token-major [B,S,H,D] memory) must give the same bits, including the
    ragged last tiles, and match the oracle."""
    B, H, S, D = 2, 4, 789, 64
    case = W.encoder_custom(805, B, H, S, D)
    q = case.q.to(DEV)

    def strided(t, width):  # the same values in rows of `width` elements
        buf = torch.zeros(B, H, S, width, dtype=t.dtype)
        buf[..., :D] = t
        return buf.to(DEV)[..., :D]

    def token_major(t):  # [B, S, H, D] memory, viewed as [B, H, S, D]
        return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)

    layouts = {
        "contiguous": (case.k.to(DEV), case.v.to(DEV)),
        "72-wide rows": (strided(case.k, 72), strided(case.v, 72)),
        "token-major": (token_major(case.k), token_major(case.v)),
        "mixed": (token_major(case.k), strided(case.v, 72)),
    }
    outs = {}
    for name, (k, v) in layouts.items():
        _say(f"[encoder-variant] key row strides: {name} k.stride={k.stride()} v.stride={v.stride()}")
        r = gpu_lib.attn_encoder_fwd(q, k, v, case.scale, None, lse=torch.empty(B, H, S, device=DEV), want_ln=False)
        torch.cuda.synchronize()
        outs[name] = (r["out"].cpu(), r["lse"].cpu())
    for name, (o, l) in outs.items():
        assert torch.equal(o, outs["contiguous"][0]) and torch.equal(l, outs["contiguous"][1]), f"{name} differs"
    ref = oracle.encoder_block(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta, case.eps)
    assert_close(outs["contiguous"][0], ref["attn"], "strided key rows: attention")


@pytest.mark.parametrize("fp32,masked", [(False, False), (True, False), (False, True)])
def test_residual_in_place(gpu_lib, fp32, masked):
    """residual_out may alias residual (the header allows it): the in-place
    block gives the bits of the out-of-place one, on the direct-copy path and
    on the register-staged paths (fp32 inputs, an additive mask)."""
    case = W.encoder_custom(990, 2, 4, 333, masked_lens=[333, 120] if masked else None, fp32_inputs=fp32)
    d = lambda t: None if t is None else t.to(DEV)
    _say(f"[encoder-variant] residual in place fp32={fp32} masked={masked}")
    ref = _run_block(gpu_lib, case)
    res = case.residual.to(DEV).clone()
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(case.mask), residual=res,
                                 residual_out=res, gamma=d(case.gamma), beta=d(case.beta), eps=case.eps)
    torch.cuda.synchronize()
    assert r["residual_out"].data_ptr() == res.data_ptr()
    for key in ("out", "residual_out", "ln_out", "ln_mean", "ln_rstd"):
        assert torch.equal(r[key], ref[key]), key
