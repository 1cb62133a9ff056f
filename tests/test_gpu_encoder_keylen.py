"""Right padding given as key lengths (attn_encoder_fwd's key_len) against the
fp64 oracle with the equivalent additive mask (0 on keys below the length,
-inf past it), through the C ABI.

The gte encoder page's "Constraints" (right padding only, a 0/1 attention
mask) and the ViT page's padded-key skipping: key tiles past a row's length
are never read, so K/V there may hold anything (NaN/inf poison below).
Covers the direct-copy bf16 path (32- and 64-key tiles), the register-staged
fp32 path, lengths 0, 1, S_kv and past S_kv (clamped), negative (clamped to
0), S_q != S_kv, the residual + LayerNorm epilogue and the lse.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import LSE_ABS, assert_close, assert_ln_stats, metrics

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _mask_of(lens, B, Skv):
    m = torch.zeros(B, 1, 1, Skv)
    for b, n in enumerate(lens):
        m[b, 0, 0, max(min(n, Skv), 0):] = float("-inf")
    return m


def _run(taa, case, lens, with_res=True, lse=True, k=None, v=None):
    d = lambda t: None if t is None else t.to(DEV)
    B, H, Sq = case.q.shape[:3]
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    lse_t = torch.empty(B, H, Sq, device=DEV) if lse else None
    r = taa.attn_encoder_fwd(d(case.q), d(case.k if k is None else k), d(case.v if v is None else v), case.scale,
                             None, key_len=kl, lse=lse_t, residual=d(case.residual) if with_res else None,
                             gamma=d(case.gamma), beta=d(case.beta), eps=case.eps, want_ln=with_res)
    torch.cuda.synchronize()
    return r


def _check(r, case, lens, what, with_res=True):
    B, Skv = case.q.shape[0], case.k.shape[2]
    mask = _mask_of(lens, B, Skv)
    ref, lse = oracle.sdpa(case.q, case.k, case.v, case.scale, mask, return_lse=True)
    assert_close(r["out"], ref, f"{what} out")
    live = torch.tensor([min(max(n, 0), Skv) > 0 for n in lens])
    got_lse = r["lse"].cpu().double().numpy()
    assert np.all(np.isneginf(got_lse[~live.numpy()])), f"{what}: rows with no key need lse = -inf"
    if live.any():
        assert metrics(r["lse"].cpu()[live], lse[live.numpy()])["max_abs"] < LSE_ABS, f"{what} lse"
    if with_res:
        blk = oracle.encoder_block(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta,
                                   case.eps, mask)
        assert_close(r["residual_out"], blk["res_out"], f"{what} residual_out")
        assert_close(r["ln_out"], blk["ln_out"], f"{what} ln_out")
        assert_ln_stats(r["residual_out"], r["ln_mean"], r["ln_rstd"], case.gamma, case.beta, case.eps, what)


@pytest.mark.parametrize("B,H,S,lens", [
    (4, 12, 512, [6, 512, 300, 129]),    # gte-base at L 512: ragged, one unpadded
    (3, 2, 200, [0, 1, 200]),            # no key, one key, all keys
    (2, 2, 96, [500, -3]),               # clamped to S_kv and to 0
    (3, 2, 192, [64, 65, 128]),          # one, two and exactly two key steps (64 keys per step)
])
def test_keylen_bf16_block(gpu_lib, B, H, S, lens):
    case = W.encoder_custom(900 + S, B, H, S, masked_lens=None)
    _say(f"[encoder-keylen] bf16 B={B} H={H} S={S} lens={lens}")
    _check(_run(gpu_lib, case, lens), case, lens, f"bf16 S={S}")


@pytest.mark.parametrize("B,H,lens", [
    (1, 16, [1537]),
    (2, 8, [1, 129]),     # one and two key steps (128 keys per step)
    (2, 8, [128, 300]),   # exactly one, and three
])
def test_keylen_64key_tiles(gpu_lib, B, H, lens):
    """One workgroup per CU and at least 1536 keys: the 64-key tile geometry."""
    case = W.encoder_custom(930 + B, B, H, 2048)
    _say(f"[encoder-keylen] 64-key tiles B={B} H={H} S=2048 lens={lens}")
    _check(_run(gpu_lib, case, lens), case, lens, f"64-key tiles lens={lens}")


def test_keylen_fp32_inputs(gpu_lib):
    case = W.encoder_custom(931, 2, 2, 160, fp32_inputs=True)
    lens = [97, 0]
    _say(f"[encoder-keylen] fp32 inputs lens={lens}")
    _check(_run(gpu_lib, case, lens), case, lens, "fp32 inputs")


def test_keylen_cross_lengths(gpu_lib):
    """S_q != S_kv: 100 query rows over 300 keys, lengths below S_kv."""
    case = W.encoder_custom(932, 2, 3, 300)
    case.q = case.q[:, :, :100].contiguous()
    case.residual = case.residual[:, :100].contiguous()
    lens = [257, 31]
    _say(f"[encoder-keylen] S_q=100 S_kv=300 lens={lens}")
    _check(_run(gpu_lib, case, lens), case, lens, "cross lengths")


def test_keylen_never_reads_padding(gpu_lib):
    """K/V past each row's length poisoned with NaN and inf: the outputs are
    finite and bit-identical to those over clean padding."""
    case = W.encoder_custom(933, 2, 4, 256)
    lens = [70, 193]
    kp, vp = case.k.clone(), case.v.clone()
    for b, n in enumerate(lens):
        kp[b, :, n:] = float("nan")
        vp[b, :, n:] = float("inf")
    _say(f"[encoder-keylen] poisoned padding lens={lens}")
    clean = _run(gpu_lib, case, lens)
    dirty = _run(gpu_lib, case, lens, k=kp, v=vp)
    for key in ("out", "lse", "residual_out", "ln_out"):
        assert torch.equal(clean[key], dirty[key]), f"{key} read the padding"
    _check(clean, case, lens, "poison reference")
