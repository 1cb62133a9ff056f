"""Additive masks that carry finite biases, not only 0 / -inf.

The decode page's "Input contract" defines the mask as additive; the entry
points add any finite value to the scaled score (a relative-position bias,
say) and remove keys at -inf.  Biases here are N(0, 2^2) with a few large ones
(+-40, far beyond the lazy-rescale threshold) and some removed keys.
"""
import sys

import pytest
import torch

import oracle
import workloads as W
from parity import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bias(seed, B, S):
    g = torch.Generator().manual_seed(seed)
    m = torch.randn(B, 1, 1, S, generator=g) * 2.0
    m[..., 5] = 40.0
    m[..., 17] = -40.0
    drop = torch.rand(B, 1, 1, S, generator=g) < 0.1
    m[drop] = float("-inf")
    m[:, ..., 5] = 40.0  # keep the large positive bias live
    return m


@pytest.mark.parametrize("fp32", [False, True])
def test_encoder_finite_bias(gpu_lib, fp32):
    case = W.encoder_custom(1400 + fp32, 2, 3, 300, fp32_inputs=fp32)
    mask = _bias(1402, 2, 300)
    _say(f"[bias] encoder B=2 H=3 S=300 fp32={fp32}")
    d = lambda t: t.to(DEV)
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(mask), want_ln=False)
    torch.cuda.synchronize()
    assert_close(r["out"], oracle.sdpa(case.q, case.k, case.v, case.scale, mask), "encoder with biases")


@pytest.mark.parametrize("D", [256, 512])
def test_decode_finite_bias(gpu_lib, D):
    case = W.decode_gemma(1410 + D, 3, 8, 4, 1500, D=D)
    mask = _bias(1411, 3, 1500)
    _say(f"[bias] decode B=3 S_ctx=1500 D={D}")
    d = lambda t: t.to(DEV)
    out = gpu_lib.attn_decode_gqa(d(case.q), d(case.k), d(case.v), d(mask), case.scale, case.G)
    torch.cuda.synchronize()
    assert_close(out, oracle.sdpa(case.q, case.k, case.v, case.scale, mask), f"decode with biases D={D}")
    beg, end = [0, 700, 1200], [1500, 1500, 1300]
    kb, ke = (torch.tensor(x, dtype=torch.int32, device=DEV) for x in (beg, end))
    outw = gpu_lib.attn_decode_gqa_window(d(case.q), d(case.k), d(case.v), d(mask), kb, ke, 600, case.scale, case.G)
    torch.cuda.synchronize()
    ref = oracle.decode_window(case.q, case.k, case.v, case.scale, mask, beg, end, 600)
    assert_close(outw, ref, f"decode window with biases D={D}")


def test_encoder_mask_row_shared_by_the_batch(gpu_lib):
    """A [1,1,1,S_kv] mask (batch stride 0) applies its one row to every
    batch entry: the same result as the row repeated per batch entry."""
    case = W.encoder_custom(1420, 3, 2, 200)
    row = _bias(1421, 1, 200)
    _say("[bias] encoder B=3 H=2 S=200, one mask row for the batch")
    d = lambda t: t.to(DEV)
    shared = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(row), want_ln=False)["out"]
    full = row.expand(3, 1, 1, 200).contiguous()
    per_b = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, d(full), want_ln=False)["out"]
    torch.cuda.synchronize()
    assert torch.equal(shared, per_b)
    assert_close(shared, oracle.sdpa(case.q, case.k, case.v, case.scale, full), "encoder with a shared mask row")
