"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties one oracle function to brute force on tiny inputs, to a library
routine it reduces to in a special case, to a closed form, or to an invariant
the definition implies.  The tolerances are fp64 round-off (1e-12 relative)
unless the invariant is exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

torch.set_default_dtype(torch.float32)


def _rand(g, *shape):
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _torch_sdpa64(q, k, v, scale, mask=None):
    """torch CPU fp64 SDPA with GQA expanded by repeat_interleave (contiguous groups)."""
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    am = None if mask is None else mask.to(torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=scale).numpy()


def _relmax(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- decoders


def test_bf16_decoder_all_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode(bits.view(torch.bfloat16))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_decoder_all_patterns():
    bits = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode(bits.view(torch.float8_e4m3fn))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # closed-form points of the OCP e4m3fn definition
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2


# ----------------------------------------------------------------------------- SDPA


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,D,masked", [
    (1, 1, 1, 3, 5, 4, False),
    (2, 4, 2, 4, 7, 8, True),
    (1, 6, 3, 1, 16, 8, True),
    (2, 2, 1, 5, 1, 3, False),
])
def test_sdpa_matches_brute_force(B, Hq, Hkv, Sq, Skv, D, masked):
    g = torch.Generator().manual_seed(7 + Skv)
    q, k, v = _rand(g, B, Hq, Sq, D), _rand(g, B, Hkv, Skv, D), _rand(g, B, Hkv, Skv, D)
    mask = None
    if masked:
        mask = torch.zeros(B, 1, 1, Skv, dtype=torch.float64)
        mask[:, 0, 0, Skv // 2 + 1:] = -math.inf
        mask[0, 0, 0, 0] = -0.75  # a finite additive entry as well
    scale = 0.37
    got = oracle.sdpa(q, k, v, scale, mask)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            ref = brute.softmax_attention(q[b, h].tolist(), k[b, h // G].tolist(), v[b, h // G].tolist(), scale,
                                          None if mask is None else mask[b, 0, 0].tolist())
            assert _relmax(got[b, h], ref) < 1e-12


@pytest.mark.parametrize("in_dtype", [torch.float64, torch.float32, torch.bfloat16])
def test_sdpa_matches_torch_fp64_gqa(in_dtype):
    g = torch.Generator().manual_seed(11)
    B, Hq, Hkv, Sq, Skv, D = 2, 8, 2, 33, 45, 16
    q, k, v = (_rand(g, B, h, s, D).to(in_dtype) for h, s in ((Hq, Sq), (Hkv, Skv), (Hkv, Skv)))
    lens = [45, 17]
    mask = torch.zeros(B, 1, 1, Skv, dtype=torch.float64)
    for b, n in enumerate(lens):
        mask[b, 0, 0, n:] = -math.inf
    got, lse = oracle.sdpa(q, k, v, 0.25, mask, return_lse=True)
    ref = _torch_sdpa64(q, k, v, 0.25, mask)
    assert _relmax(got, ref) < 1e-12
    # lse against the log-sum-exp of the torch fp64 scores
    kk = k.to(torch.float64).repeat_interleave(Hq // Hkv, 1)
    s = 0.25 * q.to(torch.float64) @ kk.transpose(-1, -2) + mask
    assert _relmax(lse, torch.logsumexp(s, -1).numpy()) < 1e-12


# ----------------------------------------------------------------------------- invariants


def _case(seed, B=1, H=2, Sq=9, Skv=13, D=8):
    g = torch.Generator().manual_seed(seed)
    return _rand(g, B, H, Sq, D), _rand(g, B, H, Skv, D), _rand(g, B, H, Skv, D)


def test_probability_rows_sum_to_one():
    # V = identity (Skv == D) makes o_i the probability row P_i itself.
    q, k, _ = _case(1, Skv=8, D=8)
    v = torch.eye(8, dtype=torch.float64).expand(1, 2, 8, 8).contiguous()
    P = oracle.sdpa(q, k, v, 0.5)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-14


def test_constant_v_returns_constant():
    q, k, _ = _case(2)
    v = torch.full((1, 2, 13, 8), 3.25, dtype=torch.float64)
    o = oracle.sdpa(q, k, v, 0.3)
    assert np.max(np.abs(o - 3.25)) < 1e-13


def test_kv_permutation_invariance():
    q, k, v = _case(3)
    mask = torch.zeros(1, 1, 1, 13, dtype=torch.float64)
    mask[..., 4] = -math.inf
    mask[..., 7] = 0.5
    perm = torch.randperm(13, generator=torch.Generator().manual_seed(9))
    o1 = oracle.sdpa(q, k, v, 0.4, mask)
    o2 = oracle.sdpa(q, k[:, :, perm], v[:, :, perm], 0.4, mask[..., perm])
    assert np.max(np.abs(o1 - o2)) < 1e-14


def test_masked_keys_are_ignored_bitwise():
    q, k, v = _case(4)
    mask = torch.zeros(1, 1, 1, 13, dtype=torch.float64)
    mask[..., 9:] = -math.inf
    o1 = oracle.sdpa(q, k, v, 0.4, mask)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 9:] = 1e30
    v2[:, :, 9:] = -1e300
    o2 = oracle.sdpa(q, k2, v2, 0.4, mask)
    assert np.array_equal(o1, o2)


def test_one_hot_score_selects_single_value_row():
    # q = 8000 e_t, k_{j*} = e_t, other keys orthogonal to e_t, scale 1/8 -> s_{j*} = 1000.
    D, Skv, t, jstar = 8, 11, 3, 6
    g = torch.Generator().manual_seed(5)
    k = _rand(g, 1, 1, Skv, D)
    k[..., t] = 0.0
    k[0, 0, jstar] = 0.0
    k[0, 0, jstar, t] = 1.0
    q = torch.zeros(1, 1, 1, D, dtype=torch.float64)
    q[..., t] = 8000.0
    v = _rand(g, 1, 1, Skv, D)
    o = oracle.sdpa(q, k, v, 1.0 / 8.0)
    assert np.array_equal(o[0, 0, 0], v[0, 0, jstar].numpy())


def test_zero_scale_gives_mean_of_unmasked_values():
    q, k, v = _case(6)
    mask = torch.zeros(1, 1, 1, 13, dtype=torch.float64)
    mask[..., 10:] = -math.inf
    o = oracle.sdpa(q, k, v, 0.0, mask)
    ref = v[:, :, :10].mean(2, keepdim=True).expand_as(torch.as_tensor(o)).numpy()
    assert np.max(np.abs(o - ref)) < 1e-14


def test_single_key_returns_its_value():
    q, k, v = _case(7, Skv=1)
    o = oracle.sdpa(q, k, v, 0.9)
    assert np.array_equal(o, v.expand(1, 2, 9, 8).numpy())


def test_fully_masked_row_is_zero_with_neg_inf_lse():
    q, k, v = _case(8)
    mask = torch.full((1, 1, 1, 13), -math.inf, dtype=torch.float64)
    o, lse = oracle.sdpa(q, k, v, 0.5, mask, return_lse=True)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_lse_merge_of_two_key_halves():
    # attention over S1 u S2 equals the LSE-weighted merge of the two halves
    q, k, v = _case(10, Skv=20)
    o, lse = oracle.sdpa(q, k, v, 0.35, return_lse=True)
    o1, l1 = oracle.sdpa(q, k[:, :, :7], v[:, :, :7], 0.35, return_lse=True)
    o2, l2 = oracle.sdpa(q, k[:, :, 7:], v[:, :, 7:], 0.35, return_lse=True)
    M = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - M), np.exp(l2 - M)
    merged = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    assert _relmax(merged, o) < 1e-13
    assert np.max(np.abs(M + np.log(w1 + w2) - lse)) < 1e-13


# ----------------------------------------------------------------------------- LayerNorm


def test_layernorm_matches_torch_and_brute():
    g = torch.Generator().manual_seed(12)
    x = _rand(g, 7, 48) * 3 + 1.5
    gamma, beta = _rand(g, 48), _rand(g, 48)
    y, mean, rstd = oracle.layernorm(x, gamma, beta, 1e-6)
    ref = torch.nn.functional.layer_norm(x, (48,), gamma, beta, 1e-6).numpy()
    assert _relmax(y, ref) < 1e-12
    for r in range(7):
        by, bm, br = brute.layernorm_row(x[r].tolist(), gamma.tolist(), beta.tolist(), 1e-6)
        assert _relmax(y[r], by) < 1e-12
        assert abs(mean[r] - bm) <= 1e-12 * abs(bm) and abs(rstd[r] - br) <= 1e-12 * br


def test_layernorm_closed_forms():
    g = torch.Generator().manual_seed(13)
    x = _rand(g, 5, 64)
    eps = 1e-3
    y, _, _ = oracle.layernorm(x, None, None, eps)
    var = x.var(-1, unbiased=False).numpy()
    assert np.max(np.abs(y.mean(-1))) < 1e-14
    assert np.max(np.abs((y ** 2).mean(-1) - var / (var + eps))) < 1e-13
    # shift invariance: LN(x + c) == LN(x)
    y2, _, _ = oracle.layernorm(x + 17.0, None, None, eps)
    assert np.max(np.abs(y2 - y)) < 1e-12
    # constant row -> beta
    beta = _rand(g, 64)
    y3, m3, _ = oracle.layernorm(torch.full((2, 64), 4.0, dtype=torch.float64), None, beta, eps)
    assert np.array_equal(y3, beta.expand(2, 64).numpy()) and np.all(m3 == 4.0)


def test_encoder_block_matches_torch_chain():
    g = torch.Generator().manual_seed(14)
    B, H, S, D = 2, 3, 10, 8
    q, k, v = (_rand(g, B, H, S, D).to(torch.bfloat16) for _ in range(3))
    res = torch.randn(B, S, H * D, generator=g)
    gamma, beta = torch.rand(H * D, generator=g) + 0.5, torch.randn(H * D, generator=g)
    mask = torch.zeros(B, 1, 1, S)
    mask[1, ..., 6:] = -math.inf
    out = oracle.encoder_block(q, k, v, 0.3, res, gamma, beta, 1e-6, mask)
    attn = _torch_sdpa64(q, k, v, 0.3, mask.to(torch.float64))
    x = res.to(torch.float64) + torch.from_numpy(attn).permute(0, 2, 1, 3).reshape(B, S, H * D)
    ln = torch.nn.functional.layer_norm(x, (H * D,), gamma.double(), beta.double(), 1e-6)
    assert _relmax(out["attn"], attn) < 1e-12
    assert np.max(np.abs(out["res_out"] - x.numpy())) < 1e-13
    assert _relmax(out["ln_out"], ln.numpy()) < 1e-12


def test_encoder_block_queries_and_keys_of_different_lengths():
    """S_q != S_kv: attention of S_q query tokens over S_kv keys, then the
    residual stream of S_q rows, against the torch fp64 chain."""
    g = torch.Generator().manual_seed(15)
    B, H, Sq, Skv, D = 2, 2, 7, 12, 8
    q = _rand(g, B, H, Sq, D).to(torch.bfloat16)
    k, v = (_rand(g, B, H, Skv, D).to(torch.bfloat16) for _ in range(2))
    res = torch.randn(B, Sq, H * D, generator=g)
    gamma, beta = torch.rand(H * D, generator=g) + 0.5, torch.randn(H * D, generator=g)
    mask = torch.zeros(B, 1, 1, Skv)
    mask[0, ..., 9:] = -math.inf
    out = oracle.encoder_block(q, k, v, 0.4, res, gamma, beta, 1e-5, mask)
    attn = _torch_sdpa64(q, k, v, 0.4, mask.to(torch.float64))
    x = res.to(torch.float64) + torch.from_numpy(attn).permute(0, 2, 1, 3).reshape(B, Sq, H * D)
    ln = torch.nn.functional.layer_norm(x, (H * D,), gamma.double(), beta.double(), 1e-5)
    assert out["attn"].shape == (B, H, Sq, D)
    assert _relmax(out["attn"], attn) < 1e-12
    assert np.max(np.abs(out["res_out"] - x.numpy())) < 1e-13
    assert _relmax(out["ln_out"], ln.numpy()) < 1e-12


def _complex_rotate(x, theta, pairing):
    """x [..., S, D] fp64 with each lane pair taken as one complex number and
    multiplied by e^{i theta[s, k]} (torch complex arithmetic)."""
    D = x.shape[-1]
    if pairing == "half":
        z = torch.complex(x[..., : D // 2], x[..., D // 2:])
    else:
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
    r = z * torch.polar(torch.ones_like(theta), theta)
    if pairing == "half":
        return torch.cat([r.real, r.imag], dim=-1)
    return torch.view_as_real(r).reshape(x.shape)


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
@pytest.mark.parametrize("Sq,Skv", [(9, 9), (6, 11)])
def test_encoder_block_rope_matches_complex_rotation_chain(pairing, Sq, Skv):
    """The encoder block on rotated q/k: query token i turns by table row i and
    key j by row j (the tables hold more rows than either length), rotation as
    complex multiplication, then torch fp64 SDPA, the token-major residual add
    and torch LayerNorm."""
    g = torch.Generator().manual_seed(31 + Sq)
    B, H, D, rows = 2, 3, 8, 14
    q = _rand(g, B, H, Sq, D).to(torch.bfloat16)
    k, v = (_rand(g, B, H, Skv, D).to(torch.bfloat16) for _ in range(2))
    res = torch.randn(B, Sq, H * D, generator=g)
    gamma, beta = torch.rand(H * D, generator=g) + 0.5, torch.randn(H * D, generator=g)
    mask = torch.zeros(B, 1, 1, Skv)
    mask[1, ..., Skv - 2:] = -math.inf
    th = _angles(rows, D // 2, 32)
    out = oracle.encoder_block_rope(q, k, v, 0.35, res, gamma, beta, 1e-6, mask, torch.cos(th), torch.sin(th),
                                    pairing)
    qr = _complex_rotate(q.double(), th[:Sq], pairing)
    kr = _complex_rotate(k.double(), th[:Skv], pairing)
    attn = torch.nn.functional.scaled_dot_product_attention(qr, kr, v.double(), attn_mask=mask.double(),
                                                            scale=0.35)
    x = res.double() + attn.permute(0, 2, 1, 3).reshape(B, Sq, H * D)
    ln = torch.nn.functional.layer_norm(x, (H * D,), gamma.double(), beta.double(), 1e-6)
    assert _relmax(out["attn"], attn.numpy()) < 1e-12
    assert np.max(np.abs(out["res_out"] - x.numpy())) < 1e-12
    assert _relmax(out["ln_out"], ln.numpy()) < 1e-12
    # a plausible slip, the key rows of the table taken from the query rows'
    # end, is caught: the result moves far beyond round-off
    if Sq != Skv:
        wrong = _complex_rotate(k.double(), th[rows - Skv:], pairing)
        a2 = torch.nn.functional.scaled_dot_product_attention(qr, wrong, v.double(), attn_mask=mask.double(),
                                                              scale=0.35)
        assert _relmax(out["attn"], a2.numpy()) > 1e-3


# ----------------------------------------------------------------------------- paged prefill


def test_paged_prefill_equals_dense_on_logical_kv():
    """Scatter a logical KV sequence into physical blocks through a random
    permutation; the paged oracle must equal dense fp64 SDPA over the first
    L_act logical keys (GQA heads contiguous)."""
    g = torch.Generator().manual_seed(15)
    Hq, Hkv, Lq, D, bs, nb, L_act = 8, 2, 6, 16, 8, 7, 37
    q = _rand(g, Hq, Lq, D).to(torch.bfloat16)
    logical_k = (torch.randn(nb * bs, Hkv, D, generator=g) * 2).to(torch.float8_e4m3fn)
    logical_v = (torch.randn(nb * bs, Hkv, D, generator=g) * 2).to(torch.float8_e4m3fn)
    bt = torch.randperm(nb, generator=g).to(torch.int32)
    kc = torch.empty(nb, Hkv, bs, D, dtype=torch.float8_e4m3fn)
    vc = torch.empty_like(kc)
    for i in range(nb):  # logical block i lives in physical block bt[i]
        kc[bt[i]] = logical_k[i * bs:(i + 1) * bs].transpose(0, 1)
        vc[bt[i]] = logical_v[i * bs:(i + 1) * bs].transpose(0, 1)
    ks, vs = 0.5, 0.125
    rows = torch.tensor([5, 0, 3])
    out, lse = oracle.prefill_paged(q, kc, vc, ks, vs, bt, L_act, 0.2, rows, return_lse=True)
    kd = (logical_k[:L_act].to(torch.float64) * ks).transpose(0, 1)[None]
    vd = (logical_v[:L_act].to(torch.float64) * vs).transpose(0, 1)[None]
    ref = _torch_sdpa64(q[None, :, rows].to(torch.float64), kd, vd, 0.2)[0]
    assert _relmax(out, ref) < 1e-12
    # physical rows past L_act are ignored bitwise
    kc2, vc2 = kc.clone(), vc.clone()
    last = int(bt[L_act // bs])
    kc2[last, :, L_act % bs:] = torch.tensor(448.0).to(torch.float8_e4m3fn)
    for i in range(L_act // bs + 1, nb):
        vc2[int(bt[i])] = torch.tensor(-448.0).to(torch.float8_e4m3fn)
    out2 = oracle.prefill_paged(q, kc2, vc2, ks, vs, bt, L_act, 0.2, rows)
    assert np.array_equal(out, out2)


# ----------------------------------------------------------------------------- windowed decode


@pytest.mark.parametrize("beg,end,W,expect", [
    (5, 70, 1000, (5, 70)),      # range inside the cache, wider window: unchanged
    (0, 100, 16, (84, 100)),     # cut to its last 16 keys
    (-3, 50, 1000, (0, 50)),     # begin clamped to 0
    (10, 500, 1000, (10, 128)),  # end clamped to S_ctx = 128
    (90, 40, 1000, (40, 40)),    # begin past end: empty
    (0, -7, 8, (0, 0)),          # end before the cache: empty
    (120, 128, 1, (127, 128)),   # one-key window
])
def test_window_range_worked_cases(beg, end, W, expect):
    """Worked by hand from the reading: clamp to [0, S_ctx], keep the last W."""
    assert oracle.window_range(128, 1, [beg], [end], W) == [expect]


def test_window_range_defaults():
    assert oracle.window_range(77, 2) == [(0, 77), (0, 77)]
    assert oracle.window_range(77, 1, None, [60], 16) == [(44, 60)]
    assert oracle.window_range(77, 1, [70], None, None) == [(70, 77)]


def test_decode_window_equals_attention_over_the_slice():
    """Windowed decode of each sequence equals torch fp64 SDPA over K/V sliced
    to that sequence's range, with the caller's mask sliced alongside."""
    g = torch.Generator().manual_seed(16)
    B, Hq, Hkv, S, D = 3, 4, 2, 90, 8
    q, k, v = _rand(g, B, Hq, 1, D), _rand(g, B, Hkv, S, D), _rand(g, B, Hkv, S, D)
    mask = torch.zeros(B, 1, 1, S, dtype=torch.float64)
    mask[1, ..., 60:64] = -math.inf
    mask[2, ..., 7] = 0.75  # a finite additive bias inside the window
    beg, end, W = [10, 0, 3], [50, 90, 40], 32
    out = oracle.decode_window(q, k, v, 0.4, mask, beg, end, W)
    slices = [(18, 50), (58, 90), (8, 40)]  # the last 32 keys of [10,50), [0,90), [3,40)
    for b, (s, e) in enumerate(slices):
        ref = _torch_sdpa64(q[b:b + 1], k[b:b + 1, :, s:e], v[b:b + 1, :, s:e], 0.4, mask[b:b + 1, ..., s:e])
        assert _relmax(out[b:b + 1], ref) < 1e-12
    # keys outside every window may hold anything
    k2, v2 = k.clone(), v.clone()
    k2[0, :, :18] = 1e6
    v2[0, :, 50:] = -1e6
    k2[2, :, 40:] = -3e5
    assert np.array_equal(oracle.decode_window(q, k2, v2, 0.4, mask, beg, end, W), out)


def test_decode_window_empty_range_is_zero():
    g = torch.Generator().manual_seed(17)
    q, k, v = _rand(g, 2, 2, 1, 4), _rand(g, 2, 1, 10, 4), _rand(g, 2, 1, 10, 4)
    out = oracle.decode_window(q, k, v, 1.0, None, [6, 0], [6, 10], 4)
    assert np.all(out[0] == 0.0)
    ref = _torch_sdpa64(q[1:], k[1:, :, 6:], v[1:, :, 6:], 1.0)
    assert _relmax(out[1:], ref) < 1e-12


# ----------------------------------------------------------------------------- prefill with current tokens


def _paged_case(seed, Hq=8, Hkv=2, Lq=12, D=16, bs=8, nb=5, L_act=29):
    g = torch.Generator().manual_seed(seed)
    q = _rand(g, Hq, Lq, D).to(torch.bfloat16)
    logical_k = (torch.randn(nb * bs, Hkv, D, generator=g) * 2).to(torch.float8_e4m3fn)
    logical_v = (torch.randn(nb * bs, Hkv, D, generator=g) * 2).to(torch.float8_e4m3fn)
    bt = torch.randperm(nb, generator=g).to(torch.int32)
    kc = torch.empty(nb, Hkv, bs, D, dtype=torch.float8_e4m3fn)
    vc = torch.empty_like(kc)
    for i in range(nb):
        kc[bt[i]] = logical_k[i * bs:(i + 1) * bs].transpose(0, 1)
        vc[bt[i]] = logical_v[i * bs:(i + 1) * bs].transpose(0, 1)
    k_cur = _rand(g, Hkv, Lq, D).to(torch.bfloat16)
    v_cur = _rand(g, Hkv, Lq, D).to(torch.bfloat16)
    return q, logical_k, logical_v, bt, kc, vc, k_cur, v_cur


def test_prefill_causal_without_history_is_causal_sdpa():
    """L_act = 0: plain causal self-attention of the current tokens (torch
    fp64 SDPA with is_causal, GQA heads contiguous)."""
    q, _, _, bt, kc, vc, k_cur, v_cur = _paged_case(18)
    rows = torch.tensor([0, 1, 7, 11])
    out = oracle.prefill_causal(q, kc, vc, 0.5, 0.25, bt, 0, k_cur, v_cur, 0.3, rows)
    G = q.shape[0] // k_cur.shape[0]
    kq = k_cur.to(torch.float64).repeat_interleave(G, dim=0)[None]
    vq = v_cur.to(torch.float64).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q.to(torch.float64)[None], kq, vq, is_causal=True,
                                                           scale=0.3)[0]
    assert _relmax(out, ref[:, rows].numpy()) < 1e-12
    # token 0 sees exactly one key: its own value row
    assert _relmax(out[:, 0], v_cur.to(torch.float64).repeat_interleave(G, dim=0)[:, 0].numpy()) < 1e-15


def test_prefill_causal_equals_dense_masked_sdpa_over_joined_keys():
    """History keys (dequantised, first L_act logical keys) joined with the
    current keys, with an explicit -inf on current keys after the query's own
    token; torch fp64 SDPA on that."""
    q, lk, lv, bt, kc, vc, k_cur, v_cur = _paged_case(19)
    L_act, Lq, ks, vs = 29, q.shape[1], 0.5, 0.125
    rows = torch.tensor([11, 0, 4, 5])
    out, lse = oracle.prefill_causal(q, kc, vc, ks, vs, bt, L_act, k_cur, v_cur, 0.2, rows, return_lse=True)
    kd = torch.cat([(lk[:L_act].to(torch.float64) * ks).transpose(0, 1), k_cur.to(torch.float64)], dim=1)
    vd = torch.cat([(lv[:L_act].to(torch.float64) * vs).transpose(0, 1), v_cur.to(torch.float64)], dim=1)
    mask = torch.zeros(Lq, L_act + Lq, dtype=torch.float64)
    for t in range(Lq):
        mask[t, L_act + t + 1:] = -math.inf
    G = q.shape[0] // kd.shape[0]
    qs = q.to(torch.float64)[:, rows]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qs[None], kd.repeat_interleave(G, dim=0)[None], vd.repeat_interleave(G, dim=0)[None],
        attn_mask=mask[rows][None, None], scale=0.2)[0]
    assert _relmax(out, ref.numpy()) < 1e-12
    s = 0.2 * torch.einsum("hrd,hkd->hrk", qs, kd.repeat_interleave(G, dim=0)) + mask[rows][None]
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def test_prefill_causal_is_the_lse_merge_of_history_and_current():
    """The joined softmax equals the log-sum-exp merge of the history-only
    result (oracle.prefill_paged) and causal attention over the current
    tokens alone: o = (e^{lse_h} o_h + e^{lse_c} o_c) / (e^{lse_h} + e^{lse_c})."""
    q, _, _, bt, kc, vc, k_cur, v_cur = _paged_case(20)
    rows = torch.tensor([0, 6, 11])
    o, lse = oracle.prefill_causal(q, kc, vc, 0.5, 0.125, bt, 29, k_cur, v_cur, 0.2, rows, return_lse=True)
    oh, lh = oracle.prefill_paged(q, kc, vc, 0.5, 0.125, bt, 29, 0.2, rows, return_lse=True)
    oc, lc = oracle.prefill_causal(q, kc, vc, 0.5, 0.125, bt, 0, k_cur, v_cur, 0.2, rows, return_lse=True)
    M = np.maximum(lh, lc)
    wh, wc = np.exp(lh - M), np.exp(lc - M)
    merged = (wh[..., None] * oh + wc[..., None] * oc) / (wh + wc)[..., None]
    assert _relmax(o, merged) < 1e-12
    assert np.max(np.abs(lse - (M + np.log(wh + wc)))) < 1e-12


def test_prefill_causal_ignores_future_tokens_bitwise():
    q, _, _, bt, kc, vc, k_cur, v_cur = _paged_case(21)
    rows = torch.tensor([0, 3, 5])
    o1 = oracle.prefill_causal(q, kc, vc, 0.5, 0.125, bt, 29, k_cur, v_cur, 0.2, rows)
    k2, v2 = k_cur.clone(), v_cur.clone()
    k2[:, 6:] = 3e4
    v2[:, 6:] = -3e4
    assert np.array_equal(oracle.prefill_causal(q, kc, vc, 0.5, 0.125, bt, 29, k2, v2, 0.2, rows), o1)


# ----------------------------------------------------------------------------- rotary embedding


def _angles(S, P, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.rand(S, P, generator=g, dtype=torch.float64) * 6.0 - 3.0


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_identity_tables_leave_x(pairing):
    g = torch.Generator().manual_seed(22)
    x = _rand(g, 2, 3, 5, 8)
    out = oracle.rope(x, np.ones((5, 4)), np.zeros((5, 4)), pairing)
    assert np.array_equal(out, x.numpy())


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_is_complex_multiplication(pairing):
    """Pair k as the complex number a + ib turns by e^{i theta}: (a + ib) e^{i theta}."""
    g = torch.Generator().manual_seed(23)
    S, D = 7, 16
    x = _rand(g, 2, S, D).numpy()
    th = _angles(S, D // 2, 24).numpy()
    out = oracle.rope(x, np.cos(th), np.sin(th), pairing)
    if pairing == "half":
        z = x[..., : D // 2] + 1j * x[..., D // 2:]
        r = z * np.exp(1j * th)
        want = np.concatenate([r.real, r.imag], axis=-1)
    else:
        z = x[..., 0::2] + 1j * x[..., 1::2]
        r = z * np.exp(1j * th)
        want = np.stack([r.real, r.imag], axis=-1).reshape(x.shape)
    assert _relmax(out, want) < 1e-14


def test_rope_pairings_differ_by_a_lane_permutation():
    """Interleaved RoPE equals rotate-half RoPE conjugated by the lane
    permutation (k, k + D/2) <-> (2k, 2k + 1)."""
    g = torch.Generator().manual_seed(25)
    S, D = 6, 12
    x = _rand(g, 3, S, D).numpy()
    th = _angles(S, D // 2, 26).numpy()
    perm = np.empty(D, dtype=np.int64)  # interleaved lane -> half lane
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    xi = x[..., perm]  # half layout -> interleaved layout
    out_i = oracle.rope(xi, np.cos(th), np.sin(th), "interleaved")
    out_h = oracle.rope(x, np.cos(th), np.sin(th), "half")
    assert np.array_equal(out_i, out_h[..., perm])


def test_rope_scores_depend_on_relative_position_only():
    """With angles pos * omega_k (1D RoPE), q_m . k_n depends on m - n only."""
    g = torch.Generator().manual_seed(27)
    D, S = 16, 40
    omega = 10000.0 ** (-np.arange(D // 2) / (D // 2))
    th = np.arange(S)[:, None] * omega[None, :]
    q, k = _rand(g, D).numpy(), _rand(g, D).numpy()
    for pairing in ("half", "interleaved"):
        qr = oracle.rope(np.broadcast_to(q, (S, D)), np.cos(th), np.sin(th), pairing)
        kr = oracle.rope(np.broadcast_to(k, (S, D)), np.cos(th), np.sin(th), pairing)
        s1 = qr[12] @ kr[5]
        s2 = qr[30] @ kr[23]
        assert abs(s1 - s2) < 1e-12 * max(1.0, abs(s1))
        assert abs(qr[12] @ kr[12] - q @ k) < 1e-12 * max(1.0, abs(q @ k))  # same position: no rotation left


def test_rope_rotation_keeps_pair_norms():
    g = torch.Generator().manual_seed(28)
    x = _rand(g, 4, 9, 10).numpy()
    th = _angles(9, 5, 29).numpy()
    out = oracle.rope(x, np.cos(th), np.sin(th), "half")
    n0 = x[..., :5] ** 2 + x[..., 5:] ** 2
    n1 = out[..., :5] ** 2 + out[..., 5:] ** 2
    assert _relmax(n1, n0) < 1e-14
