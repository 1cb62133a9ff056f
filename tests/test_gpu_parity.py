"""HIP path vs the fp64 oracle, element by element, on the same seeded inputs.

Every test goes through the C ABI (the ctypes binding) and compares with the
oracle at the tolerances in tests/parity.py.  Sizes span several tiles and a
ragged tail; the five workload shapes run at full size (the paged prefill is
checked on sampled query tokens, all 32 heads).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import prefill_full
import workloads as W
from parity import LSE_ABS, assert_close, assert_ln_stats, metrics, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _enc_run(taa, case, out_strides_token_major=False, with_ln=True, lse=False):
    dev = lambda t: None if t is None else t.to(DEV)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    res = dev(case.residual)
    B, H, S, D = case.B, case.H, case.S, case.D
    out = None
    if out_strides_token_major:
        buf = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=DEV)
        out = buf.permute(0, 2, 1, 3)  # [B,H,S,D] view of token-major storage
    lse_t = torch.empty(B, H, S, device=DEV) if lse else None
    r = taa.attn_encoder_fwd(q, k, v, case.scale, dev(case.mask), out=out, lse=lse_t, residual=res,
                             gamma=dev(case.gamma), beta=dev(case.beta), eps=case.eps, want_ln=with_ln)
    torch.cuda.synchronize()
    return r


def _enc_check(taa, case, what, **kw):
    _say(f"[encoder] {what}: B={case.B} H={case.H} S={case.S} D={case.D} dtype={case.q.dtype}")
    r = _enc_run(taa, case, **kw)
    ref = oracle.encoder_block(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta, case.eps,
                               case.mask)
    m = assert_close(r["out"], ref["attn"], f"{what} attention")
    assert_close(r["residual_out"], ref["res_out"], f"{what} residual_out")
    assert_close(r["ln_out"], ref["ln_out"], f"{what} ln_out")
    assert_ln_stats(r["residual_out"], r["ln_mean"], r["ln_rstd"], case.gamma, case.beta, case.eps, what)
    # the residual add itself is exact fp32 arithmetic on the GPU's own fp32 attention
    return r, ref, m


# ----------------------------------------------------------------------------- encoder


def test_encoder_tiny_fp32_inputs(gpu_lib):
    _enc_check(gpu_lib, W.encoder_tiny(), "tiny fp32 S=128")


def test_encoder_vjepa2_full(gpu_lib):
    _enc_check(gpu_lib, W.encoder_vjepa2(), "V-JEPA2 S=2048")


def test_encoder_dinov3_full_ragged_tail(gpu_lib):
    _enc_check(gpu_lib, W.encoder_dinov3(), "DINOv3 S=789")


@pytest.mark.parametrize("B,H,S,lens,fp32", [
    (1, 1, 1, None, False),
    (1, 1, 7, None, True),
    (2, 3, 33, [33, 17], False),
    (1, 2, 200, [150], False),
    (3, 2, 130, [1, 129, 64], False),
    (2, 1, 327, None, True),
    (1, 4, 640, [600], False),
])
def test_encoder_small_cases(gpu_lib, B, H, S, lens, fp32):
    case = W.encoder_custom(77 + S, B, H, S, masked_lens=lens, fp32_inputs=fp32)
    _enc_check(gpu_lib, case, f"custom B{B} H{H} S{S} mask={lens} fp32={fp32}")


@pytest.mark.parametrize("B,H,Sq,Skv", [
    (1, 2, 100, 1),     # one key; a single, short row tile
    (2, 1, 129, 31),    # fewer keys than one tile; two row tiles, the second of one row
    (1, 3, 64, 65),     # one key past a whole key step
    (2, 2, 300, 129),   # both ragged
    (1, 4, 200, 1600),  # long enough for 64-key tiles; ragged last tile
    (2, 3, 130, 2000),  # 64-key tiles, both ragged
])
def test_encoder_cross_lengths_block(gpu_lib, B, H, Sq, Skv):
    """S_q != S_kv, bf16, no mask (the tiles copied global -> LDS directly,
    the residual rows with them), the whole block checked: the key tail and
    the last row tile's missing rows come from the loads' range checks."""
    g = torch.Generator().manual_seed(9000 + Sq + Skv)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    D = 64
    q, k, v = bf(B, H, Sq, D), bf(B, H, Skv, D), bf(B, H, Skv, D)
    res = torch.randn(B, Sq, H * D, generator=g)
    gamma, beta = torch.rand(H * D, generator=g) + 0.5, torch.randn(H * D, generator=g) * 0.3
    _say(f"[encoder] cross lengths B={B} H={H} Sq={Sq} Skv={Skv}")
    r = gpu_lib.attn_encoder_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 0.125, None, residual=res.to(DEV),
                                 gamma=gamma.to(DEV), beta=beta.to(DEV), eps=1e-6, want_ln=True)
    torch.cuda.synchronize()
    ref = oracle.encoder_block(q, k, v, 0.125, res, gamma, beta, 1e-6)
    what = f"cross Sq={Sq} Skv={Skv}"
    assert_close(r["out"], ref["attn"], f"{what} attention")
    assert_close(r["residual_out"], ref["res_out"], f"{what} residual_out")
    assert_close(r["ln_out"], ref["ln_out"], f"{what} ln_out")
    assert_ln_stats(r["residual_out"], r["ln_mean"], r["ln_rstd"], gamma, beta, 1e-6, what)


def test_encoder_token_major_output_and_lse(gpu_lib):
    case = W.encoder_custom(5, 2, 4, 300, masked_lens=[300, 211])
    _say("[encoder] token-major out + lse")
    r = _enc_run(gpu_lib, case, out_strides_token_major=True, with_ln=False, lse=True)
    ref, lse = oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask, return_lse=True)
    assert_close(r["out"], ref, "token-major out")
    assert r["out"].permute(0, 2, 1, 3).is_contiguous()
    m = metrics(r["lse"], lse)
    assert m["max_abs"] < LSE_ABS, m


def test_encoder_fully_masked_rows(gpu_lib):
    case = W.encoder_custom(6, 2, 2, 96, masked_lens=[96, 0])
    _say("[encoder] fully masked batch row")
    r = _enc_run(gpu_lib, case, with_ln=False, lse=True)
    assert torch.all(r["out"][1] == 0)
    assert torch.all(torch.isneginf(r["lse"][1]))
    ref = oracle.sdpa(case.q[:1], case.k[:1], case.v[:1], case.scale, case.mask[:1])
    assert_close(r["out"][:1], ref, "unmasked batch row")


def test_encoder_deterministic_and_batch_independent(gpu_lib):
    case = W.encoder_custom(8, 3, 4, 257, masked_lens=[257, 200, 100])
    _say("[encoder] determinism / batch independence")
    r1 = _enc_run(gpu_lib, case)
    r2 = _enc_run(gpu_lib, case)
    for k in ("out", "residual_out", "ln_out", "ln_mean", "ln_rstd"):
        assert torch.equal(r1[k], r2[k]), k
    case.q[1] = -case.q[1]
    case.k[1] = case.k[1] * 3
    case.v[1] = 7.0
    r3 = _enc_run(gpu_lib, case)
    for b in (0, 2):
        assert torch.equal(r1["out"][b], r3["out"][b])
        assert torch.equal(r1["ln_out"][b], r3["ln_out"][b])


def test_encoder_masked_keys_poisoned(gpu_lib):
    case = W.encoder_custom(9, 1, 2, 190, masked_lens=[150])
    _say("[encoder] masked-key poisoning")
    r1 = _enc_run(gpu_lib, case, with_ln=False)
    case.k[:, :, 150:] = float("nan")
    case.v[:, :, 150:] = float("inf")
    r2 = _enc_run(gpu_lib, case, with_ln=False)
    assert torch.equal(r1["out"], r2["out"])


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1e-3, 2.5])
def test_encoder_scale_sign_and_magnitude(gpu_lib, scale):
    case = W.encoder_custom(10, 2, 2, 160, masked_lens=[160, 97], scale=scale)
    _say(f"[encoder] softmax_scale={scale}")
    r = _enc_run(gpu_lib, case, with_ln=False, lse=True)
    ref, lse = oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask, return_lse=True)
    assert_close(r["out"], ref, f"scale {scale}")
    assert metrics(r["lse"], lse)["max_abs"] < LSE_ABS
    nomask = W.encoder_custom(10, 2, 2, 160, scale=scale)
    r = _enc_run(gpu_lib, nomask, with_ln=False)
    assert_close(r["out"], oracle.sdpa(nomask.q, nomask.k, nomask.v, nomask.scale), f"scale {scale}, no mask")


def test_encoder_one_hot_selects_value_row(gpu_lib):
    # q = 8000 e_t, k_{j*} = e_t, other keys orthogonal to e_t, scale 1/8 -> s_{j*} = 1000
    S, D, t, jstar = 70, 64, 5, 41
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, 1, S, D, generator=g)
    k[..., t] = 0
    k[0, 0, jstar] = 0
    k[0, 0, jstar, t] = 1
    q = torch.zeros(1, 1, S, D)
    q[..., t] = 8000.0
    v = torch.randn(1, 1, S, D, generator=g)
    case = W.EncoderCase("onehot", 1, 1, S, D, 0.125, 1e-6, q.bfloat16(), k.bfloat16(), v.bfloat16(),
                         torch.zeros(1, S, D), None, None)
    r = _enc_run(gpu_lib, case, with_ln=False)
    want = v.bfloat16()[0, 0, jstar].float()
    assert torch.equal(r["out"][0, 0].float().cpu(), want.expand(S, D))


# ----------------------------------------------------------------------------- res_ln


@pytest.mark.parametrize("rows,hidden,xdt,affine,ydt", [
    (777, 1024, torch.bfloat16, True, torch.bfloat16),
    (64, 128, torch.float32, False, torch.float32),
    (5, 4104, None, True, torch.float32),
])
def test_res_ln_standalone(gpu_lib, rows, hidden, xdt, affine, ydt):
    _say(f"[res_ln] rows={rows} hidden={hidden} x={xdt}")
    g = torch.Generator().manual_seed(rows + hidden)
    res = torch.randn(rows, hidden, generator=g) * 2 + 0.5
    x = None if xdt is None else torch.randn(rows, hidden, generator=g).to(xdt)
    gamma = torch.rand(hidden, generator=g) + 0.5 if affine else None
    beta = torch.randn(hidden, generator=g) * 0.3 if affine else None
    dev = lambda t: None if t is None else t.to(DEV)
    res_out = torch.empty(rows, hidden, device=DEV)
    mean = torch.empty(rows, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    y = gpu_lib.res_ln(dev(res), dev(x), dev(gamma), dev(beta), 1e-6, residual_out=res_out, y_dtype=ydt,
                       mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    xin = res.double().numpy() + (0 if x is None else to64(x))
    assert np.array_equal(to64(res_out), (res + (0 if x is None else x.float())).double().numpy())
    yref, _, _ = oracle.layernorm(xin, gamma, beta, 1e-6)
    assert_close(y, yref, "res_ln y")
    assert_ln_stats(res_out, mean, rstd, gamma, beta, 1e-6, "res_ln")


# ----------------------------------------------------------------------------- decode


def _dec_run(taa, case, mask=True):
    dev = lambda t: t.to(DEV)
    out = taa.attn_decode_gqa(dev(case.q), dev(case.k), dev(case.v), dev(case.mask) if mask else None, case.scale,
                              case.G)
    torch.cuda.synchronize()
    return out


def _dec_check(taa, case, what, mask=True):
    _say(f"[decode] {what}: B={case.B} Hq={case.Hq} Hkv={case.Hkv} S_ctx={case.S_ctx} lens={case.lens.tolist()}")
    out = _dec_run(taa, case, mask)
    ref = oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask if mask else None)
    return assert_close(out, ref, what), out


def test_decode_gemma_full(gpu_lib):
    _dec_check(gpu_lib, W.decode_gemma(), "Gemma d256 B8 ctx4096")


@pytest.mark.parametrize("B,Hq,Hkv,S,lens", [
    (4, 16, 8, 4096, [1, 4096, 128, 129]),
    (2, 4, 4, 1000, [999, 1]),
    (3, 32, 8, 700, [700, 384, 17]),
    (2, 16, 2, 2048, [2048, 1500]),
])
def test_decode_edge_cases(gpu_lib, B, Hq, Hkv, S, lens):
    _dec_check(gpu_lib, W.decode_gemma(40 + S, B, Hq, Hkv, S, lens=lens), f"edge G={Hq // Hkv}")


def test_decode_without_mask(gpu_lib):
    case = W.decode_gemma(41, 2, 8, 4, 640)
    _dec_check(gpu_lib, case, "no mask", mask=False)


def test_decode_masked_kv_poison_and_determinism(gpu_lib):
    case = W.decode_gemma(42, 3, 16, 8, 1024, lens=[1024, 333, 2])
    o1 = _dec_run(gpu_lib, case)
    o2 = _dec_run(gpu_lib, case)
    assert torch.equal(o1, o2)
    for b, n in enumerate(case.lens.tolist()):
        case.k[b, :, n:] = float("nan")
        case.v[b, :, n:] = float("inf")
    o3 = _dec_run(gpu_lib, case)
    assert torch.equal(o1, o3)


def test_decode_single_key_returns_value(gpu_lib):
    case = W.decode_gemma(43, 2, 4, 2, 256, lens=[1, 1])
    out = _dec_run(gpu_lib, case)
    want = case.v[:, :, :1].repeat_interleave(2, dim=1)
    assert torch.equal(out.cpu(), want)


# ----------------------------------------------------------------------------- prefill


def _pre_run(taa, case, want_lse=False):
    dev = lambda t: t.to(DEV)
    r = taa.attn_prefill_paged(dev(case.q), dev(case.k_cache), dev(case.v_cache), case.k_scale, case.v_scale,
                               dev(case.block_table), case.L_act, case.scale, case.G, want_lse=want_lse)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("Hq,Hkv,Lq,nb,bs,L", [
    (4, 2, 100, 10, 64, 333),
    (8, 1, 37, 6, 128, 700),
    (16, 2, 64, 8, 512, 4096),
    (6, 3, 260, 5, 64, 1),
])
def test_prefill_small_full_check(gpu_lib, Hq, Hkv, Lq, nb, bs, L):
    case = W.prefill_paged(50 + Lq, Hq, Hkv, Lq, 256, nb, bs, L, n_rows=Lq)
    _say(f"[prefill] Hq={Hq} Hkv={Hkv} Lq={Lq} blocks={nb}x{bs} L_act={L}")
    out, lse = _pre_run(gpu_lib, case, want_lse=True)
    rows = torch.arange(Lq)
    ref, rlse = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                                     case.block_table, case.L_act, case.scale, rows, return_lse=True)
    assert_close(out, ref, "prefill out")
    assert metrics(lse, rlse)["max_abs"] < LSE_ABS


def test_prefill_full_config_sampled_rows(gpu_lib):
    # all 256 sampled token positions x all 32 heads (the workload's stated check)
    case = prefill_full.case()
    rows = case.rows
    _say(f"[prefill] full cfg: Lq={case.Lq} Hq={case.Hq} L_act={case.L_act}, checking {len(rows)} tokens x all heads")
    out, lse = _pre_run(gpu_lib, case, want_lse=True)
    ref, rlse = prefill_full.history_ref()
    r = rows.to(out.device)
    assert_close(out[:, r], ref, "prefill full (256 sampled rows)")
    assert metrics(lse[:, r], rlse)["max_abs"] < LSE_ABS
    o2 = _pre_run(gpu_lib, case)
    assert torch.equal(out, o2)


@pytest.mark.parametrize("scale", [-0.05, 0.0])
def test_prefill_scale_sign(gpu_lib, scale):
    case = W.prefill_paged(61, 4, 2, 50, 256, 4, 64, 210, n_rows=50, scale=scale)
    out = _pre_run(gpu_lib, case)
    ref = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table,
                               case.L_act, case.scale, torch.arange(case.Lq))
    assert_close(out, ref, f"prefill scale {scale}")


def test_prefill_poisoned_tail_ignored(gpu_lib):
    case = W.prefill_paged(60, 8, 2, 70, 256, 6, 64, 200)
    out1 = _pre_run(gpu_lib, case)
    nan = torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)
    bt = case.block_table.tolist()
    last = bt[case.L_act // case.block_size]
    case.k_cache[last, :, case.L_act % case.block_size:] = nan
    case.v_cache[last, :, case.L_act % case.block_size:] = nan
    for i in range(case.L_act // case.block_size + 1, len(bt)):
        case.k_cache[bt[i]] = nan
        case.v_cache[bt[i]] = nan
    out2 = _pre_run(gpu_lib, case)
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("token_major", [False, True])
def test_encoder_fp32_outputs(gpu_lib, token_major):
    """out and ln_out in fp32 (out_dtype / ln_dtype ATTN_F32), the attention
    output head-major or token-major by strides."""
    case = W.encoder_custom(21, 2, 4, 300, masked_lens=None)
    d = lambda t: None if t is None else t.to(DEV)
    B, H, S, D = case.B, case.H, case.S, case.D
    out = (torch.empty(B, S, H, D, device=DEV).permute(0, 2, 1, 3) if token_major
           else torch.empty(B, H, S, D, device=DEV))
    _say(f"[encoder] fp32 out and ln_out, token_major={token_major}")
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None, out=out,
                                 residual=d(case.residual), gamma=d(case.gamma), beta=d(case.beta), eps=case.eps,
                                 ln_dtype=torch.float32)
    torch.cuda.synchronize()
    assert r["out"].dtype == torch.float32 and r["ln_out"].dtype == torch.float32
    ref = oracle.encoder_block(case.q, case.k, case.v, case.scale, case.residual, case.gamma, case.beta, case.eps)
    assert_close(r["out"], ref["attn"], "fp32 out")
    assert_close(r["residual_out"], ref["res_out"], "fp32 out residual_out")
    assert_close(r["ln_out"], ref["ln_out"], "fp32 ln_out")
    # the fp32 output is the attention before its bf16 rounding: the bf16 call's output is its rounding
    rb = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None, want_ln=False)
    torch.cuda.synchronize()
    assert torch.equal(rb["out"], r["out"].to(torch.bfloat16))
