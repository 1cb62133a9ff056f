"""The Python binding rejects tensors whose shape, dtype or layout differ from
what the kernels read and write, before any device work (CPU tier: the checks
run before the device check, on CPU tensors, so no GPU and no library call is
needed).  Each case changes one argument of an otherwise valid call."""
import pytest
import torch

import transformer_attention_attn_amd as taa

bf, f32, f8 = torch.bfloat16, torch.float32, torch.float8_e4m3fn


def _enc(**over):
    B, H, S, D = 2, 4, 40, 64
    kw = dict(q=torch.zeros(B, H, S, D, dtype=bf), k=torch.zeros(B, H, S, D, dtype=bf),
              v=torch.zeros(B, H, S, D, dtype=bf), softmax_scale=0.125)
    kw.update(over)
    return kw


def _call_enc(**over):
    kw = _enc(**over)
    return taa.attn_encoder_fwd(kw.pop("q"), kw.pop("k"), kw.pop("v"), kw.pop("softmax_scale"), **kw)


def test_encoder_valid_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        _call_enc(mask=torch.zeros(2, 1, 1, 40), residual=torch.zeros(2, 40, 256))
    with pytest.raises(ValueError, match="on the GPU"):  # one mask row for the whole batch
        _call_enc(mask=torch.zeros(1, 1, 1, 40))


@pytest.mark.parametrize("over,msg", [
    (dict(k=torch.zeros(2, 4, 40, 32, dtype=bf)), "k must have shape"),
    (dict(v=torch.zeros(2, 4, 39, 64, dtype=bf)), "v must have shape"),
    (dict(k=torch.zeros(1, 4, 40, 64, dtype=bf)), "k must have shape"),
    (dict(k=torch.zeros(2, 4, 40, 64, dtype=f32)), "share a dtype"),
    (dict(mask=torch.zeros(3, 1, 1, 40)), "mask must be"),
    (dict(mask=torch.zeros(2, 1, 1, 41)), "mask must be"),
    (dict(mask=torch.zeros(2, 1, 1, 40, dtype=bf)), "mask must be"),
    (dict(mask=torch.zeros(2, 1, 40)), "mask must be"),
    (dict(out=torch.zeros(2, 4, 40, 32, dtype=bf)), "out must have shape"),
    (dict(out=torch.zeros(2, 4, 40, 64, dtype=f8)), "out must be"),
    (dict(lse=torch.zeros(2, 4, 39)), "lse must have shape"),
    (dict(residual=torch.zeros(2, 40, 255)), "residual must hold"),
    (dict(residual=torch.zeros(2, 40, 256, dtype=bf)), "residual must be"),
    (dict(residual=torch.zeros(2, 40, 256), residual_out=torch.zeros(2, 40, 128)), "residual_out must hold"),
    (dict(residual_out=torch.zeros(2, 40, 256)), "residual_out needs residual"),
    (dict(residual=torch.zeros(2, 40, 256), gamma=torch.zeros(255)), "gamma must hold"),
    (dict(residual=torch.zeros(2, 40, 256), beta=torch.zeros(256, dtype=bf)), "beta must be"),
    (dict(residual=torch.zeros(2, 40, 256), ln_out=torch.zeros(2, 40, 250, dtype=bf)), "ln_out must hold"),
    (dict(residual=torch.zeros(2, 40, 256), ln_out=torch.zeros(2, 40, 256, dtype=bf),
          ln_mean=torch.zeros(79)), "ln_mean must hold"),
    (dict(residual=torch.zeros(2, 40, 256), ln_out=torch.zeros(2, 40, 256, dtype=bf),
          ln_rstd=torch.zeros(80, dtype=bf)), "ln_rstd must be"),
    (dict(rope="sideways"), "rope must be one of"),
    (dict(rope="half", rope_cos=torch.zeros(40, 32), rope_sin=torch.zeros(40, 31)), "rope_sin must be"),
    (dict(rope="half", rope_cos=torch.zeros(30, 32), rope_sin=torch.zeros(30, 32)), "needs at least"),
    (dict(rope="half", rope_cos=torch.zeros(3, 40, 32), rope_sin=torch.zeros(3, 40, 32)), "rope_cos must be"),
])
def test_encoder_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        _call_enc(**over)


def _dec(**over):
    B, Hq, Hkv, S, D = 3, 8, 4, 100, 256
    kw = dict(q=torch.zeros(B, Hq, 1, D, dtype=bf), k=torch.zeros(B, Hkv, S, D, dtype=bf),
              v=torch.zeros(B, Hkv, S, D, dtype=bf), attn_mask=torch.zeros(B, 1, 1, S))
    kw.update(over)
    return kw


def test_decode_valid_shapes_reach_the_device_check():
    kw = _dec()
    with pytest.raises(ValueError, match="on the GPU"):
        taa.attn_decode_gqa(kw["q"], kw["k"], kw["v"], kw["attn_mask"], 1.0, 2)


@pytest.mark.parametrize("over,msg", [
    (dict(attn_mask=torch.zeros(1, 1, 1, 100)), "attn_mask must have shape"),
    (dict(attn_mask=torch.zeros(3, 1, 1, 99)), "attn_mask must have shape"),
    (dict(attn_mask=torch.zeros(3, 1, 1, 100, dtype=bf)), "attn_mask must be"),
    (dict(attn_mask=torch.zeros(3, 1, 1, 200)[..., ::2]), "attn_mask must be contiguous"),
    (dict(k=torch.zeros(3, 4, 100, 128, dtype=bf)), "k must have shape"),
    (dict(v=torch.zeros(3, 4, 99, 256, dtype=bf)), "v must have shape"),
    (dict(k=torch.zeros(2, 4, 100, 256, dtype=bf)), "k must have shape"),
    (dict(q=torch.zeros(3, 8, 2, 256, dtype=bf)), r"q must be \[B, Hq, 1, D\]"),
    (dict(q=torch.zeros(3, 8, 1, 256)), "q must be"),
    (dict(k=torch.zeros(3, 4, 100, 256)), "k must be"),
])
def test_decode_rejects(over, msg):
    kw = _dec(**over)
    with pytest.raises(ValueError, match=msg):
        taa.attn_decode_gqa(kw["q"], kw["k"], kw["v"], kw["attn_mask"], 1.0, 2)


@pytest.mark.parametrize("out,msg", [
    (torch.zeros(3, 8, 1, 128, dtype=bf), "out must have shape"),
    (torch.zeros(3, 8, 1, 256), "out must be"),
])
def test_decode_rejects_out(out, msg):
    kw = _dec()
    with pytest.raises(ValueError, match=msg):
        taa.attn_decode_gqa(kw["q"], kw["k"], kw["v"], kw["attn_mask"], 1.0, 2, out=out)


def test_decode_window_rejects_ranges():
    kw = _dec()
    with pytest.raises(ValueError, match="key_begin must be"):
        taa.attn_decode_gqa_window(kw["q"], kw["k"], kw["v"], None, torch.zeros(2, dtype=torch.int32), None, 64,
                                   1.0, 2)
    with pytest.raises(ValueError, match="key_end must be"):
        taa.attn_decode_gqa_window(kw["q"], kw["k"], kw["v"], None, None, torch.zeros(3, dtype=torch.int64), 64,
                                   1.0, 2)
    with pytest.raises(ValueError, match="attn_mask must have shape"):
        taa.attn_decode_gqa_window(kw["q"], kw["k"], kw["v"], torch.zeros(3, 1, 1, 5), None, None, 64, 1.0, 2)


def _pre(**over):
    Hq, Hkv, Lq, D, nb, bs = 8, 2, 50, 256, 4, 64
    kw = dict(q=torch.zeros(Hq, Lq, D, dtype=bf), k=torch.zeros(nb, Hkv, bs, D, dtype=f8),
              v=torch.zeros(nb, Hkv, bs, D, dtype=f8), bt=torch.zeros(nb, dtype=torch.int32))
    kw.update(over)
    return kw


def _call_pre(fn, out=None, lse=None, **over):
    kw = _pre(**over)
    return fn(kw["q"], kw["k"], kw["v"], 1.0, 1.0, kw["bt"], 100, 0.0625, 4, out=out, lse=lse)


@pytest.mark.parametrize("fn", [taa.attn_prefill_paged, taa.attn_prefill_paged_expanded])
def test_prefill_valid_shapes_reach_the_device_check(fn):
    with pytest.raises(ValueError, match="on the GPU"):
        _call_pre(fn)


@pytest.mark.parametrize("fn", [taa.attn_prefill_paged, taa.attn_prefill_paged_expanded])
@pytest.mark.parametrize("over,msg", [
    (dict(v=torch.zeros(4, 2, 32, 256, dtype=f8)), "v_cache must have shape"),
    (dict(k=torch.zeros(4, 2, 64, 128, dtype=f8), v=torch.zeros(4, 2, 64, 128, dtype=f8)), "share head_dim"),
    (dict(q=torch.zeros(8, 50, 256)), "q must be"),
    (dict(k=torch.zeros(4, 2, 64, 256, dtype=bf)), "k_cache must be"),
    (dict(bt=torch.zeros(4, dtype=torch.int64)), "block_table must be"),
    (dict(q=torch.zeros(8, 50, 512, dtype=bf)[..., ::2]), "q must be contiguous"),
    (dict(out=torch.zeros(8, 50, 128, dtype=bf)), "out must have shape"),
    (dict(out=torch.zeros(8, 50, 256)), "out must be"),
    (dict(lse=torch.zeros(8, 49)), "lse must have shape"),
    (dict(lse=torch.zeros(8, 50, dtype=bf)), "lse must be"),
])
def test_prefill_rejects(fn, over, msg):
    with pytest.raises(ValueError, match=msg):
        _call_pre(fn, **over)


@pytest.mark.parametrize("kc,vc,msg", [
    (torch.zeros(2, 49, 256, dtype=bf), torch.zeros(2, 50, 256, dtype=bf), "k_cur must have shape"),
    (torch.zeros(2, 50, 256, dtype=bf), torch.zeros(2, 50, 256), "v_cur must be"),
    (None, torch.zeros(2, 50, 256, dtype=bf), "k_cur and v_cur are required"),
])
def test_prefill_causal_rejects(kc, vc, msg):
    kw = _pre()
    with pytest.raises(ValueError, match=msg):
        taa.attn_prefill_paged_causal(kw["q"], kw["k"], kw["v"], 1.0, 1.0, kw["bt"], 100, kc, vc, 0.0625, 4)


@pytest.mark.parametrize("over,msg", [
    (dict(x=torch.zeros(6, 127)), "x must have shape"),
    (dict(gamma=torch.zeros(127)), "gamma must hold"),
    (dict(beta=torch.zeros(128, dtype=bf)), "beta must be"),
    (dict(residual_out=torch.zeros(5, 128)), "residual_out must hold"),
    (dict(y=torch.zeros(6, 128, dtype=f8)), "y must be"),
    (dict(mean=torch.zeros(5)), "mean must hold"),
    (dict(rstd=torch.zeros(6, dtype=bf)), "rstd must be"),
])
def test_res_ln_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        taa.res_ln(torch.zeros(6, 128), **over)


def test_res_ln_rejects_non_fp32_residual():
    with pytest.raises(ValueError, match="residual must be"):
        taa.res_ln(torch.zeros(6, 128, dtype=bf))
    with pytest.raises(ValueError, match="on the GPU"):
        taa.res_ln(torch.zeros(6, 128), torch.zeros(6, 128, dtype=bf), torch.ones(128), torch.zeros(128))
