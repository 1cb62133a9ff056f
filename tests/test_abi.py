"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, maps one HIP runtime, and rejects bad arguments on the host
before any launch.  Every call below fails validation, so nothing is launched.
"""
import ctypes
import os
import re

import pytest
import torch

import transformer_attention_attn_amd as taa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355attn.h")

BAD = 0x1001          # misaligned fake device address (never dereferenced: validation rejects first)
FAKE = 0x100000       # 16-byte-aligned fake address, only used where another argument is invalid


def _declared_functions():
    text = open(HEADER).read()
    text = text.split("extern \"C\" {", 1)[1]
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return taa.load()


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("attn_encoder_fwd", "attn_decode_gqa", "attn_prefill_paged", "res_ln",
              "attn_decode_gqa_workspace_size", "attn_decode_gqa_window", "attn_decode_gqa_window_workspace_size",
              "attn_prefill_paged_causal", "attn_prefill_paged_causal_workspace_size",
              "attn_prefill_paged_expanded", "attn_prefill_paged_expanded_workspace_size",
              "attn_prefill_paged_causal_expanded", "attn_prefill_paged_causal_expanded_workspace_size",
              "attn_encoder_rope_workspace_size", "attn_status_string", "attn_version", "attn_decode_gqa_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_single_hip_runtime_mapped(lib):
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    real = {os.path.realpath(p) for p in paths}
    assert len(real) == 1, real


def test_status_strings(lib):
    for s in range(5):
        assert taa.attn_status_string(s).startswith(("ATTN_OK", "ATTN_ERR"))
    assert taa.attn_status_string(99) == "unknown attn status"
    assert taa.attn_version() == 10400


def _enc(**kw):
    a = taa.EncoderArgs()
    a.q, a.k, a.v = FAKE, FAKE, FAKE
    a.in_dtype = taa.ATTN_BF16
    a.B, a.H, a.S_q, a.S_kv, a.D = 1, 2, 128, 128, 64
    for i, s in enumerate((2 * 128 * 64, 128 * 64, 64, 1)):
        a.q_stride[i] = a.k_stride[i] = a.v_stride[i] = a.out_stride[i] = s
    a.softmax_scale = 0.125
    a.out = FAKE
    a.out_dtype = taa.ATTN_BF16
    for k, v in kw.items():
        if k.endswith("_stride"):
            for i, s in enumerate(v):
                getattr(a, k)[i] = s
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(B=0), taa.ATTN_ERR_INVALID_ARG),
    (dict(S_kv=-1), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(in_dtype=taa.ATTN_FP8_E4M3FN), taa.ATTN_ERR_UNSUPPORTED),
    (dict(q=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(k_stride=(0, 0, 64, 2)), taa.ATTN_ERR_INVALID_ARG),
    (dict(v_stride=(0, 0, 60, 1)), taa.ATTN_ERR_INVALID_ARG),
    (dict(out=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(residual=FAKE), taa.ATTN_ERR_INVALID_ARG),           # residual without residual_out
    (dict(ln_out=FAKE), taa.ATTN_ERR_INVALID_ARG),             # LayerNorm needs the residual stream
    (dict(rope=3), taa.ATTN_ERR_UNSUPPORTED),                  # no such pairing
    (dict(rope=1), taa.ATTN_ERR_INVALID_ARG),                  # pairing without tables
    (dict(rope=2, rope_cos=FAKE), taa.ATTN_ERR_INVALID_ARG),   # sin table missing
    (dict(rope=1, rope_cos=FAKE, rope_sin=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(rope=1, rope_cos=FAKE, rope_sin=FAKE, rope_stride_b=-4), taa.ATTN_ERR_INVALID_ARG),
    (dict(rope=2, rope_cos=FAKE, rope_sin=FAKE, rope_stride_b=6), taa.ATTN_ERR_INVALID_ARG),  # 16-byte rows
    (dict(rope=1, rope_cos=FAKE, rope_sin=FAKE), taa.ATTN_ERR_WORKSPACE),                    # no K workspace
    (dict(rope=2, rope_cos=FAKE, rope_sin=FAKE, rope_workspace=FAKE, rope_workspace_bytes=100),
     taa.ATTN_ERR_WORKSPACE),
    (dict(rope=2, rope_cos=FAKE, rope_sin=FAKE, rope_workspace=FAKE + 16, rope_workspace_bytes=1 << 30),
     taa.ATTN_ERR_INVALID_ARG),                                                             # 256-byte alignment
    (dict(softmax_scale=float("nan")), taa.ATTN_ERR_INVALID_ARG),
    (dict(key_len=FAKE, mask=FAKE), taa.ATTN_ERR_INVALID_ARG),   # key lengths replace the mask
    (dict(key_len=FAKE + 2), taa.ATTN_ERR_INVALID_ARG),          # 4-byte alignment
    (dict(out_dtype=taa.ATTN_FP8_E4M3FN), taa.ATTN_ERR_UNSUPPORTED),
])
def test_encoder_validation(lib, kw, expect):
    a = _enc(**kw)
    assert lib.attn_encoder_fwd(ctypes.byref(a), None) == expect
    assert lib.attn_encoder_fwd(None, None) == taa.ATTN_ERR_INVALID_ARG


def _dec(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, mask=None, scale=1.0, G=2, B=8, Hq=16, Hkv=8, S=4096, D=256,
                out=FAKE, ws=None, wsb=0)
    args.update(kw)
    return (args["q"], args["k"], args["v"], args["mask"], args["scale"], args["G"], args["B"], args["Hq"],
            args["Hkv"], args["S"], args["D"], args["out"], args["ws"], args["wsb"], None)


def test_decode_workspace_size(lib):
    n = taa.attn_decode_gqa_workspace_size(8, 16, 4096, 256)
    chunks = 4096 // 128
    assert n >= 8 * 16 * chunks * (256 + 2) * 4
    assert taa.attn_decode_gqa_workspace_size(0, 16, 4096, 256) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(Hq=15), taa.ATTN_ERR_INVALID_ARG),                   # Hq != Hkv * G
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(D=512), taa.ATTN_ERR_WORKSPACE),                     # head_dim 512 passes the shape checks
    (dict(G=16, Hq=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(G=3, Hq=24), taa.ATTN_ERR_UNSUPPORTED),
    (dict(k=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(), taa.ATTN_ERR_WORKSPACE),                          # no workspace
    (dict(ws=FAKE, wsb=100), taa.ATTN_ERR_WORKSPACE),          # too small
    (dict(ws=FAKE + 16, wsb=1 << 30), taa.ATTN_ERR_INVALID_ARG),  # misaligned workspace
    (dict(scale=float("inf")), taa.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), taa.ATTN_ERR_INVALID_ARG),
])
def test_decode_validation(lib, kw, expect):
    assert lib.attn_decode_gqa(*_dec(**kw)) == expect


def _win(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, mask=None, kb=FAKE, ke=FAKE, W=1024, scale=1.0, G=2, B=8, Hq=16, Hkv=8, S=4096,
             D=256, out=FAKE, ws=None, wsb=0)
    a.update(kw)
    return (a["q"], a["k"], a["v"], a["mask"], a["kb"], a["ke"], a["W"], a["scale"], a["G"], a["B"], a["Hq"],
            a["Hkv"], a["S"], a["D"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("S,W,chunks", [
    (4096, 1024, 17),   # a 1024-key window starting anywhere touches at most 17 chunks of 64
    (4096, 64, 2),
    (4096, 1, 2),
    (4096, 4096, 64),   # never more chunks than the cache holds
    (4096, 100000, 64),
    (100, 50, 2),
    (100, 64, 2),
])
def test_window_workspace_size(S, W, chunks):
    n = taa.attn_decode_gqa_window_workspace_size(2, 4, S, W, 512)
    parts = 2 * 4 * chunks
    assert n == (parts * 512 * 4 + 255) // 256 * 256 + parts * 2 * 4
    assert taa.attn_decode_gqa_window_workspace_size(2, 4, S, 0, 512) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(W=0), taa.ATTN_ERR_INVALID_ARG),
    (dict(W=-5), taa.ATTN_ERR_INVALID_ARG),
    (dict(kb=FAKE + 2), taa.ATTN_ERR_INVALID_ARG),             # int32 arrays need 4-byte alignment
    (dict(ke=FAKE + 1), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(Hq=15), taa.ATTN_ERR_INVALID_ARG),
    (dict(), taa.ATTN_ERR_WORKSPACE),
    (dict(kb=None, ke=None, D=512), taa.ATTN_ERR_WORKSPACE),  # both ranges optional
    (dict(ws=FAKE, wsb=100), taa.ATTN_ERR_WORKSPACE),
    (dict(scale=float("nan")), taa.ATTN_ERR_INVALID_ARG),
])
def test_window_validation(lib, kw, expect):
    assert lib.attn_decode_gqa_window(*_win(**kw)) == expect


def _pre(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=1.0, vs=1.0, bt=FAKE, maxb=256, nb=256, bs=512, L=120000, scale=0.0625,
             G=16, Hq=32, Hkv=2, Lq=4096, D=256, out=FAKE, lse=None)
    a.update(kw)
    return (a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["maxb"], a["nb"], a["bs"], a["L"], a["scale"],
            a["G"], a["Hq"], a["Hkv"], a["Lq"], a["D"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(bt=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=0), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=256 * 512 + 1), taa.ATTN_ERR_INVALID_ARG),
    (dict(Hq=31), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(bs=100, L=1000), taa.ATTN_ERR_UNSUPPORTED),
    (dict(ks=0.0), taa.ATTN_ERR_INVALID_ARG),
    (dict(ks=float("nan")), taa.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), taa.ATTN_ERR_INVALID_ARG),
    (dict(out=BAD), taa.ATTN_ERR_INVALID_ARG),
])
def test_prefill_validation(lib, kw, expect):
    assert lib.attn_prefill_paged(*_pre(**kw)) == expect


def _pex(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=1.0, vs=1.0, bt=FAKE, maxb=256, nb=256, bs=512, L=120000, scale=0.0625,
             G=16, Hq=32, Hkv=2, Lq=4096, D=256, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return (a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["maxb"], a["nb"], a["bs"], a["L"], a["scale"],
            a["G"], a["Hq"], a["Hkv"], a["Lq"], a["D"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(bt=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=0), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=256 * 512 + 1), taa.ATTN_ERR_INVALID_ARG),
    (dict(Hq=31), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(ks=0.0), taa.ATTN_ERR_INVALID_ARG),
    (dict(out=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), taa.ATTN_ERR_WORKSPACE),
    (dict(wsb=2 * 3750 * 32768 - 1), taa.ATTN_ERR_WORKSPACE),   # one byte short of the live history's tiles
    (dict(ws=FAKE + 16), taa.ATTN_ERR_INVALID_ARG),             # workspace must be 256-byte aligned
])
def test_prefill_expanded_validation(lib, kw, expect):
    assert lib.attn_prefill_paged_expanded(*_pex(**kw)) == expect


def test_prefill_causal_expanded_workspace_size():
    # the causal hand-off state (rounded up to 256 bytes), then the history's tile images, then the
    # current tokens' (32768 bytes per KV head and 32 keys each)
    hand = 32 * 4096 * 256 * 4 + 32 * 4096 * 4
    assert taa.attn_prefill_paged_causal_expanded_workspace_size(32, 2, 4096, 120000, 256) == \
        hand + 2 * 3750 * 32768 + 2 * 128 * 32768
    hand = (6 * 100 * 256 * 4 + 6 * 100 * 4 + 255) // 256 * 256  # 616800 bytes, rounded up to 616960
    assert hand == 616960
    cur = 2 * 4 * 32768  # ceil(100 / 32) tiles per KV head
    assert taa.attn_prefill_paged_causal_expanded_workspace_size(6, 2, 100, 33, 256) == hand + 2 * 2 * 32768 + cur
    assert taa.attn_prefill_paged_causal_expanded_workspace_size(6, 2, 100, 0, 256) == hand + cur  # no history
    assert taa.attn_prefill_paged_causal_expanded_workspace_size(6, 4, 100, 33, 256) == 0
    assert taa.attn_prefill_paged_causal_expanded_workspace_size(6, 2, 100, 33, 128) == 0


def test_prefill_expanded_workspace_size():
    # per KV head, one 32768-byte image (16 KiB of K, 16 KiB of V^T) per 32 live keys
    assert taa.attn_prefill_paged_expanded_workspace_size(2, 120000, 256) == 2 * 3750 * 32768
    assert taa.attn_prefill_paged_expanded_workspace_size(3, 33, 256) == 3 * 2 * 32768
    assert taa.attn_prefill_paged_expanded_workspace_size(1, 1, 256) == 32768
    assert taa.attn_prefill_paged_expanded_workspace_size(2, 0, 256) == 0
    assert taa.attn_prefill_paged_expanded_workspace_size(2, 100, 128) == 0


def _prc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=1.0, vs=1.0, bt=FAKE, maxb=256, nb=256, bs=512, L=120000, kc=FAKE, vc=FAKE,
             scale=0.0625, G=16, Hq=32, Hkv=2, Lq=4096, D=256, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return (a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["maxb"], a["nb"], a["bs"], a["L"], a["kc"],
            a["vc"], a["scale"], a["G"], a["Hq"], a["Hkv"], a["Lq"], a["D"], a["out"], a["lse"], a["ws"], a["wsb"],
            None)


@pytest.mark.parametrize("kw,expect", [
    (dict(kc=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(vc=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(kc=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=-1), taa.ATTN_ERR_INVALID_ARG),
    (dict(L=256 * 512 + 1), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(Hq=31), taa.ATTN_ERR_INVALID_ARG),
    (dict(vs=float("inf")), taa.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), taa.ATTN_ERR_WORKSPACE),
    (dict(wsb=1000), taa.ATTN_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), taa.ATTN_ERR_INVALID_ARG),             # workspace must be 256-byte aligned
])
def test_prefill_causal_validation(lib, kw, expect):
    assert lib.attn_prefill_paged_causal(*_prc(**kw)) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, None, 0, None, None, 1e-6, 4, 64, None, FAKE, 1, None, None, None), taa.ATTN_ERR_INVALID_ARG),
    ((FAKE, None, 0, None, None, 1e-6, 4, 60, None, FAKE, 1, None, None, None), taa.ATTN_ERR_INVALID_ARG),
    ((FAKE, None, 0, None, None, 1e-6, 4, 16384, None, FAKE, 1, None, None, None), taa.ATTN_ERR_UNSUPPORTED),
    ((FAKE, None, 0, None, None, 1e-6, 4, 64, None, FAKE, 2, None, None, None), taa.ATTN_ERR_UNSUPPORTED),
    ((FAKE, None, 0, None, None, -1.0, 4, 64, None, FAKE, 1, None, None, None), taa.ATTN_ERR_INVALID_ARG),
    ((FAKE, None, 0, None, None, float("nan"), 4, 64, None, FAKE, 1, None, None, None), taa.ATTN_ERR_INVALID_ARG),
    ((FAKE, None, 0, None, None, 1e-6, 4, 64, None, BAD, 1, None, None, None), taa.ATTN_ERR_INVALID_ARG),
])
def test_res_ln_validation(lib, args, expect):
    assert lib.res_ln(*args, None) == expect


def test_binding_raises_instead_of_falling_back():
    with pytest.raises(ValueError):
        taa.attn_decode_gqa(torch.zeros(1, 2, 1, 256), torch.zeros(1, 1, 8, 256), torch.zeros(1, 1, 8, 256), None,
                            1.0, 2)


def test_prefill_causal_workspace_size():
    # fp32 history output [Hq*Lq, D] (rounded up to 256 bytes), then its lse per row
    n = taa.attn_prefill_paged_causal_workspace_size(32, 2, 4096, 256)
    assert n == 32 * 4096 * 256 * 4 + 32 * 4096 * 4
    assert taa.attn_prefill_paged_causal_workspace_size(6, 2, 100, 256) == 6 * 100 * 256 * 4 + 6 * 100 * 4
    assert taa.attn_prefill_paged_causal_workspace_size(1, 1, 3, 256) == 3 * 256 * 4 + 3 * 4
    assert taa.attn_prefill_paged_causal_workspace_size(6, 4, 100, 256) == 0  # Hq not a multiple of Hkv


def test_encoder_rope_workspace_size():
    assert taa.attn_encoder_rope_workspace_size(1, 16, 2048, 64) == 16 * 2048 * 64 * 2
    assert taa.attn_encoder_rope_workspace_size(2, 3, 100, 64, torch.float32) == 2 * 3 * 100 * 64 * 4
    assert taa.attn_encoder_rope_workspace_size(0, 3, 100, 64) == 0


def _dec_na(**kw):
    a = _dec(**kw)
    return a[:12] + (None,)  # no workspace arguments


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(out=None), taa.ATTN_ERR_INVALID_ARG),
    (dict(Hq=15), taa.ATTN_ERR_INVALID_ARG),
    (dict(D=128), taa.ATTN_ERR_UNSUPPORTED),
    (dict(G=3, Hq=24), taa.ATTN_ERR_UNSUPPORTED),
    (dict(k=BAD), taa.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), taa.ATTN_ERR_INVALID_ARG),
    # partials beyond the library's scratch: 8 x 64 heads x 64 chunks x (512 + 2) x 4 B = 67 MB
    (dict(D=512, Hq=64, Hkv=8, G=8), taa.ATTN_ERR_WORKSPACE),
    (dict(S=131072), taa.ATTN_ERR_WORKSPACE),
])
def test_decode_noalloc_validation(lib, kw, expect):
    """Every argument is checked, and the scratch limit enforced, before the
    device is touched (these calls run without a GPU)."""
    assert lib.attn_decode_gqa_noalloc(*_dec_na(**kw)) == expect


def test_decode_noalloc_limit_matches_the_header(lib):
    text = open(HEADER).read()
    assert "#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text
    assert taa.DECODE_NOALLOC_SCRATCH_BYTES == 32 << 20
    # the bench's decode (8 x 16 heads, 4096 keys, D 256) and the D 512 one fit
    assert taa.attn_decode_gqa_workspace_size(8, 16, 4096, 256) <= taa.DECODE_NOALLOC_SCRATCH_BYTES
    assert taa.attn_decode_gqa_workspace_size(8, 16, 4096, 512) <= taa.DECODE_NOALLOC_SCRATCH_BYTES
