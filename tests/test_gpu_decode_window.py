"""Decode at head_dim 512 and over per-sequence key ranges, HIP path vs the
fp64 oracle through the C ABI.

- head_dim 512, the global-layer size of the decode page's introduction, at
  the full Gemma-style decode shape and at every supported group count;
- key ranges (the page's "Future performance follow-on": sliding-window layers
  need only the last window of keys): windows at unaligned starts, ranges cut
  to max_keys, clamped, empty, combined with the additive mask;
- keys outside a range are never read (poisoned with NaN/inf, bit-identical
  output); a range covering the whole cache gives the unranged result bitwise.
"""
import sys

import numpy as np
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


def _i32(x):
    return None if x is None else torch.tensor(x, dtype=torch.int32, device=DEV)


def _full(taa, case, mask=True):
    d = lambda t: t.to(DEV)
    out = taa.attn_decode_gqa(d(case.q), d(case.k), d(case.v), d(case.mask) if mask else None, case.scale, case.G)
    torch.cuda.synchronize()
    return out


def _win(taa, case, beg, end, max_keys, mask=True):
    d = lambda t: t.to(DEV)
    out = taa.attn_decode_gqa_window(d(case.q), d(case.k), d(case.v), d(case.mask) if mask else None, _i32(beg),
                                     _i32(end), max_keys, case.scale, case.G)
    torch.cuda.synchronize()
    return out


def test_decode_d512_full_shape(gpu_lib):
    case = W.decode_gemma(1005, D=512)
    _say(f"[decode-d512] B=8 Hq=16 Hkv=8 S_ctx=4096 lens={case.lens.tolist()}")
    assert_close(_full(gpu_lib, case), oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask), "d512 full")


@pytest.mark.parametrize("B,Hq,Hkv,S,lens", [
    (2, 4, 4, 1000, [999, 1]),        # G=1, ragged tail
    (3, 16, 4, 700, [700, 384, 17]),  # G=4
    (2, 16, 2, 2048, [2048, 1500]),   # G=8 (merge buffer reuses the query/score LDS)
])
def test_decode_d512_groups(gpu_lib, B, Hq, Hkv, S, lens):
    case = W.decode_gemma(50 + S, B, Hq, Hkv, S, D=512, lens=lens)
    _say(f"[decode-d512] G={Hq // Hkv} B={B} S_ctx={S} lens={lens}")
    assert_close(_full(gpu_lib, case), oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask), "d512 groups")


def test_decode_d256_g8_shared_lds(gpu_lib):
    case = W.decode_gemma(60, 2, 32, 4, 1100, lens=[1100, 65])
    _say("[decode] d256 G=8 with the aliased merge buffer")
    assert_close(_full(gpu_lib, case), oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask), "d256 G=8")


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("beg,end,max_keys", [
    ([100, 0, 3000, 17], [1124, 4096, 4000, 18], 1024),   # sliding windows at unaligned starts
    ([0, 0, 0, 0], [4096, 2000, 63, 4096], 63),           # window shorter than one chunk
    ([-50, 4000, 1, 4095], [5000, 4100, 1, 4096], 65),    # clamped ends, an empty range, one key
    (None, [4096, 1, 2049, 3333], 1),                     # one-key windows, default begin
    ([129, 2, 700, 64], None, 4096),                      # default end, window past the cache
])
def test_decode_window_ranges(gpu_lib, D, beg, end, max_keys):
    case = W.decode_gemma(70 + D, 4, 8, 4, 4096, D=D, lens=[4096, 3000, 4096, 2500])
    _say(f"[decode-window] D={D} beg={beg} end={end} max_keys={max_keys}")
    out = _win(gpu_lib, case, beg, end, max_keys)
    ref = oracle.decode_window(case.q, case.k, case.v, case.scale, case.mask, beg, end, max_keys)
    assert_close(out, ref, f"window D={D}")


@pytest.mark.parametrize("D", [256, 512])
def test_decode_window_gemma_sliding(gpu_lib, D):
    """Every sequence attends the last 1024 keys of its own length (G=2, the
    bench shape), no mask."""
    case = W.decode_gemma(80 + D, D=D)
    lens = case.lens.tolist()
    beg, end = [max(n - 1024, 0) for n in lens], lens
    _say(f"[decode-window] sliding 1024 D={D} lens={lens}")
    out = _win(gpu_lib, case, beg, end, 1024, mask=False)
    ref = oracle.decode_window(case.q, case.k, case.v, case.scale, None, beg, end, 1024)
    assert_close(out, ref, f"sliding D={D}")


def test_decode_window_never_reads_outside(gpu_lib):
    case = W.decode_gemma(90, 3, 8, 4, 2048, D=512, lens=[2048, 2048, 2048])
    beg, end, Wk = [500, 0, 1900], [1524, 700, 2048], 1024
    o1 = _win(gpu_lib, case, beg, end, Wk, mask=False)
    for b in range(3):
        s, e = oracle.window_range(2048, 3, beg, end, Wk)[b]
        case.k[b, :, :s] = float("nan")
        case.v[b, :, e:] = float("inf")
        case.k[b, :, e:] = float("nan")
        case.v[b, :, :s] = float("-inf")
    o2 = _win(gpu_lib, case, beg, end, Wk, mask=False)
    assert torch.equal(o1, o2)
    assert torch.isfinite(o1.float()).all()


@pytest.mark.parametrize("D", [256, 512])
def test_decode_window_whole_cache_is_bitwise_unranged(gpu_lib, D):
    case = W.decode_gemma(95 + D, 3, 8, 4, 1000, D=D, lens=[1000, 640, 3])
    o_full = _full(gpu_lib, case)
    o_win = _win(gpu_lib, case, [0, 0, 0], [1000, 1000, 1000], 1000)
    assert torch.equal(o_full, o_win)
    # the lengths as a range instead of a mask: same live keys, same chunks, same bits
    o_len = _win(gpu_lib, case, None, case.lens.tolist(), 1000, mask=False)
    assert torch.equal(o_full, o_len)


def test_decode_window_range_changes_on_device(gpu_lib):
    """One workspace, two calls whose ranges differ only in device memory."""
    taa = gpu_lib
    case = W.decode_gemma(99, 2, 4, 2, 1536, lens=[1536, 1536])
    d = lambda t: t.to(DEV)
    q, k, v = d(case.q), d(case.k), d(case.v)
    ws = torch.zeros(taa.attn_decode_gqa_window_workspace_size(2, 4, 1536, 256, 256), dtype=torch.uint8, device=DEV)
    kb, ke = _i32([0, 0]), _i32([256, 256])
    outs = []
    for rng in (([10, 1000], [266, 1200]), ([1280, 77], [1536, 300])):
        kb.copy_(torch.tensor(rng[0], dtype=torch.int32))
        ke.copy_(torch.tensor(rng[1], dtype=torch.int32))
        o = taa.attn_decode_gqa_window(q, k, v, None, kb, ke, 256, case.scale, case.G, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.clone(), rng))
    for o, (b_, e_) in outs:
        ref = oracle.decode_window(case.q, case.k, case.v, case.scale, None, b_, e_, 256)
        assert_close(o, ref, f"device range {b_}-{e_}")


def test_one_workspace_for_decodes_of_different_shapes(gpu_lib):
    """The workspace's arrival counters sit at a fixed place: calls of
    different shapes (larger, smaller, larger again; plain and windowed)
    share one zero-filled workspace and each matches the oracle."""
    taa = gpu_lib
    big = W.decode_gemma(1530, B=8, Hq=16, Hkv=8, S_ctx=2048)
    small = W.decode_gemma(1531, B=2, Hq=8, Hkv=2, S_ctx=700, lens=[700, 3])
    n = max(taa.attn_decode_gqa_workspace_size(c.B, c.Hq, c.S_ctx, c.D) for c in (big, small))
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    d = lambda t: t.to(DEV)
    for case in (big, small, big):
        _say(f"[decode] shared workspace: B={case.B} Hq={case.Hq} Hkv={case.Hkv} S_ctx={case.S_ctx}")
        out = taa.attn_decode_gqa(d(case.q), d(case.k), d(case.v), d(case.mask), case.scale, case.G, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out, oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask), f"shared ws {case.name}")
    beg, end = [0, 200], [700, 650]
    kb, ke = (torch.tensor(x, dtype=torch.int32, device=DEV) for x in (beg, end))
    out = taa.attn_decode_gqa_window(d(small.q), d(small.k), d(small.v), None, kb, ke, 300, small.scale, small.G,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, oracle.decode_window(small.q, small.k, small.v, small.scale, None, beg, end, 300),
                 "shared ws window")


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("scale", [8.0, -1.5, 0.0])
def test_decode_softmax_scales(gpu_lib, D, scale):
    """Sharp (scores of tens of log2 units, the running max moves between key
    groups and waves), negative and zero (uniform weights) softmax scales at
    two and four query heads per KV head, ragged lengths."""
    for B, Hq, Hkv, S, lens in ((3, 16, 8, 1500, [1500, 700, 65]), (2, 16, 4, 900, [900, 33])):
        case = W.decode_gemma(70 + S, B, Hq, Hkv, S, D=D, lens=lens)
        case.scale = scale
        _say(f"[decode] D={D} scale={scale} G={Hq // Hkv} B={B} S_ctx={S} lens={lens}")
        assert_close(_full(gpu_lib, case), oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask),
                     f"d{D} scale {scale}")


def test_decode_finite_additive_mask(gpu_lib):
    """An additive mask with finite entries (uniform in [-6, 0]) besides the
    -inf of removed keys, at both head sizes."""
    for D in (256, 512):
        case = W.decode_gemma(81, 2, 16, 8, 1200, D=D, lens=[1200, 517])
        g = torch.Generator().manual_seed(82)
        finite = -6.0 * torch.rand(case.mask.shape, generator=g)
        case.mask = torch.where(torch.isinf(case.mask), case.mask, finite)
        _say(f"[decode] D={D} finite additive mask, lens=[1200, 517]")
        assert_close(_full(gpu_lib, case), oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask),
                     f"d{D} finite mask")
