"""The paged prefill through the expanded-history workspace
(attn_prefill_paged_expanded) against the fp64 oracle, and bit for bit against
attn_prefill_paged: both feed the same exactly expanded bf16 values to the
same MFMA sequence, only where the keys sit on chip differs.
"""
import sys

import pytest
import torch

import oracle
import prefill_full
import workloads as W
from parity import LSE_ABS, assert_close, metrics

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(taa, case, want_lse=False, workspace=None):
    d = lambda t: t.to(DEV)
    q, k, v, bt = d(case.q), d(case.k_cache), d(case.v_cache), d(case.block_table)
    args = (q, k, v, case.k_scale, case.v_scale, bt, case.L_act, case.scale, case.G)
    plain = taa.attn_prefill_paged(*args, want_lse=want_lse)
    exp = taa.attn_prefill_paged_expanded(*args, want_lse=want_lse, workspace=workspace)
    torch.cuda.synchronize()
    return plain, exp


@pytest.mark.parametrize("Hq,Hkv,Lq,nb,bs,L", [
    (4, 2, 100, 10, 64, 333),
    (8, 1, 37, 6, 128, 700),
    (16, 2, 64, 8, 512, 4096),
    (6, 3, 260, 5, 64, 1),
    (4, 2, 300, 3, 64, 160),   # five tiles: one pass of the six-step loop, cut short
    (4, 2, 40, 4, 64, 193),    # seven tiles: a second pass, ragged last tile
    (4, 2, 50, 2, 64, 64),     # exactly two tiles
    (4, 2, 70, 3, 64, 90),     # three tiles, ragged last tile
])
def test_expanded_small_full_check(gpu_lib, Hq, Hkv, Lq, nb, bs, L):
    case = W.prefill_paged(150 + Lq, Hq, Hkv, Lq, 256, nb, bs, L, n_rows=Lq)
    _say(f"[expanded] Hq={Hq} Hkv={Hkv} Lq={Lq} blocks={nb}x{bs} L_act={L}")
    (po, pl), (eo, el) = _both(gpu_lib, case, want_lse=True)
    ref, rlse = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                                     case.block_table, case.L_act, case.scale, torch.arange(Lq), return_lse=True)
    assert_close(eo, ref, "expanded prefill out")
    assert metrics(el, rlse)["max_abs"] < LSE_ABS
    assert torch.equal(eo, po), "expanded and plain paths differ"
    assert torch.equal(el, pl)


def test_expanded_full_config_sampled_rows(gpu_lib):
    # the bench's entry point at the full shape: all 256 sampled token
    # positions x all 32 heads against the oracle, bit for bit the plain path
    case = prefill_full.case()
    rows = case.rows
    _say(f"[expanded] full cfg: Lq={case.Lq} Hq={case.Hq} L_act={case.L_act}, {len(rows)} tokens x all heads")
    (po, pl), (eo, el) = _both(gpu_lib, case, want_lse=True)
    ref, rlse = prefill_full.history_ref()
    r = rows.to(eo.device)
    assert_close(eo[:, r], ref, "expanded prefill full (256 sampled rows)")
    assert metrics(el[:, r], rlse)["max_abs"] < LSE_ABS
    assert torch.equal(eo, po) and torch.equal(el, pl)


def test_expanded_poisoned_tail_ignored(gpu_lib):
    case = W.prefill_paged(160, 8, 2, 70, 256, 6, 64, 200)
    _, out1 = _both(gpu_lib, case)
    nan = torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)
    bt = case.block_table.tolist()
    last = bt[case.L_act // case.block_size]
    case.k_cache[last, :, case.L_act % case.block_size:] = nan
    case.v_cache[last, :, case.L_act % case.block_size:] = nan
    for i in range(case.L_act // case.block_size + 1, len(bt)):
        case.k_cache[bt[i]] = nan
        case.v_cache[bt[i]] = nan
    _, out2 = _both(gpu_lib, case)
    assert torch.equal(out1, out2)


def test_expanded_workspace_reused_for_a_shorter_history(gpu_lib):
    taa = gpu_lib
    big = W.prefill_paged(170, 8, 2, 64, 256, 8, 128, 1000)
    ws = torch.empty(taa.attn_prefill_paged_expanded_workspace_size(big.Hkv, big.L_act, big.D), dtype=torch.uint8,
                     device=DEV)
    ws.fill_(0xFF)  # NaN bf16 everywhere the first call does not write
    _, e1 = _both(taa, big, workspace=ws)
    small = W.prefill_paged(171, 8, 2, 64, 256, 8, 128, 77)
    p2, e2 = _both(taa, small, workspace=ws)
    ref = oracle.prefill_paged(small.q, small.k_cache, small.v_cache, small.k_scale, small.v_scale,
                               small.block_table, small.L_act, small.scale, torch.arange(small.Lq))
    assert_close(e2, ref, "expanded prefill, reused workspace")
    assert torch.equal(e2, p2)
    assert torch.isfinite(e1.float()).all()


def test_expanded_workspace_too_small_is_an_error(gpu_lib):
    taa = gpu_lib
    case = W.prefill_paged(172, 4, 2, 16, 256, 4, 64, 200)
    need = taa.attn_prefill_paged_expanded_workspace_size(case.Hkv, case.L_act, case.D)
    ws = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        _both(taa, case, workspace=ws)


@pytest.mark.parametrize("L", [700, 0])
def test_causal_expanded_equals_causal(gpu_lib, L):
    taa = gpu_lib
    case = W.prefill_paged(180 + L, 8, 2, 300, 256, 6, 128, max(L, 1))
    case.L_act = L
    kc, vc = (t.to(DEV) for t in W.prefill_current_kv(181, 2, 300))
    d = lambda t: t.to(DEV)
    args = (d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale, case.v_scale, d(case.block_table), L, kc, vc,
            case.scale, case.G)
    _say(f"[expanded] causal L_act={L}")
    po, pl = taa.attn_prefill_paged_causal(*args, want_lse=True)
    eo, el = taa.attn_prefill_paged_causal_expanded(*args, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(eo, po) and torch.equal(el, pl)
    ref = oracle.prefill_causal(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table, L,
                                kc.cpu(), vc.cpu(), case.scale, torch.arange(case.Lq))
    assert_close(eo, ref, "causal expanded")


def test_causal_expanded_workspace_too_small_is_an_error(gpu_lib):
    taa = gpu_lib
    case = W.prefill_paged(182, 4, 2, 16, 256, 4, 64, 200)
    kc, vc = (t.to(DEV) for t in W.prefill_current_kv(183, 2, 16))
    need = taa.attn_prefill_paged_causal_expanded_workspace_size(case.Hq, case.Hkv, case.Lq, case.L_act, case.D)
    ws = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    d = lambda t: t.to(DEV)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        taa.attn_prefill_paged_causal_expanded(d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale,
                                               case.v_scale, d(case.block_table), case.L_act, kc, vc, case.scale,
                                               case.G, workspace=ws)


def test_expanded_shared_physical_blocks(gpu_lib):
    # logical blocks that share physical blocks (a shared prefix): the table is
    # read per tile, so every logical key still resolves to its own row
    case = W.prefill_paged(190, 8, 4, 48, 256, 4, 64, 600)
    case.block_table = torch.tensor([2, 0, 2, 1, 0, 3, 2, 1, 0, 2], dtype=torch.int32)
    _say("[expanded] shared physical blocks, L_act=600 over a 10-entry table of 4 blocks")
    plain, exp = _both(gpu_lib, case)
    ref = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table,
                               case.L_act, case.scale, torch.arange(case.Lq))
    assert_close(exp, ref, "expanded prefill, shared blocks")
    assert torch.equal(exp, plain)


def test_expanded_many_kv_heads(gpu_lib):
    case = W.prefill_paged(191, 32, 8, 72, 256, 12, 128, 1400, n_rows=72)
    _say("[expanded] Hq=32 Hkv=8 Lq=72 L_act=1400")
    plain, exp = _both(gpu_lib, case)
    ref = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table,
                               case.L_act, case.scale, torch.arange(case.Lq))
    assert_close(exp, ref, "expanded prefill, 8 KV heads")
    assert torch.equal(exp, plain)


def test_causal_expanded_full_config(gpu_lib):
    # the causal call over tile images at the full prefill shape: bit for bit
    # the converting path, and all 256 sampled token positions (plus the
    # first and last) x all heads against the oracle
    taa = gpu_lib
    case = prefill_full.case()
    kc, vc = (t.to(DEV) for t in prefill_full.current_kv())
    rows = prefill_full.causal_rows()
    d = lambda t: t.to(DEV)
    args = (d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale, case.v_scale, d(case.block_table), case.L_act,
            kc, vc, case.scale, case.G)
    _say(f"[expanded] causal full cfg Lq={case.Lq} L_act={case.L_act}, {len(rows)} tokens x all heads")
    po, pl = taa.attn_prefill_paged_causal(*args, want_lse=True)
    eo, el = taa.attn_prefill_paged_causal_expanded(*args, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(eo, po) and torch.equal(el, pl)
    ref, rlse = prefill_full.causal_ref()
    r = rows.to(DEV)
    assert_close(eo[:, r], ref, "causal expanded full (sampled rows)")
    assert metrics(el[:, r], rlse)["max_abs"] < LSE_ABS
