"""Paged history plus causal current-token prefill, HIP path vs the fp64
oracle (``oracle.prefill_causal``) through the C ABI.

Prefill Context-Parallel Attention POC for Trainium2: its first version
leaves attention among the current tokens out; here token t also attends the
current tokens 0..t, one softmax over history and current keys (the
log-sum-exp merge of the two parts).  Cases: full checks with ragged lengths,
workgroups whose rows span two heads, no history at all, fewer tokens than a
key tile; the full configuration on sampled tokens; future tokens poisoned;
a negative scale.
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


def _run(taa, case, kc, vc, want_lse=False):
    d = lambda t: t.to(DEV)
    r = taa.attn_prefill_paged_causal(d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale, case.v_scale,
                                      d(case.block_table), case.L_act, d(kc), d(vc), case.scale, case.G,
                                      want_lse=want_lse)
    torch.cuda.synchronize()
    return r


def _ref(case, kc, vc, rows, lse=False):
    return oracle.prefill_causal(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table,
                                 case.L_act, kc, vc, case.scale, rows, return_lse=lse)


@pytest.mark.parametrize("Hq,Hkv,Lq,nb,bs,L", [
    (4, 2, 100, 10, 64, 333),    # Lq < 256: one workgroup's rows span several heads
    (8, 1, 300, 6, 128, 700),    # rows of a workgroup cross a head boundary mid-tile
    (16, 2, 512, 8, 512, 4096),  # whole workgroups per head
    (6, 3, 260, 5, 64, 0),       # no history: plain causal self-attention
    (4, 4, 17, 3, 64, 65),       # fewer tokens than a key tile
])
def test_prefill_causal_small_full_check(gpu_lib, Hq, Hkv, Lq, nb, bs, L):
    case = W.prefill_paged(150 + Lq, Hq, Hkv, Lq, 256, nb, bs, L, n_rows=Lq)
    kc, vc = W.prefill_current_kv(250 + Lq, Hkv, Lq)
    _say(f"[prefill-causal] Hq={Hq} Hkv={Hkv} Lq={Lq} blocks={nb}x{bs} L_act={L}")
    out, lse = _run(gpu_lib, case, kc, vc, want_lse=True)
    rows = torch.arange(Lq)
    ref, rlse = _ref(case, kc, vc, rows, lse=True)
    assert_close(out, ref, "prefill causal out")
    assert metrics(lse, rlse)["max_abs"] < LSE_ABS


def test_prefill_causal_full_config_sampled_rows(gpu_lib):
    case = prefill_full.case()
    kc, vc = prefill_full.current_kv()
    rows = prefill_full.causal_rows()
    _say(f"[prefill-causal] full cfg Lq={case.Lq} L_act={case.L_act}, {len(rows)} tokens x all heads")
    out, lse = _run(gpu_lib, case, kc, vc, want_lse=True)
    ref, rlse = prefill_full.causal_ref()
    r = rows.to(DEV)
    assert_close(out[:, r], ref, "prefill causal full (sampled rows)")
    assert metrics(lse[:, r], rlse)["max_abs"] < LSE_ABS
    assert torch.equal(out, _run(gpu_lib, case, kc, vc))


def test_prefill_causal_future_tokens_leave_no_trace(gpu_lib):
    case = W.prefill_paged(170, 8, 2, 300, 256, 6, 64, 200)
    kc, vc = W.prefill_current_kv(171, 2, 300)
    o1 = _run(gpu_lib, case, kc, vc)
    T = 140  # tokens after T change; rows 0..T must not
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, T + 1:] = 3e4
    vc2[:, T + 1:] = -3e4
    o2 = _run(gpu_lib, case, kc2, vc2)
    assert torch.equal(o1[:, :T + 1], o2[:, :T + 1])


@pytest.mark.parametrize("scale", [-0.05, 0.0])
def test_prefill_causal_scale_sign(gpu_lib, scale):
    case = W.prefill_paged(180, 4, 2, 90, 256, 4, 64, 210, n_rows=90, scale=scale)
    kc, vc = W.prefill_current_kv(181, 2, 90)
    out = _run(gpu_lib, case, kc, vc)
    assert_close(out, _ref(case, kc, vc, torch.arange(90)), f"prefill causal scale {scale}")


def test_prefill_causal_rows_independent(gpu_lib):
    """Changing some tokens' queries leaves the other tokens' rows
    bit-identical (per-row softmax decisions, same key tiles)."""
    case = W.prefill_paged(190, 8, 2, 256, 256, 4, 64, 150)
    kc, vc = W.prefill_current_kv(191, 2, 256)
    o1 = _run(gpu_lib, case, kc, vc)
    case.q[:, 1::3] *= 4.0
    o2 = _run(gpu_lib, case, kc, vc)
    keep = [t for t in range(256) if t % 3 != 1]
    assert torch.equal(o1[:, keep], o2[:, keep])
