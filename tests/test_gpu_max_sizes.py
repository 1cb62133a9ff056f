"""The largest shapes of each entry point against the fp64 oracle.

- the paged prefill with the whole 131072-token history live (every block
  full, no partial tile) at the target shape, sampled query tokens x all heads,
  and through the expanded-history workspace (bit for bit the same);
- decode over a 32768-key cache (512 chunks per sequence) at head_dim 256 and
  512, and a 4096-key window at the end of it;
- an encoder launch of 4096 workgroups (B 64, H 16, S 512), sampled batches.
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


def test_prefill_whole_history_live(gpu_lib):
    case = W.prefill_paged(1300, L_act=256 * 512)
    rows = torch.cat([case.rows[:64], torch.tensor([0, case.Lq - 1])])
    _say(f"[max] prefill L_act={case.L_act} (all {case.num_blocks} blocks), {len(rows)} tokens x all heads")
    d = lambda t: t.to(DEV)
    out = gpu_lib.attn_prefill_paged(d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale, case.v_scale,
                                     d(case.block_table), case.L_act, case.scale, case.G)
    torch.cuda.synchronize()
    ref = oracle.prefill_paged(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.block_table,
                               case.L_act, case.scale, rows)
    assert_close(out[:, rows.to(DEV)], ref, "prefill whole history")
    exp = gpu_lib.attn_prefill_paged_expanded(d(case.q), d(case.k_cache), d(case.v_cache), case.k_scale,
                                              case.v_scale, d(case.block_table), case.L_act, case.scale, case.G)
    torch.cuda.synchronize()
    assert torch.equal(exp, out), "expanded history differs from the direct path"


@pytest.mark.parametrize("D", [256, 512])
def test_decode_long_context(gpu_lib, D):
    S = 32768
    case = W.decode_gemma(1310 + D, 2, 8, 4, S, D=D, lens=[S, 20001])
    _say(f"[max] decode S_ctx={S} D={D} lens={case.lens.tolist()}")
    d = lambda t: t.to(DEV)
    out = gpu_lib.attn_decode_gqa(d(case.q), d(case.k), d(case.v), d(case.mask), case.scale, case.G)
    torch.cuda.synchronize()
    assert_close(out, oracle.sdpa(case.q, case.k, case.v, case.scale, case.mask), f"decode S={S} D={D}")
    # the last 4096 keys of each sequence through the range entry point
    beg, end = [n - 4096 for n in case.lens.tolist()], case.lens.tolist()
    kb, ke = (torch.tensor(x, dtype=torch.int32, device=DEV) for x in (beg, end))
    outw = gpu_lib.attn_decode_gqa_window(d(case.q), d(case.k), d(case.v), None, kb, ke, 4096, case.scale, case.G)
    torch.cuda.synchronize()
    ref = oracle.decode_window(case.q, case.k, case.v, case.scale, None, beg, end, 4096)
    assert_close(outw, ref, f"decode window 4096 of S={S} D={D}")


def test_encoder_many_workgroups(gpu_lib):
    case = W.encoder_custom(1320, 64, 16, 512)
    _say("[max] encoder B=64 H=16 S=512: 4096 workgroups")
    d = lambda t: t.to(DEV)
    r = gpu_lib.attn_encoder_fwd(d(case.q), d(case.k), d(case.v), case.scale, None, want_ln=False)
    torch.cuda.synchronize()
    for b in (0, 31, 63):
        ref = oracle.sdpa(case.q[b:b + 1], case.k[b:b + 1], case.v[b:b + 1], case.scale)
        assert_close(r["out"][b:b + 1], ref, f"encoder batch {b}")
