"""The entry points inside HIP graphs (stream capture through torch).

The library allocates nothing, never synchronizes and enqueues only kernel
launches on the caller's stream, so a serving loop can capture a call once and
replay it.  Each graph is replayed several times with eager work and
synchronizations between the replays (a replay must not depend on state left
by the previous one), and every replay is compared bit for bit with the eager
result of the same call.  Buffers are allocated before capture; every
workload is first run eagerly once (one-time function attributes are set
outside the capture).
"""
import sys

import pytest
import torch

import workloads as W
from transformer_attention_attn_amd.rope import grid_positions, rope_tables

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _replays_match(call, out, eager, n=3):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call()
    for i in range(n):
        out.zero_()  # eager work between the replays, on the current stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"


def test_decode_in_a_graph(gpu_lib):
    taa = gpu_lib
    case = W.decode_gemma(1200, 4, 16, 8, 2048)
    d = lambda t: t.to(DEV)
    q, k, v, m = d(case.q), d(case.k), d(case.v), d(case.mask)
    out = torch.empty_like(q)
    ws = torch.empty(taa.attn_decode_gqa_workspace_size(case.B, case.Hq, case.S_ctx, case.D), dtype=torch.uint8,
                     device=DEV)
    call = lambda: taa.attn_decode_gqa(q, k, v, m, case.scale, case.G, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    _say("[graph] decode split + combine")
    _replays_match(call, out, eager)


def test_causal_prefill_in_a_graph(gpu_lib):
    taa = gpu_lib
    case = W.prefill_paged(1201, 8, 2, 300, 256, 6, 128, 700)
    kc, vc = (t.to(DEV) for t in W.prefill_current_kv(1202, 2, 300))
    d = lambda t: t.to(DEV)
    q, k, v, bt = d(case.q), d(case.k_cache), d(case.v_cache), d(case.block_table)
    out = torch.empty_like(q)
    lse = torch.empty(case.Hq, case.Lq, device=DEV)
    ws = torch.empty(taa.attn_prefill_paged_causal_workspace_size(case.Hq, case.Hkv, case.Lq, case.D),
                     dtype=torch.uint8, device=DEV)
    call = lambda: taa.attn_prefill_paged_causal(q, k, v, case.k_scale, case.v_scale, bt, case.L_act, kc, vc,
                                                 case.scale, case.G, out=out, lse=lse, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager, eager_lse = out.clone(), lse.clone()
    _say("[graph] history prefill + current-token kernel")
    _replays_match(call, out, eager)
    assert torch.equal(lse, eager_lse)


def test_causal_expanded_prefill_in_a_graph(gpu_lib):
    taa = gpu_lib
    case = W.prefill_paged(1205, 8, 2, 300, 256, 6, 128, 700)
    kc, vc = (t.to(DEV) for t in W.prefill_current_kv(1206, 2, 300))
    d = lambda t: t.to(DEV)
    q, k, v, bt = d(case.q), d(case.k_cache), d(case.v_cache), d(case.block_table)
    out = torch.empty_like(q)
    ws = torch.empty(taa.attn_prefill_paged_causal_expanded_workspace_size(case.Hq, case.Hkv, case.Lq, case.L_act,
                                                                         case.D), dtype=torch.uint8, device=DEV)
    call = lambda: taa.attn_prefill_paged_causal_expanded(q, k, v, case.k_scale, case.v_scale, bt, case.L_act, kc,
                                                          vc, case.scale, case.G, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    _say("[graph] causal prefill over tile images (four kernels)")
    _replays_match(call, out, eager)


def test_expanded_prefill_in_a_graph(gpu_lib):
    taa = gpu_lib
    case = W.prefill_paged(1204, 8, 2, 300, 256, 6, 128, 700)
    d = lambda t: t.to(DEV)
    q, k, v, bt = d(case.q), d(case.k_cache), d(case.v_cache), d(case.block_table)
    out = torch.empty_like(q)
    ws = torch.empty(taa.attn_prefill_paged_expanded_workspace_size(case.Hkv, case.L_act, case.D),
                     dtype=torch.uint8, device=DEV)
    call = lambda: taa.attn_prefill_paged_expanded(q, k, v, case.k_scale, case.v_scale, bt, case.L_act, case.scale,
                                                   case.G, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    _say("[graph] tile-image pass + prefill key loop")
    _replays_match(call, out, eager)


def test_encoder_rope_block_in_a_graph(gpu_lib):
    taa = gpu_lib
    case = W.encoder_custom(1203, 2, 4, 300, masked_lens=[300, 200])
    pos, _ = grid_positions(15, 20)
    c, s = (torch.from_numpy(t).to(DEV) for t in rope_tables(pos, 64))
    d = lambda t: t.to(DEV)
    q, k, v, m = d(case.q), d(case.k), d(case.v), d(case.mask)
    res, gam, bet = d(case.residual), d(case.gamma), d(case.beta)
    out = torch.empty_like(q)
    res_out = torch.empty_like(res)
    ln = torch.empty(case.B, case.S, case.H * case.D, dtype=torch.bfloat16, device=DEV)
    rws = torch.empty(taa.attn_encoder_rope_workspace_size(case.B, case.H, case.S, case.D), dtype=torch.uint8,
                      device=DEV)
    call = lambda: taa.attn_encoder_fwd(q, k, v, case.scale, m, out=out, residual=res, residual_out=res_out,
                                        gamma=gam, beta=bet, eps=case.eps, ln_out=ln, rope="interleaved",
                                        rope_cos=c, rope_sin=s, rope_workspace=rws)
    call()
    torch.cuda.synchronize()
    eager, eager_ln = out.clone(), ln.clone()
    _say("[graph] RoPE pass + encoder attention + residual/LayerNorm")
    _replays_match(call, out, eager)
    assert torch.equal(ln, eager_ln)


def test_encoder_block_direct_copies_in_a_graph(gpu_lib):
    """The bf16 block without a mask (K, V and the residual rows copied global
    -> LDS directly) then the LayerNorm pass, DINOv3's ragged shape: every
    output of every replay equals the eager call's."""
    taa = gpu_lib
    case = W.encoder_dinov3()
    d = lambda t: t.to(DEV)
    q, k, v, res, gam, bet = d(case.q), d(case.k), d(case.v), d(case.residual), d(case.gamma), d(case.beta)
    out = torch.empty_like(q)
    res_out = torch.empty_like(res)
    ln = torch.empty(case.B, case.S, case.H * case.D, dtype=torch.bfloat16, device=DEV)
    mean = torch.empty(case.B * case.S, device=DEV)
    rstd = torch.empty(case.B * case.S, device=DEV)
    call = lambda: taa.attn_encoder_fwd(q, k, v, case.scale, None, out=out, residual=res, residual_out=res_out,
                                        gamma=gam, beta=bet, eps=case.eps, ln_out=ln, ln_mean=mean, ln_rstd=rstd)
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, res_out, ln, mean, rstd)]
    _say("[graph] encoder block over direct copies + LayerNorm (DINOv3 shape)")
    outs, names = (out, res_out, ln, mean, rstd), ("out", "residual_out", "ln_out", "mean", "rstd")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call()
    for i in range(3):
        for t in outs:
            t.zero_()  # eager work between the replays; every output must be rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e, name in zip(outs, eager, names):
            assert torch.equal(t, e), f"replay {i}: {name} differs from the eager call"


def test_encoder_key_lengths_in_a_graph(gpu_lib):
    """Right padding as key lengths (a device int32 array read by the kernel):
    the lengths changed between replays change the replayed result exactly as
    they change the eager one."""
    taa = gpu_lib
    case = W.encoder_custom(1100, 4, 12, 512)
    d = lambda t: t.to(DEV)
    q, k, v = d(case.q), d(case.k), d(case.v)
    out = torch.empty_like(q)
    kl = torch.tensor([512, 300, 17, 0], dtype=torch.int32, device=DEV)
    call = lambda: taa.attn_encoder_fwd(q, k, v, case.scale, None, key_len=kl, out=out, want_ln=False)
    call()
    torch.cuda.synchronize()
    _say("[graph] encoder with key lengths, lengths changed between replays")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call()
    for lens in ([512, 300, 17, 0], [1, 2, 3, 512], [256, 256, 256, 256]):
        kl.copy_(torch.tensor(lens, dtype=torch.int32))
        call()
        torch.cuda.synchronize()
        eager = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay with lengths {lens} differs from the eager call"
