"""The full paged FP8 prefill workload (4096 query tokens, 32 query heads over
2 KV heads, head_dim 256, 131072 history tokens in 512-token blocks under a
permuted block table, 120000 live) and its fp64 oracle rows.

The workload states that the oracle checks 256 random query rows: here all
256 sampled token positions x all 32 heads (8192 (head, token) rows, about
1 TFLOP of fp64 work), computed once per test process and shared by every
test of this shape.  The causal variant adds the current tokens' K/V and the
first and last token positions.
"""
import functools

import torch

import oracle
import workloads as W


@functools.lru_cache(maxsize=1)
def case():
    return W.prefill_paged()


@functools.lru_cache(maxsize=1)
def history_ref():
    """(out [Hq, 256, D], lse [Hq, 256]) fp64 for case().rows."""
    c = case()
    return oracle.prefill_paged(c.q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.block_table, c.L_act, c.scale,
                                c.rows, return_lse=True)


@functools.lru_cache(maxsize=1)
def current_kv():
    c = case()
    return W.prefill_current_kv(1105, c.Hkv, c.Lq, c.D)


@functools.lru_cache(maxsize=1)
def causal_rows():
    c = case()
    return torch.cat([c.rows, torch.tensor([0, c.Lq - 1])])


@functools.lru_cache(maxsize=1)
def causal_ref():
    """(out, lse) fp64 of the history plus causal current tokens for causal_rows()."""
    c = case()
    kc, vc = current_kv()
    return oracle.prefill_causal(c.q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.block_table, c.L_act, kc, vc,
                                 c.scale, causal_rows(), return_lse=True)
