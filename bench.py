#!/usr/bin/env python3
"""Benchmark of the flash-attention hot path on one MI355X.

One step = one pass over every kernel of the path, each on its workload:
  * encoder blocks: V-JEPA2 ViT-L attention (B=1, 16 heads, 2048 tokens,
    D=64) and DINOv3 ViT-L/16 at 448 px (B=2, 16 heads, 789 tokens: ragged
    tiles), bf16, each + residual add into the fp32 [B,S,1024] stream +
    LayerNorm;
  * GQA decode: B=8, 16 query / 8 KV heads, head_dim 256, S_ctx 4096,
    ragged lengths len_b ~ U{1..4096};
  * paged FP8 prefill: 4096 query tokens x 32 heads over 2 KV heads, D=256,
    512-token blocks under a permuted block table, 120000 live history keys,
    through its workspace (the live history expanded to bf16 tile images,
    then the key loop; both kernels inside the timed call).
All inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line.  `value` is the step's attention throughput (QK^T + PV
FLOPs of the four attention calls over the step time); `parts` gives each
call's own metric (TFLOP/s and % of the bf16 MFMA peak, or GB/s and % of HBM
peak) from HIP events recorded on the stream the kernels run on, with
min/median/mean/P90/max; each encoder block also gets its attention alone
(epilogue pointers null) and the softmax's VALU bound; `roofline` is the
dominant call's (the prefill: its two kernels).  `cpu_baseline` times the
fp64 oracle on the host cores: workloads 1-4 whole, the prefill on its 256
sampled tokens x 32 heads.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from workloads import accounting as acc  # noqa: E402


COPY_BYTES = 1 << 30


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C/C++/HIP source with comments removed and whitespace runs collapsed to
    one space: the text the compiler acts on, up to layout.  String and
    character literals are kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        ch = src[i]
        if ch in "\"'":
            j = i + 1
            while j < n and src[j] != ch:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the HIP sources' code (comments and layout ignored): measured
    HBM traffic is only reported for the exact kernels it was counted on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_attention_attn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode() + b"\0" + code_text(open(os.path.join(csrc, f)).read()).encode() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (rocprofv3
    FETCH_SIZE + WRITE_SIZE scaled by a plain copy), or None when the file is
    missing or was measured on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


class Timer:
    """Accumulates HIP-event durations for one kernel family on the current stream."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cases, pre, n_rows: int, reps: int = 3):
    """The fp64 oracle on the host cores: the tiny, V-JEPA2 and DINOv3 encoder
    blocks and the decode computed whole (median of `reps` runs each), the
    prefill on its first n_rows sampled tokens x all heads (one run).  Input
    generation is outside the timings."""
    import oracle

    oracle.build()
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    per = {}

    def timed(fn, n):
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    for key, c in cases.items():
        if key == "gemma_gqa_decode_d256_ctx4096":
            dt = timed(lambda: oracle.sdpa(c.q, c.k, c.v, c.scale, c.mask), reps)
            f = 4 * int(c.lens.sum()) * c.Hq * c.D
        else:
            dt = timed(lambda: oracle.encoder_block(c.q, c.k, c.v, c.scale, c.residual, c.gamma, c.beta, c.eps,
                                                    c.mask), reps)
            f = acc.encoder_flops(c.B, c.H, c.S, c.S, c.D)
        per[key] = {"s": dt, "gflops": f / dt / 1e9, "scope": "whole output", "runs": reps}
    rows = pre.rows[:n_rows]
    t0 = time.perf_counter()
    oracle.prefill_paged(pre.q, pre.k_cache, pre.v_cache, pre.k_scale, pre.v_scale, pre.block_table, pre.L_act,
                         pre.scale, rows)
    dt = time.perf_counter() - t0
    f = acc.prefill_flops(len(rows), pre.Hq, pre.L_act, pre.D)
    per["paged_fp8_prefill_q4096_hist120000"] = {
        "s": dt, "gflops": f / dt / 1e9, "rows_per_s": len(rows) * pre.Hq / dt, "runs": 1,
        "scope": f"{len(rows)} sampled tokens x {pre.Hq} heads x {pre.L_act} keys (of {pre.Lq} tokens; "
                 f"all {pre.Lq} would take about {dt * pre.Lq / len(rows):.0f} s, extrapolated)"}
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, cores), "kind": "oracle",
            "sample": f"fp64 C oracle (OpenMP over rows): paged FP8 prefill on {len(rows)} sampled query tokens x "
                      f"{pre.Hq} heads x {pre.L_act} keys incl. the KV decode ({dt:.1f} s) = value; workloads "
                      f"1-4 whole in per_config",
            "cpu_model": _cpu_model(), "per_config": per}


def time_next_workloads(taa, dev, flush, pre_dev, reps: int = 20):
    """Workload variants beyond the step (reported, not part of `value`):
    the 64-frame V-JEPA 2 clip (8192 tokens), a gte-base batch right-padded to
    512 tokens with ragged real lengths (as an additive key mask, and as key
    lengths), all timed as back-to-back launches between two HIP events after
    3 warm-up calls; and
    the decode at head_dim 512 (global layers) and over a 1024-key sliding
    window at head_dim 256, each call timed alone after the cache flush; and
    the paged prefill with causal attention among the 4096 current tokens
    (the history inputs of the step, already on the device; history through
    its tile images), and the step's prefill without a workspace."""
    out = {}

    def timed_flushed(fn):
        for _ in range(3):
            fn()
        ms = []
        for _ in range(reps):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return statistics.median(ms)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    c = W.encoder_custom(803, 1, 16, 8192)
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    o = torch.empty_like(q)
    ms = timed(lambda: taa.attn_encoder_fwd(q, k, v, c.scale, None, out=o, want_ln=False))
    f = acc.encoder_flops(1, 16, 8192, 8192, 64)
    out["vjepa2_clip64_s8192_attention"] = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12,
                                            "frac_bf16_peak": f / (ms * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS}
    g = torch.Generator().manual_seed(900)
    lens = torch.randint(6, 513, (8,), generator=g).tolist()
    c = W.encoder_custom(900, 8, 12, 512, masked_lens=lens)
    q, k, v, m = c.q.to(dev), c.k.to(dev), c.v.to(dev), c.mask.to(dev)
    res, gam, bet = c.residual.to(dev), c.gamma.to(dev), c.beta.to(dev)
    ms = timed(lambda: taa.attn_encoder_fwd(q, k, v, c.scale, m, residual=res, gamma=gam, beta=bet, eps=c.eps))
    dense = acc.encoder_flops(8, 12, 512, 512, 64)
    live = 4 * 512 * sum(lens) * 12 * 64
    out["gte_base_padded_L512_b8_block"] = {"ms": ms, "lens": lens, "dense_equiv_tflops": dense / (ms * 1e-3) / 1e12,
                                            "live_key_tflops": live / (ms * 1e-3) / 1e12,
                                            "kernels": "attention+mask+residual, res_ln"}
    # the same batch with its right padding given as key lengths: same result,
    # the padded key tiles are never read
    kl = torch.tensor(lens, dtype=torch.int32, device=dev)
    ms = timed(lambda: taa.attn_encoder_fwd(q, k, v, c.scale, None, key_len=kl, residual=res, gamma=gam, beta=bet,
                                            eps=c.eps))
    out["gte_base_padded_L512_b8_block_key_len"] = {
        "ms": ms, "lens": lens, "dense_equiv_tflops": dense / (ms * 1e-3) / 1e12,
        "live_key_tflops": live / (ms * 1e-3) / 1e12, "kernels": "attention+residual over the live keys, res_ln"}

    c = W.decode_gemma(1005, D=512)
    q, k, v, m = c.q.to(dev), c.k.to(dev), c.v.to(dev), c.mask.to(dev)
    o = torch.empty_like(q)
    ws = torch.empty(taa.attn_decode_gqa_workspace_size(c.B, c.Hq, c.S_ctx, c.D), dtype=torch.uint8, device=dev)
    ms = timed_flushed(lambda: taa.attn_decode_gqa(q, k, v, m, c.scale, c.G, out=o, workspace=ws))
    b = acc.decode_bytes(c.lens.tolist(), c.Hkv, c.Hq, c.S_ctx, c.D)
    out["gemma_gqa_decode_d512_b8_ctx4096"] = {"median_ms": ms, "lens": c.lens.tolist(), "bytes": b,
                                              "gbps": b / (ms * 1e-3) / 1e9,
                                              "frac_hbm_peak": b / (ms * 1e-3) / 1e9 / acc.PEAK_HBM_GBPS}
    del k, v
    c = W.decode_gemma(1006)
    win = 1024
    lens = c.lens.tolist()
    beg = torch.tensor([max(n - win, 0) for n in lens], dtype=torch.int32, device=dev)
    end = torch.tensor(lens, dtype=torch.int32, device=dev)
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    o = torch.empty_like(q)
    ws = torch.empty(taa.attn_decode_gqa_window_workspace_size(c.B, c.Hq, c.S_ctx, win, c.D), dtype=torch.uint8,
                     device=dev)
    ms = timed_flushed(lambda: taa.attn_decode_gqa_window(q, k, v, None, beg, end, win, c.scale, c.G, out=o,
                                                          workspace=ws))
    b = acc.decode_window_bytes([min(n, win) for n in lens], c.Hkv, c.Hq, c.D)
    out["gemma_sliding_window1024_decode_d256_b8_ctx4096"] = {
        "median_ms": ms, "lens": lens, "window": win, "bytes": b, "gbps": b / (ms * 1e-3) / 1e9,
        "frac_hbm_peak": b / (ms * 1e-3) / 1e9 / acc.PEAK_HBM_GBPS}
    del q, k, v

    # the encoder attention with RoPE (K rotated by its pass, q rows as the
    # attention kernel loads them; the step's V-JEPA2 inputs and the DINOv3
    # shape; attention alone, back to back, both kernels timed)
    from transformer_attention_attn_amd.rope import grid_positions, rope_tables
    for name, case, grid, prefix, pairing in (("vjepa2_s2048_rope3d_interleaved", W.encoder_vjepa2(), (8, 16, 16), 0,
                                               "interleaved"),
                                              ("dinov3_s789_rope2d_half", W.encoder_dinov3(), (28, 28), 5, "half")):
        pos, rot = grid_positions(*grid, prefix_tokens=prefix)
        c, s_ = (torch.from_numpy(t).to(dev) for t in rope_tables(pos, case.D, rotate=rot))
        q, k, v = case.q.to(dev), case.k.to(dev), case.v.to(dev)
        o = torch.empty_like(q)
        rws = torch.empty(taa.attn_encoder_rope_workspace_size(case.B, case.H, case.S, case.D), dtype=torch.uint8,
                          device=dev)
        ms_r = timed(lambda: taa.attn_encoder_fwd(q, k, v, case.scale, None, out=o, want_ln=False, rope=pairing,
                                                  rope_cos=c, rope_sin=s_, rope_workspace=rws))
        ms_0 = timed(lambda: taa.attn_encoder_fwd(q, k, v, case.scale, None, out=o, want_ln=False))
        f = acc.encoder_flops(case.B, case.H, case.S, case.S, case.D)
        out[f"{name}_attention"] = {"ms": ms_r, "ms_without_rope": ms_0, "tflops": f / (ms_r * 1e-3) / 1e12,
                                    "frac_bf16_peak": f / (ms_r * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS}

    pre, p_q, p_k, p_v, p_bt = pre_dev
    kc, vc = (t.to(dev) for t in W.prefill_current_kv(1105, pre.Hkv, pre.Lq, pre.D))
    o = torch.empty_like(p_q)
    r3 = max(3, reps // 5)

    def timed_b2b(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    pws = torch.empty(taa.attn_prefill_paged_causal_expanded_workspace_size(pre.Hq, pre.Hkv, pre.Lq, pre.L_act,
                                                                            pre.D), dtype=torch.uint8, device=dev)
    ms = timed_b2b(lambda: taa.attn_prefill_paged_causal_expanded(p_q, p_k, p_v, pre.k_scale, pre.v_scale, p_bt,
                                                                  pre.L_act, kc, vc, pre.scale, pre.G, out=o,
                                                                  workspace=pws), r3)
    f_hist = acc.prefill_flops(pre.Lq, pre.Hq, pre.L_act, pre.D)
    f_cur = acc.causal_flops(pre.Lq, pre.Hq, pre.D)
    tf = (f_hist + f_cur) / (ms * 1e-3) / 1e12
    out["paged_fp8_prefill_q4096_hist120000_plus_causal_current"] = {
        "ms": ms, "tflops": tf, "frac_bf16_peak": tf / acc.PEAK_BF16_TFLOPS, "flops_history": f_hist,
        "flops_current": f_cur}
    # the step's prefill without a workspace: the key loop converts each fp8
    # tile itself (attn_prefill_paged)
    ms = timed_b2b(lambda: taa.attn_prefill_paged(p_q, p_k, p_v, pre.k_scale, pre.v_scale, p_bt, pre.L_act,
                                                  pre.scale, pre.G, out=o), r3)
    tf = f_hist / (ms * 1e-3) / 1e12
    out["paged_fp8_prefill_q4096_hist120000_no_workspace"] = {
        "ms": ms, "tflops": tf, "frac_bf16_peak": tf / acc.PEAK_BF16_TFLOPS, "flops": f_hist}
    return out


def pcp_shapes(reps: int = 10) -> None:
    """The paged prefill at the PCP page's Q-scaling shapes (32 query heads over 2 KV
    heads, head_dim 256, 8192 history keys in 512-token blocks, Lq 1024 .. 16384):
    both entry points timed back to back on one GPU, printed as a markdown table
    beside the page's 4-chip times (another machine: context only)."""
    import transformer_attention_attn_amd as taa

    taa.load()
    dev = torch.device("cuda:0")
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_throughput_figures.json")))
    page = {row[0]: row[1] for row in gold["pcp_q_scaling_hist8192"]["rows"]}
    print("| Lq | expanded ms | TFLOP/s | % bf16 peak | no-workspace ms | TFLOP/s | page, 4 chips (ms) |")
    print("|---|---|---|---|---|---|---|")
    for Lq in (1024, 4096, 8192, 16384):
        case = W.prefill_paged(2000 + Lq, 32, 2, Lq, 256, 16, 512, 8192, n_rows=1)
        q, k, v, bt = (t.to(dev) for t in (case.q, case.k_cache, case.v_cache, case.block_table))
        out = torch.empty_like(q)
        ws = torch.empty(taa.attn_prefill_paged_expanded_workspace_size(case.Hkv, case.L_act, case.D),
                         dtype=torch.uint8, device=dev)
        args = (q, k, v, case.k_scale, case.v_scale, bt, case.L_act, case.scale, case.G)
        f = acc.prefill_flops(Lq, case.Hq, case.L_act, case.D)
        res = []
        for fn in (lambda: taa.attn_prefill_paged_expanded(*args, out=out, workspace=ws),
                   lambda: taa.attn_prefill_paged(*args, out=out)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / reps)
        tf = [f / (ms * 1e-3) / 1e12 for ms in res]
        print(f"| {Lq} | {res[0]:.3f} | {tf[0]:.0f} | {100 * tf[0] / acc.PEAK_BF16_TFLOPS:.1f} | {res[1]:.3f} | "
              f"{tf[1]:.0f} | {page[Lq]} |", flush=True)
        del q, k, v, bt, out, ws


def _short(name: str) -> str:
    """Kernel family name from a demangled rocprofv3 kernel name."""
    for k in ("prefill_paged_kernel", "prefill_tile_images_kernel", "prefill_current_kernel", "encoder_fwd_kernel",
              "res_ln_kernel", "rope_k_kernel", "decode_split_kernel", "decode_combine_kernel", "copyBuffer"):
        if k in name:
            return k
    return None


def _grid(row: dict) -> str:
    """Launch grid of a rocprofv3 CSV row in work-items (the kernel trace gives
    Grid_Size_X/Y/Z, the counter collection their product as Grid_Size)."""
    if row.get("Grid_Size") not in (None, ""):
        return str(int(float(row["Grid_Size"])))
    n = 1
    for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"):
        if row.get(k) not in (None, ""):
            n *= int(float(row[k]))
    return str(n)


def _pct(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


def _launches(rows):
    """This library's launches of one rocprofv3 CSV (one row per dispatch, or
    one per (dispatch, counter)), in dispatch order, each with its role: an
    encoder launch followed by a LayerNorm launch belongs to a fused block,
    any other encoder launch is attention alone."""
    by_id = {}
    for r in rows:
        f = _short(r["Kernel_Name"])
        if not f:
            continue
        d = int(r["Dispatch_Id"])
        e = by_id.setdefault(d, {"family": f, "grid": _grid(r), "kernel": r["Kernel_Name"], "row": r, "value": 0.0})
        if "Counter_Value" in r:
            e["value"] += float(r["Counter_Value"])
            if r.get("Counter_Name"):
                c = e.setdefault("counters", {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ordered = [by_id[d] for d in sorted(by_id)]
    ours = [e for e in ordered if e["family"] != "copyBuffer"]
    for i, e in enumerate(ours):
        nxt = ours[i + 1]["family"] if i + 1 < len(ours) else None
        e["role"] = e["family"]
        if e["family"] == "encoder_fwd_kernel":
            e["role"] = "encoder_fwd_kernel" if nxt == "res_ln_kernel" else "encoder_fwd_kernel(alone)"
    return ordered


# Workloads of the step as they appear in a kernel trace: the encoder blocks in
# step order (V-JEPA2 first), then the decode and the prefill.
PROFILE_WORKLOADS = [
    ("encoder_fwd_kernel__vjepa2_s2048_block", "vjepa2_encoder_block_s2048", 0),
    ("encoder_fwd_kernel__dinov3_s789_block", "dinov3_encoder_block_s789", 1),
    ("decode_gqa__gemma_d256_b8_ctx4096", "gemma_gqa_decode_d256_ctx4096", None),
    ("prefill_paged_kernel__paged_fp8_prefill_q4096_hist120000", "paged_fp8_prefill_q4096_hist120000", None),
]

PROFILE_COMMANDS = """cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o bench -- python3 <repo>/bench.py --steps 10 --warmup 3 --cpu-rows 0 --no-next
cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/FETCH_SIZE -o bench -- python3 <repo>/bench.py --steps 2 --warmup 1 --cpu-rows 0 --no-next
cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/WRITE_SIZE -o bench -- python3 <repo>/bench.py --steps 2 --warmup 1 --cpu-rows 0 --no-next
cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/FETCH_SIZE_copy -o copy -- python3 <repo>/bench.py --copy-calibration
cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/WRITE_SIZE_copy -o copy -- python3 <repo>/bench.py --copy-calibration
python3 <repo>/bench.py --summarize <out>      # writes profiles/traffic.json and these summaries"""

# Two counter passes over the same bench step (each within the per-block limits
# of one rocprofv3 pass: at most 8 SQ and 2 GRBM counters).
PMC_PASSES = {
    "pmc1": "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
            "SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_INSTS_VALU GRBM_GUI_ACTIVE",
    "pmc2": "SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_ACTIVE_INST_ANY "
            "SQ_INSTS_SALU SQ_INSTS_VALU_CVT GRBM_GUI_ACTIVE",
}
N_SE = 32  # shader engines of the MI355X (4 per XCD)
PMC_COMMANDS = "\n".join(f"cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out>/{d} -o run -- python3 "
                         "<repo>/bench.py --steps 2 --warmup 1 --cpu-rows 0 --no-next" for d, c in PMC_PASSES.items())
NEXT_COMMAND = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_next -o next -- "
                "python3 <repo>/bench.py --only next --cpu-rows 0")
PCP_COMMAND = "python3 <repo>/bench.py --pcp-shapes > <out>/pcp.md"


def summarize(prof_dir: str) -> None:
    """Turn the rocprofv3 CSV output of the profiling commands (kernel trace in
    <dir>/trace, FETCH_SIZE / WRITE_SIZE passes of the bench in <dir>/<C> and of
    --copy-calibration in <dir>/<C>_copy) into profiles/traffic.json, and, when
    <dir>/bench.json holds the bench line of the same lease, into one markdown
    summary per workload of the step under profiles/.  Launches are grouped by
    role (see _launches) and launch grid (the two encoder workloads share one
    kernel).  Reads CSV and JSON only; no GPU."""
    import csv
    import glob

    def one(pattern):
        hits = sorted(glob.glob(os.path.join(prof_dir, pattern)))
        if not hits:
            raise SystemExit(f"summarize: no {pattern} under {prof_dir}")
        return hits[0]

    def groups(path, field):
        g = {}
        for e in _launches(list(csv.DictReader(open(path)))):
            key = (e.get("role", e["family"]), e["grid"])
            g.setdefault(key, {"kernel": e["kernel"], "vals": [], "first": int(e["row"]["Dispatch_Id"])})
            g[key]["vals"].append(field(e))
        return g

    trace = groups(one("trace/*kernel_trace.csv"),
                   lambda e: float(e["row"]["End_Timestamp"]) - float(e["row"]["Start_Timestamp"]))
    roles = {}
    for (r, gr) in trace:
        roles.setdefault(r, []).append(gr)
    label = {(r, gr): (r if len(roles[r]) == 1 else f"{r}@{gr}") for (r, gr) in trace}

    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        d = groups(one(f"{c}_copy/*counter_collection.csv"), lambda e: e["value"])
        # the 1 GiB copies: the copyBuffer launches of the largest grid
        copies = sorted((int(gr), statistics.fmean(v["vals"])) for (r, gr), v in d.items() if r == "copyBuffer")
        cal[c] = copies[-1][1] * 1024 / COPY_BYTES
    fetch = {k: statistics.fmean(v["vals"]) for k, v in
             groups(one("FETCH_SIZE/*counter_collection.csv"), lambda e: e["value"]).items()}
    write = {k: statistics.fmean(v["vals"]) for k, v in
             groups(one("WRITE_SIZE/*counter_collection.csv"), lambda e: e["value"]).items()}
    kernels = {}
    for key, st in sorted(trace.items(), key=lambda kv: kv[1]["first"]):
        if key[0] == "copyBuffer":
            continue
        ns = st["vals"]
        entry = {"kernel": st["kernel"], "role": key[0], "grid_work_items": int(key[1]), "launches": len(ns),
                 "first_dispatch": st["first"],
                 "avg_duration_ns": statistics.fmean(ns), "min_duration_ns": min(ns),
                 "median_duration_ns": statistics.median(ns), "p90_duration_ns": _pct(ns, 0.9),
                 "max_duration_ns": max(ns)}
        if key in fetch and key in write:
            entry.update({"fetch_kib_raw": fetch[key], "write_kib_raw": write[key],
                          "hbm_bytes_per_launch": int(fetch[key] * 1024 / cal["FETCH_SIZE"]
                                                      + write[key] * 1024 / cal["WRITE_SIZE"])})
        kernels[label[key]] = entry
    out = {"source_hash": kernel_source_hash(),
           "note": "rocprofv3 kernel trace (per-launch durations) and FETCH_SIZE/WRITE_SIZE (KiB per dispatch, "
                   "L2 <-> memory fabric) divided by the ratio the same counter reads for a 1 GiB device copy; "
                   "launches grouped by role and grid (work-items)",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_ratio": cal["FETCH_SIZE"], "write_ratio": cal["WRITE_SIZE"]},
           "kernels": kernels}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"wrote {path} (sources {out['source_hash']}; copy calibration fetch x{cal['FETCH_SIZE']:.4f}, "
          f"write x{cal['WRITE_SIZE']:.4f})")
    bench_path = os.path.join(prof_dir, "bench.json")
    if os.path.exists(bench_path):
        _write_profiles(json.load(open(bench_path)), kernels, cal)
    _write_pmc_profile(prof_dir, kernels)
    _write_next_profile(prof_dir)
    _write_pcp_profile(prof_dir)


def _hash_line():
    return (f"Measured on one MI355X (gfx950, 256 CUs) in the same lease as the other summaries, kernel code hash "
            f"`{kernel_source_hash()}` (comments and layout ignored; `bench.py` -> `kernel_source_hash()`).")


def _write_pmc_profile(prof_dir, kernels):
    """profiles/pmc_instruction_mix__bench_step.md from the two counter passes
    (<dir>/pmc1, <dir>/pmc2) and the kernel trace's durations (kernels)."""
    import csv
    import glob

    merged, order = {}, []
    for d in PMC_PASSES:
        hits = sorted(glob.glob(os.path.join(prof_dir, d, "*counter_collection.csv")))
        if not hits:
            return
        for e in _launches(list(csv.DictReader(open(hits[0])))):
            if e["family"] == "copyBuffer":
                continue
            key = (e["role"], e["grid"])
            if key not in merged:
                merged[key] = {}
                order.append(key)
            for c, v in e.get("counters", {}).items():
                merged[key].setdefault(c, []).append(v)
    dur = {(e["role"], str(e["grid_work_items"])): e["avg_duration_ns"] for e in kernels.values()}
    names = {(e["role"], str(e["grid_work_items"])): e["kernel"] for e in kernels.values()}
    L = ["# Instruction mix and MFMA occupancy of the bench step (rocprofv3 counters)", "", _hash_line(), "",
         "Commands (repository root copy `<repo>`, output dir `<out>`; two passes, each within the per-block counter "
         "limits; the durations come from the kernel trace of the same lease):", "", "```", PMC_COMMANDS, "```", "",
         "Per launch (mean over the launches of each kernel and grid), wave-level instruction counts. "
         "`SQ_INSTS_VALU` counts the MFMA instructions too; the VALU column is `SQ_INSTS_VALU - SQ_INSTS_MFMA`. "
         "MFMA busy: `SQ_VALU_MFMA_BUSY_CYCLES` (cycles the matrix cores are busy, summed over the 1024 SIMDs) over "
         f"the SIMD cycles of the kernel's active time, `SQ_BUSY_CYCLES` / {N_SE} x 1024 (`SQ_BUSY_CYCLES` sums the "
         f"{N_SE} shader engines: over the 12 ms prefill it reads about 30.5 x `GRBM_GUI_ACTIVE` / 8, i.e. {N_SE} "
         "engines busy ~95% of the time; `GRBM_GUI_ACTIVE` itself also counts each dispatch's idle overhead under "
         f"counter collection, which dominates a 5-30 us kernel).  Clock: `SQ_BUSY_CYCLES` / {N_SE} over the traced "
         "duration.", "",
         "| kernel (role, grid) | MFMA insts | VALU insts | VALU / MFMA | exp2 (trans) / MFMA | cvt / MFMA | "
         "LDS insts / MFMA | LDS bank conflicts | wait-any / wave cycles | MFMA busy | clock (GHz) |",
         "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in order:
        c = {k: statistics.fmean(v) for k, v in merged[key].items()}
        mf, va = c.get("SQ_INSTS_MFMA", 0.0), c.get("SQ_INSTS_VALU", 0.0) - c.get("SQ_INSTS_MFMA", 0.0)
        per = (lambda x: f"{x / mf:.2f}") if mf else (lambda x: "-")
        sq, t = c.get("SQ_BUSY_CYCLES"), dur.get(key)
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (sq / N_SE * 1024) if sq else None
        clk = sq / N_SE / t if sq and t else None
        wa = c.get("SQ_WAIT_INST_ANY", 0.0) / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else None
        L.append(f"| `{key[0]}` ({key[1]}) | {mf:.4g} | {va:.4g} | {per(va)} | {per(c.get('SQ_INSTS_VALU_TRANS_F32', 0))} | "
                 f"{per(c.get('SQ_INSTS_VALU_CVT', 0))} | {per(c.get('SQ_INSTS_LDS', 0))} | "
                 f"{c.get('SQ_LDS_BANK_CONFLICT', 0):.3g} | {'-' if wa is None else f'{wa:.2f}'} | "
                 f"{'-' if busy is None else f'{100 * busy:.0f}%'} | {'-' if clk is None else f'{clk:.2f}'} |")
    L += ["", "Full kernel names:", ""]
    L += [f"- `{k[0]}` ({k[1]}): `{names.get(k, '?')}`" for k in order]
    L += ["", "Raw counter means per launch:", "", "| kernel (role, grid) | " + " | ".join(
        sorted({n for k in order for n in merged[k]})) + " |"]
    cols = sorted({n for k in order for n in merged[k]})
    L.append("|---|" + "---|" * len(cols))
    for key in order:
        L.append(f"| `{key[0]}` ({key[1]}) | " + " | ".join(
            f"{statistics.fmean(merged[key][n]):.4g}" if n in merged[key] else "-" for n in cols) + " |")
    with open(os.path.join(ROOT, "profiles", "pmc_instruction_mix__bench_step.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    print("wrote profiles/pmc_instruction_mix__bench_step.md")


def _write_next_profile(prof_dir):
    """profiles/next_workloads__kernel_trace.md from <dir>/trace_next (one call
    of time_next_workloads under the kernel trace)."""
    import csv
    import glob

    hits = sorted(glob.glob(os.path.join(prof_dir, "trace_next", "*kernel_trace.csv")))
    if not hits:
        return
    by = {}
    for r in csv.DictReader(open(hits[0])):
        by.setdefault(r["Kernel_Name"], []).append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3)
    L = ["# Workload variants reported under `parts.next` (kernel trace)", "", _hash_line(), "",
         "Command (repository root copy `<repo>`, output dir `<out>`):", "", "```", NEXT_COMMAND, "```", "",
         "One call of `time_next_workloads` (each workload: warm-up calls, then timed calls): the V-JEPA2 64-frame "
         "clip (8192 tokens, attention alone); a gte-base batch right-padded to 512 tokens (mask, residual, "
         "LayerNorm; then the same with key lengths); decode at head_dim 512 and over a 1024-key sliding window at head_dim 256; V-JEPA2 and DINOv3 "
         "attention with RoPE (`rope_k_kernel` rotates K once); the paged prefill with causal current tokens. "
         "Kernels by total time:", "",
         "| kernel | calls | avg (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        L.append(f"| `{name}` | {len(v)} | {statistics.fmean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    with open(os.path.join(ROOT, "profiles", "next_workloads__kernel_trace.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    print("wrote profiles/next_workloads__kernel_trace.md")


def _write_pcp_profile(prof_dir):
    """profiles/prefill_pcp_q_scaling__hist8192.md from <dir>/pcp.md (the
    --pcp-shapes table of the same lease)."""
    path = os.path.join(prof_dir, "pcp.md")
    if not os.path.exists(path):
        return
    table = [l.rstrip("\n") for l in open(path) if l.startswith("|")]
    L = ["# Paged prefill at the PCP page's Q-scaling shapes (32 Q / 2 KV heads, D 256, 8192 history keys)", "",
         _hash_line(), "", "Command (repository root copy `<repo>`, output dir `<out>`):", "", "```", PCP_COMMAND,
         "```", "",
         "Each entry point is timed over 10 back-to-back calls after 3 warm-up calls, with HIP events on the stream "
         "the library launches on; inputs are seeded synthetic tensors of the shapes, 512-token blocks under a "
         "permuted block table.  FLOPs are 4 * Lq * 32 * 8192 * 256 (QK^T + PV).  The page's column is its own "
         "table, on four Trainium2 chips: another machine, context only.", ""] + table
    with open(os.path.join(ROOT, "profiles", "prefill_pcp_q_scaling__hist8192.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    print("wrote profiles/prefill_pcp_q_scaling__hist8192.md")


def _kernel_rows(ks):
    t = ["| kernel | launches | min (us) | median (us) | mean (us) | P90 (us) | max (us) | HBM bytes / launch |",
         "|---|---|---|---|---|---|---|---|"]
    for name, e in ks:
        hb = e.get("hbm_bytes_per_launch")
        t.append(f"| `{name}` | {e['launches']} | {e['min_duration_ns'] / 1e3:.2f} | {e['median_duration_ns'] / 1e3:.2f} | "
                 f"{e['avg_duration_ns'] / 1e3:.2f} | {e['p90_duration_ns'] / 1e3:.2f} | "
                 f"{e['max_duration_ns'] / 1e3:.2f} | {'-' if hb is None else f'{hb / 1e6:.1f} MB'} |")
    t.append("")
    t.append("Full kernel names (grid in work-items):")
    t.append("")
    for name, e in ks:
        t.append(f"- `{name}`: `{e['kernel']}`, grid {e['grid_work_items']}")
    return t


def _write_profiles(line, kernels, cal):
    """One markdown summary per workload of the step: the same lease's bench
    line (HIP events) beside the kernel trace and the traffic counters."""
    parts = line["parts"]
    by_role = {}
    for name, e in sorted(kernels.items(), key=lambda kv: kv[1]["first_dispatch"]):
        by_role.setdefault(e["role"], []).append((name, e))
    head = ["Measured on one MI355X (gfx950, 256 CUs) in one lease: the bench line and the rocprofv3 runs below, "
            f"kernel code hash `{kernel_source_hash()}` (comments and layout ignored; `bench.py` -> "
            "`kernel_source_hash()`).", "",
            "Commands (run from the repository root copy `<repo>`, output dir `<out>`; the bench line comes from "
            "`python3 <repo>/bench.py > <out>/bench.json` in the same lease):", "", "```", PROFILE_COMMANDS, "```", "",
            f"Traffic scaling: a 1 GiB device copy reads FETCH_SIZE = {cal['FETCH_SIZE']:.4f} x and WRITE_SIZE = "
            f"{cal['WRITE_SIZE']:.4f} x its true byte count; the counters see L2 <-> memory fabric traffic "
            "(Infinity Cache hits included), per dispatch, summed over all XCDs.", ""]
    for fname, key, enc_idx in PROFILE_WORKLOADS:
        p = parts.get(key)
        if p is None:
            continue
        L = []
        if enc_idx is not None:
            enc = by_role.get("encoder_fwd_kernel", [])
            lns = by_role.get("res_ln_kernel", [])
            alone = by_role.get("encoder_fwd_kernel(alone)", [])
            if len(enc) <= enc_idx or len(lns) <= enc_idx:
                continue
            ks = [enc[enc_idx], lns[enc_idx]] + ([alone[enc_idx]] if len(alone) > enc_idx else [])
            sh = p["shape"]
            t_blk = (ks[0][1]["avg_duration_ns"] + ks[1][1]["avg_duration_ns"]) / 1e3
            t_att = ks[2][1]["avg_duration_ns"] / 1e3 if len(ks) > 2 else None
            L += [f"# Encoder block, {key} (B {sh['B']}, H {sh['H']}, S {sh['S']}, D {sh['D']}, fused residual add, "
                  f"then LayerNorm over {sh['hidden']})", ""] + head
            L += ["## Bench line of the same lease (HIP events, warm)", "",
                  "| call | mean (us) | median (us) | min (us) | P90 (us) | TFLOP/s | % bf16 peak |", "|---|---|---|---|---|---|---|",
                  f"| block (attention + residual, LayerNorm) | {p['mean_ms'] * 1e3:.1f} | {p['median_ms'] * 1e3:.1f} | "
                  f"{p['min_ms'] * 1e3:.1f} | {p['p90_ms'] * 1e3:.1f} | {p['tflops']:.0f} | {100 * p['frac_bf16_peak']:.1f} |",
                  f"| attention alone | {p['attention_only']['mean_ms'] * 1e3:.1f} | {p['attention_only']['median_ms'] * 1e3:.1f} | "
                  f"{p['attention_only']['min_ms'] * 1e3:.1f} | {p['attention_only']['p90_ms'] * 1e3:.1f} | "
                  f"{p['attention_only']['tflops']:.0f} | {100 * p['attention_only']['frac_bf16_peak']:.1f} |", ""]
            if "back_to_back_ms" in p:
                L += [f"Back to back (50 calls between two events, per call): block {p['back_to_back_ms'] * 1e3:.1f} us "
                      f"({100 * p['back_to_back_frac_bf16_peak']:.1f}% of the bf16 peak), attention alone "
                      f"{p['attention_only']['back_to_back_ms'] * 1e3:.1f} us "
                      f"({100 * p['attention_only']['back_to_back_frac_bf16_peak']:.1f}%).", ""]
            L += ["## Kernel trace", ""] + _kernel_rows(ks) + [""]
            L += [f"Algorithmic work: {p['flops'] / 1e9:.2f} GFLOP of attention (QK^T + PV); MFMA bound at the "
                  f"bf16 peak {p['mfma_bound_us']:.2f} us; softmax VALU bound {p['valu_bound']['us']:.2f} us "
                  f"({p['valu_bound']['per_score']}).  From the trace: block {t_blk:.1f} us = "
                  f"{p['flops'] / (t_blk * 1e-6) / 1e12:.0f} TFLOP/s ({100 * p['flops'] / (t_blk * 1e-6) / 1e12 / acc.PEAK_BF16_TFLOPS:.1f}% "
                  "of bf16 peak)" + (f"; attention alone {t_att:.1f} us = {p['flops'] / (t_att * 1e-6) / 1e12:.0f} "
                                     f"TFLOP/s ({100 * p['flops'] / (t_att * 1e-6) / 1e12 / acc.PEAK_BF16_TFLOPS:.1f}%), "
                                     f"{100 * p['valu_bound']['us'] / t_att:.0f}% of the VALU bound's speed"
                                     if t_att else "") + ".", ""]
        elif key.startswith("gemma"):
            ks = by_role.get("decode_split_kernel", []) + by_role.get("decode_combine_kernel", [])
            if not ks:
                continue
            t = sum(e["avg_duration_ns"] for _, e in ks) / 1e3
            L += ["# Gemma-style GQA decode (B 8, 16 Q / 8 KV heads, D 256, S_ctx 4096, per-row lengths from the seed)",
                  ""] + head
            L += ["## Bench line of the same lease (HIP events, 512 MiB written before each call)", "",
                  "| mean (us) | median (us) | min (us) | P90 (us) | GB/s | % HBM peak |", "|---|---|---|---|---|---|",
                  f"| {p['mean_ms'] * 1e3:.1f} | {p['median_ms'] * 1e3:.1f} | {p['min_ms'] * 1e3:.1f} | "
                  f"{p['p90_ms'] * 1e3:.1f} | {p['gbps']:.0f} | {100 * p['frac_hbm_peak']:.1f} |", "",
                  "## Kernel trace", ""] + _kernel_rows(ks) + [""]
            L += [f"Algorithmic bytes: the live K/V rows (sum_b len_b x 8 KV heads x 256 x 2 B x 2) plus mask, q and "
                  f"out: {p['bytes'] / 1e6:.1f} MB.  From the trace: the kernels take {t:.1f} us = "
                  f"{p['bytes'] / (t * 1e-6) / 1e9:.0f} GB/s ({100 * p['bytes'] / (t * 1e-6) / 1e9 / acc.PEAK_HBM_GBPS:.1f}% "
                  "of 8 TB/s).", ""]
        else:
            ks = by_role.get("prefill_tile_images_kernel", []) + by_role.get("prefill_paged_kernel", [])
            if not ks:
                continue
            t = sum(e["avg_duration_ns"] for _, e in ks) / 1e3
            tmin = sum(e["min_duration_ns"] for _, e in ks) / 1e3
            r = line.get("roofline") or {}
            L += ["# Paged FP8 prefill (4096 query tokens x 32 heads over 2 KV heads, D 256, 120000 of 131072 "
                  "history keys, 512-token blocks)", ""] + head
            L += ["## Bench line of the same lease (HIP events, warm)", "",
                  "| mean (ms) | median (ms) | min (ms) | P90 (ms) | TFLOP/s | % bf16 peak |", "|---|---|---|---|---|---|",
                  f"| {p['mean_ms']:.3f} | {p['median_ms']:.3f} | {p['min_ms']:.3f} | {p['p90_ms']:.3f} | "
                  f"{p['tflops']:.0f} | {100 * p['frac_bf16_peak']:.1f} |", "",
                  f"The line's `ms_per_step` (all four calls of the step, wall clock) is {line['ms_per_step']:.2f} ms.",
                  "", "## Kernel trace", ""] + _kernel_rows(ks) + [""]
            tr = sum(e.get("hbm_bytes_per_launch", 0) for _, e in ks)
            L += [f"Algorithmic work: {p['flops'] / 1e12:.3f} TFLOP (QK^T + PV over the live keys).  From the trace: "
                  f"image pass + key loop {t / 1e3:.3f} ms mean ({tmin / 1e3:.3f} ms min) = "
                  f"{p['flops'] / (t * 1e-6) / 1e12:.0f} TFLOP/s, {100 * p['flops'] / (t * 1e-6) / 1e12 / acc.PEAK_BF16_TFLOPS:.1f}% "
                  f"of the bf16 MFMA peak (the bench line: {100 * p['frac_bf16_peak']:.1f}%).  HBM-side traffic "
                  f"{tr / 1e6:.0f} MB per call against {r.get('algorithmic_bytes', 0) / 1e6:.0f} MB of algorithmic "
                  f"bytes (q, out, the live fp8 K/V once): "
                  f"{tr / r['algorithmic_bytes'] if r.get('algorithmic_bytes') else float('nan'):.1f}x, the image pass "
                  "writing the bf16 images and the key loop re-reading them from each XCD; at under 0.2 TB/s this is "
                  "not what bounds the call.", ""]
        with open(os.path.join(ROOT, "profiles", fname + ".md"), "w") as f:
            f.write("\n".join(L))
        print(f"wrote profiles/{fname}.md")


def _stats(ms):
    return {"mean_ms": statistics.fmean(ms), "median_ms": statistics.median(ms), "min_ms": min(ms),
            "p90_ms": _pct(ms, 0.9), "max_ms": max(ms)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="prefill tokens in the CPU-baseline sample (256: the workload's sampled rows; 0: skip "
                         "the CPU baseline)")
    ap.add_argument("--only", choices=["all", "vjepa2", "dinov3", "decode", "prefill", "next"], default="all",
                    help="run a single workload of the step (profiling runs)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the workload variants reported under parts.next (profiling runs of the step)")
    ap.add_argument("--pcp-shapes", action="store_true",
                    help="only time the paged prefill at the PCP page's Q-scaling shapes (markdown table)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 4 times (scales the rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="no GPU: write profiles/traffic.json and print tables from rocprofv3 CSV output in DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 4}))
        return
    if args.pcp_shapes:
        pcp_shapes()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import transformer_attention_attn_amd as taa

    taa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _log("[bench] generating inputs")
    encs = {"vjepa2_encoder_block_s2048": W.encoder_vjepa2(), "dinov3_encoder_block_s789": W.encoder_dinov3()}
    dec = W.decode_gemma()
    pre = W.prefill_paged()

    class EncDev:
        def __init__(self, c):
            self.c = c
            self.q, self.k, self.v = (t.to(dev) for t in (c.q, c.k, c.v))
            self.res, self.g, self.b = c.residual.to(dev), c.gamma.to(dev), c.beta.to(dev)
            self.out = torch.empty_like(self.q)
            self.rout = torch.empty_like(self.res)
            self.ln = torch.empty(c.B, c.S, c.H * c.D, dtype=torch.bfloat16, device=dev)
            self.mean = torch.empty(c.B * c.S, device=dev)
            self.rstd = torch.empty(c.B * c.S, device=dev)

        def block(self):
            c = self.c
            taa.attn_encoder_fwd(self.q, self.k, self.v, c.scale, None, out=self.out, residual=self.res,
                                 residual_out=self.rout, gamma=self.g, beta=self.b, eps=c.eps, ln_out=self.ln,
                                 ln_mean=self.mean, ln_rstd=self.rstd)

        def attention(self):
            taa.attn_encoder_fwd(self.q, self.k, self.v, self.c.scale, None, out=self.out, want_ln=False)

    which = {"vjepa2": "vjepa2_encoder_block_s2048", "dinov3": "dinov3_encoder_block_s789"}
    run_enc = [k for k in encs if args.only == "all" or which.get(args.only) == k]
    run_dec = args.only in ("all", "decode")
    run_pre = args.only in ("all", "prefill")
    if args.only == "next":
        args.steps = args.warmup = 0
    e_dev = {k: EncDev(encs[k]) for k in run_enc}

    d_q, d_k, d_v, d_m = (t.to(dev) for t in (dec.q, dec.k, dec.v, dec.mask))
    d_out = torch.empty_like(d_q)
    d_ws = torch.empty(taa.attn_decode_gqa_workspace_size(dec.B, dec.Hq, dec.S_ctx, dec.D), dtype=torch.uint8,
                       device=dev)

    p_q, p_k, p_v, p_bt = (t.to(dev) for t in (pre.q, pre.k_cache, pre.v_cache, pre.block_table))
    p_out = torch.empty_like(p_q)
    p_ws = torch.empty(taa.attn_prefill_paged_expanded_workspace_size(pre.Hkv, pre.L_act, pre.D), dtype=torch.uint8,
                       device=dev)
    # 512 MiB written before every decode call (outside its timer), so its
    # ~134 MB of K/V come from HBM and not from the 256 MB Infinity Cache.
    # The encoder blocks and the prefill are timed warm (compute-bound: their
    # inputs are re-read from L2/MALL many times within one call anyway).
    flush = torch.empty(512 * 1024 * 1024 // 4, device=dev)
    torch.cuda.synchronize()

    t_enc = {k: Timer() for k in run_enc}
    t_dec, t_pre = Timer(), Timer()

    def step(timed: bool):
        for k in run_enc:
            s_ = t_enc[k].start() if timed else None
            e_dev[k].block()
            if timed:
                t_enc[k].stop(s_)
        if run_dec:
            flush.zero_()
            s_ = t_dec.start() if timed else None
            taa.attn_decode_gqa(d_q, d_k, d_v, d_m, dec.scale, dec.G, out=d_out, workspace=d_ws)
            if timed:
                t_dec.stop(s_)
        if run_pre:
            s_ = t_pre.start() if timed else None
            taa.attn_prefill_paged_expanded(p_q, p_k, p_v, pre.k_scale, pre.v_scale, p_bt, pre.L_act, pre.scale,
                                            pre.G, out=p_out, workspace=p_ws)
            if timed:
                t_pre.stop(s_)

    _log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    _log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps if args.steps else 0.0

    lens = dec.lens.tolist()
    f_dec = 4 * sum(lens) * dec.Hq * dec.D  # each query head attends len_b keys of its batch row
    f_pre = acc.prefill_flops(pre.Lq, pre.Hq, pre.L_act, pre.D)
    b_dec = acc.decode_bytes(lens, dec.Hkv, dec.Hq, dec.S_ctx, dec.D)
    f_enc = {k: acc.encoder_flops(c.B, c.H, c.S, c.S, c.D) for k, c in encs.items()}
    total_flops = sum(f_enc[k] for k in run_enc) + (f_dec if run_dec else 0) + (f_pre if run_pre else 0)

    parts = {}

    def gpu_timed(fn, n):
        """Per-call GPU time of fn: a spin kernel (about 60 us) holds the stream
        while the host enqueues the start event, the call and the end event, so
        each event window holds the call's kernels only, not the host's
        enqueue time (which exceeds a 20 us kernel)."""
        t = Timer()
        for _ in range(n):
            torch.cuda._sleep(150_000)
            s_ = t.start()
            fn()
            t.stop(s_)
        torch.cuda.synchronize()
        return t.ms()

    # the encoder blocks and their attention alone (epilogue pointers null),
    # timed after the step loop, warm; in the step itself a block's events
    # also cover the host's enqueue time
    for k in run_enc:
        if not args.steps:
            break
        e = e_dev[k]
        for _ in range(3):
            e.attention()
        # at least 50 calls each (~0.1 ms apiece): the mean of a few 20-40 us
        # calls moves by several percent with one slow call
        ms_b = gpu_timed(e.block, max(args.steps, 50))
        ms_a = gpu_timed(e.attention, max(args.steps, 50))

        def back_to_back(fn, n=50):
            """Mean GPU time per call of n calls enqueued back to back between
            two events (as in a model's layer loop: each launch overlaps the
            previous call's tail)."""
            torch.cuda._sleep(150_000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        bb_b, bb_a = back_to_back(e.block), back_to_back(e.attention)
        c = encs[k]
        tf_b = f_enc[k] / (statistics.fmean(ms_b) * 1e-3) / 1e12
        tf_a = f_enc[k] / (statistics.fmean(ms_a) * 1e-3) / 1e12
        scores = c.B * c.H * c.S * c.S
        bound_us = acc.softmax_valu_bound_us(scores)
        parts[k] = {
            **_stats(ms_b), "tflops": tf_b, "frac_bf16_peak": tf_b / acc.PEAK_BF16_TFLOPS, "flops": f_enc[k],
            "kernels": "attention + fp32 residual epilogue, res_ln (LayerNorm over H*D)",
            "shape": {"B": c.B, "H": c.H, "S": c.S, "D": c.D, "hidden": c.H * c.D},
            "attention_only": {**_stats(ms_a), "tflops": tf_a, "frac_bf16_peak": tf_a / acc.PEAK_BF16_TFLOPS,
                               "back_to_back_ms": bb_a,
                               "back_to_back_frac_bf16_peak": f_enc[k] / (bb_a * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS},
            "back_to_back_ms": bb_b,
            "back_to_back_frac_bf16_peak": f_enc[k] / (bb_b * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS,
            "epilogue_and_ln_ms": statistics.fmean(ms_b) - statistics.fmean(ms_a),
            "in_step_events_mean_ms": statistics.fmean(t_enc[k].ms()),
            "timing": "per call, HIP events behind a spin kernel (GPU time of the call's kernels), warm; "
                      "back_to_back_*: 50 calls between two events, per call",
            "mfma_bound_us": f_enc[k] / acc.PEAK_BF16_TFLOPS / 1e6,
            "valu_bound": {"us": bound_us, "scores": scores,
                           "per_score": f"{acc.SOFTMAX_EXP_PER_SCORE:g} exp2 (16 cycles per wave64) + "
                                        f"{acc.SOFTMAX_FULL_RATE_PER_SCORE:g} full-rate VALU ops (4 cycles): FMA, "
                                        "half a max3, half a bf16 pack, half a dot2 row sum",
                           "attention_frac_of_bound": bound_us / (statistics.fmean(ms_a) * 1e3)},
        }
    if run_dec and args.steps:
        ms = t_dec.ms()
        gbs = b_dec / (statistics.fmean(ms) * 1e-3) / 1e9
        parts["gemma_gqa_decode_d256_ctx4096"] = {
            **_stats(ms), "gbps": gbs, "frac_hbm_peak": gbs / acc.PEAK_HBM_GBPS, "bytes": b_dec,
            "dense_equiv_gbps": acc.decode_dense_bytes(dec.B, dec.Hkv, dec.Hq, dec.S_ctx, dec.D)
            / (statistics.fmean(ms) * 1e-3) / 1e9, "kernels": "split-K, combine",
            "timing": "512 MiB written before each call (outside its events): K/V come from HBM"}
    if run_pre and args.steps:
        ms = t_pre.ms()
        tf = f_pre / (statistics.fmean(ms) * 1e-3) / 1e12
        parts["paged_fp8_prefill_q4096_hist120000"] = {
            **_stats(ms), "tflops": tf, "frac_bf16_peak": tf / acc.PEAK_BF16_TFLOPS, "flops": f_pre,
            "tflops_at_131072_convention": acc.prefill_flops(pre.Lq, pre.Hq, 131072, pre.D)
            / (statistics.fmean(ms) * 1e-3) / 1e12,
            "kernels": "tile images (fp8 history -> bf16), key loop"}

    roofline = None
    if run_pre and args.steps:
        p = parts["paged_fp8_prefill_q4096_hist120000"]
        # one prefill call = the tile-image pass + the key loop; both count
        # toward its time (achieved) and its HBM bytes (traffic)
        t_img, t_loop = measured_traffic("prefill_tile_images_kernel"), measured_traffic("prefill_paged_kernel")
        # algorithmic bytes: q and out bf16, the live fp8 history K/V once
        alg = 2 * pre.Hq * pre.Lq * pre.D * 2 + 2 * pre.Hkv * pre.L_act * pre.D
        traffic = t_img + t_loop if t_img is not None and t_loop is not None else None
        roofline = {"bound": "mfma", "achieved": p["tflops"], "peak": acc.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": p["tflops"] / acc.PEAK_BF16_TFLOPS, "traffic": traffic,
                    "algorithmic_bytes": alg, "traffic_over_algorithmic": traffic / alg if traffic else None,
                    "kernel": "prefill_tile_images_kernel + prefill_paged_kernel",
                    "kernel_source_hash": kernel_source_hash()}
    elif run_enc and args.steps:
        p = parts[run_enc[0]]
        roofline = {"bound": "mfma", "achieved": p["tflops"], "peak": acc.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": p["frac_bf16_peak"], "traffic": None, "kernel": "encoder_fwd_kernel+res_ln_kernel"}
    elif run_dec and args.steps:
        p = parts["gemma_gqa_decode_d256_ctx4096"]
        roofline = {"bound": "hbm", "achieved": p["gbps"], "peak": acc.PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": p["frac_hbm_peak"], "traffic": None, "kernel": "decode_split_kernel+decode_combine_kernel"}

    if args.only in ("all", "next") and not args.no_next:
        _log("[bench] workload variants")
        parts["next"] = time_next_workloads(taa, dev, flush, (pre, p_q, p_k, p_v, p_bt))

    cpu = None
    if args.cpu_rows > 0 and args.only == "all":
        _log(f"[bench] cpu baseline: oracle on workloads 1-4 and {args.cpu_rows} prefill tokens")
        cases = {"tiny_sdpa_s128_block": W.encoder_tiny(), **encs, "gemma_gqa_decode_d256_ctx4096": dec}
        cpu = cpu_baseline(cases, pre, args.cpu_rows)

    line = {
        "metric": "attn TFLOP/s & % MFMA peak (encoder/prefill); decode GB/s & % HBM peak",
        "value": total_flops / (ms_step * 1e-3) / 1e12 if ms_step else 0.0,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' workloads, no weights or datasets)",
        "config": {
            "workload": "vjepa2_encoder_block_s2048 + dinov3_encoder_block_s789 + gemma_gqa_decode_d256_ctx4096 + "
                        "paged_fp8_prefill_q4096_hist120000" if args.only == "all" else args.only,
            "encoders": {k: {"B": c.B, "H": c.H, "S": c.S, "D": c.D, "residual_ln_hidden": c.H * c.D}
                         for k, c in encs.items()},
            "decode": {"B": dec.B, "Hq": dec.Hq, "Hkv": dec.Hkv, "S_ctx": dec.S_ctx, "D": dec.D, "sum_len": sum(lens)},
            "prefill": {"Lq": pre.Lq, "Hq": pre.Hq, "Hkv": pre.Hkv, "D": pre.D, "block_size": pre.block_size,
                        "actual_history_len": pre.L_act, "kv": "fp8_e4m3fn"},
            "parallelism": "single GPU",
        },
        "parts": parts,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
