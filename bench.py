#!/usr/bin/env python3
"""Benchmark of the flash-attention hot path on one MI355X.

One step = one pass over every kernel of the path, each on its workload:
  * encoder block: V-JEPA2 ViT-L attention (B=1, 16 heads, 2048 tokens, D=64,
    bf16) + residual add into the fp32 [2048,1024] stream + LayerNorm;
  * GQA decode: B=8, 16 query / 8 KV heads, head_dim 256, S_ctx 4096,
    ragged lengths len_b ~ U{1..4096};
  * paged FP8 prefill: 4096 query tokens x 32 heads over 2 KV heads, D=256,
    512-token blocks under a permuted block table, 120000 live history keys,
    through its workspace (the live history expanded to bf16 tile images,
    then the key loop; both kernels inside the timed call).
All inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line.  `value` is the step's attention throughput (QK^T + PV
FLOPs of the three attention calls over the step time); `parts` gives each
kernel's own metric (TFLOP/s and % of the bf16 MFMA peak, or GB/s and % of
HBM peak) from HIP events recorded on the stream the kernels run on;
`roofline` is the dominant call's (the prefill: its two kernels).  `cpu_baseline` times the
fp64 oracle on a bounded sample of the prefill workload on the host cores.
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


def cpu_baseline(pre, n_rows: int):
    """Time the fp64 oracle on n_rows query tokens x all heads of the prefill."""
    import oracle

    oracle.build()
    rows = pre.rows[:n_rows]
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    t0 = time.perf_counter()
    oracle.prefill_paged(pre.q, pre.k_cache, pre.v_cache, pre.k_scale, pre.v_scale, pre.block_table, pre.L_act,
                         pre.scale, rows)
    dt = time.perf_counter() - t0
    flops = acc.prefill_flops(len(rows), pre.Hq, pre.L_act, pre.D)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, cores), "kind": "oracle",
            "sample": f"paged FP8 prefill, {len(rows)} query tokens x {pre.Hq} heads x {pre.L_act} keys "
                      f"(fp64 C oracle incl. KV decode), {dt:.1f} s wall"}


def time_next_workloads(taa, dev, flush, pre_dev, reps: int = 20):
    """Workload variants beyond the step (reported, not part of `value`):
    the 64-frame V-JEPA 2 clip (8192 tokens), a gte-base batch right-padded to
    512 tokens with ragged real lengths (additive key mask), both timed as
    back-to-back launches between two HIP events after 3 warm-up calls; and
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
    for k in ("prefill_paged_kernel", "prefill_tile_images_kernel", "encoder_fwd_kernel", "res_ln_kernel",
              "decode_split_kernel", "decode_combine_kernel", "copyBuffer"):
        if k in name:
            return k
    return None


def summarize(prof_dir: str) -> None:
    """Turn the rocprofv3 CSV output of the profiling commands (kernel trace in
    <dir>/trace, FETCH_SIZE / WRITE_SIZE passes of the bench in <dir>/<C> and of
    --copy-calibration in <dir>/<C>_copy) into profiles/traffic.json, and print
    the per-kernel duration and traffic tables.  Reads CSV only; no GPU."""
    import csv
    import glob

    def one(pattern):
        hits = sorted(glob.glob(os.path.join(prof_dir, pattern)))
        if not hits:
            raise SystemExit(f"summarize: no {pattern} under {prof_dir}")
        return hits[0]

    def per_dispatch(path):
        vals = {}
        for r in csv.DictReader(open(path)):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        fam = {}
        for (_, name), v in vals.items():
            if _short(name):
                fam.setdefault(_short(name), []).append(v)
        return {k: statistics.fmean(v) for k, v in fam.items()}

    stats = {}
    for r in csv.DictReader(open(one("trace/*kernel_stats.csv"))):
        if not _short(r["Name"]):  # not one of this library's kernels (e.g. the cache flush)
            continue
        if _short(r["Name"]) in stats:
            raise SystemExit(f"summarize: two kernels of family {_short(r['Name'])} in the trace; profile the "
                             "step alone (bench.py --no-next)")
        stats[_short(r["Name"])] = {"kernel": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                                    "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        kib = per_dispatch(one(f"{c}_copy/*counter_collection.csv"))["copyBuffer"]
        cal[c] = kib * 1024 / COPY_BYTES
    fetch = per_dispatch(one("FETCH_SIZE/*counter_collection.csv"))
    write = per_dispatch(one("WRITE_SIZE/*counter_collection.csv"))
    kernels = {}
    for k, st in stats.items():
        if k == "copyBuffer" or k not in fetch or k not in write:
            continue
        kernels[k] = {"kernel": st["kernel"], "fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
                      "hbm_bytes_per_launch": int(fetch[k] * 1024 / cal["FETCH_SIZE"] + write[k] * 1024 / cal["WRITE_SIZE"]),
                      "avg_duration_ns": st["avg_ns"]}
    out = {"source_hash": kernel_source_hash(),
           "note": "rocprofv3 FETCH_SIZE/WRITE_SIZE (KiB per dispatch, L2 <-> memory fabric) divided by the ratio "
                   "the same counter reads for a 1 GiB device copy",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_ratio": cal["FETCH_SIZE"], "write_ratio": cal["WRITE_SIZE"]},
           "kernels": kernels}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"wrote {path} (sources {out['source_hash']}; copy calibration fetch x{cal['FETCH_SIZE']:.4f}, "
          f"write x{cal['WRITE_SIZE']:.4f})")
    print("\n| kernel | calls | avg (us) | min (us) | max (us) |\n|---|---|---|---|---|")
    for k, st in sorted(stats.items(), key=lambda kv: -kv[1]["avg_ns"] * kv[1]["calls"]):
        print(f"| `{st['kernel']}` | {st['calls']} | {st['avg_ns'] / 1e3:.2f} | {st['min_ns'] / 1e3:.2f} | "
              f"{st['max_ns'] / 1e3:.2f} |")
    print("\n| kernel | FETCH_SIZE raw (KiB) | WRITE_SIZE raw (KiB) | scaled bytes / launch |\n|---|---|---|---|")
    for k, v in kernels.items():
        print(f"| {k} | {v['fetch_kib_raw']:.1f} | {v['write_kib_raw']:.1f} | {v['hbm_bytes_per_launch'] / 1e6:.1f} MB |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=160,
                    help="query tokens in the CPU-baseline sample, about 10 s of oracle work on 16 cores (0: skip)")
    ap.add_argument("--only", choices=["all", "encoder", "decode", "prefill", "next"], default="all",
                    help="run a single kernel family (profiling runs)")
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
    enc = W.encoder_vjepa2()
    dec = W.decode_gemma()
    pre = W.prefill_paged()

    e_q, e_k, e_v = (t.to(dev) for t in (enc.q, enc.k, enc.v))
    e_res, e_g, e_b = enc.residual.to(dev), enc.gamma.to(dev), enc.beta.to(dev)
    e_out = torch.empty_like(e_q)
    e_rout = torch.empty_like(e_res)
    e_ln = torch.empty(enc.B, enc.S, enc.H * enc.D, dtype=torch.bfloat16, device=dev)
    e_mean = torch.empty(enc.B * enc.S, device=dev)
    e_rstd = torch.empty(enc.B * enc.S, device=dev)

    d_q, d_k, d_v, d_m = (t.to(dev) for t in (dec.q, dec.k, dec.v, dec.mask))
    d_out = torch.empty_like(d_q)
    d_ws = torch.empty(taa.attn_decode_gqa_workspace_size(dec.B, dec.Hq, dec.S_ctx, dec.D), dtype=torch.uint8,
                       device=dev)

    p_q, p_k, p_v, p_bt = (t.to(dev) for t in (pre.q, pre.k_cache, pre.v_cache, pre.block_table))
    p_out = torch.empty_like(p_q)
    p_ws = torch.empty(taa.attn_prefill_paged_expanded_workspace_size(pre.Hkv, pre.L_act, pre.D), dtype=torch.uint8,
                       device=dev)
    # 512 MiB written before every decode call (outside its timer), so its
    # ~134 MB of K/V come from HBM and not from the 256 MB Infinity Cache
    flush = torch.empty(512 * 1024 * 1024 // 4, device=dev)
    torch.cuda.synchronize()

    t_enc, t_dec, t_pre = Timer(), Timer(), Timer()
    run_enc = args.only in ("all", "encoder")
    run_dec = args.only in ("all", "decode")
    run_pre = args.only in ("all", "prefill")
    if args.only == "next":
        args.steps = args.warmup = 0

    def step(timed: bool):
        if run_enc:
            s = t_enc.start() if timed else None
            taa.attn_encoder_fwd(e_q, e_k, e_v, enc.scale, None, out=e_out, residual=e_res, residual_out=e_rout,
                                 gamma=e_g, beta=e_b, eps=enc.eps, ln_out=e_ln, ln_mean=e_mean, ln_rstd=e_rstd)
            if timed:
                t_enc.stop(s)
        if run_dec:
            flush.zero_()
            s = t_dec.start() if timed else None
            taa.attn_decode_gqa(d_q, d_k, d_v, d_m, dec.scale, dec.G, out=d_out, workspace=d_ws)
            if timed:
                t_dec.stop(s)
        if run_pre:
            s = t_pre.start() if timed else None
            taa.attn_prefill_paged_expanded(p_q, p_k, p_v, pre.k_scale, pre.v_scale, p_bt, pre.L_act, pre.scale,
                                            pre.G, out=p_out, workspace=p_ws)
            if timed:
                t_pre.stop(s)

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

    f_enc = acc.encoder_flops(enc.B, enc.H, enc.S, enc.S, enc.D)
    lens = dec.lens.tolist()
    f_dec = 4 * sum(lens) * dec.Hq * dec.D  # each query head attends len_b keys of its batch row
    f_pre = acc.prefill_flops(pre.Lq, pre.Hq, pre.L_act, pre.D)
    b_dec = acc.decode_bytes(lens, dec.Hkv, dec.Hq, dec.S_ctx, dec.D)
    total_flops = (f_enc if run_enc else 0) + (f_dec if run_dec else 0) + (f_pre if run_pre else 0)

    parts = {}

    def summ(ms):
        return {"mean_ms": statistics.fmean(ms), "median_ms": statistics.median(ms), "min_ms": min(ms),
                "max_ms": max(ms)}

    if run_enc:
        ms = t_enc.ms()
        tf = f_enc / (statistics.fmean(ms) * 1e-3) / 1e12
        parts["encoder_block"] = {**summ(ms), "tflops": tf, "frac_bf16_peak": tf / acc.PEAK_BF16_TFLOPS,
                                  "flops": f_enc, "kernels": "attention+residual, res_ln"}
    if run_dec:
        ms = t_dec.ms()
        gbs = b_dec / (statistics.fmean(ms) * 1e-3) / 1e9
        parts["decode"] = {**summ(ms), "gbps": gbs, "frac_hbm_peak": gbs / acc.PEAK_HBM_GBPS, "bytes": b_dec,
                           "dense_equiv_gbps": acc.decode_dense_bytes(dec.B, dec.Hkv, dec.Hq, dec.S_ctx, dec.D)
                           / (statistics.fmean(ms) * 1e-3) / 1e9, "kernels": "split-K, combine"}
    if run_pre:
        ms = t_pre.ms()
        tf = f_pre / (statistics.fmean(ms) * 1e-3) / 1e12
        parts["prefill"] = {**summ(ms), "tflops": tf, "frac_bf16_peak": tf / acc.PEAK_BF16_TFLOPS, "flops": f_pre,
                            "tflops_at_131072_convention": acc.prefill_flops(pre.Lq, pre.Hq, 131072, pre.D)
                            / (statistics.fmean(ms) * 1e-3) / 1e12,
                            "kernels": "tile images (fp8 history -> bf16), key loop"}

    roofline = None
    if run_pre:
        p = parts["prefill"]
        # one prefill call = the tile-image pass + the key loop; both count
        # toward its time (achieved) and its HBM bytes (traffic)
        t_img, t_loop = measured_traffic("prefill_tile_images_kernel"), measured_traffic("prefill_paged_kernel")
        roofline = {"bound": "mfma", "achieved": p["tflops"], "peak": acc.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": p["tflops"] / acc.PEAK_BF16_TFLOPS,
                    "traffic": t_img + t_loop if t_img is not None and t_loop is not None else None,
                    "kernel": "prefill_tile_images_kernel + prefill_paged_kernel",
                    "kernel_source_hash": kernel_source_hash()}
    elif run_enc:
        p = parts["encoder_block"]
        roofline = {"bound": "mfma", "achieved": p["tflops"], "peak": acc.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": p["frac_bf16_peak"], "traffic": None, "kernel": "encoder_fwd_kernel+res_ln_kernel"}
    elif run_dec:
        p = parts["decode"]
        roofline = {"bound": "hbm", "achieved": p["gbps"], "peak": acc.PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": p["frac_hbm_peak"], "traffic": None, "kernel": "decode_split_kernel+decode_combine_kernel"}

    if args.only in ("all", "next") and not args.no_next:
        parts["next"] = time_next_workloads(taa, dev, flush, (pre, p_q, p_k, p_v, p_bt))

    cpu = None
    if args.cpu_rows > 0 and run_pre:
        _log(f"[bench] cpu baseline: oracle on {args.cpu_rows} prefill tokens")
        cpu = cpu_baseline(pre, args.cpu_rows)

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
            "workload": "vjepa2_encoder_block_s2048 + gemma_gqa_decode_d256_ctx4096 + paged_fp8_prefill_q4096_hist120000"
            if args.only == "all" else args.only,
            "encoder": {"B": enc.B, "H": enc.H, "S": enc.S, "D": enc.D, "residual_ln_hidden": enc.H * enc.D},
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
