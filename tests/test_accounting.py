"""The FLOP accounting reproduces the throughput arithmetic the pages print."""
import json
import os

from workloads import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_throughput_figures.json")))


def test_vit_l_closed_form_flops_and_mfu():
    g = GOLD["vjepa2_encoder"]
    f = acc.vit_encoder_flops(**g["geometry"])
    assert abs(f - g["model_flops"]) / g["model_flops"] < 5e-5
    peak = g["peak_tflops_per_logical_core"] * 1e12
    for key in ("stock", "kernels"):
        mfu = 100 * f / (g["latency_ms"][key] * 1e-3) / peak
        assert abs(mfu - g["mfu_percent"][key]) < 0.1


def test_attention_is_a_quarter_of_vit_l():
    g = GOLD["vjepa2_encoder"]["geometry"]
    att = g["layers"] * acc.encoder_flops(1, 16, g["tokens"], g["tokens"], 64)
    assert abs(att / acc.vit_encoder_flops(**g) - 0.249) < 0.001


def test_pcp_mfu_tables():
    for key in ("pcp_q_scaling_hist8192",):
        g = GOLD[key]
        peak = g["chips"] * g["peak_tflops_per_chip"] * 1e12
        for Lq, ms, mfu in g["rows"]:
            f = acc.prefill_flops(Lq, g["Hq"], g["history"], g["D"])
            assert abs(100 * f / (ms * 1e-3) / peak - mfu) < 0.01
    g = GOLD["pcp_ladder_q1k"]
    peak = g["chips"] * g["peak_tflops_per_chip"] * 1e12
    f = acc.prefill_flops(g["Lq"], g["Hq"], g["history"], g["D"])
    for ms, mfu in g["rows"]:
        assert abs(100 * f / (ms * 1e-3) / peak - mfu) < 0.005


def test_pcp_full_machine():
    g = GOLD["pcp_full_machine"]
    f = acc.prefill_flops(g["Lq"], g["Hq"], g["history"], g["D"])
    assert abs(100 * f / (g["device_ms"] * 1e-3) / (g["chips"] * g["peak_tflops_per_chip"] * 1e12)
               - g["mfu_percent"]) < 0.01
    assert abs(g["Lq"] / (g["mean_ms"] * 1e-3) - g["tokens_per_s"]) < 1.0


def test_decode_bytes():
    # one KV head, one row of 3 keys, D=4: K+V 3*4*2*2, mask 8*4, q+out 2*1*4*2
    assert acc.decode_bytes([3], 1, 1, 8, 4) == 48 + 32 + 16


def test_decode_window_bytes():
    # two sequences of 3 and 5 in-range keys, 2 KV / 4 query heads, D=8:
    # K+V 8*2*8*2*2, q+out 2*2*4*8*2, no mask
    assert acc.decode_window_bytes([3, 5], 2, 4, 8) == 512 + 256


def test_causal_flops():
    # 3 tokens see 1, 2, 3 keys: 6 (query, key) pairs, 4*D FLOPs each, 2 heads
    assert acc.causal_flops(3, 2, 8) == 6 * 4 * 8 * 2
