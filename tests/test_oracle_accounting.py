"""Pins of the oracle's byte accounting against the figures the page prints
(tests/golden/page3_figures.json, each entry citing its page section).
GB is 10**9 bytes; printed values are compared at their printed rounding."""
import json
import os

import pytest

from oracle import accounting as acc


@pytest.fixture(scope="module")
def page(golden_dir):
    raw = json.load(open(os.path.join(golden_dir, "page3_figures.json")))
    return {k: v["value"] for k, v in raw.items() if not k.startswith("_")}


def rounds_to(x, printed, decimals):
    return round(x, decimals) == pytest.approx(printed, abs=10 ** -(decimals + 3))


def test_layer_slab_is_exactly_three_bits_per_weight(page):
    assert acc.weights_per_layer() == 192_937_984
    assert acc.slab_bytes() == page["slab_bytes"]
    assert page["slab_bytes"] * 8 == 3 * acc.weights_per_layer()


def test_attention_feed_forward_split(page):
    assert rounds_to(100 * acc.attention_share(), page["attention_pct"], 1)
    assert rounds_to(100 * acc.feed_forward_share(), page["feed_forward_pct"], 1)
    assert acc.attention_share() + acc.feed_forward_share() == pytest.approx(1.0, abs=1e-15)


def test_ternary_lane_vocab_tables_and_file(page):
    assert acc.N_LAYERS == page["n_layers"]
    assert acc.VOCAB == page["vocab_rows"] and acc.HIDDEN == page["vocab_cols"]
    assert rounds_to(acc.ternary_lane_bytes() / 1e9, page["ternary_lane_gb"], 2)
    assert rounds_to(acc.vocab_table_bytes() / 1e9, page["vocab_tables_gb"], 2)
    assert acc.METADATA_BYTES == page["metadata_mb"] * 10 ** 6
    assert rounds_to(acc.file_bytes() / 1e9, page["file_gb"], 2)
    assert rounds_to(100 * acc.ternary_lane_bytes() / acc.file_bytes(), page["ternary_lane_pct"], 1)
    assert rounds_to(100 * acc.vocab_table_bytes() / acc.file_bytes(), page["vocab_tables_pct"], 1)


def test_fp16_size_is_about_sixteen_gb_and_four_times_the_file(page):
    assert round(acc.fp16_bytes() / 1e9) == page["fp16_gb_about"]
    assert round(acc.fp16_bytes() / acc.file_bytes()) == page["fp16_ratio_about"]


def test_quoted_traffic_rates_are_file_size_times_token_rate(page):
    assert round(acc.file_traffic_rate(page["h100_tok_s"]) / 1e12, 1) == page["h100_tb_s_about"]
    # "about 97": the printed 3.88 GB file times 24.9 tok/s is 96.6 GB/s
    assert round(page["file_gb"] * page["m5_cpu_tok_s"]) == page["m5_cpu_gb_s_about"]
    assert abs(acc.file_traffic_rate(page["m5_cpu_tok_s"]) / 1e9 - page["m5_cpu_gb_s_about"]) < 1.0


def test_kv_cache_accounting(page):
    assert acc.KV_HEADS == page["kv_heads"] and acc.HEAD_DIM == page["head_dim"]
    assert acc.kv_bytes_per_position() == page["kv_bytes_per_position"]
    assert acc.kv_bytes_per_position() == page["kv_kib_per_position"] * 1024
    for tokens, gb in page["kv_gb_at_tokens"].items():
        assert rounds_to(acc.kv_bytes(int(tokens)) / 1e9, gb, 2)
    cross = acc.kv_crossover_tokens()
    assert acc.kv_bytes(cross) > acc.file_bytes() >= acc.kv_bytes(cross - 1)
    assert round(cross, -3) == page["kv_crossover_tokens_about"]
    assert acc.Q_HEADS == page["kv_all_query_heads"]
    assert acc.kv_all_heads_ratio() == page["kv_all_heads_ratio"]


def test_speculative_cycle_bytes_are_about_one_fifth(page):
    f = acc.draft_cycle_fraction(6, page["draft_bytes_ratio"])
    assert round(f, 1) == page["draft_cycle_fraction_about"]


def test_build_format_step_bytes():
    """The 2-bit format's per-step bytes: closed form from the shapes."""
    b = acc.step_bytes()
    assert b["ternary_weights"] == 36 * 192_937_984 // 4 == 1_736_441_856
    assert b["ternary_scales"] == 36 * 38_912 * 4
    assert b["output_table"] == 151_936 * 4096 + 151_936 * 4
    assert b["total"] == 2_364_986_884
    assert acc.level_bytes(6144, 4096) == 6_316_032
    assert acc.level_bytes(24576, 4096) == 25_264_128
    assert acc.level_bytes(4096, 12288) == 12_599_296
    assert acc.step_bytes(bits_per_weight=3)["total"] == 3_233_207_812
