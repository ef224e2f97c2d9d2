"""Oracle cell-size helpers against every byte count the pages print.

Fixture: tests/golden/cell_sizes.json (each case cites its page and section).
"""
import json
import os

import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cell_sizes.json")))


@pytest.mark.parametrize("case", GOLD["gqa"], ids=lambda c: c["name"])
def test_gqa_cell_bytes(case):
    per_tok = oracle.kv_cell_bytes(case["L"], case["h_kv"], case["d_h"], case["b"])
    assert per_tok * case["tokens"] == case["bytes"]


@pytest.mark.parametrize("case", GOLD["mla"], ids=lambda c: c["name"])
def test_mla_cell_bytes(case):
    per_tok = oracle.mla_cell_bytes(case["L"], case["d_c"], case["d_R"], case["b"])
    assert per_tok * case["tokens"] == case["bytes"]


@pytest.mark.parametrize("case", GOLD["ratios"], ids=lambda c: c["name"])
def test_printed_ratios(case):
    m, l = case["mha"], case["mla"]
    r = oracle.kv_cell_bytes(m["L"], m["h_kv"], m["d_h"], m["b"]) / \
        oracle.mla_cell_bytes(l["L"], l["d_c"], l["d_R"], l["b"])
    assert round(r, case["decimals"]) == case["printed"]


def test_cell_second_route_llama3_8b():
    # "The KV cache size formula": one K vector is 8 x 128 elements at 2 bytes
    # = 2 KiB, K plus V 4 KiB per layer, 32 layers = 128 KiB.
    k_vec = 8 * 128 * 2
    assert k_vec == 2048
    assert oracle.kv_cell_bytes(1, 8, 128, 2) == 2 * k_vec
    assert oracle.kv_cell_bytes(32, 8, 128, 2) == 32 * 2 * k_vec == 128 * 1024


def test_gqa_formula_on_mla_logical_shape_overestimates_71x():
    # "The KV cache size formula": plugging DeepSeek-V3's logical shapes into
    # the GQA formula, 61 x 128 x (192 + 128) x 2, gives 4.77 MiB, 71x too much.
    logical = 61 * 128 * (192 + 128) * 2
    assert round(logical / 2**20, 2) == 4.77
    assert round(logical / oracle.mla_cell_bytes(61, 512, 64, 2)) == 71
