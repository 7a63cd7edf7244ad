"""Pins of the work and byte conventions the benchmark reports throughput with."""

import json
import os

import numpy as np
import pytest

import oracle
from scaled_dot_product_flash_amd import work

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_flop_table_of_kv_cache_section():
    # Last-step FLOPs printed for a 64-dim single-layer attention: without a
    # cache, Q/K/V projections of all n tokens (6nD^2), dense n x n attention
    # and the output projection of the new token (2D^2); with a cache, four
    # projections of one token (8D^2) and attention of one query over n keys.
    t = _load("p5_flop_table.json")
    D = t["D"]
    for row in t["rows"]:
        n = row["n"]
        assert 6 * n * D * D + work.attention_flops(n * n, D) + 2 * D * D == row["no_cache"]
        assert 8 * D * D + work.attention_flops(n, D) == row["cache"]


def test_kv_bytes_table():
    t = _load("p5_kv_bytes_table.json")
    for row in t["rows"]:
        per_token = t["layers"] * work.kv_bytes_per_token(row["kv_heads"], t["head_dim"], t["elem_bytes"])
        assert per_token == row["bytes_per_token"]
        assert per_token * 131072 / 2**30 == row["gib_at_131072"]


@pytest.mark.parametrize("Sq,Sk,causal,window", [
    (1, 1, False, 0), (7, 7, True, 0), (5, 13, True, 0), (64, 64, True, 1), (64, 64, True, 17),
    (30, 90, True, 40), (100, 100, True, 1000), (9, 31, False, 0), (1, 50, True, 8),
])
def test_visible_pairs_counts_the_oracle_mask(Sq, Sk, causal, window):
    assert work.visible_pairs(Sq, Sk, causal, window) == int(oracle.visible(Sq, Sk, causal, window).sum())


def test_workload_flops_match_closed_forms():
    # pairs per head of the benchmark workloads, from their sizes
    assert work.visible_pairs(1024, 1024, True, 0) == 1024 * 1025 // 2
    assert work.visible_pairs(4096, 4096, True, 0) == 4096 * 4097 // 2
    assert work.visible_pairs(16384, 16384, True, 4096) == 4096 * 4097 // 2 + (16384 - 4096) * 4096
    assert work.prefill_flops(4, 32, 4096, 4096, 128, True, 0) == 4 * 4 * 32 * 128 * (4096 * 4097 // 2)


def test_decode_bytes():
    lens = np.array([512, 8192, 1000])
    assert work.decode_kv_bytes(lens, 8, 128) == int(lens.sum()) * 2 * 8 * 128 * 2


def test_decode_window_bytes():
    from scaled_dot_product_flash_amd import work

    lens = [1, 100, 4096, 5000]
    per = work.kv_bytes_per_token(8, 128, 2)
    assert work.decode_window_kv_bytes(lens, 8, 128, 0) == work.decode_kv_bytes(lens, 8, 128)
    assert work.decode_window_kv_bytes(lens, 8, 128, 4096) == (1 + 100 + 4096 + 4096) * per
    assert work.decode_window_kv_bytes(lens, 8, 128, 1) == 4 * per
    # the windowed pair count of one query at the end of n keys is min(n, W)
    for n in lens:
        assert work.visible_pairs(1, n, True, 4096) == min(n, 4096)


def test_backward_flops_is_five_products_per_pair():
    # five matrix products of 2·D flop per visible pair = 2.5x the forward's 4·D
    for args in [(4, 32, 4096, 4096, 128, True, 0), (1, 2, 100, 300, 64, False, 0), (1, 4, 50, 50, 128, True, 7)]:
        assert work.backward_flops(*args) * 2 == 5 * work.prefill_flops(*args)
    assert work.backward_flops(1, 1, 3, 3, 2, True, 0) == 10 * 2 * 6
