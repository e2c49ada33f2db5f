"""The FLOP/byte model reproduces the figures the pages print (tests/golden/pages_figures.json)."""
import json
import os

import pytest

from block_sparse_attention_head_amd import perfmodel as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_per_token_compute_reduction_28_4x():
    r = P.per_token_compute_ratio(N=2 ** 20, h_q=64, h_idx=4, d=128, d_idx=128, top_k=16, block=128)
    assert round(r, 1) == GOLD["per_token_compute_reduction"]["value"]
    assert r == pytest.approx(28.44, abs=0.01)


def test_kv_outer_vs_q_outer_intensity():
    g = GOLD["kv_outer_intensity"]
    assert round(P.kv_outer_intensity(g["block"], 128)) == g["value"]
    assert P.q_outer_intensity(g["group"]) == g["q_outer_value"]


def test_tokens_per_query():
    # attended keys: top_k - 1 full blocks plus the causal part of the query's own block
    assert 16 * 128 == GOLD["tokens_per_query"]["value"]
    N = 128 * 40
    s = P.sum_attended_keys(N, 16)
    # brute force
    brute = sum(128 * (min(16, t // 128 + 1) - 1) + t % 128 + 1 for t in range(N))
    assert s == brute
    assert P.sum_valid_blocks(N, 16) == sum(min(16, t // 128 + 1) for t in range(N))


def test_flops_of_the_128k_workload():
    s = P.Shape(batch=1, seqlen=131072, h_q=64, h_kv=4, top_k=16)
    assert P.index_flops(s) == pytest.approx(8.796e12, rel=1e-3)
    brute_keys = sum(128 * (min(16, t // 128 + 1) - 1) + t % 128 + 1 for t in range(0, 131072))
    assert P.main_flops(s) == 4 * 128 * 64 * brute_keys
    assert P.bwd_flops(s) == 2.5 * P.main_flops(s)
    assert P.pair_rows(s) == 4 * 16 * sum(min(16, t // 128 + 1) for t in range(131072))


def test_stage_bytes_with_the_local_block_in_the_combine():
    # top_k <= 16: each query's own block leaves the partial phase (one row per query
    # head and position), and the combine reads the query rows and each block's K/V once
    s = P.Shape(batch=1, seqlen=4096, h_q=8, h_kv=2, top_k=4)
    pairs = 8 * sum(min(4, t // 128 + 1) for t in range(4096))
    entries = 2 * sum(min(4, t // 128 + 1) for t in range(4096))
    kv = 2 * 32 * 2 * 128 * 128 * 2
    local = 8 * 4096
    assert P.partial_bytes(s) == (pairs - local) * (256 + 256 + 4) + kv + (entries - 2 * 4096) * 4
    out = 4096 * 8 * (256 + 4)
    sel = 2 * 4096 * 4 * 4
    assert P.combine_bytes(s) == (pairs - local) * (256 + 4) + sel + out + 4096 * 8 * 256 + kv
    # the own block's keys up to each position: 128 * 129 / 2 per block of positions
    assert P.local_block_flops(s) == 4 * 128 * 8 * 32 * (128 * 129 // 2)
    assert P.partial_flops(s) == P.main_flops(s) - P.local_block_flops(s)
    # past 16 slots every pair goes through the partial phase and its record
    t = P.Shape(batch=1, seqlen=4096, h_q=8, h_kv=2, top_k=17)
    pt = 8 * sum(min(17, u // 128 + 1) for u in range(4096))
    assert P.combine_bytes(t) == pt * (256 + 4) + 2 * 4096 * 17 * 4 + out
    assert P.partial_flops(t) == P.main_flops(t)


def test_decode_bytes_closed_form():
    from block_sparse_attention_head_amd.perfmodel import decode_bytes

    # L = 1000: t = 999, c_loc = 7; top_k = 4 -> blocks 3 full + local keys 896..999 (104)
    b = decode_bytes([1000], h_q=8, h_kv=2, top_k=4)
    assert b["index"] == 1000 * 256 + 2 * 256 + 2 * 8 * 4
    assert b["topk"] == 2 * (7 * 4 + 4 * 4)
    assert b["attn"] == 2 * ((3 * 128 + 104) * 512 + 16) + 8 * (512 + 4)
    # short sequence: every block, an empty one adds nothing
    s = decode_bytes([200, 0], h_q=4, h_kv=1, top_k=16)
    assert s["attn"] == (128 + 72) * 512 + 64 + 4 * 516


def test_index_bwd_flops_closed_form():
    from block_sparse_attention_head_amd.perfmodel import Shape, index_bwd_flops, sum_attended_keys

    s = Shape(batch=2, seqlen=1024, h_q=8, h_kv=2, top_k=4)
    # per attended (position, group, key): the G = 4 main heads' scores plus three index products
    assert index_bwd_flops(s) == 2 * sum_attended_keys(1024, 4) * (2 * 128 * 8 + 3 * 2 * 128 * 2)
