"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: a hand-worked
example, a closed form, a special case that reduces to a library attention
routine (torch's scaled_dot_product_attention, float64 on the CPU), brute force
on tiny inputs, or an invariant. Chosen so that a dropped term, a wrong sign,
an off-by-one at a block edge or a transposed operand fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth.msa_inputs import WORKLOADS, make_inputs, small_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _nullinf(x):
    return np.array([[[-np.inf if v is None else v for v in row] for row in head] for head in x], dtype=np.float64)


# ---------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_worked_example.json)
# ---------------------------------------------------------------------------
def test_hand_example_pooled_and_topk():
    g = _golden("hand_worked_example.json")
    B = g["block_size"]
    k_idx = np.array(g["k_idx"], dtype=np.float64)[None]              # [1, N, D]
    q_idx = np.array(g["q_idx_heads"]["values"], dtype=np.float64)[None]  # [1, N, H, D]
    pooled = O.index_scores(q_idx, k_idx, block_size=B)
    np.testing.assert_array_equal(pooled[0], _nullinf(g["expected_pooled"]["values"]))
    for key, k in (("k1", 1), ("k2", 2), ("k3", 3)):
        exp = g["expected_topk"][key]
        exp = exp["values"] if isinstance(exp, dict) else exp
        got = O.block_topk(pooled, k, block_size=B)
        np.testing.assert_array_equal(got[0], np.array(exp, dtype=np.int32), err_msg=key)


def test_hand_example_uniform_attention():
    g = _golden("hand_worked_example.json")
    B, N = g["block_size"], g["seqlen"]
    sel = np.array(g["expected_topk"]["k2"]["values"][0], dtype=np.int32)[None, None]  # [1,1,N,2]
    q = np.zeros((1, N, 1, 1))
    k = np.zeros((1, N, 1, 1))
    v = np.arange(N, dtype=np.float64).reshape(1, N, 1, 1)
    out, lse = O.sparse_attention(q, k, v, sel, softmax_scale=1.0, block_size=B)
    np.testing.assert_allclose(out[0, :, 0, 0], g["uniform_attention"]["expected_O"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(g["uniform_attention"]["expected_n_keys"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Index scores: brute force and a closed form
# ---------------------------------------------------------------------------
def test_index_scores_brute_force_python_loops():
    rng = np.random.default_rng(11)
    Bsz, N, H, D, blk = 2, 13, 3, 5, 4
    q = rng.standard_normal((Bsz, N, H, D))
    k = rng.standard_normal((Bsz, N, D))
    got = O.index_scores(q, k, block_size=blk)
    nblk = -(-N // blk)
    for b in range(Bsz):
        for g in range(H):
            for t in range(N):
                for c in range(nblk):
                    vals = []
                    for j in range(c * blk, min((c + 1) * blk, N)):
                        if j <= t:
                            vals.append(sum(q[b, t, g, e] * k[b, j, e] for e in range(D)))
                    want = max(vals) if vals else -math.inf
                    assert got[b, g, t, c] == pytest.approx(want, abs=1e-12), (b, g, t, c)


def test_index_scores_positions_subset_matches_full():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 300, 2, 8))
    k = rng.standard_normal((1, 300, 8))
    full = O.index_scores(q, k)
    pos = [0, 5, 127, 128, 129, 255, 256, 299]
    part = O.index_scores(q, k, positions=pos)
    np.testing.assert_array_equal(part, full[:, :, pos])


def test_index_scores_monotone_key_closed_form():
    # q = e_0 and k[j, 0] = j: the pooled score of a block is its last visible position.
    N, blk = 700, 128
    q = np.zeros((1, N, 2, 16))
    q[..., 0] = 1.0
    k = np.random.default_rng(0).standard_normal((1, N, 16))
    k[..., 0] = np.arange(N)
    q[..., 1:] = 0.0
    got = O.index_scores(q, k, block_size=blk)
    nblk = -(-N // blk)
    want = np.full((N, nblk), -np.inf)
    for t in range(N):
        for c in range(t // blk + 1):
            want[t, c] = min(c * blk + blk - 1, t)
    np.testing.assert_array_equal(got[0, 0], want)
    np.testing.assert_array_equal(got[0, 1], want)


# ---------------------------------------------------------------------------
# Top-k: brute force, order-statistic certificate, ties, invariants
# ---------------------------------------------------------------------------
def _brute_topk_row(scores, c_loc, k):
    if c_loc + 1 <= k:
        sel = list(range(c_loc + 1))
    else:
        sel = sorted(range(c_loc), key=lambda c: (-scores[c], c))[: k - 1] + [c_loc]
    sel = sorted(sel)
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("k", [1, 2, 4, 7, 8, 9])
def test_topk_brute_force_tiny_workload(k):
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    pooled = O.index_scores(x["q_idx"], x["k_idx"])
    got = O.block_topk(pooled, k)
    for t in range(w.seqlen):
        want = _brute_topk_row(pooled[0, 0, t], t // 128, k)
        assert list(got[0, 0, t]) == want, t


def test_topk_order_statistic_certificate():
    rng = np.random.default_rng(5)
    # integer-valued scores force many exact ties
    pooled = rng.integers(-3, 4, size=(1, 2, 1500, 12)).astype(np.float64)
    k = 5
    got = O.block_topk(pooled, k)
    for g in range(2):
        for t in range(1500):
            cl = t // 128
            sel = [c for c in got[0, g, t] if c >= 0]
            assert cl in sel
            assert len(sel) == min(k, cl + 1)
            if cl + 1 > k:
                chosen = [c for c in sel if c != cl]
                rest = [c for c in range(cl) if c not in chosen]
                keyf = lambda c: (pooled[0, g, t, c], -c)  # larger is better
                assert min(keyf(c) for c in chosen) > max(keyf(c) for c in rest)


def test_topk_zero_scores_tie_closed_form():
    # Q_idx == 0 makes every visible pooled score exactly 0: the lowest blocks win.
    w = small_workload(2048, 4, 1, 5, seed=3)
    x = make_inputs(w)
    q_idx = torch.zeros_like(x["q_idx"])
    pooled = O.index_scores(q_idx, x["k_idx"])
    vis = np.isfinite(pooled)
    assert np.all(pooled[vis] == 0.0)
    got = O.block_topk(pooled, w.top_k)
    for t in range(w.seqlen):
        cl = t // 128
        want = list(range(cl + 1)) if cl + 1 <= w.top_k else list(range(w.top_k - 1)) + [cl]
        assert list(got[0, 0, t][: len(want)]) == want


def test_topk_duplicate_block_lower_index_wins():
    # Key block 5 is an exact copy of block 2, so their full-block pooled scores tie exactly.
    w = small_workload(2048, 4, 1, 4, seed=4)
    x = make_inputs(w)
    k_idx = x["k_idx"].clone()
    k_idx[:, 5 * 128:6 * 128] = k_idx[:, 2 * 128:3 * 128]
    pooled = O.index_scores(x["q_idx"], k_idx)
    got = O.block_topk(pooled, w.top_k)
    rows = np.arange(6 * 128, w.seqlen)
    assert np.all(pooled[0, 0, rows, 5] == pooled[0, 0, rows, 2])
    for t in rows:
        sel = set(got[0, 0, t].tolist())
        if 5 in sel:
            assert 2 in sel, t
    # and the tie is actually exercised: some rows keep block 2 but not block 5
    assert any((2 in got[0, 0, t]) and (5 not in got[0, 0, t]) for t in rows)


def test_topk_local_block_invariants_all_workload_rows():
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    pooled = O.index_scores(x["q_idx"], x["k_idx"])
    sel = O.block_topk(pooled, w.top_k)
    for t in range(w.seqlen):
        cl = t // 128
        row = sel[0, 0, t]
        valid = row[row >= 0]
        assert cl in valid
        assert len(valid) == min(w.top_k, cl + 1)
        assert np.all(np.diff(valid) > 0)          # ascending, no duplicates
        assert valid.max() <= cl
        assert np.all(row[len(valid):] == -1)      # padding only at the end


# ---------------------------------------------------------------------------
# Main attention: reductions to dense attention (torch SDPA, float64)
# ---------------------------------------------------------------------------
def _sdpa_ref(q, k, v, mask, scale):
    """torch float64 attention with an explicit boolean mask [N, N] (True = attend), GQA by repeat."""
    qt = torch.as_tensor(q).permute(0, 2, 1, 3)  # [B, Hq, N, D]
    G = q.shape[2] // k.shape[2]
    kt = torch.as_tensor(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
    vt = torch.as_tensor(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
    m = torch.as_tensor(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    s = (qt @ kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


def _rand_qkv(rng, Bsz, N, Hq, Hkv, D):
    return (rng.standard_normal((Bsz, N, Hq, D)), rng.standard_normal((Bsz, N, Hkv, D)),
            rng.standard_normal((Bsz, N, Hkv, D)))


def test_dense_reduction_when_topk_covers_all_blocks():
    rng = np.random.default_rng(7)
    N, Hq, Hkv, D, blk = 300, 4, 2, 16, 128  # ragged last block
    q, k, v = _rand_qkv(rng, 1, N, Hq, Hkv, D)
    nblk = -(-N // blk)
    pooled = rng.standard_normal((1, Hkv, N, nblk))
    sel = O.block_topk(pooled, nblk, block_size=blk)
    scale = D ** -0.5
    out, lse = O.sparse_attention(q, k, v, sel, scale, block_size=blk)
    mask = np.tril(np.ones((N, N), dtype=bool))
    ref, ref_lse = _sdpa_ref(q, k, v, mask, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_top1_is_blockwise_local_causal_attention():
    rng = np.random.default_rng(8)
    N, Hq, Hkv, D, blk = 384, 2, 1, 8, 128
    q, k, v = _rand_qkv(rng, 1, N, Hq, Hkv, D)
    pooled = rng.standard_normal((1, Hkv, N, N // blk))
    sel = O.block_topk(pooled, 1, block_size=blk)
    scale = 0.3
    out, lse = O.sparse_attention(q, k, v, sel, scale, block_size=blk)
    for c in range(N // blk):
        sl = slice(c * blk, (c + 1) * blk)
        ref, ref_lse = _sdpa_ref(q[:, sl], k[:, sl], v[:, sl], np.tril(np.ones((blk, blk), dtype=bool)), scale)
        np.testing.assert_allclose(out[:, sl], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, sl], ref_lse, rtol=1e-12, atol=1e-12)


def test_random_selection_matches_masked_sdpa():
    rng = np.random.default_rng(9)
    N, Hq, Hkv, D, blk, k_sel = 640, 6, 2, 16, 128, 3
    q, k, v = _rand_qkv(rng, 2, N, Hq, Hkv, D)
    pooled = rng.standard_normal((2, Hkv, N, N // blk))
    sel = O.block_topk(pooled, k_sel, block_size=blk)
    scale = D ** -0.5
    out, lse = O.sparse_attention(q, k, v, sel, scale, block_size=blk)
    G = Hq // Hkv
    for b in range(2):
        for g in range(Hkv):
            mask = np.zeros((N, N), dtype=bool)
            for t in range(N):
                for c in sel[b, g, t]:
                    if c >= 0:
                        mask[t, c * blk:(c + 1) * blk] = True
            mask &= np.tril(np.ones((N, N), dtype=bool))
            hs = slice(g * G, (g + 1) * G)
            ref, ref_lse = _sdpa_ref(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1], mask, scale)
            np.testing.assert_allclose(out[b:b + 1, :, hs], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b:b + 1, hs], ref_lse, rtol=1e-12, atol=1e-12)


def test_uniform_scores_give_mean_over_attended_keys():
    # Closed form: with all keys zero every attended key has the same weight.
    rng = np.random.default_rng(10)
    N, Hq, Hkv, D, blk, ksel = 1000, 4, 2, 8, 128, 3
    q = rng.standard_normal((1, N, Hq, D))
    k = np.zeros((1, N, Hkv, D))
    v = rng.standard_normal((1, N, Hkv, D))
    sel = O.block_topk(rng.standard_normal((1, Hkv, N, 8)), ksel, block_size=blk)
    out, lse = O.sparse_attention(q, k, v, sel, 1.0, block_size=blk)
    G = Hq // Hkv
    for t in range(0, N, 37):
        for g in range(Hkv):
            keys = [j for c in sel[0, g, t] if c >= 0 for j in range(c * blk, min((c + 1) * blk, t + 1))]
            for h in range(g * G, (g + 1) * G):
                np.testing.assert_allclose(out[0, t, h], v[0, keys, g].mean(axis=0), rtol=1e-12, atol=1e-13)
                assert lse[0, h, t] == pytest.approx(math.log(len(keys)), abs=1e-13)


def test_one_hot_value_probe_mass_only_on_selected_blocks():
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    N = w.seqlen
    v = np.zeros((1, N, 1, 128))
    v[0, np.arange(N), 0, np.arange(N) // 128] = 1.0
    pooled = O.index_scores(x["q_idx"], x["k_idx"])
    sel = O.block_topk(pooled, w.top_k)
    out, _ = O.sparse_attention(x["q"], x["k"], v, sel, w.softmax_scale)
    for t in range(N):
        s = set(int(c) for c in sel[0, 0, t] if c >= 0)
        mass = out[0, t, :, :w.nblk]            # [H_q, nblk]
        for c in range(128):
            if c not in s:
                assert np.all(out[0, t, :, c] == 0.0), (t, c)
        np.testing.assert_allclose(mass.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
        assert np.all(mass[:, sorted(s)] > 0)


def test_lse_and_output_bounds():
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    pos = np.arange(0, w.seqlen, 7)
    bi, out, lse, _ = O.msa_forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.top_k,
                                    w.softmax_scale, positions=pos)
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    v = x["v"].double().numpy()
    for i, t in enumerate(pos):
        keys = O.attended_keys(bi[0, 0, i], int(t))
        z = w.softmax_scale * q[0, t] @ k[0, keys, 0].T     # [H_q, n]
        zmax = z.max(axis=-1)
        assert np.all(zmax <= lse[0, :, i] + 1e-12)
        assert np.all(lse[0, :, i] <= zmax + math.log(len(keys)) + 1e-12)
        lo = v[0, keys, 0].min(axis=0)
        hi = v[0, keys, 0].max(axis=0)
        assert np.all(out[0, i] >= lo - 1e-12) and np.all(out[0, i] <= hi + 1e-12)


def test_msa_forward_positions_subset_consistent():
    w = small_workload(1024, 8, 2, 3, seed=12)
    x = make_inputs(w)
    full = O.msa_forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.top_k, w.softmax_scale)
    pos = [0, 1, 127, 128, 383, 384, 700, 1023]
    part = O.msa_forward(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], w.top_k, w.softmax_scale,
                         positions=pos)
    np.testing.assert_array_equal(part[0], full[0][:, :, pos])
    np.testing.assert_array_equal(part[1], full[1][:, pos])
    np.testing.assert_array_equal(part[2], full[2][:, :, pos])


# ---------------------------------------------------------------------------
# Near-tie classification used by the parity tests
# ---------------------------------------------------------------------------
def test_near_tie_classification():
    pooled = np.array([[[[5.0, 4.0, 3.0, 3.002, 1.0, 9.0]]]])  # one row, t in block 5
    pos = [5 * 128]
    ref = O.block_topk(pooled, 4, positions=pos)
    assert list(ref[0, 0, 0]) == [0, 1, 3, 5]
    swapped = np.array([[[[0, 1, 2, 5]]]], dtype=np.int32)     # 3.0 vs 3.002: within 1e-3 relative
    far = np.array([[[[0, 1, 4, 5]]]], dtype=np.int32)         # 1.0 is far from the boundary
    nolocal = np.array([[[[0, 1, 2, 3]]]], dtype=np.int32)
    assert O.near_tie_rows(pooled, swapped, ref, 4, positions=pos)[:2] == (1, 1)
    n, nt, bad = O.near_tie_rows(pooled, far, ref, 4, positions=pos)
    assert (n, nt, bad) == (1, 0, [(0, 0, 0)])
    assert O.near_tie_rows(pooled, nolocal, ref, 4, positions=pos)[1] == 0
    assert O.near_tie_rows(pooled, ref, ref, 4, positions=pos) == (0, 0, [])


def test_near_tie_rejects_a_wrong_exact_tie_break():
    # block 2 and block 3 score exactly 3.0; the lower block must win, so picking
    # block 3 is a wrong tie-break, not a near-tie
    pooled = np.array([[[[5.0, 4.0, 3.0, 3.0, 1.0, 9.0]]]])
    pos = [5 * 128]
    ref = O.block_topk(pooled, 4, positions=pos)
    assert list(ref[0, 0, 0]) == [0, 1, 2, 5]
    wrong = np.array([[[[0, 1, 3, 5]]]], dtype=np.int32)
    assert O.near_tie_rows(pooled, wrong, ref, 4, positions=pos) == (1, 0, [(0, 0, 0)])
    # with a third block just below the tied pair: trading a tied block for it is a
    # near-tie, trading one tied block for the other is not
    pooled = np.array([[[[5.0, 4.0, 3.0, 3.0, 2.999, 9.0]]]])
    ref = O.block_topk(pooled, 4, positions=pos)
    assert list(ref[0, 0, 0]) == [0, 1, 2, 5]
    below = np.array([[[[0, 1, 4, 5]]]], dtype=np.int32)
    assert O.near_tie_rows(pooled, below, ref, 4, positions=pos)[:2] == (1, 1)
    assert O.near_tie_rows(pooled, wrong, ref, 4, positions=pos)[:2] == (1, 0)
    # -0.0 and +0.0 are equal scores: a higher block over a lower one is no near-tie
    pooled = np.array([[[[1.0, -0.0, 0.0, -2.0, 9.0]]]])
    pos = [4 * 128]
    ref = O.block_topk(pooled, 3, positions=pos)
    assert list(ref[0, 0, 0]) == [0, 1, 4]
    assert O.near_tie_rows(pooled, np.array([[[[0, 2, 4]]]], dtype=np.int32), ref, 3, positions=pos)[:2] == (1, 0)


def test_empty_selection_gives_zero_output_and_minus_inf_lse():
    # R9: an empty sum of exp is 0, so LSE = log 0 = -inf; O is taken as 0.
    rng = np.random.default_rng(13)
    q, k, v = _rand_qkv(rng, 1, 256, 2, 1, 8)
    sel = np.full((1, 1, 256, 2), -1, dtype=np.int32)
    sel[0, 0, 200] = [1, -1]
    sel[0, 0, 10] = [1, -1]   # block after the local block: nothing attendable
    out, lse = O.sparse_attention(q, k, v, sel, 0.5)
    empty = np.ones(256, dtype=bool)
    empty[200] = False
    assert np.all(out[0, empty] == 0.0) and np.all(lse[0, :, empty] == -np.inf)
    keys = np.arange(128, 201)
    z = 0.5 * q[0, 200] @ k[0, keys, 0].T
    np.testing.assert_allclose(lse[0, :, 200], np.log(np.exp(z).sum(-1)), rtol=1e-12)
