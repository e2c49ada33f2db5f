"""GPU parity of the decode step (msa_decode and its three stages) against the CPU oracle.

Cache rows at or past each sequence's length are NaN (poisoned) in most cases:
any read of them would show up as a non-finite output. Every test prints its
case before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth.msa_inputs import DECODE_WORKLOADS, make_decode_inputs, small_decode_workload
from tests._parity import check_attn, check_pooled, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def msa():
    from block_sparse_attention_head_amd import msa as m

    m.lib()
    return m


def _gpu(x):
    return {k: v.to(DEV) for k, v in x.items()}


def _check_selection(sel_g, pooled_g, pooled_r, lengths, top_k, tag):
    """GPU selection == the oracle's selection on the GPU's pooled scores; against the oracle's own
    scores only near-ties may differ. Returns (mismatching rows, near-ties)."""
    n_mis = n_tie = 0
    for b, L in enumerate(lengths):
        if L <= 0:
            assert (sel_g[b] == -1).all(), f"{tag}: empty sequence {b} selected blocks"
            continue
        t = L - 1
        nb = t // 128 + 1
        same = O.block_topk(pooled_g[b][None, :, None, :nb].astype(np.float64), top_k, positions=[t])
        assert np.array_equal(same[0, :, 0], sel_g[b]), f"{tag}: sequence {b} differs on identical scores"
        ref = O.block_topk(pooled_r[b][None, :, None, :nb], top_k, positions=[t])
        m, k, bad = O.near_tie_rows(pooled_r[b][None, :, None, :nb], sel_g[b][None, :, None], ref, top_k,
                                    positions=[t])
        assert not bad, f"{tag}: sequence {b}: selection differs beyond near-ties"
        n_mis += m
        n_tie += k
    return n_mis, n_tie


def _parity(msa, w, x, tag):
    xg = _gpu(x)
    lengths = [int(v) for v in x["seqlens"]]
    C, K = w.capacity, w.top_k
    _say(tag, "stages")
    pooled = msa.decode_index_scores(xg["q_idx"], xg["k_idx"], xg["seqlens"])
    sel = msa.decode_topk(pooled, xg["seqlens"], K, C)
    # with a workspace the attention spreads each group's blocks over several workgroups
    # when there are few sequences (as msa_decode does); without, one workgroup per group
    ws = msa.alloc_workspace(msa.make_shape(w.batch, C, w.h_q, w.h_kv, K, w.softmax_scale), msa.OP_DECODE,
                             xg["q"].device)
    o, lse = msa.decode_attn(xg["q"], xg["k"], xg["v"], xg["seqlens"], sel, w.softmax_scale, workspace=ws)
    o1, lse1 = msa.decode_attn(xg["q"], xg["k"], xg["v"], xg["seqlens"], sel, w.softmax_scale)
    _say(tag, "msa_decode")
    bi, o2, lse2 = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], K,
                              w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(bi, sel) and torch.equal(o2, o) and torch.equal(lse2, lse)
    pg, sg, og, lg = to_np(pooled), to_np(sel), to_np(o), to_np(lse)
    _say(tag, "oracle")
    cpu = {k: v for k, v in x.items()}
    sel_r, _, _, pooled_r = O.msa_decode(cpu["q_idx"], cpu["k_idx"], cpu["q"], cpu["k"], cpu["v"], cpu["seqlens"],
                                         K, w.softmax_scale)
    _, _, _, bound = O.msa_decode(cpu["q_idx"].abs(), cpu["k_idx"].abs(), cpu["q"], cpu["k"], cpu["v"],
                                  cpu["seqlens"], K, w.softmax_scale)
    bound = 127 * 2.0 ** -24 * np.where(np.isfinite(bound), bound, 0.0) + 1e-6
    check_pooled(pg, pooled_r, bound, tag, check_upper=True)
    mis = _check_selection(sg, pg, pooled_r, lengths, K, tag)
    _, o_r, lse_r, _ = O.msa_decode(cpu["q_idx"], cpu["k_idx"], cpu["q"], cpu["k"], cpu["v"], cpu["seqlens"], K,
                                    w.softmax_scale, block_idx=sg)
    do, dl = check_attn(og, lg, o_r, lse_r, tag)
    check_attn(to_np(o1), to_np(lse1), o_r, lse_r, tag + "/one-workgroup-per-group")
    assert np.isfinite(og).all()
    _say(tag, f"O err {do:.2e} LSE err {dl:.2e} selection mismatches/near-ties {mis}")
    return sg, og, lg


DEC_SHAPES = [
    # (capacity, h_q, h_kv, top_k, batch): G = 4, 16, 4 with 8 heads, 1, 128 (8 head tiles), 2,
    # top_k = 65 (64 ranked), top_k = 1
    (1024, 8, 2, 4, 6),
    (2048, 64, 4, 16, 5),
    (4096, 32, 8, 16, 3),
    (1024, 4, 4, 3, 4),
    (1024, 128, 1, 5, 3),
    (640, 6, 3, 2, 4),
    (16384, 16, 1, 65, 2),
    (2048, 8, 2, 1, 3),
]


@pytest.mark.parametrize("C,hq,hkv,k,b", DEC_SHAPES)
def test_decode_parity(msa, C, hq, hkv, k, b):
    w = small_decode_workload(C, hq, hkv, k, seed=400 + C + hq + k, batch=b)
    edge = [C, 0, 1, 129, 128, 127]
    rng = np.random.default_rng(C + hq)
    lengths = [edge[i] if i < len(edge) else int(rng.integers(1, C + 1)) for i in range(b)]
    x = make_decode_inputs(w, lengths=lengths, poison_tail=True)
    _parity(msa, w, x, w.name)


def test_decode_lengths_past_capacity_read_as_capacity(msa):
    w = small_decode_workload(1024, 8, 2, 4, seed=5, batch=2)
    x = make_decode_inputs(w, lengths=[1024, 1024])
    xg = _gpu(x)
    _say(w.name, "length past capacity")
    a = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], 4, w.softmax_scale)
    over = torch.tensor([5000, 1 << 30], dtype=torch.int32, device=DEV)
    b = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], over, 4, w.softmax_scale)
    neg = torch.tensor([-7, 0], dtype=torch.int32, device=DEV)
    c = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], neg, 4, w.softmax_scale)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert (c[0] == -1).all() and (c[1] == 0).all() and torch.isneginf(c[2]).all()


def test_decode_ties_take_lower_blocks(msa):
    # closed form: with zero index queries every pooled score is exactly 0, so each row keeps
    # blocks 0 .. top_k-2 and its own block; rows of 1024 and 8192 blocks run the four-wave
    # selection with every block a candidate. A copy of block 2's index keys in block 5 ties
    # the two exactly; the lower block must win.
    for C, lengths in ((131072, [131072, 70001, 2000]), (1 << 20, [1 << 20, 600000])):
        w = small_decode_workload(C, 8, 2, 16, seed=77, batch=len(lengths))
        x = make_decode_inputs(w, lengths=lengths)
        x["q_idx"] = torch.zeros_like(x["q_idx"])
        xg = _gpu(x)
        _say(w.name, f"decode all-tied selection, rows of {C // 128} blocks")
        bi, _, _ = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], 16,
                              w.softmax_scale)
        torch.cuda.synchronize()
        got = to_np(bi)
        for b, L in enumerate(lengths):
            cl = (L - 1) // 128
            want = list(range(15)) + [cl]
            assert (got[b] == np.array(want)[None, :]).all(), (C, b, got[b])
    # an exact tie at the selection boundary: blocks 7 and 9 (keys x8) lead, blocks 2 and 5
    # (the same keys x4, an exact copy) tie for the last of the top_k - 1 = 3 places, and the
    # lower block must win; scaling by a power of two is exact in bf16
    w = small_decode_workload(131072, 8, 2, 4, seed=78, batch=1)
    x = make_decode_inputs(w, lengths=[131072])
    ki = x["k_idx"][0]
    for c, f in ((7, 8.0), (9, 8.0), (2, 4.0)):
        ki[c * 128:(c + 1) * 128] = ki[c * 128:(c + 1) * 128] * f
    ki[5 * 128:6 * 128] = ki[2 * 128:3 * 128]
    xg = _gpu(x)
    _say(w.name, "decode tie at the selection boundary")
    pooled = msa.decode_index_scores(xg["q_idx"], xg["k_idx"], xg["seqlens"])
    bi = msa.decode_topk(pooled, xg["seqlens"], 4, 131072)
    torch.cuda.synchronize()
    gp, gi = to_np(pooled), to_np(bi)
    for h in range(w.h_kv):
        assert gp[0, h, 5] == gp[0, h, 2]  # identical inputs, identical sums
        order = sorted(range(1023), key=lambda c: (-float(gp[0, h, c]), c))
        assert order[:4] in ([7, 9, 2, 5], [9, 7, 2, 5]), (h, order[:6])  # the case is exercised
        assert list(gi[0, h]) == [2, 7, 9, 1023], (h, gi[0, h])


def test_decode_attn_invalid_and_repeated_entries(msa):
    w = small_decode_workload(2048, 16, 2, 6, seed=6, batch=3)
    lengths = [2000, 300, 1025]
    x = make_decode_inputs(w, lengths=lengths, poison_tail=True)
    rng = np.random.default_rng(3)
    given = rng.integers(-3, 18, size=(3, 2, 6)).astype(np.int32)
    given[0, 0] = [4, 4, 4, 15, -1, 20]
    given[1, 1] = [3, 9, -1, -2, 17, 5]  # nothing visible for L = 300
    xg = _gpu(x)
    _, o_r, lse_r, _ = O.msa_decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], 6,
                                    w.softmax_scale, block_idx=given)
    ws = msa.alloc_workspace(msa.make_shape(3, 2048, 16, 2, 6, w.softmax_scale), msa.OP_DECODE, xg["q"].device)
    # without a workspace (one workgroup per group), then with one (the group's slots split over
    # several workgroups, some of which see no valid entry)
    for label, wsp in (("one workgroup", None), ("split", ws)):
        _say(w.name, f"caller's selection, {label}")
        o, lse = msa.decode_attn(xg["q"], xg["k"], xg["v"], xg["seqlens"], torch.from_numpy(given).to(DEV),
                                 w.softmax_scale, workspace=wsp)
        torch.cuda.synchronize()
        og, lg = to_np(o), to_np(lse)
        check_attn(og, lg, o_r, lse_r, f"{w.name}/{label}")
        assert not og[1, 8:].any() and np.isneginf(lg[1, 8:]).all()


def test_decode_deterministic(msa):
    w = small_decode_workload(4096, 64, 4, 16, seed=7, batch=8)
    xg = _gpu(make_decode_inputs(w))
    _say(w.name, "determinism")
    r1 = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], 16, w.softmax_scale)
    ws = msa.alloc_workspace(msa.make_shape(8, 4096, 64, 4, 16, w.softmax_scale), msa.OP_DECODE, torch.device(DEV))
    ws.fill_(0x7F)
    r2 = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], 16, w.softmax_scale,
                    workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,n_check", [("dec_b128_n128k", 3), ("dec_b16_n1m", 0)])
def test_decode_full_size_sampled(msa, name, n_check):
    """The benchmark workloads, drawn on the GPU; a few sequences are checked in full
    against the oracle (pooled scores, selection, attention on the GPU's blocks)."""
    w = DECODE_WORKLOADS[name]
    _say(name, "generating inputs on the GPU")
    xg = make_decode_inputs(w, device=DEV)
    _say(name, "msa_decode")
    bi, o, lse = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], w.top_k,
                            w.softmax_scale)
    pooled = msa.decode_index_scores(xg["q_idx"], xg["k_idx"], xg["seqlens"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    picks = sorted(set([0, w.batch - 1] + np.random.default_rng(w.seed).integers(0, w.batch, n_check).tolist()))
    picks = picks[:n_check + 1]  # the float64 oracle widens whole caches: one sequence at 1M tokens
    sub = {k: v[picks].cpu() for k, v in xg.items()}
    _say(name, f"oracle on sequences {picks}, lengths {sub['seqlens'].tolist()}")
    sg = to_np(bi[picks])
    sel_r, _, _, pooled_r = O.msa_decode(sub["q_idx"], sub["k_idx"], sub["q"], sub["k"], sub["v"], sub["seqlens"],
                                         w.top_k, w.softmax_scale)
    _, _, _, bound = O.msa_decode(sub["q_idx"].abs(), sub["k_idx"].abs(), sub["q"], sub["k"], sub["v"],
                                  sub["seqlens"], w.top_k, w.softmax_scale)
    bound = 127 * 2.0 ** -24 * np.where(np.isfinite(bound), bound, 0.0) + 1e-6
    pg = to_np(pooled[picks])
    check_pooled(pg, pooled_r, bound, name, check_upper=True)
    mis = _check_selection(sg, pg, pooled_r, sub["seqlens"].tolist(), w.top_k, name)
    _, o_r, lse_r, _ = O.msa_decode(sub["q_idx"], sub["k_idx"], sub["q"], sub["k"], sub["v"], sub["seqlens"],
                                    w.top_k, w.softmax_scale, block_idx=sg)
    do, dl = check_attn(to_np(o[picks]), to_np(lse[picks]), o_r, lse_r, name)
    _say(name, f"O err {do:.2e} LSE err {dl:.2e} selection mismatches/near-ties {mis}")


def test_decode_rejects_bad_arguments(msa):
    qi = torch.zeros(2, 2, 128, dtype=torch.bfloat16, device=DEV)
    ki = torch.zeros(2, 1024, 128, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(2, 1024, 2, 128, dtype=torch.bfloat16, device=DEV)
    sl = torch.ones(2, dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        msa.decode(qi, ki, q, k, k, sl.long(), 4, 0.1)
    with pytest.raises(ValueError):
        msa.decode(qi[:, :1], ki, q, k, k, sl, 4, 0.1)
    with pytest.raises(msa.MsaError) as e:
        msa.decode(qi, ki, q, k, k, sl, 66, 0.1)
    assert e.value.status == 2
    small = torch.empty(8, dtype=torch.uint8, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.decode(qi, ki, q, k, k, sl, 4, 0.1, workspace=small)
    assert e.value.status == 3
