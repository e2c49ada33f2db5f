"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test prints the case it is about to run before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth.msa_inputs import WORKLOADS, make_inputs, small_workload
from tests._parity import (check_attn, check_pooled, check_topk, pooled_bound, sample_positions, to_np)

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


def _run_stages(msa, w, xg):
    """Index scores, top-k, then sparse attention, each through its own entry point."""
    pooled = msa.index_scores(xg["q_idx"], xg["k_idx"])
    bi = msa.block_topk(pooled, w.top_k)
    o, lse = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], bi, w.softmax_scale)
    torch.cuda.synchronize()
    return pooled, bi, o, lse


def _full_parity(msa, w, x):
    xg = _gpu(x)
    _say(w.name, "stages")
    pooled, bi, o, lse = _run_stages(msa, w, xg)
    _say(w.name, "msa_fwd")
    bi2, o2, lse2 = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    # msa_fwd runs the same kernels: identical bits
    assert torch.equal(bi, bi2) and torch.equal(o, o2) and torch.equal(lse, lse2)

    ref_pooled = O.index_scores(x["q_idx"], x["k_idx"])
    gp = to_np(pooled)
    check_pooled(gp, ref_pooled, pooled_bound(x["q_idx"], x["k_idx"]), w.name, check_upper=True)
    gi = to_np(bi)
    n_mis, n_tie = check_topk(gi, gp, ref_pooled, w.top_k, tag=w.name)
    _say(w.name, f"index rows differing from the oracle: {n_mis} (all near-ties: {n_tie})")
    for label, sel in (("oracle-indices", O.block_topk(ref_pooled, w.top_k)), ("gpu-indices", gi)):
        if label == "oracle-indices":
            og, lg = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], torch.from_numpy(sel).to(DEV), w.softmax_scale)
            torch.cuda.synchronize()
        else:
            og, lg = o, lse
        ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], sel, w.softmax_scale)
        do, dl = check_attn(to_np(og), to_np(lg), ro, rl, f"{w.name}/{label}")
        _say(w.name, label, f"max|dO|={do:.2e} max|dLSE|={dl:.2e}")


def test_mfma_full_parity_tiny(msa):
    w = WORKLOADS["tiny_n1k"]
    _full_parity(msa, w, make_inputs(w))


def test_full_parity_n8k(msa):
    w = WORKLOADS["n8k"]
    _full_parity(msa, w, make_inputs(w))


SHAPES = [
    # (seqlen, h_q, h_kv, top_k, batch): ragged index tiles (3 heads), G = 1, 2, 32, 128,
    # top_k = 1, top_k > blocks (dense), one block, batch 2
    (640, 6, 3, 3, 1),
    (1024, 4, 4, 2, 1),
    (2048, 32, 1, 5, 2),
    (512, 8, 2, 16, 1),
    (1024, 8, 2, 1, 1),
    (128, 4, 1, 4, 1),
    (768, 128, 1, 3, 1),
    (3072, 16, 2, 7, 1),
]


@pytest.mark.parametrize("N,hq,hkv,k,b", SHAPES)
def test_shapes_parity(msa, N, hq, hkv, k, b):
    w = small_workload(N, hq, hkv, k, seed=100 + N + hq + k, batch=b)
    _full_parity(msa, w, make_inputs(w))


FUSED_SHAPES = SHAPES + [
    # list length at the register cap (17), past it (two kernels), many heads, full length
    (4096, 8, 2, 17, 1), (4096, 8, 2, 18, 1), (8192, 32, 8, 16, 1), (131072, 4, 4, 16, 1)]


@pytest.mark.parametrize("N,hq,hkv,k,b", FUSED_SHAPES)
def test_fused_index_topk_matches_the_two_stages(msa, N, hq, hkv, k, b):
    # one pass (scores, pool and a running per-row list) against msa_index_scores +
    # msa_block_topk: the same pooled arithmetic and the same order, so identical indices
    w = small_workload(N, hq, hkv, k, seed=300 + N + hq + k, batch=b)
    x = make_inputs(w)
    qi, ki = x["q_idx"].to(DEV), x["k_idx"].to(DEV)
    _say(w.name, "fused index top-k")
    fused = msa.index_topk(qi, ki, k)
    staged = msa.block_topk(msa.index_scores(qi, ki, visible_only=True), k)
    again = msa.index_topk(qi, ki, k)
    torch.cuda.synchronize()
    assert torch.equal(fused, staged)
    assert torch.equal(fused, again)


def test_fused_index_topk_ties_take_lower_blocks(msa):
    # key blocks repeat with period 3, so every row's block scores tie in threes
    # (and q_idx = 0 rows tie everywhere): equal scores go to the lower block
    w = small_workload(4096, 8, 2, 9, seed=41)
    x = make_inputs(w)
    qi, ki = x["q_idx"].clone(), x["k_idx"].clone()
    for c in range(3, w.nblk):
        ki[:, c * 128:(c + 1) * 128] = ki[:, (c % 3) * 128:(c % 3 + 1) * 128]
    qi[:, 2000:2100] = 0
    qi, ki = qi.to(DEV), ki.to(DEV)
    _say(w.name, "fused index top-k with ties")
    fused = msa.index_topk(qi, ki, w.top_k)
    staged = msa.block_topk(msa.index_scores(qi, ki, visible_only=True), w.top_k)
    torch.cuda.synchronize()
    assert torch.equal(fused, staged)
    zero_rows = to_np(fused)[0, :, 2000:2100]
    t = np.arange(2000, 2100)
    want = np.concatenate([np.tile(np.arange(8), (100, 1)), (t // 128)[:, None]], axis=1)
    assert (zero_rows == want[None]).all()


@pytest.mark.parametrize("N,hq,hkv,k,chunk", [(4096, 8, 2, 4, 1024), (1024, 4, 1, 3, 384), (2048, 64, 4, 16, 128)])
def test_forward_in_position_chunks_matches_one_pass(msa, N, hq, hkv, k, chunk):
    # a workspace for `chunk` query positions runs the sparse attention chunk by chunk
    # (the last one ragged); every (t, slot) record and every combine reads only its own
    # row's inputs, so the result is identical bit for bit
    w = small_workload(N, hq, hkv, k, seed=700 + N + chunk)
    xg = {kk: v.to(DEV) for kk, v in make_inputs(w).items()}
    _say(w.name, f"forward in chunks of {chunk} positions")
    shape = msa.make_shape(1, N, hq, hkv, k, w.softmax_scale)
    bi1, o1, l1 = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], k, w.softmax_scale)
    small = msa.make_shape(1, chunk, hq, hkv, k, w.softmax_scale)
    # the chunked workspace: the forward's for `chunk` positions, plus the plan's per-tile arrays of all N
    n_ws = msa.workspace_size(small, msa.OP_SPARSE_ATTN_FWD) + msa.workspace_size(shape, msa.OP_INDEX_TOPK) + \
        16 * 4 * (N // 128) * hkv + (1 << 16)
    assert n_ws < msa.workspace_size(shape, msa.OP_FWD)
    ws = torch.empty(n_ws, dtype=torch.uint8, device=DEV)
    bi2, o2, l2 = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], k, w.softmax_scale, workspace=ws)
    o3, l3 = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], bi1, w.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bi1, bi2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    with pytest.raises(msa.MsaError) as e:  # the stage-wise calls need the whole sequence in one pass
        msa.sparse_attn_plan(shape, bi1, ws)
    assert e.value.status == 3


def test_dense_reduction_on_gpu(msa):
    # top_k covering every block: the GPU path must equal dense causal GQA attention
    w = small_workload(1024, 8, 2, 8, seed=21)
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "dense")
    bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    q = x["q"].double().permute(0, 2, 1, 3)
    kk = x["k"].double().permute(0, 2, 1, 3).repeat_interleave(4, dim=1)
    vv = x["v"].double().permute(0, 2, 1, 3).repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=w.softmax_scale)
    s = (q @ kk.transpose(-1, -2)) * w.softmax_scale
    s = s.masked_fill(~torch.ones(w.seqlen, w.seqlen, dtype=torch.bool).tril(), float("-inf"))
    check_attn(to_np(o), to_np(lse), ref.permute(0, 2, 1, 3).numpy(), torch.logsumexp(s, -1).numpy(), "dense")


LONG_ROWS = small_workload(1040 * 128, 2, 1, 16, seed=31)  # 1040 blocks: the general (two-pass) top-k path


@pytest.mark.parametrize("name", ["n32k_b2", "n128k", "n64k_train", "long_rows"])
def test_full_size_sampled_rows(msa, name):
    w = LONG_ROWS if name == "long_rows" else WORKLOADS[name]
    _say(name, "generating inputs")
    x = make_inputs(w)
    xg = _gpu(x)
    _say(name, "msa_fwd + index scores")
    bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    pooled = msa.index_scores(xg["q_idx"], xg["k_idx"], visible_only=True)
    torch.cuda.synchronize()
    pos = sample_positions(w.seqlen, 40, seed=w.seed)
    _say(name, f"oracle on {len(pos)} sampled positions")
    gp = to_np(pooled[:, :, pos])
    ref_pooled = O.index_scores(x["q_idx"], x["k_idx"], positions=pos)
    vis = np.isfinite(ref_pooled)
    gp = np.where(vis, gp, -np.inf)
    check_pooled(gp, ref_pooled, pooled_bound(x["q_idx"], x["k_idx"], positions=pos), name)
    gi = to_np(bi[:, :, pos])
    n_mis, n_tie = check_topk(gi, gp, ref_pooled, w.top_k, positions=pos, tag=name)
    _say(name, f"sampled index rows differing from the oracle: {n_mis} (near-ties: {n_tie})")
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], gi, w.softmax_scale, positions=pos)
    do, dl = check_attn(to_np(o[:, pos]), to_np(lse[:, :, pos]), ro, rl, name)
    _say(name, f"max|dO|={do:.2e} max|dLSE|={dl:.2e}")
    # properties that hold at every position: local block present, count, order
    bic = to_np(bi).astype(np.int64)
    t = np.arange(w.seqlen)
    cl = t // 128
    valid = bic >= 0
    assert np.all(valid.sum(-1) == np.minimum(w.top_k, cl + 1)[None, None])
    assert np.all(np.take_along_axis(bic, (valid.sum(-1, keepdims=True) - 1), -1)[..., 0] == cl[None, None])
    assert np.all(np.where(valid[..., 1:], np.diff(bic, axis=-1) > 0, True))
    assert np.all(np.isfinite(to_np(lse)))


@pytest.mark.timeout(900)
def test_full_rows_n32k_b2(msa):
    """Every index row of the 32K two-batch workload (2 x 8 heads x 32768 positions): bit-exact
    against the oracle's selection on the GPU's own pooled scores; against the oracle's float64
    scores only near-ties may differ, and they are counted and printed. O and LSE on 640 positions."""
    w = WORKLOADS["n32k_b2"]
    _say(w.name, "generating inputs")
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "msa_fwd + index scores")
    bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    pooled = msa.index_scores(xg["q_idx"], xg["k_idx"], visible_only=True)
    torch.cuda.synchronize()
    gi = to_np(bi)
    gp = pooled.cpu().numpy()
    del pooled
    torch.cuda.empty_cache()
    _say(w.name, "oracle selection on the GPU's pooled scores, every row")
    same = O.block_topk(gp.astype(np.float64), w.top_k)   # reads only the visible part
    bad = np.argwhere(np.any(same != gi, axis=-1))
    assert bad.size == 0, f"selection differs from the oracle on identical scores at rows {bad[:5].tolist()}"
    del same
    q64, k64 = x["q_idx"].double().numpy(), x["k_idx"].double().numpy()
    n_mis = n_tie = 0
    step = 4096
    for b in range(w.batch):
        for p0 in range(0, w.seqlen, step):
            pos = np.arange(p0, p0 + step)
            ref_pooled = O.index_scores(q64[b:b + 1], k64[b:b + 1], positions=pos)
            ref_idx = O.block_topk(ref_pooled, w.top_k, positions=pos)
            m, t, not_tie = O.near_tie_rows(ref_pooled, gi[b:b + 1, :, p0:p0 + step], ref_idx, w.top_k,
                                            positions=pos)
            assert not not_tie, f"batch {b}: {len(not_tie)} rows differ beyond near-ties, e.g. {not_tie[:5]}"
            n_mis += m
            n_tie += t
            _say(w.name, f"batch {b} positions {p0}..{p0 + step - 1}: float64 rows differing {m} (near-ties {t})")
    rows = w.batch * w.h_idx * w.seqlen
    _say(w.name, f"index rows differing from the float64 oracle: {n_mis} of {rows} (all near-ties: {n_tie})")
    pos = sample_positions(w.seqlen, 628, seed=w.seed + 1)
    assert len(pos) >= 512
    _say(w.name, f"attention oracle on {len(pos)} positions")
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], gi[:, :, pos], w.softmax_scale, positions=pos)
    do, dl = check_attn(to_np(o[:, pos]), to_np(lse[:, :, pos]), ro, rl, w.name)
    _say(w.name, f"max|dO|={do:.2e} max|dLSE|={dl:.2e}")


def test_fused_index_topk_exact_integer_scores_long_rows(msa):
    """Index queries and keys drawn from {-1, 0, 1}: every dot product is a small integer, exact
    in fp32 and float64 alike, so the GPU's pooled scores equal the oracle's and the selection
    must match bit for bit, with no near-tie allowance, on rows of up to 8192 blocks where exact
    ties between blocks are everywhere (equal scores must go to the lower block)."""
    N, H, K = 1 << 20, 4, 16
    gen = torch.Generator(device=DEV).manual_seed(91)
    _say("integer index scores 2^20", "drawing")
    qi = torch.randint(-1, 2, (1, N, H, 128), generator=gen, device=DEV).to(torch.bfloat16)
    ki = torch.randint(-1, 2, (1, N, 128), generator=gen, device=DEV).to(torch.bfloat16)
    _say("integer index scores 2^20", "fused index top-k")
    bi = msa.index_topk(qi, ki, K)
    torch.cuda.synchronize()
    pos = sample_positions(N, 28, seed=91)
    pos_t = torch.from_numpy(pos).to(DEV)
    got = to_np(bi[:, :, pos_t])
    bic = to_np(bi).astype(np.int64)
    q_h, k_h = qi.cpu(), ki.cpu()
    del bi, qi, ki
    torch.cuda.empty_cache()
    _say("integer index scores 2^20", f"oracle on {len(pos)} positions")
    ref_pooled = O.index_scores(q_h, k_h, positions=pos)
    assert np.all(ref_pooled[np.isfinite(ref_pooled)] == np.round(ref_pooled[np.isfinite(ref_pooled)]))
    ref = O.block_topk(ref_pooled, K, positions=pos)
    # the case is exercised: many rows have a tie across the selection boundary
    cl = pos // 128
    ties = 0
    for i, t in enumerate(pos):
        if cl[i] >= K:
            for h in range(H):
                row = ref_pooled[0, h, i, :cl[i]]
                chosen = row[ref[0, h, i, :K - 1]]
                ties += int(np.sum(row == chosen.min()) > np.sum(chosen == chosen.min()))
    _say("integer index scores 2^20", f"rows with an exact tie across the boundary: {ties}")
    assert ties >= 20
    np.testing.assert_array_equal(got, ref)
    valid = bic >= 0
    c_all = np.arange(N) // 128
    assert np.all(valid.sum(-1) == np.minimum(K, c_all + 1)[None, None])
    assert np.all(np.take_along_axis(bic, (valid.sum(-1, keepdims=True) - 1), -1)[..., 0] == c_all[None, None])
    assert np.all(np.where(valid[..., 1:], np.diff(bic, axis=-1) > 0, True))


def test_long_context_sampled_rows(msa):
    # 2^20 tokens with the 128K workload's heads, as the benchmark's long-context line runs it:
    # the one-pass selection over rows of up to 8192 blocks and the sparse attention in query
    # chunks inside the library's own workspace; sampled positions against the oracle
    w = WORKLOADS["n1m"]
    _say(w.name, "generating inputs on the GPU")
    xg = make_inputs(w, device=DEV)
    _say(w.name, "msa_fwd")
    bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    pos = sample_positions(w.seqlen, 12, seed=w.seed)
    pos_t = torch.from_numpy(pos).to(DEV)
    gi = to_np(bi[:, :, pos_t])
    go, gl = to_np(o[:, pos_t]), to_np(lse[:, :, pos_t])
    bic = bi.cpu().numpy().astype(np.int64)
    lse_finite = bool(torch.isfinite(lse).all())
    del bi, o, lse
    x = {name: t.cpu() for name, t in xg.items()}  # host copies for the oracle
    del xg
    torch.cuda.empty_cache()
    _say(w.name, f"oracle on {len(pos)} sampled positions")
    ref_pooled = O.index_scores(x["q_idx"], x["k_idx"], positions=pos)
    ref_idx = O.block_topk(ref_pooled, w.top_k, positions=pos)
    n_mis, n_tie, not_tie = O.near_tie_rows(ref_pooled, gi, ref_idx, w.top_k, positions=pos)
    assert not not_tie, f"{w.name}: {len(not_tie)} mismatching rows are not near-ties, e.g. {not_tie[:5]}"
    _say(w.name, f"sampled index rows differing from the oracle: {n_mis} (near-ties: {n_tie})")
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], gi, w.softmax_scale, positions=pos)
    do, dl = check_attn(go, gl, ro, rl, w.name)
    _say(w.name, f"max|dO|={do:.2e} max|dLSE|={dl:.2e}")
    # every row: local block last, min(top_k, c_loc + 1) ascending entries
    cl = np.arange(w.seqlen) // 128
    valid = bic >= 0
    assert np.all(valid.sum(-1) == np.minimum(w.top_k, cl + 1)[None, None])
    assert np.all(np.take_along_axis(bic, (valid.sum(-1, keepdims=True) - 1), -1)[..., 0] == cl[None, None])
    assert np.all(np.where(valid[..., 1:], np.diff(bic, axis=-1) > 0, True))
    assert lse_finite


def test_zero_index_queries_tie_to_lowest_blocks(msa):
    w = small_workload(2048, 4, 1, 5, seed=3)
    x = make_inputs(w)
    xg = _gpu(x)
    xg["q_idx"].zero_()
    _say(w.name, "zero q_idx")
    pooled = msa.index_scores(xg["q_idx"], xg["k_idx"])
    bi = msa.block_topk(pooled, w.top_k)
    torch.cuda.synchronize()
    gi = to_np(bi)[0, 0]
    for t in range(w.seqlen):
        cl = t // 128
        want = list(range(cl + 1)) if cl + 1 <= w.top_k else list(range(w.top_k - 1)) + [cl]
        assert list(gi[t][: len(want)]) == want


def test_duplicate_block_exact_tie_lower_index_wins(msa):
    w = small_workload(2048, 4, 1, 4, seed=4)
    x = make_inputs(w)
    x["k_idx"][:, 5 * 128:6 * 128] = x["k_idx"][:, 2 * 128:3 * 128]
    xg = _gpu(x)
    _say(w.name, "duplicate key block")
    pooled = msa.index_scores(xg["q_idx"], xg["k_idx"])
    bi = msa.block_topk(pooled, w.top_k)
    torch.cuda.synchronize()
    gp, gi = to_np(pooled), to_np(bi)
    rows = np.arange(6 * 128, w.seqlen)
    assert np.array_equal(gp[0, 0, rows, 5], gp[0, 0, rows, 2])  # identical inputs, identical sums
    np.testing.assert_array_equal(gi, O.block_topk(gp.astype(np.float64), w.top_k))
    assert any(2 in gi[0, 0, t] and 5 not in gi[0, 0, t] for t in rows)


def test_block_topk_full_length_rows_every_path(msa):
    """msa_block_topk on 1024-block rows (N = 131072) against the oracle, bit-exact, on five
    kinds of row, each sampled at every local block from 16 to 1023: normal scores; every score
    negative; five positive scores among negative ones; scores on three levels (ties, more
    candidates than the kernel's list); and constant rows of +0 and -0 (equal scores)."""
    N, nblk, k = 131072, 1024, 16
    g = torch.Generator(device=DEV).manual_seed(77)
    _say("block_topk 1024-block rows", "drawing")
    p = torch.randn(1, 1, N, nblk, device=DEV, generator=g)
    kind = ((torch.arange(N, device=DEV) // 7) % 5).view(1, 1, N, 1)
    neg = -p.abs() - 0.5
    few = torch.where(torch.rand(1, 1, N, nblk, device=DEV, generator=g) < 5.0 / 1024, p.abs() + 1.0, neg)
    levels = p.round().clamp(-1.0, 1.0)
    zeros = torch.where(torch.rand(1, 1, N, nblk, device=DEV, generator=g) < 0.5, -0.0, 0.0)
    p = torch.where(kind == 1, neg, p)
    p = torch.where(kind == 2, few, p)
    p = torch.where(kind == 3, levels, p)
    p = torch.where(kind == 4, zeros, p)
    del neg, few, levels, zeros
    _say("block_topk 1024-block rows", "select")
    bi = msa.block_topk(p, k)
    torch.cuda.synchronize()
    rows = np.array([cl * 128 + 7 * c for cl in range(16, nblk) for c in range(5)])
    sample = p[:, :, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    got = to_np(bi)[:, :, rows]
    del p, bi
    torch.cuda.empty_cache()
    kinds = (rows // 7) % 5
    assert all(np.sum(kinds == c) >= 900 for c in range(5))
    _say("block_topk 1024-block rows", f"oracle on {len(rows)} rows")
    np.testing.assert_array_equal(got, O.block_topk(sample.astype(np.float64), k, positions=rows))


def test_one_hot_value_probe(msa):
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    N = w.seqlen
    v = torch.zeros(1, N, 1, 128, dtype=torch.bfloat16)
    v[0, torch.arange(N), 0, torch.arange(N) // 128] = 1.0
    xg = _gpu(x)
    _say(w.name, "one-hot V")
    bi = msa.block_topk(msa.index_scores(xg["q_idx"], xg["k_idx"]), w.top_k)
    o, _ = msa.sparse_attn_fwd(xg["q"], xg["k"], v.to(DEV), bi, w.softmax_scale)
    torch.cuda.synchronize()
    og, gi = to_np(o)[0], to_np(bi)[0, 0]
    for t in range(N):
        sel = set(int(c) for c in gi[t] if c >= 0)
        off = [c for c in range(128) if c not in sel]
        assert np.all(og[t][:, off] == 0.0), t
        np.testing.assert_allclose(og[t][:, :w.nblk].sum(-1), 1.0, atol=2e-2)


def test_invalid_and_empty_selections(msa):
    # entries < 0 or > t//128 are padding; repeats count twice; rows with no valid entry give O = 0, LSE = -inf
    w = small_workload(1024, 8, 2, 4, seed=5)
    x = make_inputs(w)
    rng = np.random.default_rng(0)
    sel = rng.integers(-3, 10, size=(1, 2, w.seqlen, 4)).astype(np.int32)
    sel[0, 0, 300] = -1
    sel[0, 1, 900] = [7, 100, -1, -5]
    sel[0, 0, 500] = [3, 3, 1, -1]  # the query's own block (500 // 128 = 3) twice
    sel[0, 1, 640] = [2, 0, 2, 4]   # an earlier block twice; its own block (5) absent, 4 is
    sel[0, 0, 130] = [9, 8, 2, 1]   # only later blocks and its own (1): one valid entry
    xg = _gpu(x)
    _say(w.name, "invalid entries")
    o, lse = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], torch.from_numpy(sel).to(DEV), w.softmax_scale)
    torch.cuda.synchronize()
    og, lg = to_np(o), to_np(lse)
    assert np.all(og[0, 300, 0:4] == 0.0) and np.all(lg[0, 0:4, 300] == -np.inf)
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], sel, w.softmax_scale)
    assert (rl == -np.inf).sum() > 100  # the case is exercised
    assert np.array_equal(og[rl.transpose(0, 2, 1) == -np.inf], np.zeros_like(og[rl.transpose(0, 2, 1) == -np.inf]))
    check_attn(og, lg, ro, rl, "invalid-entries")


def test_sparse_attention_past_sixteen_slots(msa):
    # top_k > 16: every slot, the query's own block included, goes through the partial
    # phase and the records-only combine (the local block is computed in the combine only
    # up to 16 slots); caller selections with padding and repeats, against the oracle
    w = small_workload(4096, 16, 2, 20, seed=11)
    x = make_inputs(w)
    rng = np.random.default_rng(3)
    t = np.arange(w.seqlen)
    sel = rng.integers(-2, w.nblk, size=(1, 2, w.seqlen, 20)).astype(np.int32)
    sel[..., 0] = t // 128  # the local block, as the method's selections hold it
    sel[0, 1, 2000, 5] = sel[0, 1, 2000, 6] = 3  # a repeated block counts twice
    xg = _gpu(x)
    _say(w.name, "20 slots")
    o, lse = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], torch.from_numpy(sel).to(DEV), w.softmax_scale)
    torch.cuda.synchronize()
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], sel, w.softmax_scale)
    check_attn(to_np(o), to_np(lse), ro, rl, "20-slots")


def test_own_block_in_the_combine_matches_the_records_path(msa):
    # the same selection through the two combine paths: 16 slots (the combine computes each
    # query's own block) and the same 16 plus one padding slot (every slot through the
    # partial phase and its record); both round per-slot outputs to bf16 and merge in fp32
    w = small_workload(4096, 32, 2, 16, seed=23)
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "own block: combine against records")
    bi = msa.index_topk(xg["q_idx"], xg["k_idx"], 16)
    o1, l1 = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], bi, w.softmax_scale)
    pad = torch.full(bi.shape[:-1] + (1,), -1, dtype=torch.int32, device=DEV)
    o2, l2 = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], torch.cat([bi, pad], -1).contiguous(), w.softmax_scale)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-5
    ro, rl = O.sparse_attention(x["q"], x["k"], x["v"], to_np(bi), w.softmax_scale)
    check_attn(to_np(o1), to_np(l1), ro, rl, "own-block")


def test_deterministic_and_stage_calls_match(msa):
    w = WORKLOADS["n8k"]
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "determinism")
    r1 = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    r2 = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    shape = msa.make_shape(1, w.seqlen, w.h_q, w.h_kv, w.top_k, w.softmax_scale)
    ws = msa.alloc_workspace(shape, msa.OP_SPARSE_ATTN_FWD, torch.device(DEV))
    o3 = torch.empty_like(xg["q"])
    lse3 = torch.empty_like(r1[2])
    msa.sparse_attn_plan(shape, r1[0], ws)
    msa.sparse_attn_partial(shape, xg["q"], xg["k"], xg["v"], ws)
    msa.sparse_attn_combine(shape, xg["q"], xg["k"], xg["v"], r1[0], o3, lse3, ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    assert torch.equal(o3, r1[1]) and torch.equal(lse3, r1[2])


def test_binding_rejects_bad_shapes(msa):
    q = torch.zeros(1, 256, 4, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 256, 1, 128, dtype=torch.bfloat16, device=DEV)
    bi = torch.zeros(1, 1, 256, 4, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        msa.sparse_attn_fwd(q, k, k, bi[:, :, :128], 0.1)
    with pytest.raises(TypeError):
        msa.sparse_attn_fwd(q.float(), k, k, bi, 0.1)
    q2 = torch.zeros(1, 200, 4, 128, dtype=torch.bfloat16, device=DEV)
    k2 = torch.zeros(1, 200, 1, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.sparse_attn_fwd(q2, k2, k2, torch.zeros(1, 1, 200, 4, dtype=torch.int32, device=DEV), 0.1)
    assert e.value.status == 2
