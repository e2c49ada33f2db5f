"""GPU parity of the main-branch backward (msa_sparse_attn_bwd) against the CPU oracle.

The GPU forward produces block_idx, O and LSE; the GPU backward runs on them
with a seeded dO; the oracle's sparse_attention_bwd runs in float64 on the same
bf16 inputs and the same block_idx. Every test prints its case before it
touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth.msa_inputs import WORKLOADS, make_inputs, small_workload
from tests._parity import check_grads, sample_positions, to_np

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


def _fwd_bwd(msa, w, xg, sel=None):
    if sel is None:
        bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    else:
        bi = sel
        o, lse = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], bi, w.softmax_scale)
    dq, dk, dv = msa.sparse_attn_bwd(xg["q"], xg["k"], xg["v"], o, lse, xg["d_o"], bi, w.softmax_scale)
    torch.cuda.synchronize()
    return bi, dq, dk, dv


def _full_parity(msa, w, x, sel=None):
    xg = _gpu(x)
    _say(w.name, "fwd + bwd")
    bi, dq, dk, dv = _fwd_bwd(msa, w, xg, None if sel is None else torch.from_numpy(sel).to(DEV))
    gi = to_np(bi)
    _say(w.name, "oracle backward")
    rq, rk, rv = O.sparse_attention_bwd(x["q"], x["k"], x["v"], gi, x["d_o"], w.softmax_scale)
    stats = check_grads((to_np(dq), to_np(dk), to_np(dv)), (rq, rk, rv), w.name)
    _say(w.name, stats)
    return dq, dk, dv, rq, rk, rv


BWD_SHAPES = [
    # (seqlen, h_q, h_kv, top_k, batch): G = 4, 1, 2 (3 KV heads), 32, 128, 16 with every block selected
    # (8 work items on block 0), batch 2, one block
    (1024, 4, 1, 4, 1),
    (2048, 8, 2, 4, 1),
    (1024, 4, 4, 2, 1),
    (640, 6, 3, 3, 1),
    (1024, 32, 1, 5, 1),
    (768, 128, 1, 3, 1),
    (1024, 16, 1, 8, 1),
    (1024, 8, 2, 3, 2),
    (128, 4, 1, 4, 1),
]


@pytest.mark.parametrize("N,hq,hkv,k,b", BWD_SHAPES)
def test_bwd_parity(msa, N, hq, hkv, k, b):
    w = small_workload(N, hq, hkv, k, seed=200 + N + hq + k, batch=b).replace(with_grad=True)
    _full_parity(msa, w, make_inputs(w))


def test_bwd_invalid_repeated_and_empty_selections(msa):
    # entries < 0 or after the query's block are padding; a repeated block counts twice;
    # rows with no valid entry have dQ = 0 and add nothing to dK, dV
    w = small_workload(1024, 8, 2, 4, seed=5).replace(with_grad=True)
    x = make_inputs(w)
    rng = np.random.default_rng(1)
    sel = rng.integers(-3, 10, size=(1, 2, w.seqlen, 4)).astype(np.int32)
    sel[0, 0, 300] = -1
    sel[0, 1, 900] = [7, 100, -1, -5]
    sel[0, 0, 700] = [3, 3, 5, 1]
    dq, dk, dv, rq, rk, rv = _full_parity(msa, w, x, sel)
    dead = np.array([not any(0 <= c <= t // 128 for c in sel[0, g, t]) for g in range(2) for t in range(w.seqlen)])
    dead = dead.reshape(2, w.seqlen)
    assert dead.sum() > 100  # the case is exercised
    g = to_np(dq)[0]
    for grp in range(2):
        rows = np.nonzero(dead[grp])[0]
        assert np.all(g[rows, grp * 4:(grp + 1) * 4] == 0.0)


def test_bwd_deterministic(msa):
    w = small_workload(2048, 8, 2, 4, seed=8).replace(with_grad=True)
    xg = _gpu(make_inputs(w))
    _say(w.name, "backward determinism")
    bi, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    r1 = msa.sparse_attn_bwd(xg["q"], xg["k"], xg["v"], o, lse, xg["d_o"], bi, w.softmax_scale)
    shape = msa.make_shape(1, w.seqlen, w.h_q, w.h_kv, w.top_k, w.softmax_scale)
    ws = msa.alloc_workspace(shape, msa.OP_SPARSE_ATTN_BWD, torch.device(DEV))
    ws.fill_(0xAB)  # the workspace needs no initialisation
    r2 = msa.sparse_attn_bwd(xg["q"], xg["k"], xg["v"], o, lse, xg["d_o"], bi, w.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_bwd_full_size_sampled(msa):
    """The 64K-token training shape: dQ on sampled positions; dK, dV on the last
    block (every group) and on a middle block of one group (the oracle on that
    group's slice, over the positions that selected the block)."""
    w = WORKLOADS["n64k_train"]
    _say(w.name, "generating inputs")
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "fwd + bwd")
    bi, dq, dk, dv = _fwd_bwd(msa, w, xg)
    gi = to_np(bi)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t.float()).all()), name
    pos = sample_positions(w.seqlen, 24, seed=w.seed)
    _say(w.name, f"oracle dQ on {len(pos)} positions")
    rq, _, _ = O.sparse_attention_bwd(x["q"], x["k"], x["v"], gi[:, :, pos], x["d_o"], w.softmax_scale,
                                      positions=pos)
    _say(w.name, "dQ", check_grads((to_np(dq[:, pos]),), (rq,), f"{w.name}/dq"))

    last = w.nblk - 1
    hit = O.positions_attending(gi, last)[0].any(axis=0)
    lp = np.nonzero(hit)[0]
    _say(w.name, f"oracle dK, dV of block {last} over {len(lp)} positions")
    _, rk, rv = O.sparse_attention_bwd(x["q"], x["k"], x["v"], gi[:, :, lp], x["d_o"], w.softmax_scale,
                                       positions=lp)
    rows = slice(last * 128, (last + 1) * 128)
    _say(w.name, "last block", check_grads((to_np(dk[:, rows]), to_np(dv[:, rows])),
                                           (rk[:, rows], rv[:, rows]), f"{w.name}/block{last}"))

    g, c, G = 3, w.nblk // 2, w.group
    mp = np.nonzero(O.positions_attending(gi[:, g:g + 1], c)[0, 0])[0]
    _say(w.name, f"oracle dK, dV of block {c}, group {g}, over {len(mp)} positions")
    hs = slice(g * G, (g + 1) * G)
    _, rk, rv = O.sparse_attention_bwd(x["q"][:, :, hs], x["k"][:, :, g:g + 1], x["v"][:, :, g:g + 1],
                                       gi[:, g:g + 1, mp], x["d_o"][:, :, hs], w.softmax_scale, positions=mp)
    rows = slice(c * 128, (c + 1) * 128)
    _say(w.name, "middle block", check_grads((to_np(dk[:, rows, g:g + 1]), to_np(dv[:, rows, g:g + 1])),
                                             (rk[:, rows], rv[:, rows]), f"{w.name}/block{c}/group{g}"))


def test_bwd_rejects_bad_arguments(msa):
    q = torch.zeros(1, 256, 4, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 256, 1, 128, dtype=torch.bfloat16, device=DEV)
    bi = torch.zeros(1, 1, 256, 4, dtype=torch.int32, device=DEV)
    lse = torch.zeros(1, 4, 256, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        msa.sparse_attn_bwd(q, k, k, q, lse[:, :2], q, bi, 0.1)
    with pytest.raises(TypeError):
        msa.sparse_attn_bwd(q, k, k, q, lse, q.float(), bi, 0.1)
    shape = msa.make_shape(1, 256, 4, 1, 4, 0.1)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.sparse_attn_bwd(q, k, k, q, lse, q, bi, 0.1, workspace=small)
    assert e.value.status == 3
    assert msa.workspace_size(shape, msa.OP_SPARSE_ATTN_BWD) > 0
