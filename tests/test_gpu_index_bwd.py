"""GPU parity of the index branch's KL gradient (msa_index_bwd) against the CPU oracle.

The GPU forward produces block_idx and the main LSE; msa_index_bwd runs on
them; the oracle's index_kl_grad runs in float64 on the same bf16 inputs and
the same block_idx. Every test prints its case before it touches the GPU.
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


def _run(msa, w, xg, sel=None, index_scale=None, kl_weight=1.0, workspace=None):
    if sel is None:
        bi, _, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], w.top_k, w.softmax_scale)
    else:
        bi = sel
        _, lse = msa.sparse_attn_fwd(xg["q"], xg["k"], xg["v"], bi, w.softmax_scale)
    dq, dk = msa.index_bwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], lse, bi, w.softmax_scale,
                           index_scale=index_scale, kl_weight=kl_weight, workspace=workspace)
    torch.cuda.synchronize()
    return bi, dq, dk


def _parity(msa, w, x, sel=None, index_scale=None, kl_weight=1.0):
    xg = _gpu(x)
    _say(w.name, f"fwd + index bwd (index_scale={index_scale}, kl_weight={kl_weight})")
    bi, dq, dk = _run(msa, w, xg, None if sel is None else torch.from_numpy(sel).to(DEV), index_scale, kl_weight)
    gi = to_np(bi)
    _say(w.name, "oracle")
    rq, rk, _ = O.index_kl_grad(x["q_idx"], x["k_idx"], x["q"], x["k"], gi, w.softmax_scale,
                                index_scale=index_scale, kl_weight=kl_weight)
    stats = check_grads((to_np(dq), to_np(dk)), (rq, rk), w.name)
    _say(w.name, stats)
    return gi, dq, dk


IDX_SHAPES = [
    # (seqlen, h_q, h_kv, top_k, batch): G = 4, 4 with 2 groups, 1, 2 (3 groups), 32, 8 with batch 2,
    # one block, every block selected (the dense warmup selection)
    (1024, 4, 1, 4, 1),
    (2048, 8, 2, 4, 1),
    (1024, 4, 4, 2, 1),
    (640, 6, 3, 3, 1),
    (1024, 32, 1, 5, 1),
    (1024, 16, 2, 3, 2),
    (128, 4, 1, 4, 1),
    (1024, 8, 2, 8, 1),
]


@pytest.mark.parametrize("N,hq,hkv,k,b", IDX_SHAPES)
def test_index_bwd_parity(msa, N, hq, hkv, k, b):
    w = small_workload(N, hq, hkv, k, seed=500 + N + hq + k, batch=b)
    _parity(msa, w, make_inputs(w))


@pytest.mark.parametrize("index_scale,kl_weight", [(0.2, 1.0), (None, 0.37), (0.05, -2.0)])
def test_index_bwd_scale_and_weight(msa, index_scale, kl_weight):
    w = small_workload(1024, 8, 2, 4, seed=31)
    _parity(msa, w, make_inputs(w), index_scale=index_scale, kl_weight=kl_weight)


def test_index_bwd_invalid_repeated_and_empty_selections(msa):
    w = small_workload(1024, 8, 2, 4, seed=32)
    x = make_inputs(w)
    rng = np.random.default_rng(4)
    sel = rng.integers(-3, 10, size=(1, 2, w.seqlen, 4)).astype(np.int32)
    sel[0, 0, 300] = -1
    sel[0, 1, 900] = [7, 100, -1, -5]
    sel[0, 0, 700] = [3, 3, 5, 1]
    gi, dq, dk = _parity(msa, w, x, sel)
    dead = np.array([[not any(0 <= c <= t // 128 for c in sel[0, g, t]) for t in range(w.seqlen)] for g in range(2)])
    assert dead.sum() > 100
    g = to_np(dq)[0]
    for grp in range(2):
        assert np.all(g[np.nonzero(dead[grp])[0], grp] == 0.0)


def test_index_bwd_deterministic(msa):
    w = small_workload(2048, 8, 2, 4, seed=33)
    xg = _gpu(make_inputs(w))
    _say(w.name, "index bwd determinism")
    bi, dq1, dk1 = _run(msa, w, xg)
    shape = msa.make_shape(1, w.seqlen, w.h_q, w.h_kv, w.top_k, w.softmax_scale)
    ws = msa.alloc_workspace(shape, msa.OP_INDEX_BWD, torch.device(DEV))
    ws.fill_(0xCD)
    _, dq2, dk2 = _run(msa, w, xg, sel=bi, workspace=ws)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2)


def test_index_bwd_full_size_sampled(msa):
    """The 64K-token training shape: dq_idx on sampled positions; dk_idx on the last key block and
    the one at 7/8 of the sequence (the oracle over every position that attends the block in any
    group: about 2000 here, against about 9600 for the middle block)."""
    w = WORKLOADS["n64k_train"]
    _say(w.name, "generating inputs")
    x = make_inputs(w)
    xg = _gpu(x)
    _say(w.name, "fwd + index bwd")
    bi, dq, dk = _run(msa, w, xg)
    gi = to_np(bi)
    assert bool(torch.isfinite(dq.float()).all()) and bool(torch.isfinite(dk.float()).all())
    pos = sample_positions(w.seqlen, 24, seed=w.seed)
    _say(w.name, f"oracle dq_idx on {len(pos)} positions")
    rq, _, _ = O.index_kl_grad(x["q_idx"], x["k_idx"], x["q"], x["k"], gi[:, :, pos], w.softmax_scale, positions=pos)
    _say(w.name, "dq_idx", check_grads((to_np(dq[:, pos]),), (rq,), f"{w.name}/dq_idx"))
    for c in (w.nblk - 1, 7 * w.nblk // 8):
        hit = np.nonzero(O.positions_attending(gi, c)[0].any(axis=0))[0]
        _say(w.name, f"oracle dk_idx of block {c} over {len(hit)} positions")
        _, rk, _ = O.index_kl_grad(x["q_idx"], x["k_idx"], x["q"], x["k"], gi[:, :, hit], w.softmax_scale,
                                   positions=hit)
        rows = slice(c * 128, (c + 1) * 128)
        _say(w.name, f"block {c}", check_grads((to_np(dk[:, rows]),), (rk[:, rows],), f"{w.name}/dk_idx{c}"))


def test_index_bwd_rejects_bad_arguments(msa):
    q = torch.zeros(1, 256, 4, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 256, 1, 128, dtype=torch.bfloat16, device=DEV)
    qi = torch.zeros(1, 256, 1, 128, dtype=torch.bfloat16, device=DEV)
    ki = torch.zeros(1, 256, 128, dtype=torch.bfloat16, device=DEV)
    bi = torch.zeros(1, 1, 256, 4, dtype=torch.int32, device=DEV)
    lse = torch.zeros(1, 4, 256, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        msa.index_bwd(qi, ki, q, k, lse[:, :2], bi, 0.1)
    with pytest.raises(msa.MsaError) as e:
        msa.index_bwd(qi, ki, q, k, lse, bi, 0.1, index_scale=-1.0)
    assert e.value.status == 1
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.index_bwd(qi, ki, q, k, lse, bi, 0.1, workspace=small)
    assert e.value.status == 3
    q64 = torch.zeros(1, 256, 64, 128, dtype=torch.bfloat16, device=DEV)
    lse64 = torch.zeros(1, 64, 256, dtype=torch.float32, device=DEV)
    with pytest.raises(msa.MsaError) as e:  # G = 64 heads per group
        msa.index_bwd(qi, ki, q64, k, lse64, bi, 0.1)
    assert e.value.status == 2
