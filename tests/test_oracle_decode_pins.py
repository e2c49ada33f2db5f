"""Pins for the oracle's decode step (msa_decode).

Independent references: the (separately pinned) forward oracle at the
sequence's last position, torch scaled_dot_product_attention in float64 when
the selection covers every visible block, and the defining property of the
selection checked pair by pair.
"""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth.msa_inputs import make_decode_inputs, small_decode_workload


def _np(x):
    return x.double().numpy() if torch.is_tensor(x) else np.asarray(x, dtype=np.float64)


def _prefill_row(x, b, L, rng):
    """Forward-oracle inputs for sequence b: the cache rows 0..L-1 as keys, the decode
    queries at position L-1 and random queries elsewhere."""
    Hq, D = x["q"].shape[1:]
    Hi = x["q_idx"].shape[1]
    q = rng.standard_normal((1, L, Hq, D))
    qi = rng.standard_normal((1, L, Hi, D))
    q[0, L - 1] = _np(x["q"][b])
    qi[0, L - 1] = _np(x["q_idx"][b])
    return (qi, _np(x["k_idx"][b, :L])[None], q, _np(x["k"][b, :L])[None], _np(x["v"][b, :L])[None])


@pytest.mark.parametrize("top_k", [1, 3, 5])
def test_decode_equals_forward_at_the_last_position(top_k):
    w = small_decode_workload(1024, 8, 2, top_k, seed=11, batch=9)
    lengths = [1, 127, 128, 129, 256, 383, 700, 1023, 1024]
    x = make_decode_inputs(w, lengths=lengths)
    sel, o, lse, pooled = O.msa_decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], top_k,
                                       w.softmax_scale)
    rng = np.random.default_rng(0)
    for b, L in enumerate(lengths):
        qi, ki, q, k, v = _prefill_row(x, b, L, rng)
        bi, O_ref, lse_ref, pooled_ref = O.msa_forward(qi, ki, q, k, v, top_k, w.softmax_scale, positions=[L - 1])
        nb = pooled_ref.shape[-1]
        np.testing.assert_allclose(pooled[b, :, :nb], pooled_ref[0, :, 0], rtol=1e-13, atol=1e-13)
        assert np.isneginf(pooled[b, :, nb:]).all()
        np.testing.assert_array_equal(sel[b], bi[0, :, 0])
        np.testing.assert_allclose(o[b], O_ref[0, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], lse_ref[0, :, 0], rtol=1e-12, atol=1e-13)


def test_decode_dense_when_top_k_covers_every_block():
    w = small_decode_workload(640, 6, 3, 5, seed=12, batch=4)
    lengths = [1, 130, 500, 640]
    x = make_decode_inputs(w, lengths=lengths)
    sel, o, lse, _ = O.msa_decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], 5, 0.3)
    for b, L in enumerate(lengths):
        nb = -(-L // 128)
        assert list(sel[b, 0]) == list(range(nb)) + [-1] * (5 - nb)
        q = torch.tensor(_np(x["q"][b]))[:, None, :]                         # [Hq, 1, D]
        k = torch.tensor(_np(x["k"][b, :L])).permute(1, 0, 2).repeat_interleave(2, dim=0)  # [Hq, L, D]
        v = torch.tensor(_np(x["v"][b, :L])).permute(1, 0, 2).repeat_interleave(2, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.3)[:, 0]
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-13)
        z = 0.3 * torch.einsum("hd,hjd->hj", q[:, 0], k)
        np.testing.assert_allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12, atol=1e-13)


def test_decode_selection_property_with_ties():
    # key blocks repeat with period 3 so pooled scores tie; every chosen earlier block must
    # beat every unchosen earlier block under (score desc, block asc)
    w = small_decode_workload(2048, 4, 2, 5, seed=13, batch=6)
    x = make_decode_inputs(w, lengths=[2048, 2000, 1500, 1025, 700, 640])
    for c in range(3, 16):
        x["k_idx"][:, c * 128:(c + 1) * 128] = x["k_idx"][:, (c % 3) * 128:(c % 3 + 1) * 128]
    x["q_idx"][3] = 0  # all scores equal (L = 1025: local block 8)
    sel, _, _, _ = O.msa_decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], 5, 0.1)
    ki = _np(x["k_idx"])
    for b, L in enumerate(x["seqlens"].tolist()):
        t, cl = L - 1, (L - 1) // 128
        for g in range(2):
            s = ki[b, :L] @ _np(x["q_idx"][b, g])
            pooled = [max(s[j] for j in range(c * 128, min(c * 128 + 128, L))) for c in range(cl + 1)]
            row = [int(c) for c in sel[b, g]]
            assert row[-1] == cl and row[:-1] == sorted(row[:-1]) and len(set(row)) == 5
            chosen = set(row[:-1])
            for c in chosen:
                for u in set(range(cl)) - chosen:
                    assert pooled[c] > pooled[u] or (pooled[c] == pooled[u] and c < u), (b, g, c, u)
    assert [int(c) for c in sel[3, 0]] == [0, 1, 2, 3, 8]


def test_decode_empty_sequence_and_unread_cache_tail():
    w = small_decode_workload(512, 4, 1, 3, seed=14, batch=3)
    clean = make_decode_inputs(w, lengths=[0, 200, 512])
    poisoned = make_decode_inputs(w, lengths=[0, 200, 512], poison_tail=True)
    assert torch.isnan(poisoned["k"][1, 200:]).all()
    a = O.msa_decode(*(clean[n] for n in ("q_idx", "k_idx", "q", "k", "v", "seqlens")), 3, 0.2)
    b = O.msa_decode(*(poisoned[n] for n in ("q_idx", "k_idx", "q", "k", "v", "seqlens")), 3, 0.2)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    sel, o, lse, _ = a
    assert (sel[0] == -1).all() and not o[0].any() and np.isneginf(lse[0]).all()
    assert np.isfinite(o[1:]).all() and np.isfinite(lse[1:]).all()


def test_decode_given_selection_matches_forward_sparse_attention():
    # a caller's selection with repeats, padding, out-of-range and future blocks
    w = small_decode_workload(1024, 8, 2, 4, seed=15, batch=4)
    lengths = [1000, 300, 129, 1024]
    x = make_decode_inputs(w, lengths=lengths)
    rng = np.random.default_rng(1)
    given = rng.integers(-2, 9, size=(4, 2, 4)).astype(np.int32)
    given[0, 0] = [3, 3, 7, -1]
    given[1, 1] = [5, 6, -1, -4]  # nothing visible for L = 300 (blocks 0..2)
    sel, o, lse, _ = O.msa_decode(x["q_idx"], x["k_idx"], x["q"], x["k"], x["v"], x["seqlens"], 4, 0.25,
                                  block_idx=given)
    np.testing.assert_array_equal(sel, given)
    for b, L in enumerate(lengths):
        _, _, q, k, v = _prefill_row(x, b, L, rng)
        O_ref, lse_ref = O.sparse_attention(q, k, v, given[b][None, :, None, :], 0.25, positions=[L - 1])
        np.testing.assert_allclose(o[b], O_ref[0, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], lse_ref[0, :, 0], rtol=1e-12, atol=1e-13)
    assert not o[1, 4:].any() and np.isneginf(lse[1, 4:]).all()
