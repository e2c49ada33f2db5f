"""Pins for the oracle's backward of the main branch (selection held fixed).

Independent references: torch autograd in float64 through
scaled_dot_product_attention with an explicit mask built from the selection,
the dense causal case, and central finite differences of the (pinned) forward.
"""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O


def _inputs(rng, B, N, Hq, Hkv, D):
    return (rng.standard_normal((B, N, Hq, D)), rng.standard_normal((B, N, Hkv, D)),
            rng.standard_normal((B, N, Hkv, D)), rng.standard_normal((B, N, Hq, D)))


def _torch_grads(q, k, v, d_o, sel, scale, blk):
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    mask = np.zeros((B, Hq, N, N), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for t in range(N):
                for c in sel[b, g, t]:
                    if c >= 0:
                        mask[b, g * G:(g + 1) * G, t, c * blk:(c + 1) * blk] = True
    mask &= np.tril(np.ones((N, N), dtype=bool))[None, None]
    qt = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kt = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    vt = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), attn_mask=torch.tensor(mask), scale=scale)
    (out * torch.tensor(d_o).permute(0, 2, 1, 3)).sum().backward()
    return (qt.grad.permute(0, 2, 1, 3).numpy(), kt.grad.permute(0, 2, 1, 3).numpy(),
            vt.grad.permute(0, 2, 1, 3).numpy())


@pytest.mark.parametrize("N,Hq,Hkv,k_sel", [(384, 4, 2, 2), (640, 6, 3, 3), (300, 2, 1, 2)])
def test_bwd_matches_torch_autograd_masked_sdpa(N, Hq, Hkv, k_sel):
    rng = np.random.default_rng(N + Hq)
    q, k, v, d_o = _inputs(rng, 2, N, Hq, Hkv, 16)
    nblk = -(-N // 128)
    sel = O.block_topk(rng.standard_normal((2, Hkv, N, nblk)), k_sel)
    scale = 16 ** -0.5
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, scale)
    rq, rk, rv = _torch_grads(q, k, v, d_o, sel, scale, 128)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_bwd_dense_causal_when_topk_covers_all_blocks():
    rng = np.random.default_rng(3)
    N, Hq, Hkv, D = 256, 4, 2, 8
    q, k, v, d_o = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = O.block_topk(np.zeros((1, Hkv, N, 2)), 2)
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, 0.4)
    qt = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kt = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    vt = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(2, dim=1), vt.repeat_interleave(2, dim=1), is_causal=True, scale=0.4)
    (out * torch.tensor(d_o).permute(0, 2, 1, 3)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)


def test_bwd_central_finite_differences_of_the_forward():
    rng = np.random.default_rng(4)
    N, Hq, Hkv, D = 260, 2, 1, 4
    q, k, v, d_o = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = O.block_topk(rng.standard_normal((1, Hkv, N, 3)), 2)
    scale = 0.7
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, scale)

    def loss(qq, kk, vv):
        out, _ = O.sparse_attention(qq, kk, vv, sel, scale)
        return float((out * d_o).sum())

    eps = 1e-6
    for name, grad, args, idx in (("q", dq, 0, (0, 200, 1, 2)), ("k", dk, 1, (0, 130, 0, 1)),
                                  ("v", dv, 2, (0, 5, 0, 3)), ("k", dk, 1, (0, 255, 0, 0))):
        xs = [q.copy(), k.copy(), v.copy()]
        xs[args][idx] += eps
        up = loss(*xs)
        xs[args][idx] -= 2 * eps
        dn = loss(*xs)
        assert (up - dn) / (2 * eps) == pytest.approx(grad[idx], rel=1e-6, abs=1e-8), name


def test_bwd_positions_subset_gives_complete_gradients_of_attended_blocks():
    rng = np.random.default_rng(5)
    N, Hq, Hkv, D = 768, 4, 2, 8
    q, k, v, d_o = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = O.block_topk(rng.standard_normal((1, Hkv, N, 6)), 3)
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, 0.3)
    blk = 1
    hit = O.positions_attending(sel, blk)            # [1, Hkv, N]
    pos = np.nonzero(hit[0].any(axis=0))[0]
    sq, sk, sv = O.sparse_attention_bwd(q, k, v, sel[:, :, pos], d_o, 0.3, positions=pos)
    rows = slice(blk * 128, (blk + 1) * 128)
    np.testing.assert_allclose(sk[0, rows], dk[0, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sv[0, rows], dv[0, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sq[0], dq[0, pos], rtol=1e-12, atol=1e-13)


def test_bwd_empty_rows_contribute_nothing():
    rng = np.random.default_rng(6)
    q, k, v, d_o = _inputs(rng, 1, 256, 2, 1, 4)
    sel = np.full((1, 1, 256, 2), -1, dtype=np.int32)
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, 1.0)
    assert not dq.any() and not dk.any() and not dv.any()


def test_bwd_repeated_and_out_of_range_entries_match_log_multiplicity_bias():
    # A block listed m times enters the softmax m times, which is the same as one
    # copy with log(m) added to its logits; entries < 0 or after the query's own
    # block add nothing. Reference: float64 autograd through SDPA with that bias.
    rng = np.random.default_rng(7)
    B, N, Hq, Hkv, D, blk = 1, 512, 4, 2, 8, 128
    q, k, v, d_o = _inputs(rng, B, N, Hq, Hkv, D)
    G = Hq // Hkv
    sel = rng.integers(-2, 6, size=(B, Hkv, N, 4)).astype(np.int32)
    sel[0, 0, 400] = [2, 2, 3, -1]   # block 2 twice
    sel[0, 1, 100] = [0, 0, 0, 9]    # block 0 three times, then past the end
    mult = np.zeros((B, Hq, N, N))
    for g in range(Hkv):
        for t in range(N):
            for c in sel[0, g, t]:
                if 0 <= c <= t // blk:
                    mult[0, g * G:(g + 1) * G, t, c * blk:(c + 1) * blk] += 1
    mult *= np.tril(np.ones((N, N)))[None, None]
    live = mult.sum(-1) > 0                      # rows with at least one attended key
    assert live[0, 0, 400] and not live.all()
    bias = np.where(mult > 0, np.log(np.maximum(mult, 1)), -np.inf)
    bias[~live] = 0.0                            # keep dead rows finite; their output is masked below
    qt = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kt = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    vt = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), attn_mask=torch.tensor(bias), scale=0.5)
    w = torch.tensor(d_o).permute(0, 2, 1, 3) * torch.tensor(live[..., None].astype(np.float64))
    (out * w).sum().backward()
    dq, dk, dv = O.sparse_attention_bwd(q, k, v, sel, d_o, 0.5)
    np.testing.assert_allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
