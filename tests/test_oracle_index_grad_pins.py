"""Pins for the oracle's index-branch gradient (index_kl_grad).

Independent references: torch autograd in float64 through the explicit KL
loss (teacher detached), a closed form where the proxy equals the main branch,
central finite differences, linearity in the weight, and the dense (warmup)
selection against full causal softmax written with torch.
"""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O


def _inputs(rng, B, N, Hq, Hkv, D):
    return (rng.standard_normal((B, N, Hkv, D)), rng.standard_normal((B, N, D)),
            rng.standard_normal((B, N, Hq, D)), rng.standard_normal((B, N, Hkv, D)))


def _torch_kl(qi, ki, q, k, sel, scale, s_idx, w, blk):
    """The KL alignment loss written out in torch (teacher from detached main probabilities)."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qi_t = torch.tensor(qi, requires_grad=True)
    ki_t = torch.tensor(ki, requires_grad=True)
    qt, kt = torch.tensor(q), torch.tensor(k)
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for g in range(Hkv):
            for t in range(N):
                rows = [j for c in sel[b, g, t] if c >= 0 for j in range(c * blk, min((c + 1) * blk, t + 1))]
                if not rows:
                    continue
                idx = torch.tensor(rows)
                with torch.no_grad():
                    pm = torch.softmax(scale * qt[b, t, g * G:(g + 1) * G] @ kt[b, idx, g].T, dim=-1).mean(0)
                logp = torch.log_softmax(s_idx * ki_t[b, idx] @ qi_t[b, t, g], dim=-1)
                loss = loss + w * (pm * (torch.log(pm) - logp)).sum()
    loss.backward()
    return qi_t.grad.numpy(), ki_t.grad.numpy(), float(loss.detach())


@pytest.mark.parametrize("N,Hq,Hkv,k_sel,s_idx,w", [(300, 4, 2, 2, None, 1.0), (384, 6, 3, 3, 0.2, 0.5),
                                                   (260, 2, 1, 2, 0.9, 2.0)])
def test_index_grad_matches_autograd_of_the_kl_loss(N, Hq, Hkv, k_sel, s_idx, w):
    rng = np.random.default_rng(N + Hq)
    qi, ki, q, k = _inputs(rng, 2, N, Hq, Hkv, 8)
    sel = O.block_topk(rng.standard_normal((2, Hkv, N, -(-N // 128))), k_sel)
    scale = 8 ** -0.5
    dq, dk, loss = O.index_kl_grad(qi, ki, q, k, sel, scale, index_scale=s_idx, kl_weight=w)
    rq, rk, rloss = _torch_kl(qi, ki, q, k, sel, scale, scale if s_idx is None else s_idx, w, 128)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-10, atol=1e-12)
    assert loss == pytest.approx(rloss, rel=1e-12)


def test_index_grad_vanishes_when_the_proxy_equals_the_main_branch():
    # G = 1, q_idx = q, k_idx = k, same scale: p_px = p, so the loss and both gradients are 0
    rng = np.random.default_rng(2)
    N, D = 400, 8
    q = rng.standard_normal((1, N, 1, D))
    k = rng.standard_normal((1, N, 1, D))
    sel = O.block_topk(rng.standard_normal((1, 1, N, 4)), 2)
    dq, dk, loss = O.index_kl_grad(q, k[:, :, 0], q, k, sel, 0.4)
    assert abs(loss) < 1e-12
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


def test_index_grad_central_finite_differences_and_weight():
    rng = np.random.default_rng(3)
    N, Hq, Hkv, D = 260, 4, 2, 4
    qi, ki, q, k = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = O.block_topk(rng.standard_normal((1, Hkv, N, 3)), 2)
    dq, dk, loss = O.index_kl_grad(qi, ki, q, k, sel, 0.6, index_scale=0.8)
    eps = 1e-6
    for name, arr, idx, grad in (("q_idx", qi, (0, 200, 1, 2), dq), ("k_idx", ki, (0, 130, 3), dk),
                                 ("k_idx", ki, (0, 7, 0), dk)):
        up, dn = arr.copy(), arr.copy()
        up[idx] += eps
        dn[idx] -= eps
        args_up = (up, ki) if name == "q_idx" else (qi, up)
        args_dn = (dn, ki) if name == "q_idx" else (qi, dn)
        lu = O.index_kl_grad(*args_up, q, k, sel, 0.6, index_scale=0.8)[2]
        ld = O.index_kl_grad(*args_dn, q, k, sel, 0.6, index_scale=0.8)[2]
        assert (lu - ld) / (2 * eps) == pytest.approx(grad[idx], rel=1e-6, abs=1e-9), name
    dq3, dk3, loss3 = O.index_kl_grad(qi, ki, q, k, sel, 0.6, index_scale=0.8, kl_weight=3.0)
    np.testing.assert_allclose(dq3, 3 * dq, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk3, 3 * dk, rtol=1e-13, atol=1e-15)
    assert loss3 == pytest.approx(3 * loss, rel=1e-13) and loss > 0


def test_index_grad_dense_warmup_selection():
    # every visible block selected: the teacher is full causal attention averaged over the group
    rng = np.random.default_rng(4)
    N, Hq, Hkv, D = 256, 4, 2, 8
    qi, ki, q, k = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = O.block_topk(np.zeros((1, Hkv, N, 2)), 2)
    dq, dk, _ = O.index_kl_grad(qi, ki, q, k, sel, 0.3)
    qi_t = torch.tensor(qi, requires_grad=True)
    ki_t = torch.tensor(ki, requires_grad=True)
    causal = torch.tril(torch.ones(N, N, dtype=torch.bool))
    loss = torch.zeros((), dtype=torch.float64)
    for g in range(Hkv):
        zm = 0.3 * torch.einsum("thd,jd->htj", torch.tensor(q[0, :, 2 * g:2 * g + 2]), torch.tensor(k[0, :, g]))
        pm = torch.softmax(zm.masked_fill(~causal, -torch.inf), dim=-1).mean(0)     # [t, j]
        zp = 0.3 * (qi_t[0, :, g] @ ki_t[0].T)
        logp = torch.log_softmax(zp.masked_fill(~causal, -torch.inf), dim=-1)
        loss = loss + torch.where(causal, pm * (torch.log(pm) - logp), torch.zeros(())).sum()
    loss.backward()
    np.testing.assert_allclose(dq, qi_t.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, ki_t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_index_grad_empty_rows_and_repeats():
    rng = np.random.default_rng(5)
    N, Hq, Hkv, D = 384, 2, 1, 4
    qi, ki, q, k = _inputs(rng, 1, N, Hq, Hkv, D)
    sel = np.full((1, 1, N, 3), -1, dtype=np.int32)
    dq, dk, loss = O.index_kl_grad(qi, ki, q, k, sel, 0.5)
    assert not dq.any() and not dk.any() and loss == 0.0
    sel[0, 0, 300] = [2, 2, 0]  # block 2 twice
    dq, dk, loss = O.index_kl_grad(qi, ki, q, k, sel, 0.5)
    rq, rk, rl = _torch_kl(qi, ki, q, k, sel, 0.5, 0.5, 1.0, 128)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, rk, rtol=1e-10, atol=1e-12)
    assert np.nonzero(np.abs(dq).sum(axis=(0, 2, 3)))[0].tolist() == [300]
