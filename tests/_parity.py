"""Comparison helpers shared by the GPU parity tests (test infrastructure).

Tolerances:
  * pooled scores: each is a max over fp32 dot products of 128 exact bf16
    products. fp32 summation of n terms is off by at most (n-1)*2^-24*sum|terms|,
    so the bound per element is 127*2^-24 * max_{j in block} sum_e |q_e k_je|
    (evaluated with the oracle's index_scores on |q_idx|, |k_idx|), plus 1e-6.
  * block indices: bit-exact against the oracle's selection run on the GPU's
    own pooled scores; against the oracle's float64 pooled scores, mismatching
    rows must be near-ties (reported, not failed).
  * O: max |GPU - oracle| <= 2e-2; LSE: max |GPU - oracle| <= 1e-3.
  * gradients (dQ, dK, dV of the main branch): per tensor, the largest
    elementwise error <= 1e-2 * max |oracle| and 1 - cosine similarity <= 1e-4.
    The GPU rounds P and dS to bf16 before their products (relative 2^-9 per
    term), takes D = rowsum(dO * O) from the bf16 O, and rounds each gradient
    to bf16 (2^-9): errors of a few 2^-9 of the tensor's scale, so 1e-2 leaves
    a margin of about 3. [Flash-MSA] "Correctness" compares gradients by cosine
    similarity with 0.01 as the usual bf16 tolerance; 1e-4 is far inside it.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import msa_oracle as O

O_TOL = 2e-2
LSE_TOL = 1e-3


def pooled_bound(q_idx, k_idx, positions=None):
    qa = q_idx.double().abs()
    ka = k_idx.double().abs()
    s = O.index_scores(qa, ka, positions=positions)
    s = np.where(np.isfinite(s), s, 0.0)
    return 127 * 2.0 ** -24 * s + 1e-6


def check_pooled(gpu_pooled: np.ndarray, ref_pooled: np.ndarray, bound: np.ndarray, tag="", check_upper=False):
    """Visible entries within the fp32 bound; with check_upper, the rest must be -inf."""
    vis = np.isfinite(ref_pooled)
    g = gpu_pooled[vis]
    assert np.all(np.isfinite(g)), f"{tag}: non-finite pooled score in the visible part"
    err = np.abs(g - ref_pooled[vis])
    worst = float((err / bound[vis]).max()) if err.size else 0.0
    assert worst <= 1.0, f"{tag}: pooled error exceeds the fp32 bound by x{worst:.3f}"
    if check_upper:
        assert np.all(gpu_pooled[~vis] == -np.inf), f"{tag}: blocks after the local block must be -inf"
    return float(err.max()) if err.size else 0.0


def check_topk(gpu_idx: np.ndarray, gpu_pooled: np.ndarray, ref_pooled: np.ndarray, top_k: int, positions=None,
               tag=""):
    """GPU selection == oracle selection on the GPU's pooled scores (exact);
    vs the oracle's own pooled scores, only near-ties may differ. Returns (mismatch, near_ties)."""
    same_input = O.block_topk(gpu_pooled.astype(np.float64), top_k, positions=positions)
    bad = np.argwhere(np.any(same_input != gpu_idx, axis=-1))
    assert bad.size == 0, f"{tag}: selection differs from the oracle on identical scores at rows {bad[:5].tolist()}"
    ref_idx = O.block_topk(ref_pooled, top_k, positions=positions)
    n_mis, n_tie, not_tie = O.near_tie_rows(ref_pooled, gpu_idx, ref_idx, top_k, positions=positions)
    assert not not_tie, f"{tag}: {len(not_tie)} mismatching rows are not near-ties, e.g. {not_tie[:5]}"
    return n_mis, n_tie


def check_attn(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, tag=""):
    do = float(np.abs(o_gpu - o_ref).max())
    finite = np.isfinite(lse_ref)
    assert np.array_equal(finite, np.isfinite(lse_gpu)), f"{tag}: -inf LSE pattern differs"
    dl = float(np.abs(lse_gpu[finite] - lse_ref[finite]).max()) if finite.any() else 0.0
    assert do <= O_TOL, f"{tag}: O max abs error {do:.3e} > {O_TOL}"
    assert dl <= LSE_TOL, f"{tag}: LSE max abs error {dl:.3e} > {LSE_TOL}"
    return do, dl


GRAD_REL_TOL = 1e-2
GRAD_COS_TOL = 1e-4


def check_grads(gpu, ref, tag=""):
    """Compare tuples of gradient tensors; returns a printable summary."""
    out = []
    for i, (g, r) in enumerate(zip(gpu, ref)):
        g = np.asarray(g, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        assert g.shape == r.shape, f"{tag}[{i}]: shape {g.shape} vs {r.shape}"
        assert np.all(np.isfinite(g)), f"{tag}[{i}]: non-finite gradient"
        scale = float(np.abs(r).max())
        err = float(np.abs(g - r).max())
        if scale == 0.0:
            assert err == 0.0, f"{tag}[{i}]: nonzero gradient where the oracle's is zero"
            out.append(f"[{i}] zero")
            continue
        nr, ng = float(np.linalg.norm(r)), float(np.linalg.norm(g))
        cos = float((g * r).sum() / (nr * ng)) if ng > 0 else 0.0
        rel = err / scale
        assert rel <= GRAD_REL_TOL, f"{tag}[{i}]: max error {err:.3e} = {rel:.2e} of max|ref| {scale:.3e}"
        assert 1.0 - cos <= GRAD_COS_TOL, f"{tag}[{i}]: cosine similarity {cos:.8f}"
        out.append(f"[{i}] rel {rel:.2e} 1-cos {1.0 - cos:.1e}")
    return " ".join(out)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def sample_positions(N: int, n_random: int, seed: int):
    base = {0, 1, 127, 128, 129, 255, N // 2, N // 2 + 1, N - 129, N - 128, N - 2, N - 1}
    rng = np.random.default_rng(seed)
    base.update(int(x) for x in rng.integers(0, N, size=n_random))
    return np.array(sorted(p for p in base if 0 <= p < N), dtype=np.int64)
