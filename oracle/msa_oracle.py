"""Plain, slow CPU oracle for the MiniMax Sparse Attention (MSA) forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module. The product path (the HIP library and its
Python binding) never imports, calls or links it, and this module imports
nothing from the product path.

Arithmetic is float64 NumPy throughout; bfloat16 inputs are widened exactly.
Each function writes out the definition it follows; a matrix product is the
only library primitive used, plus a stable sort for selection.

Sources (web pages; cited by title and section):
  [MSA summary]   "MiniMax Sparse Attention (MSA): Turning Theoretical Sparse
                  Attention Gains into Real GPU Speedups" (forum summary of the
                  MSA paper).
  [Flash-MSA]     "Flash-MSA: Accelerating Million-Token Training with Sparse
                  Attention Kernels" (blog post).
  [flash-msa pkg] "flash-msa 0.1.0" (package page).

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes at the repository root):
  R1  index score = raw dot product of the index query head and the shared
      index key head, no scale or activation ([MSA summary] "GPU kernel
      co-design": top-k runs on raw scores; [Flash-MSA] "Proxy attention":
      proxy dot-product);
  R2  block aggregation = max over the block's causally visible tokens
      ([Flash-MSA] "About MSA" item 1: max-pooling; "Proxy attention": causal
      local max per chunk);
  R3  top_k counts the forced local block ([MSA summary] "Architecture":
      k=16 blocks of 128 give about 2048 tokens per query);
  R4  fewer visible blocks than top_k -> every visible block is selected, the
      remaining slots hold -1;
  R5  ties in the pooled score go to the lower block index;
  R6  selected blocks are stored in ascending block order;
  R7  index head g serves query heads [g*G, (g+1)*G), G = H_q / H_kv, and
      uses KV head g ([Flash-MSA] "About MSA" item 3, "Note about scheduler":
      MSA groups equal GQA groups);
  R8  LSE is the natural log of sum_j exp(scale * q.k_j) over attended keys;
  R9  a row whose selection holds no attendable key (only possible for a
      caller-supplied selection) gets O = 0 and LSE = -inf, the limits of an
      empty sum;
  R14 a decode step for a sequence of length L computes what the forward
      computes for position L - 1 over cache rows 0..L-1;
  R15-R17 the index branch's gradient (index_kl_grad): proxy logits scaled by
      the main softmax scale unless another is given, the KL term weighted by
      the caller's kl_weight, over the main branch's attended set.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

DEFAULT_BLOCK = 128


def _f64(x) -> np.ndarray:
    """Widen an array-like (NumPy array or CPU torch tensor, any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no NumPy dtype, widen in torch first
        import torch  # local import: torch is only used to unwrap tensors

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def n_blocks(seqlen: int, block_size: int = DEFAULT_BLOCK) -> int:
    return -(-seqlen // block_size)


def _positions(seqlen: int, positions: Optional[Sequence[int]]) -> np.ndarray:
    if positions is None:
        return np.arange(seqlen, dtype=np.int64)
    p = np.asarray(positions, dtype=np.int64)
    if p.ndim != 1 or (p.size and (p.min() < 0 or p.max() >= seqlen)):
        raise ValueError("positions must be a 1-D list of query positions inside the sequence")
    return p


# ---------------------------------------------------------------------------
# Stage 1+2: index scores and causal block max-pool
# ---------------------------------------------------------------------------
def index_scores(q_idx, k_idx, block_size: int = DEFAULT_BLOCK,
                 positions: Optional[Sequence[int]] = None) -> np.ndarray:
    """Pooled index scores.

    [MSA summary] "Architecture: two-stage block-sparse attention": one index
    query head per GQA group and one shared index key head score every visible
    key token, and the token scores are aggregated into blocks. [Flash-MSA]
    "About MSA" item 1 and "Proxy attention": the aggregation is a max, taken
    causally inside the query's own block.

        s[b, g, t, j]      = sum_e q_idx[b, t, g, e] * k_idx[b, j, e]     for j <= t
        pooled[b, g, t, c] = max { s[b, g, t, j] : j in block c, j <= t }  for c <= t // B
        pooled[b, g, t, c] = -inf                                         for c >  t // B

    q_idx: [B, N, H_idx, D]; k_idx: [B, N, D].
    Returns float64 [B, H_idx, P, nblk] for the P requested positions (all N by default).
    """
    q = _f64(q_idx)
    kk = _f64(k_idx)
    B, N, H, D = q.shape
    if kk.shape != (B, N, D):
        raise ValueError("k_idx must be [B, N, D] matching q_idx")
    pos = _positions(N, positions)
    nblk = n_blocks(N, block_size)
    out = np.full((B, H, pos.size, nblk), -np.inf)
    # Rows are handled in groups that share a query block only so that one
    # matrix product serves several rows; every row still gets exactly the
    # definition above.
    qblocks = pos // block_size
    for b in range(B):
        for qb in np.unique(qblocks):
            rows = np.nonzero(qblocks == qb)[0]
            ts = pos[rows]
            hi = int(ts.max()) + 1
            r = ts.size
            s = (q[b, ts].reshape(r * H, D) @ kk[b, :hi].T).reshape(r, H, hi)  # s[r, h, j] = <q_idx, k_idx_j>
            visible = np.arange(hi)[None, :] <= ts[:, None]       # [r, hi]: causal mask
            s = np.where(visible[:, None, :], s, -np.inf)
            for c in range(int(qb) + 1):
                lo_j, hi_j = c * block_size, min((c + 1) * block_size, hi)
                out[b, :, rows, c] = s[:, :, lo_j:hi_j].max(axis=-1)
    return out


# ---------------------------------------------------------------------------
# Stage 3: top-k block selection with the local block forced
# ---------------------------------------------------------------------------
def block_topk(pooled, top_k: int, block_size: int = DEFAULT_BLOCK,
               positions: Optional[Sequence[int]] = None) -> np.ndarray:
    """Selected key blocks per (batch, index head, query).

    [MSA summary] "Architecture": the top-k blocks are kept per query and
    group, and the block holding the query's own position is always kept.
    [Flash-MSA] "Proxy attention" forces the local block by giving it an
    infinite score. [MSA summary] "GPU kernel co-design": softmax keeps the
    order, so the selection runs on raw scores.

    For query t with local block c_loc = t // B:
      * if c_loc + 1 <= top_k: every block 0..c_loc is selected (R4);
      * else: c_loc plus the top_k - 1 largest pooled[c] over c < c_loc,
        ordered by (score descending, block ascending) (R5).
    The selection is written in ascending block order (R6), padded with -1.

    pooled: [B, H, P, nblk] (as from ``index_scores``); ``positions`` names
    the query position of each of the P rows (default 0..P-1).
    Returns int32 [B, H, P, top_k].
    """
    pl = _f64(pooled)
    B, H, P, nblk = pl.shape
    if top_k < 1:
        raise ValueError("top_k must be >= 1")
    pos = np.arange(P, dtype=np.int64) if positions is None else np.asarray(positions, dtype=np.int64)
    if pos.shape != (P,) or (P and (pos.min() < 0 or pos.max() // block_size >= nblk)):
        raise ValueError("positions must give one query position per pooled row, inside the blocks")
    out = np.full((B, H, P, top_k), -1, dtype=np.int32)
    cloc = pos // block_size
    for cl in np.unique(cloc):
        rows = np.nonzero(cloc == cl)[0]
        cl = int(cl)
        if cl + 1 <= top_k:
            out[:, :, rows, : cl + 1] = np.arange(cl + 1, dtype=np.int32)
            continue
        cand = pl[:, :, rows, :cl]                              # non-local visible blocks
        order = np.argsort(-cand, axis=-1, kind="stable")       # stable: lower block wins ties
        chosen = order[..., : top_k - 1]
        sel = np.concatenate([chosen, np.full(chosen.shape[:-1] + (1,), cl)], axis=-1)
        out[:, :, rows, :] = np.sort(sel, axis=-1).astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# Stage 4: exact softmax attention over the selected blocks (main branch)
# ---------------------------------------------------------------------------
def attended_keys(sel: np.ndarray, t: int, block_size: int = DEFAULT_BLOCK) -> np.ndarray:
    """Key positions a query at position t attends to: j in a selected block and j <= t."""
    parts = [np.arange(c * block_size, min((c + 1) * block_size, t + 1)) for c in sel if c >= 0]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


def sparse_attention(q, k, v, block_idx, softmax_scale: float, block_size: int = DEFAULT_BLOCK,
                     positions: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Main-branch attention restricted to the selected blocks.

    [MSA summary] "Architecture": exact softmax attention for every query head,
    computed only over the selected blocks, with no approximation inside them.
    [Flash-MSA] "Main attention": a block-sparse (causal) flash attention
    forward; "Forward": the main LSE is saved for the backward.

    For query head h (group g = h // G) at position t, with K(t) the attended
    keys (selected blocks of group g, causal):
        z_j  = scale * <q[b,t,h], k[b,j,g]>      j in K(t)
        O    = sum_j exp(z_j) v[b,j,g] / sum_j exp(z_j)
        LSE  = log sum_j exp(z_j)
    (evaluated with the usual max shift for range, which leaves both unchanged).

    q: [B, N, H_q, D]; k, v: [B, N, H_kv, D]; block_idx: [B, H_kv, P, top_k]
    rows for the P requested positions. Returns O float64 [B, P, H_q, D] and
    LSE float64 [B, H_q, P]. A row with no attended key gives O = 0, LSE = -inf (R9).
    """
    # q is widened one requested row at a time: at long lengths the whole of it
    # in float64 would not fit in host memory, and only the requested rows are read
    kk, vv = _f64(k), _f64(v)
    bi = np.asarray(block_idx)
    B, N, Hq, D = q.shape
    Hkv = kk.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    pos = _positions(N, positions)
    if bi.shape[:3] != (B, Hkv, pos.size):
        raise ValueError("block_idx must be [B, H_kv, P, top_k] for the requested positions")
    O = np.zeros((B, pos.size, Hq, D))
    LSE = np.zeros((B, Hq, pos.size))
    for b in range(B):
        for i, t in enumerate(pos):
            t = int(t)
            qt = _f64(q[b, t])                                 # [H_q, D]
            for g in range(Hkv):
                keys = attended_keys(bi[b, g, i], t, block_size)
                if keys.size == 0:  # R9: nothing to attend to
                    O[b, i, g * G:(g + 1) * G] = 0.0
                    LSE[b, g * G:(g + 1) * G, i] = -np.inf
                    continue
                qg = qt[g * G:(g + 1) * G]                     # [G, D]
                z = softmax_scale * (qg @ kk[b, keys, g].T)  # [G, n]
                m = z.max(axis=-1, keepdims=True)
                p = np.exp(z - m)
                l = p.sum(axis=-1)
                O[b, i, g * G:(g + 1) * G] = (p @ vv[b, keys, g]) / l[:, None]
                LSE[b, g * G:(g + 1) * G, i] = m[:, 0] + np.log(l)
    return O, LSE


def msa_forward(q_idx, k_idx, q, k, v, top_k: int, softmax_scale: float,
                block_size: int = DEFAULT_BLOCK, positions: Optional[Sequence[int]] = None):
    """The whole forward: index scores -> pooled -> top-k -> sparse attention.

    [Flash-MSA] "Forward": proxy (index) attention first, then the sparse main
    attention; the main output and LSE are kept, and so are the block indices.
    Returns (block_idx int32 [B,H_idx,P,top_k], O [B,P,H_q,D], LSE [B,H_q,P], pooled).
    """
    N = np.shape(q)[1]
    pos = _positions(N, positions)
    pooled = index_scores(q_idx, k_idx, block_size, pos)
    bi = block_topk(pooled, top_k, block_size, positions=pos)
    O, LSE = sparse_attention(q, k, v, bi, softmax_scale, block_size, pos)
    return bi, O, LSE, pooled


# ---------------------------------------------------------------------------
# Backward of the main branch over cached selections
# ---------------------------------------------------------------------------
def sparse_attention_bwd(q, k, v, block_idx, d_o, softmax_scale: float, block_size: int = DEFAULT_BLOCK,
                         positions: Optional[Sequence[int]] = None):
    """Gradients of the main-branch attention with the selection held fixed.

    [Flash-MSA] "Kernel Design" and "Backward": the block indices kept from
    the forward are reused, so the main branch's backward only touches the
    selected blocks. The selection itself (a top-k) has no gradient. For query
    head h at position t (group g) with attended keys K(t), P = softmax(z),
    z_j = scale * q.k_j, O = sum_j P_j v_j, and an incoming gradient dO:
        dV_j += P_j dO
        dP_j  = dO . v_j
        dS_j  = P_j (dP_j - sum_i P_i dP_i)
        dQ    = scale * sum_j dS_j k_j
        dK_j += scale * dS_j q
    (the chain rule through the softmax; LSE receives no gradient).

    block_idx: [B, H_kv, P, top_k] rows for the P query positions that
    contribute (default: all N, one row per position). dQ rows are returned for
    those positions; dK, dV hold the sum of their contributions over the whole
    sequence. Returns dQ float64 [B, P, H_q, D], dK, dV float64 [B, N, H_kv, D].
    """
    qq, kk, vv, go = _f64(q), _f64(k), _f64(v), _f64(d_o)
    bi = np.asarray(block_idx)
    B, N, Hq, D = qq.shape
    Hkv = kk.shape[2]
    G = Hq // Hkv
    pos = _positions(N, positions)
    if bi.shape[:3] != (B, Hkv, pos.size):
        raise ValueError("block_idx must be [B, H_kv, P, top_k] for the contributing positions")
    dQ = np.zeros((B, pos.size, Hq, D))
    dK = np.zeros_like(kk)
    dV = np.zeros_like(vv)
    for b in range(B):
        for i, t in enumerate(pos):
            t = int(t)
            for g in range(Hkv):
                keys = attended_keys(bi[b, g, i], t, block_size)
                if keys.size == 0:  # R9: nothing attended, nothing to differentiate
                    continue
                hs = slice(g * G, (g + 1) * G)
                qg, dog = qq[b, t, hs], go[b, t, hs]         # [G, D]
                kg, vg = kk[b, keys, g], vv[b, keys, g]      # [n, D]
                z = softmax_scale * (qg @ kg.T)              # [G, n]
                p = np.exp(z - z.max(axis=-1, keepdims=True))
                p /= p.sum(axis=-1, keepdims=True)
                dp = dog @ vg.T                              # [G, n]
                ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
                dQ[b, i, hs] = softmax_scale * (ds @ kg)
                gk = softmax_scale * (ds.T @ qg)             # [n, D], rows in the order of `keys`
                gv = p.T @ dog
                # keys is the concatenation of one contiguous run per valid selected
                # block (attended_keys); add each run back to its block, so a block
                # listed twice receives both contributions
                o = 0
                for c in bi[b, g, i]:
                    lo, hi = int(c) * block_size, min((int(c) + 1) * block_size, t + 1)
                    if c < 0 or hi <= lo:  # padding, or a block after the query: no keys
                        continue
                    dK[b, lo:hi, g] += gk[o:o + hi - lo]
                    dV[b, lo:hi, g] += gv[o:o + hi - lo]
                    o += hi - lo
    return dQ, dK, dV


def index_kl_grad(q_idx, k_idx, q, k, block_idx, softmax_scale: float, index_scale: Optional[float] = None,
                  kl_weight: float = 1.0, block_size: int = DEFAULT_BLOCK,
                  positions: Optional[Sequence[int]] = None):
    """Gradient of the index (proxy) branch from the KL alignment loss, selection held fixed.

    [MSA summary] "Training stability": the top-k has no gradient, so the index
    projections learn from a KL alignment loss whose teacher averages each
    query head's softmax over the selected tokens, the main branch detached.
    [Flash-MSA] "KL Divergence Loss": with the teacher p and the proxy
    distribution p_px over the same tokens, L = sum_t KL(p_t || p_px,t) and
    dL/dz_px,j = p_px,j - p_j, so the loss itself is never needed.
    Readings R15-R17: the proxy logits use `index_scale` (default: the main
    softmax scale, the one scale the call takes); `kl_weight` is the gradient
    of the caller's total loss with respect to L; the attended set is the main
    branch's (selected blocks, keys <= t, a repeated block twice).

    For group g, position t with attended keys A:
        p_j    = (1/G) sum_{h in g} softmax_j(softmax_scale * q[b,t,h] . k[b,j,g])
        z_j    = index_scale * q_idx[b,t,g] . k_idx[b,j]
        p_px   = softmax_j(z)
        dz_j   = kl_weight * (p_px_j - p_j)
        dq_idx[b,t,g] = index_scale * sum_j dz_j k_idx[b,j]
        dk_idx[b,j]  += index_scale * dz_j q_idx[b,t,g]   (over t and g: one shared index key head)
    block_idx: [B, H_kv, P, top_k] rows for the P positions (default all N).
    Returns dq_idx float64 [B, P, H_idx, D_idx], dk_idx float64 [B, N, D_idx], and
    the loss kl_weight * sum over (b, g, t) of sum_j p_j (log p_j - log p_px_j).
    """
    qi, ki, qq, kk = _f64(q_idx), _f64(k_idx), _f64(q), _f64(k)
    bi = np.asarray(block_idx)
    B, N, Hq, _ = qq.shape
    Hkv = kk.shape[2]
    G = Hq // Hkv
    s_idx = softmax_scale if index_scale is None else index_scale
    pos = _positions(N, positions)
    if bi.shape[:3] != (B, Hkv, pos.size):
        raise ValueError("block_idx must be [B, H_kv, P, top_k] for the requested positions")
    dq = np.zeros((B, pos.size, Hkv, qi.shape[-1]))
    dk = np.zeros_like(ki)
    loss = 0.0
    for b in range(B):
        for i, t in enumerate(pos):
            t = int(t)
            for g in range(Hkv):
                keys = attended_keys(bi[b, g, i], t, block_size)
                if keys.size == 0:
                    continue
                z_main = softmax_scale * (qq[b, t, g * G:(g + 1) * G] @ kk[b, keys, g].T)   # [G, n]
                pm = np.exp(z_main - z_main.max(axis=-1, keepdims=True))
                pm /= pm.sum(axis=-1, keepdims=True)
                teacher = pm.mean(axis=0)                                                # [n]
                z = s_idx * (ki[b, keys] @ qi[b, t, g])                                  # [n]
                log_px = z - (z.max() + np.log(np.exp(z - z.max()).sum()))
                dz = kl_weight * (np.exp(log_px) - teacher)
                dq[b, i, g] = s_idx * (dz @ ki[b, keys])
                np.add.at(dk[b], keys, s_idx * np.outer(dz, qi[b, t, g]))
                loss += kl_weight * float((teacher * (np.log(teacher) - log_px)).sum())
    return dq, dk, loss


def positions_attending(block_idx, block: int, block_size: int = DEFAULT_BLOCK):
    """Query positions (per batch and KV head) whose selection row holds `block` (attendable: block <= t/B)."""
    bi = np.asarray(block_idx)
    t = np.arange(bi.shape[2])
    hit = np.any(bi == block, axis=-1) & (block <= t // block_size)[None, None]
    return hit  # [B, H_kv, N] boolean


# ---------------------------------------------------------------------------
# Decode: one new query per sequence against its cache
# ---------------------------------------------------------------------------
def msa_decode(q_idx, k_idx, q, k, v, seqlens, top_k: int, softmax_scale: float,
               block_size: int = DEFAULT_BLOCK, block_idx=None):
    """One decode step for a batch of sequences of different lengths.

    [MSA summary] "Why long context is the bottleneck": decoding adds one token
    at a time against a KV cache that grows with the context; "Architecture"
    and "Experimental results": the same selection (k = 16 blocks of 128, local
    block kept) serves decoding. Reading R14: the step for a sequence of length
    L computes what the forward computes for its last position t = L - 1, over
    the cache rows 0..t; cache rows at or beyond L are never read.

    q_idx [B, H_idx, D_idx], q [B, H_q, D]: the new token's index query heads
    and query heads. k_idx [B, C, D_idx], k, v [B, C, H_kv, D]: caches of
    capacity C >= max(seqlens). seqlens [B]: L per sequence; L = 0 is an empty
    sequence (block_idx all -1, O = 0, LSE = -inf, as R9).

    Written per sequence and head, without the forward's helpers:
      s_j = q_idx[b,g] . k_idx[b,j] for j <= t;  pooled_c = max of s_j over
      block c's rows;  keep c_loc = t // block_size, plus the top_k - 1
      earlier blocks by (score desc, block asc), output ascending with c_loc
      last (R3-R6); if c_loc + 1 <= top_k every block 0..c_loc, then -1;
      o, lse = softmax attention of q[b,h] over the selected blocks' rows <= t.
    With ``block_idx`` [B, H_kv, top_k] given, the attention uses those blocks
    instead (entries outside [0, c_loc] ignored, a repeated block counted twice,
    as the forward's sparse attention treats a caller's selection).
    Returns block_idx int32 [B, H_idx, top_k] (the one used), O float64
    [B, H_q, D], LSE [B, H_q], and pooled float64 [B, H_idx, ceil(C/block_size)]
    (-inf for blocks after the sequence's own).
    """
    qi, ki = _f64(q_idx), _f64(k_idx)
    qq, kk, vv = _f64(q), _f64(k), _f64(v)
    L = np.asarray(seqlens, dtype=np.int64)
    B, H_idx, _ = qi.shape
    _, H_q, D = qq.shape
    H_kv = kk.shape[2]
    G = H_q // H_kv
    if H_idx != H_kv:
        raise ValueError("one index head per KV head (R7)")
    if kk.shape[1] < L.max(initial=0):
        raise ValueError("cache capacity below the longest sequence")
    sel = np.full((B, H_idx, top_k), -1, dtype=np.int32)
    pooled_all = np.full((B, H_idx, -(-kk.shape[1] // block_size)), -np.inf)
    out = np.zeros((B, H_q, D))
    lse = np.full((B, H_q), -np.inf)
    for b in range(B):
        n = int(L[b])
        if n <= 0:
            continue
        t = n - 1
        cl = t // block_size
        for g in range(H_idx):
            scores = ki[b, :n] @ qi[b, g]
            pooled = [scores[c * block_size:min((c + 1) * block_size, n)].max() for c in range(cl + 1)]
            pooled_all[b, g, :cl + 1] = pooled
            if cl + 1 <= top_k:
                chosen = list(range(cl + 1))
            else:
                ranked = sorted(range(cl), key=lambda c: (-pooled[c], c))
                chosen = sorted(ranked[:top_k - 1]) + [cl]
            sel[b, g, :len(chosen)] = chosen
        if block_idx is not None:
            sel[b] = np.asarray(block_idx[b], dtype=np.int32)
        for g in range(H_kv):
            parts = [np.arange(c * block_size, min((c + 1) * block_size, n)) for c in sel[b, g] if 0 <= c <= cl]
            if not parts:
                continue
            rows = np.concatenate(parts)
            keys, vals = kk[b, rows, g], vv[b, rows, g]
            for h in range(g * G, (g + 1) * G):
                z = softmax_scale * (keys @ qq[b, h])
                m = z.max()
                w = np.exp(z - m)
                lse[b, h] = m + np.log(w.sum())
                out[b, h] = (w / w.sum()) @ vals
    return sel, out, lse, pooled_all


# ---------------------------------------------------------------------------
# Parity helpers (comparison logic; no method arithmetic beyond the definitions above)
# ---------------------------------------------------------------------------
def near_tie_rows(pooled_ref, sel_a, sel_b, top_k: int, block_size: int = DEFAULT_BLOCK,
                  positions: Optional[Sequence[int]] = None, rel: float = 1e-3):
    """Classify rows where a selection ``sel_a`` differs from the reference ``sel_b``.

    ``sel_b`` is the oracle's selection on ``pooled_ref`` (float64 scores); ``sel_a``
    is the one under test (fp32 scores on the GPU). A differing row is a near-tie,
    a difference that fp32 rounding of the scores can explain, when
      * both selections hold the local block and the same number of valid entries, and
      * for every block x chosen only by ``sel_a`` and every block y chosen only by
        ``sel_b``: 0 < s_y - s_x <= rel * max(|s_x|, |s_y|) in the reference scores.
    Exact equality (s_y == s_x) is never a near-tie: equal scores are ordered by
    block index (lower first), so picking x over an equal-scored lower y is a
    wrong tie-break, whatever the precision. Returns (n_mismatch, n_near_tie,
    list of (b, h, row) that are mismatches but NOT near-ties).
    """
    pl = _f64(pooled_ref)
    A = np.asarray(sel_a)
    Bs = np.asarray(sel_b)
    B, H, P, _ = A.shape
    pos = np.arange(P) if positions is None else np.asarray(positions)
    diff = np.any(A != Bs, axis=-1)
    bad = []
    n_tie = 0
    for b, h, i in zip(*np.nonzero(diff)):
        cl = int(pos[i]) // block_size
        a = set(int(x) for x in A[b, h, i] if x >= 0)
        r = set(int(x) for x in Bs[b, h, i] if x >= 0)
        ok = cl in a and cl in r and len(a) == len(r)
        if ok:
            for x in a - r:
                for y in r - a:
                    sx, sy = pl[b, h, i, x], pl[b, h, i, y]
                    if not (np.isfinite(sx) and np.isfinite(sy)):
                        ok = False
                    elif not (0.0 < sy - sx <= rel * max(abs(sx), abs(sy))):
                        ok = False
        if ok:
            n_tie += 1
        else:
            bad.append((int(b), int(h), int(i)))
    return int(diff.sum()), n_tie, bad
