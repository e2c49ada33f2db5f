"""Algorithmic FLOP and byte counts of the MSA forward stages (closed forms).

These are the counts the benchmark divides by measured time. They count the
work the method needs, not what a particular kernel happens to do:

  index scores     2 * d_idx FLOP per (query, visible key, index head)
                   ([MSA summary] "Architecture": every visible key is scored)
  main attention   4 * d FLOP per (query head, attended key): QK^T and PV
  top-k            reads the non-local visible pooled scores of every row that
                   has more visible blocks than top_k, writes top_k int32
  partial (KV-outer) per (query row, selected block): read the query row (bf16),
                   write a bf16 partial O row and one fp32 LSE; per tile read
                   K and V of the block once; read the reverse-index entries
  combine          read every partial O row and LSE, read the selection rows,
                   write O (bf16) and LSE (fp32)
  with the local block in the combine (top_k <= 16, as the library does): the
                   (row, own block) pairs leave the partial phase (every query
                   has exactly one); the combine reads the query rows and K and
                   V of every block once instead of their records

Decode (one query per sequence, length L, t = L - 1, c_loc = t // B_k):
  index            read the L cached index keys (bf16) and the H_idx index
                   queries; write the c_loc + 1 visible pooled scores per head
  top-k            read the c_loc earlier pooled scores per head; write top_k int32
  attention        read the K and V rows of the selected keys (min(top_k,
                   c_loc + 1) blocks, the local one up to t), the block indices
                   and the H_q queries; write O (bf16) and LSE (fp32)

Pins (tests): with 64 query heads, 4 index heads, d = d_idx = 128, k = 16,
B_k = 128 and N = 2^20, full attention needs 28.44x the per-token FLOP of
MSA ([MSA summary] "Summary" / "Experimental results": 28.4x); KV-outer
intensity is (2/3) B_k = 85.3 FLOP/B against G for query-outer
([MSA summary] "GPU kernel co-design": 85 vs 16 for B_k = 128, G = 16).
"""
from __future__ import annotations

from dataclasses import dataclass

BLOCK = 128
HEAD_DIM = 128
BF16 = 2
FP32 = 4
INT32 = 4

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def valid_blocks(t: int, top_k: int, block: int = BLOCK) -> int:
    """Blocks a query at position t attends to: min(top_k, t // block + 1)."""
    return min(top_k, t // block + 1)


def sum_valid_blocks(N: int, top_k: int, block: int = BLOCK) -> int:
    """sum_t min(top_k, t//block + 1) over t < N (N a multiple of block)."""
    nb = N // block
    return block * sum(min(top_k, c + 1) for c in range(nb)) + (N % block) * min(top_k, nb + 1)


def sum_attended_keys(N: int, top_k: int, block: int = BLOCK) -> int:
    """sum_t n_t, n_t = keys attended by query t: block * (blocks - 1) + (t % block) + 1."""
    total = 0
    for c in range(-(-N // block)):
        rows = min(block, N - c * block)
        nb = min(top_k, c + 1)
        total += rows * block * (nb - 1) + rows * (rows + 1) // 2
    return total


@dataclass(frozen=True)
class Shape:
    batch: int
    seqlen: int
    h_q: int
    h_kv: int
    top_k: int
    h_idx: int = 0
    head_dim: int = HEAD_DIM
    idx_dim: int = HEAD_DIM
    block: int = BLOCK

    @property
    def hidx(self) -> int:
        return self.h_idx or self.h_kv

    @property
    def nblk(self) -> int:
        return -(-self.seqlen // self.block)

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv


def index_flops(s: Shape) -> float:
    return 2.0 * s.idx_dim * s.hidx * s.batch * s.seqlen * (s.seqlen + 1) / 2


def main_flops(s: Shape) -> float:
    return 4.0 * s.head_dim * s.h_q * s.batch * sum_attended_keys(s.seqlen, s.top_k, s.block)


def bwd_flops(s: Shape) -> float:
    """Backward of the main branch over cached indices: five 2*d products per (query head,
    attended key) -- S recomputed, dP, dV, dK, dQ -- i.e. 2.5 x the forward's two."""
    return 10.0 * s.head_dim * s.h_q * s.batch * sum_attended_keys(s.seqlen, s.top_k, s.block)


def index_bwd_flops(s: Shape) -> float:
    """Index branch's KL gradient: per attended (position, key) the main scores of the G heads
    (2 d G) for the teacher, then per group the proxy logits, dq_idx and dk_idx (3 x 2 d)."""
    return (2.0 * s.head_dim * s.h_q + 6.0 * s.idx_dim * s.hidx) * s.batch * sum_attended_keys(s.seqlen, s.top_k,
                                                                                                 s.block)


def index_bytes(s: Shape) -> float:
    visible = s.batch * s.hidx * sum(min(s.block, s.seqlen - c * s.block) * (c + 1) for c in range(s.nblk))
    return (s.batch * s.seqlen * s.hidx * s.idx_dim * BF16 + s.batch * s.seqlen * s.idx_dim * BF16
            + visible * FP32)


def topk_bytes(s: Shape) -> float:
    read = 0
    for c in range(s.nblk):
        if c + 1 > s.top_k:
            read += min(s.block, s.seqlen - c * s.block) * c
    rows = s.batch * s.hidx * s.seqlen
    return s.batch * s.hidx * read * FP32 + rows * s.top_k * INT32


def pair_rows(s: Shape) -> int:
    """(query head, selected block) pairs = query rows the KV-outer tiles process."""
    return s.batch * s.h_kv * sum_valid_blocks(s.seqlen, s.top_k, s.block) * s.group


FOLD_MAX_TOP_K = 16  # the library's combine computes the local block for top_k up to this


def folds_local(s: Shape) -> bool:
    return s.top_k <= FOLD_MAX_TOP_K


def local_block_flops(s: Shape) -> float:
    """The main attention's FLOP on each query's own block: 4 d per query head and key of
    that block up to the position."""
    keys = sum(r * (r + 1) // 2 for r in (min(s.block, s.seqlen - c * s.block) for c in range(s.nblk)))
    return 4.0 * s.head_dim * s.h_q * s.batch * keys


def partial_flops(s: Shape) -> float:
    """The main attention's FLOP in the partial phase (all of it unless the combine takes the local block)."""
    return main_flops(s) - (local_block_flops(s) if folds_local(s) else 0.0)


def partial_bytes(s: Shape) -> float:
    rows = pair_rows(s)
    tiles = s.batch * s.h_kv * s.nblk
    entries = s.batch * s.h_kv * sum_valid_blocks(s.seqlen, s.top_k, s.block)
    if folds_local(s):
        rows -= s.batch * s.h_q * s.seqlen
        entries -= s.batch * s.h_kv * s.seqlen
    return (rows * (s.head_dim * BF16 + s.head_dim * BF16 + FP32)
            + tiles * 2 * s.block * s.head_dim * BF16 + entries * INT32)


def combine_bytes(s: Shape) -> float:
    rows = pair_rows(s)
    extra = 0
    if folds_local(s):
        rows -= s.batch * s.h_q * s.seqlen
        extra = (s.batch * s.seqlen * s.h_q * s.head_dim * BF16
                 + s.batch * s.h_kv * s.nblk * 2 * s.block * s.head_dim * BF16)
    return (rows * (s.head_dim * BF16 + FP32) + s.batch * s.h_kv * s.seqlen * s.top_k * INT32
            + s.batch * s.seqlen * s.h_q * s.head_dim * BF16 + s.batch * s.h_q * s.seqlen * FP32 + extra)


def per_token_compute_ratio(N: int, h_q: int, h_idx: int, d: int, d_idx: int, top_k: int, block: int) -> float:
    """Full causal attention FLOP per token over MSA FLOP per token (index branch + main branch)."""
    full = h_q * 4 * d * (N + 1) / 2
    msa = h_idx * 2 * d_idx * (N + 1) / 2 + h_q * 4 * d * top_k * block
    return full / msa


def kv_outer_intensity(block: int, d: int, partial_o_bytes: int = FP32) -> float:
    """FLOP per HBM byte of one (query row, key block) pair: gather the bf16 query row, write its partial O."""
    return 4.0 * block * d / (BF16 * d + partial_o_bytes * d)


def q_outer_intensity(group: int) -> float:
    """Query-outer: a K/V block is loaded for the G heads of one query, so FLOP/byte equals G."""
    return float(group)


def decode_bytes(seqlens, h_q: int, h_kv: int, top_k: int, d: int = HEAD_DIM, block: int = BLOCK):
    """Algorithmic HBM bytes of one decode step per stage: {'index', 'topk', 'attn'}."""
    idx = topk = attn = 0.0
    for L in seqlens:
        L = int(L)
        if L <= 0:
            continue
        t = L - 1
        cl = t // block
        idx += L * d * BF16 + h_kv * d * BF16 + h_kv * (cl + 1) * FP32
        topk += h_kv * (cl * FP32 + top_k * INT32)
        keys = (valid_blocks(t, top_k, block) - 1) * block + (t % block + 1)
        attn += h_kv * (keys * 2 * d * BF16 + top_k * INT32) + h_q * (2 * d * BF16 + FP32)
    return {"index": idx, "topk": topk, "attn": attn}
