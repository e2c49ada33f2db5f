"""Seeded synthetic inputs for the MSA forward path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic, so both the CPU oracle's tests and the GPU path may use it.

Recipe (the same for every workload):
  * one ``torch.Generator('cpu')`` seeded with the workload's seed;
  * float32 standard-normal draws in this fixed order:
      1. Q      [B, N, H_q, 128]
      2. K      [B, N, H_kv, 128]
      3. V      [B, N, H_kv, 128]
      4. Q_idx  [B, N, H_idx, 128]
      5. K_idx  [B, N, 128]
      6. U      [B, nblk, 128], each row scaled to unit length
      7. dO     [B, N, H_q, 128]   (training-step workload only)
  * K_idx[b, j] += 0.5 * U[b, j // 128]  (a per-block offset that gives the
    index scores a block structure, as trained index keys would have);
  * every tensor rounded to bfloat16 (round-to-nearest-even).

Decode workloads (one new token per sequence against its cache) use their own
generator, ``make_decode_inputs``, on the CPU or on a GPU, in this order:
  1. L      [B] sequence lengths, uniform integers in [min_len, max_len]
  2. Q      [B, H_q, 128]      3. Q_idx [B, H_idx, 128]
  then per sequence b: 4. K [C, H_kv, 128]  5. V [C, H_kv, 128]
  6. K_idx [C, 128]  7. U [ceil(C/128), 128] unit rows, K_idx[j] += 0.5 U[j // 128]
with C the cache capacity; cache rows at or beyond L are drawn too (an
allocation holds whatever it holds) unless ``poison_tail`` fills them with NaN.

The pages measure on trained models and public benchmarks that are not
available here; these inputs stand in for them with the head shapes the pages
name (64 query heads, 4 KV heads, head dim 128 for the 109B model).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

BLOCK_SIZE = 128
HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    h_q: int
    h_kv: int
    h_idx: int
    top_k: int
    seed: int
    head_dim: int = HEAD_DIM
    idx_dim: int = HEAD_DIM
    block_size: int = BLOCK_SIZE
    with_grad: bool = False
    offset_scale: float = 0.5

    @property
    def nblk(self) -> int:
        return -(-self.seqlen // self.block_size)

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def softmax_scale(self) -> float:
        return self.head_dim ** -0.5

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # 1024 tokens (8 blocks), 4 query heads on 1 KV head, top-4.
    "tiny_n1k": Workload("tiny_n1k", batch=1, seqlen=1024, h_q=4, h_kv=1, h_idx=1, top_k=4, seed=0),
    # 8192 tokens (64 blocks), 32 query heads on 8 KV heads, top-16.
    "n8k": Workload("n8k", batch=1, seqlen=8192, h_q=32, h_kv=8, h_idx=8, top_k=16, seed=1),
    # batch 2 x 32768 tokens (256 blocks), 64 query heads on 8 KV heads, top-16.
    "n32k_b2": Workload("n32k_b2", batch=2, seqlen=32768, h_q=64, h_kv=8, h_idx=8, top_k=16, seed=2),
    # 131072 tokens (1024 blocks), 64 query heads on 4 KV heads (the 109B model's
    # attention shape), top-16.
    "n128k": Workload("n128k", batch=1, seqlen=131072, h_q=64, h_kv=4, h_idx=4, top_k=16, seed=3),
    # 2^20 tokens (8192 blocks) on the 128K workload's heads: the context length of the pages'
    # prefill figure (inputs drawn on the GPU)
    "n1m": Workload("n1m", batch=1, seqlen=1 << 20, h_q=64, h_kv=4, h_idx=4, top_k=16, seed=9),
    # the training step's heads at 2^20 tokens: the length of the training pages' title
    # (inputs drawn on the GPU)
    "n1m_train": Workload("n1m_train", batch=1, seqlen=1 << 20, h_q=32, h_kv=8, h_idx=8, top_k=16, seed=10,
                          with_grad=True),
    # main-branch training step: 65536 tokens, 32 query heads on 8 KV heads, top-16.
    "n64k_train": Workload("n64k_train", batch=1, seqlen=65536, h_q=32, h_kv=8, h_idx=8, top_k=16,
                           seed=4, with_grad=True),
}


def make_inputs(w: Workload, generator_seed: Optional[int] = None, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """Draw the workload's inputs as contiguous bfloat16 tensors, on the CPU by default
    (a GPU generator draws a different, equally seeded stream: for sizes the CPU
    would take minutes over).

    Returns a dict with q, k, v, q_idx, k_idx (and d_o when ``w.with_grad``).
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if generator_seed is None else generator_seed)
    B, N = w.batch, w.seqlen
    f32 = torch.float32
    q = torch.randn((B, N, w.h_q, w.head_dim), generator=g, dtype=f32, device=device)
    q = q.to(torch.bfloat16) if device != "cpu" else q
    k = torch.randn((B, N, w.h_kv, w.head_dim), generator=g, dtype=f32, device=device)
    v = torch.randn((B, N, w.h_kv, w.head_dim), generator=g, dtype=f32, device=device)
    q_idx = torch.randn((B, N, w.h_idx, w.idx_dim), generator=g, dtype=f32, device=device)
    k_idx = torch.randn((B, N, w.idx_dim), generator=g, dtype=f32, device=device)
    u = torch.randn((B, w.nblk, w.idx_dim), generator=g, dtype=f32, device=device)
    u = u / u.norm(dim=-1, keepdim=True)
    block_of = torch.arange(N, device=device) // w.block_size
    k_idx += w.offset_scale * u[:, block_of, :]
    out = {
        "q": q.to(torch.bfloat16),
        "k": k.to(torch.bfloat16),
        "v": v.to(torch.bfloat16),
        "q_idx": q_idx.to(torch.bfloat16),
        "k_idx": k_idx.to(torch.bfloat16),
    }
    del q, k, v, q_idx, k_idx
    if w.with_grad:
        out["d_o"] = torch.randn((B, N, w.h_q, w.head_dim), generator=g, dtype=f32, device=device).to(torch.bfloat16)
    return out


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    capacity: int
    h_q: int
    h_kv: int
    h_idx: int
    top_k: int
    seed: int
    min_len: int
    max_len: int
    head_dim: int = HEAD_DIM
    idx_dim: int = HEAD_DIM
    block_size: int = BLOCK_SIZE
    offset_scale: float = 0.5

    @property
    def nblk(self) -> int:
        return -(-self.capacity // self.block_size)

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def softmax_scale(self) -> float:
        return self.head_dim ** -0.5

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    # the deployment batch of the pages' selection kernel (128 sequences, top-16) on the
    # 109B model's attention shape, contexts of 64K-128K tokens
    "dec_b128_n128k": DecodeWorkload("dec_b128_n128k", batch=128, capacity=131072, h_q=64, h_kv=4, h_idx=4,
                                     top_k=16, seed=5, min_len=65536, max_len=131072),
    # 16 sequences of 768K-1M tokens: the context length of the pages' decoding figure
    "dec_b16_n1m": DecodeWorkload("dec_b16_n1m", batch=16, capacity=1048576, h_q=64, h_kv=4, h_idx=4,
                                  top_k=16, seed=6, min_len=786432, max_len=1048576),
}


def make_decode_inputs(w: DecodeWorkload, device: str = "cpu", poison_tail: bool = False,
                       lengths: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Draw a decode step's inputs on `device` (bfloat16, seqlens int32).

    Returns q, q_idx [B, H, 128]; k, v [B, C, H_kv, 128]; k_idx [B, C, 128];
    seqlens [B]. `lengths` overrides the drawn lengths (the draws still happen,
    so the other tensors do not change)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    B, C = w.batch, w.capacity
    f32, bf = torch.float32, torch.bfloat16
    seqlens = torch.randint(w.min_len, w.max_len + 1, (B,), generator=g, device=device, dtype=torch.int64)
    if lengths is not None:
        seqlens = torch.as_tensor(lengths, dtype=torch.int64, device=device).clone()
    q = torch.randn((B, w.h_q, w.head_dim), generator=g, device=device, dtype=f32).to(bf)
    q_idx = torch.randn((B, w.h_idx, w.idx_dim), generator=g, device=device, dtype=f32).to(bf)
    k = torch.empty((B, C, w.h_kv, w.head_dim), device=device, dtype=bf)
    v = torch.empty_like(k)
    k_idx = torch.empty((B, C, w.idx_dim), device=device, dtype=bf)
    nb = -(-C // w.block_size)
    block_of = torch.arange(C, device=device) // w.block_size
    for b in range(B):
        k[b] = torch.randn((C, w.h_kv, w.head_dim), generator=g, device=device, dtype=f32).to(bf)
        v[b] = torch.randn((C, w.h_kv, w.head_dim), generator=g, device=device, dtype=f32).to(bf)
        ki = torch.randn((C, w.idx_dim), generator=g, device=device, dtype=f32)
        u = torch.randn((nb, w.idx_dim), generator=g, device=device, dtype=f32)
        u = u / u.norm(dim=-1, keepdim=True)
        k_idx[b] = (ki + w.offset_scale * u[block_of]).to(bf)
        if poison_tail:
            n = int(seqlens[b])
            k[b, n:] = float("nan")
            v[b, n:] = float("nan")
            k_idx[b, n:] = float("nan")
    return {"q": q, "q_idx": q_idx, "k": k, "v": v, "k_idx": k_idx, "seqlens": seqlens.to(torch.int32)}


def small_decode_workload(capacity: int, h_q: int, h_kv: int, top_k: int, seed: int, batch: int,
                          min_len: int = 1, max_len: Optional[int] = None) -> DecodeWorkload:
    """A named-by-shape decode workload for parity tests."""
    return DecodeWorkload(f"dec_b{batch}_c{capacity}_hq{h_q}_hkv{h_kv}_k{top_k}_s{seed}", batch=batch,
                          capacity=capacity, h_q=h_q, h_kv=h_kv, h_idx=h_kv, top_k=top_k, seed=seed,
                          min_len=min_len, max_len=capacity if max_len is None else max_len)


def small_workload(seqlen: int, h_q: int, h_kv: int, top_k: int, seed: int, batch: int = 1,
                   h_idx: Optional[int] = None) -> Workload:
    """A named-by-shape workload for parity tests at sizes the oracle finishes quickly."""
    return Workload(f"b{batch}_n{seqlen}_hq{h_q}_hkv{h_kv}_k{top_k}_s{seed}", batch=batch, seqlen=seqlen,
                    h_q=h_q, h_kv=h_kv, h_idx=h_kv if h_idx is None else h_idx, top_k=top_k, seed=seed)
