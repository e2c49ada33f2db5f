#!/usr/bin/env python3
"""Benchmark of the MSA forward hot path on one MI355X.

One step = one full forward over one batch of the workload: index scores,
causal block max-pool and top-k selection (one single-pass kernel), reverse
index + tile plan, KV-outer partial attention, softmax combine. The two-kernel
selection (pooled scores through HBM, then a selection kernel) is timed beside
it on the same inputs. Inputs are seeded synthetic bf16 tensors
already resident in HBM when the timed region starts; each stage is bracketed
by HIP events on the stream the library launches on.

Prints ONE JSON line (rank 0): the contract fields, the roofline of the
dominant kernel, per-stage figures, the CPU oracle baseline, (unless
--no-backward) a "backward" object: msa_sparse_attn_bwd timed at the
64K-token training shape, (unless --no-decode) a "decode" object: one
decode step (msa_decode's three stages) for 128 sequences of 64K-128K tokens,
and (unless --no-long-context) a "long_context" object: msa_fwd at 2^20 tokens,
and a "long_training" object: forward and both backward passes at 2^20 tokens.

    python bench.py [--steps K] [--warmup W] [--workload n128k] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA fwd tokens/sec and TFLOP/s at N=131072, k=16, B_k=128 (% of MFMA peak)"
PROFILES = os.path.join(ROOT, "profiles")

# kernel behind each single-kernel stage, the source it is built from, and its roofline bound
STAGE_KERNEL = {
    "index_topk": ("k_index_topk", "k_index_pool.hip", "mfma"),
    "index_pool": ("k_index_pool", "k_index_pool.hip", "mfma"),
    "topk": ("k_block_topk", "k_block_topk.hip", "hbm"),
    "partial": ("k_sparse_partial", "k_sparse_partial.hip", "hbm"),
    "combine": ("k_combine", "k_combine.hip", "hbm"),
}
SHARED_HEADERS = ("msa_device.hpp", "msa_internal.hpp")
DECODE_KERNEL = {
    "index": ("k_dec_index", "k_decode.hip"),
    "topk": ("k_dec_topk", "k_decode.hip"),
    "attn": ("k_dec_attn", "k_decode.hip"),
}


def source_sha(fname: str) -> str:
    """Hash of a kernel's source file and the headers every kernel includes."""
    h = hashlib.sha256()
    for f in (fname, *SHARED_HEADERS):
        p = os.path.join(ROOT, "block_sparse_attention_head_amd", "csrc", f)
        h.update(open(p, "rb").read() if os.path.exists(p) else b"<missing>")
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch from the committed counter runs, or None when the kernel changed since."""
    p = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != source_sha(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu():
    """The host's CPU model and core counts, for the CPU-baseline record."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return {"cpu_model": model, "host_cpus_affinity": len(os.sched_getaffinity(0)),
            "host_cpus_total": os.cpu_count(), "blas_threads": blas}


SAMPLE_SEED = 7
PARITY_MAX_POSITIONS = 8192  # GPU rows kept for the parity check; the CPU leg samples fewer


def sample_order(n: int, seed: int = SAMPLE_SEED):
    import numpy as np

    return np.random.default_rng(seed).permutation(n)


def cpu_baseline(w, x, budget_s: float, seed: int = SAMPLE_SEED, max_positions: int = PARITY_MAX_POSITIONS):
    """The CPU oracle, as it stands, on a bounded uniform sample of query positions
    (until budget_s seconds of oracle time or max_positions positions).
    Returns the report and the oracle's outputs at the sampled positions."""
    import numpy as np

    from oracle import msa_oracle as O

    host = host_cpu()
    x64 = {k: v.double().numpy() for k, v in x.items() if k in ("q", "k", "v", "q_idx", "k_idx")}
    order = sample_order(w.seqlen, seed)
    done, t_total, chunk = 0, 0.0, 16
    outs = []
    while done < min(w.seqlen, max_positions) and t_total < budget_s:
        pos = np.sort(order[done:min(done + chunk, max_positions)])
        t0 = time.perf_counter()
        r = O.msa_forward(x64["q_idx"], x64["k_idx"], x64["q"], x64["k"], x64["v"], w.top_k, w.softmax_scale,
                          positions=pos)
        t_total += time.perf_counter() - t0
        outs.append((pos, r))
        done += len(pos)
    del x64
    cores = host["blas_threads"] or host["host_cpus_affinity"]
    report = {
        "value": w.batch * done / t_total,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{done} query positions drawn uniformly (seed {seed}) from the {w.name} workload "
                   f"(batch {w.batch}, all {w.h_idx} index heads and {w.h_q} query heads), full forward per "
                   f"position (index scores over all visible keys, top-k, sparse attention); "
                   f"{t_total:.1f} s of float64 NumPy on the host; tokens/s = positions x batch / seconds"),
        **host,
    }
    return report, outs


def parity_report(w, outs, gpu_rows):
    """The GPU's block_idx, O and LSE at the CPU leg's sampled positions against the oracle's.
    Index rows are compared exactly; rows that differ must be near-ties (pairwise rule of
    the oracle's near_tie_rows). O and LSE are compared on positions whose selections agree."""
    import numpy as np

    from oracle import msa_oracle as O

    where = {int(p): i for i, p in enumerate(gpu_rows["positions"])}
    n_pos = n_mis = n_tie = n_bad = 0
    max_o = max_l = 0.0
    for pos, (bi_r, o_r, lse_r, pooled_r) in outs:
        rows = np.array([where[int(p)] for p in pos])
        bi_g = gpu_rows["block_idx"][:, :, rows]
        mis, tie, bad = O.near_tie_rows(pooled_r, bi_g, bi_r, w.top_k, positions=pos)
        n_pos += len(pos)
        n_mis += mis
        n_tie += tie
        n_bad += len(bad)
        same = np.all(bi_g == bi_r, axis=(0, 1, 3))          # positions whose every index row agrees
        if same.any():
            o_g = gpu_rows["o"][:, rows][:, same]
            l_g = gpu_rows["lse"][:, :, rows][:, :, same]
            max_o = max(max_o, float(np.abs(o_g - o_r[:, same]).max()))
            max_l = max(max_l, float(np.abs(l_g - lse_r[:, :, same]).max()))
    return {"positions": n_pos, "index_rows": n_pos * w.batch * w.h_idx, "index_mismatch": n_mis,
            "near_ties": n_tie, "not_near_ties": n_bad, "max_abs_O": max_o, "max_abs_LSE": max_l,
            "tolerance": {"O": 2e-2, "LSE": 1e-3},
            "what": ("GPU msa_fwd outputs of the timed steps at the CPU baseline's sampled positions against "
                     "the float64 oracle: index rows bit-exact except counted near-ties; O and LSE max-abs error")}


def backward_report(w, steps: int, warmup: int):
    """Time msa_sparse_attn_bwd (dQ, dK, dV over the forward's cached block indices) with HIP events."""
    import torch

    from block_sparse_attention_head_amd import msa
    from block_sparse_attention_head_amd import perfmodel as P
    from synth.msa_inputs import make_inputs

    dev = torch.device("cuda:0")
    print(f"[bench] backward: generating {w.name} inputs", file=sys.stderr, flush=True)
    xg = {k: v.to(dev) for k, v in make_inputs(w.replace(with_grad=True)).items()}
    B, N, Hq, Hkv, K = w.batch, w.seqlen, w.h_q, w.h_kv, w.top_k
    block_idx, o, lse = msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], K, w.softmax_scale)
    shape = msa.make_shape(B, N, Hq, Hkv, K, w.softmax_scale)
    ws = msa.alloc_workspace(shape, msa.OP_SPARSE_ATTN_BWD, dev)
    dq, dk, dv = torch.empty_like(xg["q"]), torch.empty_like(xg["k"]), torch.empty_like(xg["v"])

    def bwd():
        msa.sparse_attn_bwd(xg["q"], xg["k"], xg["v"], o, lse, xg["d_o"], block_idx, w.softmax_scale, dq, dk, dv,
                            ws)

    def fwd():
        msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], K, w.softmax_scale, block_idx, o, lse)

    ws_idx = msa.alloc_workspace(shape, msa.OP_INDEX_BWD, dev)
    dq_idx, dk_idx = torch.empty_like(xg["q_idx"]), torch.empty_like(xg["k_idx"])

    def idx_bwd():
        msa.index_bwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], lse, block_idx, w.softmax_scale, dq_idx=dq_idx,
                      dk_idx=dk_idx, workspace=ws_idx)

    res = {}
    for name, fn in (("bwd", bwd), ("fwd", fwd), ("idx", idx_bwd)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    s = P.Shape(B, N, Hq, Hkv, K)
    tf = P.bwd_flops(s) / 1e12 / (res["bwd"] / 1e3)
    tf_idx = P.index_bwd_flops(s) / 1e12 / (res["idx"] / 1e3)
    del xg, ws, dq, dk, dv, block_idx, o, lse, ws_idx, dq_idx, dk_idx
    torch.cuda.empty_cache()
    return {"workload": w.name, "config": {"batch": B, "seqlen": N, "h_q": Hq, "h_kv": Hkv, "top_k": K},
            "what": "msa_sparse_attn_bwd: dQ, dK, dV of the main branch over the forward's block indices",
            "ms": round(res["bwd"], 4), "tokens_s": round(B * N / (res["bwd"] / 1e3), 1),
            "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / P.PEAK_BF16_TFLOPS, 4),
            "algorithmic_tflop": round(P.bwd_flops(s) / 1e12, 4),
            "fwd_ms_same_shape": round(res["fwd"], 4),
            "index_branch": {"what": "msa_index_bwd: dq_idx, dk_idx from the KL alignment term over the same indices",
                             "ms": round(res["idx"], 4), "tflops": round(tf_idx, 2),
                             "frac_of_bf16_peak": round(tf_idx / P.PEAK_BF16_TFLOPS, 4),
                             "algorithmic_tflop": round(P.index_bwd_flops(s) / 1e12, 4)}}


def decode_report(w, steps: int, warmup: int):
    """Time one decode step per stage with HIP events; inputs drawn on the GPU."""
    import torch

    from block_sparse_attention_head_amd import msa
    from block_sparse_attention_head_amd import perfmodel as P
    from synth.msa_inputs import make_decode_inputs

    print(f"[bench] decode: generating {w.name} inputs on the GPU", file=sys.stderr, flush=True)
    x = make_decode_inputs(w, device="cuda:0")
    B, C, Hq, Hkv, K = w.batch, w.capacity, w.h_q, w.h_kv, w.top_k
    dev = x["q"].device
    pooled = torch.empty((B, Hkv, C // 128), dtype=torch.float32, device=dev)
    bi = torch.empty((B, Hkv, K), dtype=torch.int32, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    # the attention's workspace: as in msa_decode, few sequences spread a group's blocks over
    # several workgroups whose records a second kernel merges
    ws = msa.alloc_workspace(msa.make_shape(B, C, Hq, Hkv, K, w.softmax_scale), msa.OP_DECODE, dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        msa.decode_index_scores(x["q_idx"], x["k_idx"], x["seqlens"], pooled)
        if ev is not None:
            ev[1].record()
        msa.decode_topk(pooled, x["seqlens"], K, C, bi)
        if ev is not None:
            ev[2].record()
        msa.decode_attn(x["q"], x["k"], x["v"], x["seqlens"], bi, w.softmax_scale, o, lse, workspace=ws)
        if ev is not None:
            ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for e in evs:
        step(e)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    lens = x["seqlens"].tolist()
    nbytes = P.decode_bytes(lens, Hq, Hkv, K)
    stages = {}
    for j, name in enumerate(("index", "topk", "attn")):
        ms = sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
        gbs = nbytes[name] / 1e9 / (ms / 1e3)
        kern, src = DECODE_KERNEL[name]
        stages[name] = {"ms": round(ms, 4), "algorithmic_GB": round(nbytes[name] / 1e9, 4), "achieved": round(gbs, 1),
                        "unit": "GB/s", "frac": round(gbs / P.PEAK_HBM_GBS, 4), "kernel": kern,
                        "traffic": _traffic(kern, w.name, src)}
    del x, pooled, bi, o, lse, ws
    torch.cuda.empty_cache()
    total = sum(nbytes.values())
    return {"workload": w.name,
            "config": {"batch": B, "cache_capacity": C, "seqlen_min": min(lens), "seqlen_max": max(lens),
                       "seqlen_mean": round(sum(lens) / len(lens), 1), "h_q": Hq, "h_kv": Hkv, "h_idx": w.h_idx,
                       "top_k": K, "seed": w.seed},
            "what": "msa_decode stages: one new token per sequence against its KV cache",
            "ms_per_step": round(ms_step, 4), "tokens_s": round(B / (ms_step / 1e3), 1),
            "achieved_GBs": round(total / 1e9 / (ms_step / 1e3), 1),
            "frac_of_hbm": round(total / 1e9 / (ms_step / 1e3) / P.PEAK_HBM_GBS, 4),
            "stages": stages}


def long_context_report(w, steps: int, warmup: int):
    """msa_fwd at 2^20 tokens (inputs drawn on the GPU), timed with HIP events. The per-slot
    partials of one pass would not fit in HBM, so the library runs the sparse attention in
    query chunks inside its workspace."""
    import torch

    from block_sparse_attention_head_amd import msa
    from block_sparse_attention_head_amd import perfmodel as P
    from synth.msa_inputs import make_inputs

    print(f"[bench] long context: generating {w.name} inputs on the GPU", file=sys.stderr, flush=True)
    xg = make_inputs(w, device="cuda:0")
    B, N, Hq, Hkv, K = w.batch, w.seqlen, w.h_q, w.h_kv, w.top_k
    dev = xg["q"].device
    shape = msa.make_shape(B, N, Hq, Hkv, K, w.softmax_scale)
    ws = msa.alloc_workspace(shape, msa.OP_FWD, dev)
    small = msa.make_shape(B, 1 << 17, Hq, Hkv, K, w.softmax_scale)
    block_idx = torch.empty((B, Hkv, N, K), dtype=torch.int32, device=dev)
    o = torch.empty_like(xg["q"])
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)

    def fwd():
        msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], K, w.softmax_scale, block_idx, o, lse,
                    workspace=ws)

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    finite = bool(torch.isfinite(o[:, ::4097].float()).all()) and bool(torch.isfinite(lse[:, :, ::4097]).all())
    # rows with at least top_k visible blocks end with their own block (shorter rows are padded)
    t_full = (K - 1) * 128
    local = bool((block_idx[:, :, t_full:, -1] == (torch.arange(t_full, N, device=dev) // 128)).all())
    s = P.Shape(B, N, Hq, Hkv, K)
    flop = P.index_flops(s) + P.main_flops(s)
    per_pos = msa.workspace_size(small, msa.OP_SPARSE_ATTN_FWD) / (1 << 17)
    del xg, ws, block_idx, o, lse
    torch.cuda.empty_cache()
    return {"workload": w.name, "config": {"batch": B, "seqlen": N, "h_q": Hq, "h_kv": Hkv, "top_k": K},
            "what": "msa_fwd (single-pass selection, chunked sparse attention)", "ms": round(ms, 2),
            "tokens_s": round(B * N / (ms / 1e3), 1), "tflops": round(flop / 1e12 / (ms / 1e3), 2),
            "workspace_GB": round(msa.workspace_size(shape, msa.OP_FWD) / 1e9, 2),
            "one_pass_workspace_GB": round(per_pos * N / 1e9, 1),
            "outputs_finite": finite, "local_block_last": local}


def long_training_report(w, steps: int, warmup: int):
    """One training step of the attention at 2^20 tokens: msa_fwd, msa_sparse_attn_bwd and
    msa_index_bwd, each timed with HIP events; each workspace is allocated for its phase and
    freed after it (the three do not fit in HBM at once)."""
    import torch

    from block_sparse_attention_head_amd import msa
    from block_sparse_attention_head_amd import perfmodel as P
    from synth.msa_inputs import make_inputs

    print(f"[bench] long training: generating {w.name} inputs on the GPU", file=sys.stderr, flush=True)
    xg = make_inputs(w, device="cuda:0")
    B, N, Hq, Hkv, K = w.batch, w.seqlen, w.h_q, w.h_kv, w.top_k
    dev = xg["q"].device
    shape = msa.make_shape(B, N, Hq, Hkv, K, w.softmax_scale)
    block_idx = torch.empty((B, Hkv, N, K), dtype=torch.int32, device=dev)
    o = torch.empty_like(xg["q"])
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(xg["q"]), torch.empty_like(xg["k"]), torch.empty_like(xg["v"])
    dqi, dki = torch.empty_like(xg["q_idx"]), torch.empty_like(xg["k_idx"])
    res, gb = {}, {}

    def timed(name, op, fn):
        ws = msa.alloc_workspace(shape, op, dev)
        gb[name] = round(ws.numel() / 1e9, 1)
        for _ in range(warmup):
            fn(ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn(ws)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
        del ws
        torch.cuda.empty_cache()

    timed("fwd", msa.OP_FWD, lambda ws: msa.msa_fwd(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], K,
                                                    w.softmax_scale, block_idx, o, lse, workspace=ws))
    timed("bwd", msa.OP_SPARSE_ATTN_BWD, lambda ws: msa.sparse_attn_bwd(
        xg["q"], xg["k"], xg["v"], o, lse, xg["d_o"], block_idx, w.softmax_scale, dq, dk, dv, ws))
    timed("index_bwd", msa.OP_INDEX_BWD, lambda ws: msa.index_bwd(
        xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], lse, block_idx, w.softmax_scale, dq_idx=dqi, dk_idx=dki,
        workspace=ws))
    finite = all(bool(torch.isfinite(t[:, ::4099].float()).all()) for t in (o, dq, dk, dv, dqi, dki))
    s = P.Shape(B, N, Hq, Hkv, K)
    flop = P.index_flops(s) + P.main_flops(s) + P.bwd_flops(s) + P.index_bwd_flops(s)
    step = res["fwd"] + res["bwd"] + res["index_bwd"]
    del xg, block_idx, o, lse, dq, dk, dv, dqi, dki
    torch.cuda.empty_cache()
    return {"workload": w.name, "config": {"batch": B, "seqlen": N, "h_q": Hq, "h_kv": Hkv, "h_idx": w.h_idx,
                                           "top_k": K},
            "what": "msa_fwd + msa_sparse_attn_bwd + msa_index_bwd", "ms": {k: round(v, 2) for k, v in res.items()},
            "step_ms": round(step, 2), "tokens_s": round(B * N / (step / 1e3), 1),
            "tflops": round(flop / 1e12 / (step / 1e3), 2), "workspace_GB": gb, "outputs_finite": finite}


def two_kernel_selection(msa, xg, w, block_idx_single, steps: int, warmup: int):
    """msa_index_scores (pooled scores to HBM) then msa_block_topk, on the step's inputs,
    timed with HIP events per kernel; the indices must equal the single pass's."""
    import torch

    K = w.top_k
    pooled = torch.empty((w.batch, w.h_idx, w.seqlen, w.nblk), dtype=torch.float32, device=xg["q"].device)
    bi = torch.empty_like(block_idx_single)
    for _ in range(warmup):
        msa.index_scores(xg["q_idx"], xg["k_idx"], pooled, visible_only=True)
        msa.block_topk(pooled, K, bi)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        msa.index_scores(xg["q_idx"], xg["k_idx"], pooled, visible_only=True)
        e[1].record()
        msa.block_topk(pooled, K, bi)
        e[2].record()
    torch.cuda.synchronize()
    ip = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    tk = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    same = bool(torch.equal(bi, block_idx_single))
    del pooled, bi
    torch.cuda.empty_cache()
    return {"index_pool_ms": round(ip, 4), "topk_ms": round(tk, 4), "total_ms": round(ip + tk, 4),
            "same_indices": same}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n128k")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward measurement at the 64K-token training shape")
    ap.add_argument("--backward-workload", default="n64k_train")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the backward measurement (a JSON line with the backward object), for profiling")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the 2^20-token forward and the 2^20-token training step")
    ap.add_argument("--decode-workload", default="dec_b128_n128k")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode measurement (a JSON line with the decode object), for profiling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device-to-device copy (counter calibration)")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this MSA build has no multi-GPU path (it would shard by "
              "MSA group, one KV head and its query heads per GPU); use --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from block_sparse_attention_head_amd import msa
    from block_sparse_attention_head_amd import perfmodel as P
    from synth.msa_inputs import DECODE_WORKLOADS, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 3
    if a.decode_only:
        out = {"decode": decode_report(DECODE_WORKLOADS[a.decode_workload], a.steps, a.warmup)}
        if a.copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
        print(json.dumps(out), flush=True)
        return 0
    if a.backward_only:
        print(json.dumps({"backward": backward_report(WORKLOADS[a.backward_workload], a.steps, a.warmup)}), flush=True)
        return 0
    w = WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x = make_inputs(w)
    xg = {k: v.to(dev) for k, v in x.items()}
    B, N, Hq, Hkv, K = w.batch, w.seqlen, w.h_q, w.h_kv, w.top_k
    shape = msa.make_shape(B, N, Hq, Hkv, K, w.softmax_scale)
    block_idx = torch.empty((B, Hkv, N, K), dtype=torch.int32, device=dev)
    o = torch.empty_like(xg["q"])
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = msa.alloc_workspace(shape, msa.OP_SPARSE_ATTN_FWD, dev)
    ws_sel = msa.alloc_workspace(shape, msa.OP_INDEX_TOPK, dev)
    stages = ["index_topk", "plan", "partial", "combine"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        msa.index_topk(xg["q_idx"], xg["k_idx"], K, block_idx, workspace=ws_sel)
        if ev is not None:
            ev[1].record()
        msa.sparse_attn_plan(shape, block_idx, ws)
        if ev is not None:
            ev[2].record()
        msa.sparse_attn_partial(shape, xg["q"], xg["k"], xg["v"], ws)
        if ev is not None:
            ev[3].record()
        msa.sparse_attn_combine(shape, xg["q"], xg["k"], xg["v"], block_idx, o, lse, ws)
        if ev is not None:
            ev[4].record()

    print(f"[bench] warmup {a.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(a.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(a.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / a.steps
    per_step = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    stage_ms = {s: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / a.steps for j, s in enumerate(stages)}
    # the last timed step's outputs at the positions the CPU baseline will sample (a superset)
    gpu_rows = None
    if not a.no_cpu_baseline:
        sp = torch.from_numpy(sample_order(N)[:PARITY_MAX_POSITIONS].copy()).to(dev)
        gpu_rows = {"positions": sp.cpu().numpy(), "block_idx": block_idx[:, :, sp].cpu().numpy(),
                    "o": o[:, sp].float().cpu().numpy(), "lse": lse[:, :, sp].cpu().numpy()}
    two_kernel = two_kernel_selection(msa, xg, w, block_idx, a.steps, a.warmup)

    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    s = P.Shape(B, N, Hq, Hkv, K)
    idx_f, main_f = P.index_flops(s), P.main_flops(s)
    work = {
        "index_topk": ("TFLOP/s", idx_f / 1e12, P.PEAK_BF16_TFLOPS),
        "partial": ("GB/s", P.partial_bytes(s) / 1e9, P.PEAK_HBM_GBS),
        "combine": ("GB/s", P.combine_bytes(s) / 1e9, P.PEAK_HBM_GBS),
    }
    stage_report = {}
    for name in stages:
        ms = stage_ms[name]
        r = {"ms": round(ms, 4)}
        if name in work:
            unit, amount, peak = work[name]
            ach = amount / (ms / 1e3)
            r.update({"achieved": round(ach, 2), "unit": unit, "peak": peak, "frac": round(ach / peak, 4),
                      "kernel": STAGE_KERNEL[name][0]})
        stage_report[name] = r
    stage_report["partial"]["tflops"] = round(P.partial_flops(s) / 1e12 / (stage_ms["partial"] / 1e3), 2)
    main_ms = stage_ms["plan"] + stage_ms["partial"] + stage_ms["combine"]

    dom = max(work, key=lambda n: stage_ms[n])
    kname, src, bound = STAGE_KERNEL[dom]
    unit, amount, peak = work[dom]
    ach = amount / (stage_ms[dom] / 1e3)
    traffic = _traffic(kname, w.name, src)
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                "traffic": traffic, "kernel": kname,
                "per_launch": (f"{amount:.4g} {'TFLOP' if unit == 'TFLOP/s' else 'GB'} algorithmic per launch "
                               f"/ {stage_ms[dom]:.3f} ms mean launch time (HIP events)")}

    tokens_s = B * N / (ms_step / 1e3)
    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seqlen": N, "h_q": Hq, "h_kv": Hkv, "h_idx": w.h_idx,
                   "head_dim": w.head_dim, "block_size": w.block_size, "top_k": K, "seed": w.seed},
        "tflops": round((idx_f + main_f) / 1e12 / (ms_step / 1e3), 2),
        "tflops_frac_of_bf16_peak": round((idx_f + main_f) / 1e12 / (ms_step / 1e3) / P.PEAK_BF16_TFLOPS, 4),
        "main_attention_tflops": round(main_f / 1e12 / (main_ms / 1e3), 2),
        "index_tflops": round(idx_f / 1e12 / (stage_ms["index_topk"] / 1e3), 2),
        "stages": stage_report,
        "two_kernel_selection": {
            **two_kernel, "single_pass_ms": round(stage_ms["index_topk"], 4),
            "index_pool_tflops": round(idx_f / 1e12 / (two_kernel["index_pool_ms"] / 1e3), 2),
            "topk_gbs": round(P.topk_bytes(s) / 1e9 / (two_kernel["topk_ms"] / 1e3), 2),
            "saving_ms": round(two_kernel["total_ms"] - stage_ms["index_topk"], 4)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    del xg, block_idx, o, lse, ws, ws_sel
    torch.cuda.empty_cache()
    if not a.no_backward:
        out["backward"] = backward_report(WORKLOADS[a.backward_workload], a.steps, a.warmup)
    if not a.no_decode:
        out["decode"] = decode_report(DECODE_WORKLOADS[a.decode_workload], a.steps, a.warmup)
    if not a.no_decode and not a.no_long_context:
        # decode at the pages' long context: 16 sequences of 768K-1M cached tokens
        try:
            out["decode_long"] = decode_report(DECODE_WORKLOADS["dec_b16_n1m"], a.steps, a.warmup)
        except Exception as exc:  # pragma: no cover
            out["decode_long"] = {"error": f"{type(exc).__name__}: {exc}"}
    if not a.no_long_context:
        try:  # a failure here must not cost the main line
            out["long_context"] = long_context_report(WORKLOADS["n1m"], min(a.steps, 2), min(a.warmup, 1))
        except Exception as exc:  # pragma: no cover
            out["long_context"] = {"error": f"{type(exc).__name__}: {exc}"}
        try:
            out["long_training"] = long_training_report(WORKLOADS["n1m_train"], 1, 1)
        except Exception as exc:  # pragma: no cover
            out["long_training"] = {"error": f"{type(exc).__name__}: {exc}"}
    if not a.no_cpu_baseline:
        print(f"[bench] CPU oracle baseline (~{a.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        out["cpu_baseline"], outs = cpu_baseline(w, x, a.cpu_budget)
        out["parity"] = parity_report(w, outs, gpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
