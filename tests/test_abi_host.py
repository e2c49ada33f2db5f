"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching the GPU. No compute call is
made here, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_attention_head_amd", "libmsa.so")
HEADER = os.path.join(ROOT, "include", "msa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmsa.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401  (bind to torch's HIP runtime, as the binding does)
    from block_sparse_attention_head_amd import msa

    return msa


def test_every_declared_function_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    declared = _declared()
    assert "msa_fwd" in declared and "msa_block_topk" in declared
    assert not set(declared) - exported, sorted(set(declared) - exported)


def test_library_loads_and_resolves_every_symbol(m):
    lib = m.lib()
    for name in _declared():
        assert getattr(lib, name) is not None


def _ws(m, op=None, **kw):
    base = dict(batch=1, seqlen=1024, h_q=4, h_kv=1, top_k=4, softmax_scale=128 ** -0.5)
    base.update(kw)
    s = m.make_shape(**base)
    n = ctypes.c_size_t(123)
    st = m.lib().msa_workspace_size(ctypes.byref(s), m.OP_FWD if op is None else op, ctypes.byref(n))
    return st, n.value


def test_workspace_size_valid(m):
    st, n = _ws(m)
    assert st == 0
    # reverse index + partials [1,1024,4,4,128] bf16 + lse (the selection runs in one pass)
    assert n >= 1024 * 4 * 4 * 128 * 2 + 1024 * 4 * 4 * 4
    st, n = _ws(m, op=m.OP_INDEX_SCORES)
    assert (st, n) == (0, 0)
    st, n = _ws(m, op=m.OP_BLOCK_TOPK)
    assert (st, n) == (0, 0)
    st1, n1 = _ws(m, op=m.OP_SPARSE_ATTN_FWD)
    st2, n2 = _ws(m, op=m.OP_FWD)
    assert st1 == st2 == 0 and n2 == n1
    # top_k = 18 runs index scores and selection as two kernels: pooled [1,1,4096,32] fp32 on top
    st1, n1 = _ws(m, op=m.OP_SPARSE_ATTN_FWD, top_k=18, seqlen=4096)
    st2, n2 = _ws(m, op=m.OP_FWD, top_k=18, seqlen=4096)
    assert st1 == st2 == 0 and n2 >= n1 + 4096 * 32 * 4
    # backward: reverse index + D [1,1024,4] + dQ partials [1,1024,4,4,128] bf16 + dK/dV item partials
    # index + selection: one pass without workspace for top_k <= 17, else the pooled scores
    assert _ws(m, op=m.OP_INDEX_TOPK) == (0, 0)
    st4, n4 = _ws(m, op=m.OP_INDEX_TOPK, top_k=18, seqlen=4096)
    assert st4 == 0 and n4 >= 4096 * 32 * 4
    st3, n3 = _ws(m, op=m.OP_SPARSE_ATTN_BWD)
    assert st3 == 0 and n3 >= 1024 * 4 * 4 + 1024 * 4 * 4 * 128 * 2 + 2 * 128 * 128 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 1),
    (dict(seqlen=0), 1),
    (dict(h_q=6, h_kv=4), 1),           # not a multiple
    (dict(top_k=0), 1),
    (dict(softmax_scale=0.0), 1),
    (dict(softmax_scale=float("inf")), 1),
    (dict(seqlen=1000), 2),             # not a multiple of 128
    (dict(h_q=12, h_kv=4), 2),          # G = 3 is not a power of two
    (dict(h_q=256, h_kv=1), 2),         # G > 128
    (dict(top_k=257), 2),
])
def test_workspace_size_rejects(m, kw, code):
    st, _ = _ws(m, **kw)
    assert st == code, (kw, st)


def test_unsupported_dims_and_flags(m):
    s = m.make_shape(1, 1024, 4, 1, 4, 0.1)
    n = ctypes.c_size_t()
    for field, val in (("head_dim", 64), ("idx_dim", 256), ("block_size", 64), ("h_idx", 2), ("flags", 0)):
        t = m.make_shape(1, 1024, 4, 1, 4, 0.1)
        setattr(t, field, val)
        assert m.lib().msa_workspace_size(ctypes.byref(t), m.OP_FWD, ctypes.byref(n)) == 2, field
    assert m.lib().msa_workspace_size(ctypes.byref(s), 9, ctypes.byref(n)) == 1
    assert m.lib().msa_workspace_size(ctypes.byref(s), 8, ctypes.byref(n)) == 1
    assert m.lib().msa_workspace_size(None, m.OP_FWD, ctypes.byref(n)) == 1
    assert m.lib().msa_workspace_size(ctypes.byref(s), m.OP_FWD, None) == 1


def test_null_pointers_rejected_before_any_launch(m):
    lib = m.lib()
    s = m.make_shape(1, 1024, 4, 1, 4, 0.1)
    P = ctypes.c_void_p
    one = P(16)  # never dereferenced: validation fails on the null argument first
    assert lib.msa_index_scores(ctypes.byref(s), P(0), one, one, P(0)) == 1
    assert lib.msa_block_topk(ctypes.byref(s), one, P(0), P(0), 0, P(0)) == 1
    assert lib.msa_sparse_attn_fwd(ctypes.byref(s), one, one, one, one, one, P(0), one, 1 << 40, P(0)) == 1
    # workspace too small / missing
    assert lib.msa_sparse_attn_fwd(ctypes.byref(s), one, one, one, one, one, one, P(0), 0, P(0)) == 3
    assert lib.msa_fwd(ctypes.byref(s), one, one, one, one, one, one, one, one, one, 10, P(0)) == 3
    assert lib.msa_sparse_attn_plan(ctypes.byref(s), one, one, 10, P(0)) == 3
    assert lib.msa_sparse_attn_partial(ctypes.byref(s), one, one, one, one, 10, P(0)) == 3
    assert lib.msa_sparse_attn_combine(ctypes.byref(s), one, one, one, one, one, one, one, 10, P(0)) == 3
    for i in range(6):  # each of q, k, v, block_idx, o, lse
        args = [one] * 6
        args[i] = P(0)
        assert lib.msa_sparse_attn_combine(ctypes.byref(s), *args, one, 1 << 40, P(0)) == 1
    assert lib.msa_fwd(None, one, one, one, one, one, one, one, one, one, 10, P(0)) == 1
    assert lib.msa_index_topk(ctypes.byref(s), P(0), one, one, one, 1 << 40, P(0)) == 1
    big = m.make_shape(batch=1, seqlen=4096, h_q=4, h_kv=1, top_k=18, softmax_scale=0.1)
    assert lib.msa_index_topk(ctypes.byref(big), one, one, one, P(0), 1 << 40, P(0)) == 3
    assert lib.msa_index_topk(ctypes.byref(big), one, one, one, one, 8, P(0)) == 3
    bwd = lib.msa_sparse_attn_bwd
    args = [one] * 10
    for i in range(10):  # each of q, k, v, o, lse, d_o, block_idx, dq, dk, dv
        a = list(args)
        a[i] = P(0)
        assert bwd(ctypes.byref(s), *a, one, 1 << 40, P(0)) == 1, i
    assert bwd(ctypes.byref(s), *args, P(0), 1 << 40, P(0)) == 3
    assert bwd(ctypes.byref(s), *args, one, 10, P(0)) == 3


def test_status_strings(m):
    for code in range(5):
        assert m.lib().msa_status_string(code).startswith(b"MSA_")
    assert m.lib().msa_status_string(77) == b"unknown msa_status"


def test_binding_rejects_cpu_tensors(m):
    import torch

    q = torch.zeros(1, 128, 1, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.index_scores(q, k)


def test_decode_shape_validation_and_workspace(m):
    lib = m.lib()
    P = ctypes.c_void_p
    one = P(16)  # never dereferenced: validation fails first
    n = ctypes.c_size_t(0)
    # capacity 4096 (32 blocks), 4 KV heads, batch 8: pooled [8, 4, 32] fp32
    s = m.make_shape(8, 4096, 64, 4, 16, 128 ** -0.5)
    assert lib.msa_workspace_size(ctypes.byref(s), m.OP_DECODE, ctypes.byref(n)) == 0
    assert n.value >= 8 * 4 * 32 * 4
    for kw, code in [(dict(seqlen=4000), 2), (dict(top_k=66), 2), (dict(seqlen=(1 << 21) + 128), 2),
                     (dict(h_q=48), 2), (dict(h_q=6), 1), (dict(softmax_scale=0.0), 1)]:
        args = dict(batch=8, seqlen=4096, h_q=64, h_kv=4, top_k=16, softmax_scale=0.1)
        args.update(kw)
        bad = m.make_shape(**args)
        assert lib.msa_workspace_size(ctypes.byref(bad), m.OP_DECODE, ctypes.byref(n)) == code, kw
        assert lib.msa_decode_topk(ctypes.byref(bad), one, one, one, P(0)) == code, kw
    # the decode limits differ from the forward's: a capacity of 2^23 tokens is no forward shape
    # either, but top_k = 65 at 1M tokens is a decode shape only
    ok = m.make_shape(2, 1 << 20, 64, 4, 65, 0.1)
    assert lib.msa_workspace_size(ctypes.byref(ok), m.OP_DECODE, ctypes.byref(n)) == 0
    args = [one] * 9
    for i in range(9):  # q_idx, k_idx, q, k, v, seqlens, block_idx, o, lse
        a = list(args)
        a[i] = P(0)
        assert lib.msa_decode(ctypes.byref(s), *a, one, 1 << 40, P(0)) == 1, i
    assert lib.msa_decode(ctypes.byref(s), *args, one, 8, P(0)) == 3
    assert lib.msa_decode(ctypes.byref(s), *args, P(0), 1 << 40, P(0)) == 3
    assert lib.msa_decode_index_scores(ctypes.byref(s), one, one, P(0), one, P(0)) == 1
    assert lib.msa_decode_attn(ctypes.byref(s), one, one, one, one, one, one, P(0), P(0), 0, P(0)) == 1
    # 8 sequences x 4 KV heads leave CUs idle: a workspace given to the attention must hold
    # its split records (NULL runs one workgroup per group and needs none)
    assert lib.msa_decode_attn(ctypes.byref(s), one, one, one, one, one, one, one, one, 8, P(0)) == 3


def test_index_bwd_validation(m):
    lib = m.lib()
    P = ctypes.c_void_p
    one = P(16)
    s = m.make_shape(1, 1024, 8, 2, 4, 0.1)
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(s), m.OP_INDEX_BWD, ctypes.byref(n)) == 0
    # dZ and dq_idx partials: 2 groups x 1024 positions x 4 slots x 128 keys/dims, bf16 each
    assert n.value >= 2 * (2 * 1024 * 4 * 128 * 2)
    args = [one] * 6
    for i in range(6):  # q_idx, k_idx, q, k, lse, block_idx
        a = list(args)
        a[i] = P(0)
        assert lib.msa_index_bwd(ctypes.byref(s), *a, ctypes.c_float(0.1), ctypes.c_float(1.0), one, one, one,
                                 1 << 40, P(0)) == 1, i
    call = lambda sh, sc, w, ws, nb: lib.msa_index_bwd(ctypes.byref(sh), *args, ctypes.c_float(sc), ctypes.c_float(w),
                                                       one, one, ws, nb, P(0))
    assert call(s, 0.0, 1.0, one, 1 << 40) == 1
    assert call(s, 0.1, float("nan"), one, 1 << 40) == 1
    assert call(s, 0.1, 1.0, one, 8) == 3
    assert call(m.make_shape(1, 1024, 128, 2, 4, 0.1), 0.1, 1.0, one, 1 << 40) == 2  # 64 heads per group


def test_forward_workspace_is_bounded_by_chunking(m):
    # 1M tokens, 64 query heads, top-16: one pass would need 2^20 * 16 * 64 * 260 B of per-slot
    # partials (about 280 GB); the library asks for one chunk's worth under its 64 GiB budget
    s = m.make_shape(1, 1 << 20, 64, 4, 16, 0.1)
    n = ctypes.c_size_t(0)
    assert m.lib().msa_workspace_size(ctypes.byref(s), m.OP_FWD, ctypes.byref(n)) == 0
    assert (32 << 30) < n.value <= (64 << 30)
    small = m.make_shape(1, 128 * 1024, 64, 4, 16, 0.1)
    n2 = ctypes.c_size_t(0)
    assert m.lib().msa_workspace_size(ctypes.byref(small), m.OP_FWD, ctypes.byref(n2)) == 0
    assert n2.value < n.value  # 128K tokens fit in one pass
    P = ctypes.c_void_p
    one = P(16)
    # a workspace below one chunk of 128 positions is refused before any launch
    assert m.lib().msa_fwd(ctypes.byref(s), one, one, one, one, one, one, one, one, one, 4096, P(0)) == 3
