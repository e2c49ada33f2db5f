"""msa_decode_noalloc (the decode step with the library's static device scratch)
against msa_decode (caller workspace), through the C ABI: identical outputs, bit
for bit, on two calls in a row with the second on a smaller input, and the
scratch limit rejected on the host."""
import sys

import pytest
import torch

from synth.msa_inputs import make_decode_inputs, small_decode_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def msa():
    from block_sparse_attention_head_amd import msa as m

    m.lib()
    return m


def test_decode_noalloc_matches_decode_on_two_calls(msa):
    cases = [
        # larger first: 5 sequences in a 16K cache (lengths at the edges), 16 query heads on 4 KV heads
        (small_decode_workload(16384, 16, 4, 8, seed=61, batch=5), [16384, 9000, 129, 1, 0]),
        # then a smaller one: the scratch still holds the first call's scores
        (small_decode_workload(2048, 8, 2, 4, seed=62, batch=3), [2048, 300, 128]),
    ]
    for w, lens in cases:
        x = make_decode_inputs(w, lengths=torch.tensor(lens, dtype=torch.int32))
        xg = {k: v.to(DEV) for k, v in x.items()}
        shape = msa.make_shape(w.batch, w.capacity, w.h_q, w.h_kv, w.top_k, w.softmax_scale)
        # the reference's workspace is filled with NaN: a read of anything it did not write would show
        ws = torch.full((msa.workspace_size(shape, msa.OP_DECODE) // 4,), float("nan"), dtype=torch.float32,
                        device=DEV).view(torch.uint8)
        _say(w.name, "msa_decode")
        ref = msa.decode(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], w.top_k,
                         w.softmax_scale, workspace=ws)
        _say(w.name, "msa_decode_noalloc")
        got = msa.decode_noalloc(xg["q_idx"], xg["k_idx"], xg["q"], xg["k"], xg["v"], xg["seqlens"], w.top_k,
                                 w.softmax_scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("block_idx", "o", "lse"), ref, got):
            assert torch.equal(a, b), f"{w.name}: {name} differs from msa_decode"
        nonempty = torch.tensor(lens, device=DEV) > 0
        assert bool(torch.isfinite(got[2][nonempty]).all())


def test_decode_noalloc_rejects_steps_past_its_scratch(msa):
    # 128 sequences x 8 index heads x 16384 blocks x 4 B = 64 MiB of pooled scores > 32 MiB:
    # the C ABI rejects the shape on the host, before any launch (the small buffers
    # passed here are never read)
    import ctypes

    shape = msa.make_shape(128, 1 << 21, 8, 8, 16, 128 ** -0.5)
    buf = torch.zeros(1024, dtype=torch.float32, device=DEV)
    p = ctypes.c_void_p(buf.data_ptr())
    st = msa.lib().msa_decode_noalloc(ctypes.byref(shape), p, p, p, p, p, p, p, p, p,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 3  # MSA_ERR_WORKSPACE
