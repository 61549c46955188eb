"""The decode entry point that allocates nothing, through the C ABI.

paged_decode_attention_noalloc keeps its split-K partials in the library's
own device array instead of a caller workspace. On one device its output
must be bitwise that of paged_decode_attention with the same arguments (the
same kernels and launch), call after call: the array keeps the previous
call's contents, so a second, smaller call runs over the first one's
leftovers. Both are also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import decode_attention_slot_amd as K
import workloads as W
from oracle.runner import OracleStep
from workloads import device as dev

pytestmark = pytest.mark.gpu

TOL = 1e-5  # max-abs-error against the fp64 oracle, fp32 and bf16 KV alike


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def stepped(w, cuda):
    """The workload's caches on the device after its step's write, and the oracle's."""
    s = dev.build(w, cuda)
    dev.run_step(s)
    ref = OracleStep(w, s.host_table)
    ref.write_step()
    return s, ref


def both(s, **kw):
    w = s.w
    args = (s.q, s.k_cache, s.v_cache, s.block_table, s.seq_lens, w.scale)
    a = K.paged_decode_attention(*args, **kw)
    b = K.paged_decode_attention_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_equals_workspace_call_twice(cuda):
    # first call: the 12-request block-config batch (split requests, so the
    # partials and the merge are used); second: a smaller batch
    # (the 2-request fp32 workload) over the first call's leftovers
    big = W.make_workload(1)
    small = W.make_workload(0)
    s1, r1 = stepped(big, cuda)
    s2, r2 = stepped(small, cuda)
    a1, b1 = both(s1)
    assert torch.equal(a1.view(torch.int32), b1.view(torch.int32))
    a2, b2 = both(s2)
    assert torch.equal(a2.view(torch.int32), b2.view(torch.int32))
    for w, ref, out in ((big, r1, b1), (small, r2, b2)):
        want = ref.attention(w.q())
        assert float(np.abs(out.double().cpu().numpy() - want).max()) <= TOL
    # and once more on the larger batch, with the fixed-shape walk
    a3, b3 = both(s1, flags=K.KVS_WALK_TABLE)
    assert torch.equal(a3.view(torch.int32), b3.view(torch.int32))
    assert torch.equal(b3.view(torch.int32), b1.view(torch.int32))


def test_noalloc_rejects_past_its_array(cuda):
    # 8192 requests of 64 query heads: about 290 MB of partial slots on
    # MI355X, past the 64 MiB array; rejected before anything is enqueued
    B, Hq, Hkv, D, bs = 8192, 64, 8, 128, 16
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device=cuda)
    kc = torch.zeros((2, bs, Hkv, D), dtype=torch.bfloat16, device=cuda)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=cuda)
    sl = torch.zeros(B, dtype=torch.int32, device=cuda)
    out = torch.full((B, 1, Hq, D), 7.0, device=cuda)
    with pytest.raises(K.KvslotError) as e:
        K.paged_decode_attention_noalloc(q, kc, kc, bt, sl, 1.0, out=out)
    assert e.value.name == "KVS_ENOSPACE"
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # nothing ran
