"""The no-allocation entry point (plan and partials in the library's static scratch)
against the existing pair mla_get_split_metadata + mla_decode_fwd with torch-allocated
plan buffers: the same kernels on the same plan, so the outputs must agree bit for bit
(stricter than the bf16/fp32 tolerances).  Two calls in a row per dtype, the second with
a smaller input, so the second reuses a scratch that still holds the first call's plan
and partials."""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I

from gpu_util import announce, run, to_device

pytestmark = pytest.mark.gpu

# (batch, s_q, heads, causal, lengths): the first call of each pair is the larger one;
# with the device's workgroup count every long sequence is split into several parts
PAIRS = {
    "bf16": [(8, 1, 128, False, [4096, 1, 64, 65, 3000, 8192, 777, 0]),
             (3, 2, 64, True, [300, 2, 129])],
    "f32": [(2, 2, 128, True, [2000, 700]),
            (1, 1, 16, False, [256])],
}


def noalloc(d, t):
    Bn, s_q, H, _ = t["q"].shape
    out = torch.full((Bn, s_q, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, s_q, H), 7.0, dtype=torch.float32, device="cuda")
    B.decode_fwd_noalloc(t["q"], t["kv"], t["table"], t["lens"], float(d["scale"]), out, lse,
                         causal=d["causal"])
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_planned_call_twice(dtype):
    for k, (batch, s_q, heads, causal, lens) in enumerate(PAIRS[dtype]):
        w = I.Workload("noalloc", batch, s_q, heads, max(lens), dtype, 192, causal=causal,
                       ragged=True, seed=90 + k)
        d = I.make_workload(w, seqlens=lens)
        t = to_device(d)
        announce(f"no-alloc call {k + 1} {dtype} B={batch} s_q={s_q} H={heads} lens={lens}")
        o_ref, l_ref, st, _ = run(d, t)
        assert st == 0
        o, l = noalloc(d, t)
        assert np.isfinite(o).all() and not np.isnan(l).any()
        assert np.array_equal(o, o_ref), float(np.abs(o - o_ref).max())
        assert np.array_equal(l, l_ref)


def scratch_need(nseg, nwg, row_bytes=1032):
    """Bytes of plan (rounded up to 256) and bf16 partials the call needs."""
    plan = ((32 + 8 * (nwg + nseg)) * 4 + 255) // 256 * 256
    return plan + (nwg + nseg) * 128 * row_bytes


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """The smallest batch of 128-row segments whose plan and partials exceed the fixed
    scratch (379 with 256 workgroups) is refused with a clear host-side error and
    nothing enqueued; one sequence fewer runs."""
    nwg = B.device_workgroups(0)
    batch = next(n for n in range(1, 100000)
                 if scratch_need(n, nwg) > B.NOALLOC_SCRATCH_BYTES)
    if nwg == 256:
        assert batch == 379
    q = torch.zeros((batch, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((batch, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(batch, dtype=torch.int32, device="cuda")
    out = torch.zeros((batch, 1, 128, 512), device="cuda")
    lse = torch.zeros((batch, 1, 128), device="cuda")
    with pytest.raises(B.MlaError) as e:
        B.decode_fwd_noalloc(q, kv, table, lens, 0.1, out, lse)
    assert e.value.code == B.MLA_ERR_SCRATCH
    assert "scratch" in B.status_string(B.MLA_ERR_SCRATCH)
    # one segment fewer fits
    B.decode_fwd_noalloc(q[:-1], kv, table[:-1], lens[:-1], 0.1, out[:-1], lse[:-1])
    torch.cuda.synchronize()
    o = out[:-1].cpu().numpy()
    # length 1: every query returns the single key's value row (block 0, row 0: zeros)
    assert np.array_equal(o, np.zeros_like(o))
