"""A decode step captured in a HIP graph (through torch.cuda.CUDAGraph) replays exactly.

The step is mla_get_split_metadata + mla_decode_fwd on the capturing stream: three
kernels and no memory set or copy.  The graph is replayed several times with eager
work and synchronizations between the replays; every replay must equal the eager
result bit for bit, including after the inputs (Q, and the lengths the scheduler reads)
are changed in place between replays.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I

from gpu_util import announce, to_device

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    lens = [1000, 65, 2, 777, 4096, 130]
    w = I.Workload("graph", len(lens), 1, 128, max(lens), "bf16", 192, ragged=True, seed=21)
    d = I.make_workload(w, seqlens=lens)
    t = to_device(d)
    Bn, s_q, H = w.batch, 1, 128
    plan = B.alloc_plan(Bn, s_q, H, False, t["table"].shape[1], 40)
    out = torch.empty((Bn, s_q, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((Bn, s_q, H), dtype=torch.float32, device="cuda")
    scale = float(d["scale"])

    def step():
        B.get_split_metadata(t["lens"], plan)
        B.decode_fwd(t["q"], t["kv"], t["table"], t["lens"], scale, out, lse, plan)

    def eager():
        step()
        torch.cuda.synchronize()
        assert B.read_status(plan) == 0
        return out.clone(), lse.clone()

    ref0 = eager()
    q0 = t["q"].clone()
    q1 = (t["q"].float() * -0.75).to(torch.bfloat16)
    lens1 = torch.tensor([999, 64, 3, 700, 4000, 1], dtype=torch.int32, device="cuda")
    lens0 = t["lens"].clone()
    t["q"].copy_(q1)
    ref1 = eager()
    t["lens"].copy_(lens1)
    ref2 = eager()
    t["q"].copy_(q0)
    t["lens"].copy_(lens0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i, (qv, lv, ref) in enumerate([(q0, lens0, ref0), (q1, lens0, ref1), (q1, lens1, ref2),
                                       (q0, lens0, ref0), (q0, lens0, ref0)]):
        t["q"].copy_(qv)
        t["lens"].copy_(lv)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert B.read_status(plan) == 0
        announce(f"graph replay {i}")
        assert torch.equal(out, ref[0]), f"replay {i}: O differs from eager"
        assert torch.equal(lse, ref[1]), f"replay {i}: LSE differs from eager"
