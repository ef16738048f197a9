"""GPU parity of MLA decode over a quantized (fp8) latent cache against the oracle.

The cache rows are 656 bytes: 512 fp8 e4m3 latent codes, 64 bf16 rope values and the
row's fp32 scale.  The oracle dequantizes exactly (fp64); the GPU path writes each
latent value as bf16 (value * scale, rounded to nearest even) and decodes in bf16, so the
bar is the bf16 tolerance.  Covered: ragged lengths around block boundaries, causal
multi-token queries, several row groups, forced splits, a block number outside the pool
(status bit, NaN for that sequence only) and the full 64 x 8K workload on sampled
sequences.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I
from oracle import mla_oracle as O

from gpu_util import announce, check

pytestmark = pytest.mark.gpu


def run_fp8(d, num_workgroups=None):
    q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).cuda()
    kv = torch.from_numpy(d["kv_cache"]).cuda()
    table = torch.from_numpy(d["block_table"]).cuda()
    lens = torch.from_numpy(d["seqlens"]).cuda()
    Bn, s_q, H, _ = q.shape
    plan = B.alloc_fp8_plan(Bn, s_q, H, d["causal"], table.shape[1], num_workgroups)
    out = torch.full((Bn, s_q, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, s_q, H), 7.0, dtype=torch.float32, device="cuda")
    B.decode_fp8_fwd(q, kv, table, lens, float(d["scale"]), out, lse, plan)
    status = B.read_status(plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), status


def oracle(d, batches=None):
    return O.mla_decode_fp8(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], d["scale"],
                            d["causal"], batches=batches)


SMALL = [
    # heads, s_q, causal, seqlens, workgroups
    (128, 1, False, [1, 63, 64, 65, 777], None),
    (128, 2, True, [2, 130, 1000], 40),          # causal pair, forced splits
    (64, 1, False, [300, 5, 129], 7),            # few workgroups: long ranges
    (48, 3, True, [200, 3, 90], None),           # 144 rows: two row groups
]


@pytest.mark.parametrize("heads,s_q,causal,lens,nwg", SMALL)
def test_fp8_small_cases(heads, s_q, causal, lens, nwg):
    w = I.Workload("fp8", len(lens), s_q, heads, max(lens), "bf16", 192, causal=causal,
                   ragged=True, seed=60 + heads + s_q)
    d = I.make_fp8_workload(w, seqlens=lens)
    announce(f"fp8 H={heads} s_q={s_q} causal={causal} lens={lens} nwg={nwg}")
    ref_o, ref_l = oracle(d)
    out, lse, status = run_fp8(d, nwg)
    assert status == 0
    check(out, lse, ref_o, ref_l, "bf16", what="fp8")


def test_fp8_bad_block_flags_only_its_sequence():
    w = I.Workload("fp8bad", 3, 1, 128, 500, "bf16", 192, ragged=True, seed=71)
    d = I.make_fp8_workload(w, seqlens=[500, 200, 300])
    d["block_table"][1, 2] = d["kv_cache"].shape[0] + 3
    announce("fp8 bad block")
    out, lse, status = run_fp8(d)
    assert status & B.MLA_STATUS_BAD_BLOCK
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref_o, ref_l = oracle(d, batches=[0, 2])
    check(out, lse, ref_o, ref_l, "bf16", batches=[0, 2], what="fp8 good sequences")


def test_fp8_full_size_workload():
    w = I.FP8_WORKLOADS["fp8_b64_l8192"]
    d = I.make_fp8_workload(w)
    batches = I.sample_sequences(w.batch, 6, w.seed)
    announce(f"fp8 full size, sampled sequences {batches.tolist()}")
    out, lse, status = run_fp8(d)
    assert status == 0 and np.isfinite(out).all() and np.isfinite(lse).all()
    ref_o, ref_l = oracle(d, batches=batches)
    check(out, lse, ref_o, ref_l, "bf16", batches=batches, what="fp8 full size")
