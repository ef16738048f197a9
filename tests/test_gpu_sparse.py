"""GPU parity of sparse MLA decode (keys at listed token positions) against the oracle.

Small cases are compared element by element in full, covering padding entries, lists
longer than the sequence, positions at or past the length, duplicates, empty
selections and forced splits; the 128K / top-2048 workload is compared on every
sequence.  Device-side errors (a block number outside the pool, an invalid length)
must set the status bit and turn only the affected sequence into NaN.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I
from oracle import mla_oracle as O

from gpu_util import announce, check

pytestmark = pytest.mark.gpu


def to_device(d):
    return {
        "q": torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).cuda(),
        "kv": torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16).cuda(),
        "table": torch.from_numpy(d["block_table"]).cuda(),
        "lens": torch.from_numpy(d["seqlens"]).cuda(),
        "idx": torch.from_numpy(np.ascontiguousarray(d["indices"])).cuda(),
    }


def run_sparse(d, num_workgroups=None):
    t = to_device(d)
    Bn, _, H, _ = t["q"].shape
    topk = t["idx"].shape[1]
    plan = B.alloc_sparse_plan(Bn, H, topk, num_workgroups)
    out = torch.full((Bn, 1, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, 1, H), 7.0, dtype=torch.float32, device="cuda")
    B.decode_sparse_fwd(t["q"], t["kv"], t["table"], t["lens"], t["idx"], float(d["scale"]),
                        out, lse, plan)
    status = B.read_status(plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), status


def oracle(d, batches=None):
    return O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"],
                               d["indices"], d["scale"], batches=batches)


SMALL = [
    # heads, context, topk, seqlens override, pad, workgroups
    (128, 5000, 256, None, 20, None),
    (128, 1000, 128, [1000, 64, 1, 0, 300], 10, None),     # lists longer than sequences
    (16, 3000, 192, None, 0, 7),                           # few workgroups: long ranges
    (64, 900, 128, [900, 200, 129], 30, 40),               # many workgroups: split parts
]


@pytest.mark.parametrize("heads,context,topk,lens,pad,nwg", SMALL)
def test_sparse_small_cases(heads, context, topk, lens, pad, nwg):
    w = I.SparseWorkload("small", 3 if lens is None else len(lens), heads, context, topk,
                         seed=heads + topk)
    d = I.make_sparse_workload(w, seqlens=lens, pad=pad)
    announce(f"sparse heads={heads} topk={topk} lens={d['seqlens'].tolist()} nwg={nwg}")
    out, lse, st = run_sparse(d, nwg)
    assert st == 0
    ref_o, ref_l = oracle(d)
    check(out, lse, ref_o, ref_l, "bf16", what=f"sparse h{heads} k{topk}")


def test_sparse_lists_longer_than_eight_rounds():
    """topk = 4160: 17 rounds of 256 list entries, which the index kernel places eight
    rounds at a time.  Sequence 0's valid entries are spread over all rounds; sequence
    1's last list entry is valid (the padding row comes from the final round); sequence
    2's valid entries all sit in the first 2048 entries, so the later rounds select
    nothing and the padding row must come from the first eight."""
    w = I.SparseWorkload("long_list", 3, 32, 6000, 4160, seed=44)
    d = I.make_sparse_workload(w, seqlens=[6000, 3000, 100], pad=50)
    idx = d["indices"]
    ok1 = np.flatnonzero((idx[1] >= 0) & (idx[1] < 3000))
    idx[1, [ok1[0], -1]] = idx[1, [-1, ok1[0]]]
    v = idx[2][(idx[2] >= 0) & (idx[2] < 100)]
    idx[2, :] = -1
    idx[2, :len(v)] = v
    assert 0 < len(v) <= 2048 and 0 <= idx[1, -1] < 3000
    announce("sparse lists of 17 rounds")
    ref_o, ref_l = oracle(d)
    for nwg in (None, 11):
        out, lse, st = run_sparse(d, nwg)
        assert st == 0
        check(out, lse, ref_o, ref_l, "bf16", what=f"sparse k4160 nwg={nwg}")


def test_sparse_duplicates_and_empty_selection():
    w = I.SparseWorkload("dup", 3, 128, 700, 128, seed=41)
    d = I.make_sparse_workload(w)
    idx = d["indices"]
    idx[0, 64:] = idx[0, :64]              # every selected key twice
    idx[1, :] = -1                         # nothing selected
    idx[2, :] = 699                        # one key, 128 times
    announce("sparse duplicates / empty")
    out, lse, st = run_sparse(d)
    assert st == 0
    ref_o, ref_l = oracle(d)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    check(out, lse, ref_o, ref_l, "bf16", what="sparse duplicates")


def test_sparse_full_list_matches_dense_path():
    """Every position listed once: the sparse call gives the dense call's result."""
    w = I.SparseWorkload("all", 2, 128, 512, 512, seed=42)
    d = I.make_sparse_workload(w)
    announce("sparse full list vs dense")
    out, lse, st = run_sparse(d)
    assert st == 0
    dd = dict(d, causal=False, workload=I.Workload("all", 2, 1, 128, 512, "bf16", 192))
    from gpu_util import run
    out_d, lse_d, st_d, _ = run(dd)
    assert st_d == 0
    check(out, lse, out_d.astype(np.float64), lse_d.astype(np.float64), "bf16",
          what="sparse vs dense path")


def test_sparse_bad_block_and_bad_length_flag_only_their_sequence():
    w = I.SparseWorkload("bad", 3, 128, 640, 128, seed=43)
    d = I.make_sparse_workload(w)
    sel = int(d["indices"][1][d["indices"][1] >= 0][0])
    d["block_table"][1, sel // 64] = 10 ** 6           # a selected block outside the pool
    announce("sparse bad block")
    out, lse, st = run_sparse(d)
    assert st & B.MLA_STATUS_BAD_BLOCK
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref_o, ref_l = oracle(d, batches=[0, 2])
    check(out, lse, ref_o, ref_l, "bf16", batches=[0, 2], what="sparse, others of bad block")

    d = I.make_sparse_workload(w)
    ref_o, ref_l = oracle(d, batches=[0, 1])
    d["seqlens"][2] = 64 * d["block_table"].shape[1] + 1   # longer than its block table
    announce("sparse bad length")
    out, lse, st = run_sparse(d)
    assert st & B.MLA_STATUS_BAD_SEQLEN
    assert np.isnan(out[2]).all() and np.isnan(lse[2]).all()
    check(out, lse, ref_o, ref_l, "bf16", batches=[0, 1], what="sparse, others of bad length")


def test_sparse_full_size_workload():
    w = I.SPARSE_WORKLOADS["sparse_b64_l131072_topk2048"]
    announce(f"full-size {w.name}: generating")
    d = I.make_sparse_workload(w)
    announce(f"full-size {w.name}: GPU run")
    out, lse, st = run_sparse(d)
    assert st == 0
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref_o, ref_l = oracle(d)
    check(out, lse, ref_o, ref_l, "bf16", what=w.name)


def test_sparse_pool_beyond_32bit_offsets_uses_packed_rows():
    """A pool too large for 32-bit row byte offsets (more than 58,254 blocks of 64 x 576
    bf16) takes the two-pass form (rows copied into packed blocks first).  The drawn
    blocks are placed above that limit in a 4.3 GB device pool whose other blocks are
    zero, the block table shifted to match; the result must equal the oracle's on the
    drawn pool and table."""
    w = I.SparseWorkload("big_pool", 3, 128, 2000, 256, seed=31)
    d = I.make_sparse_workload(w, pad=12)
    ref_o, ref_l = oracle(d)
    t = to_device(d)
    nb = t["kv"].shape[0]
    limit = 0xFFFFFFFF // (64 * 576 * 2)
    base = limit + 1 - nb // 2            # drawn blocks straddle the limit
    big = torch.zeros((base + nb, 64, 576), dtype=torch.bfloat16, device="cuda")
    big[base:] = t["kv"]
    table = torch.where(t["table"] >= 0, t["table"] + base, t["table"])
    announce(f"sparse pool of {base + nb} blocks (limit {limit})")
    Bn, _, H, _ = t["q"].shape
    plan = B.alloc_sparse_plan(Bn, H, t["idx"].shape[1])
    out = torch.full((Bn, 1, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, 1, H), 7.0, dtype=torch.float32, device="cuda")
    B.decode_sparse_fwd(t["q"], big, table, t["lens"], t["idx"], float(d["scale"]), out, lse,
                        plan)
    assert B.read_status(plan) == 0
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "bf16", what="big pool")
    del big
