"""GPU parity of MLA decode over a quantized (fp8) latent cache against the oracle.

The cache rows are 656 bytes: 512 fp8 e4m3 latent codes, 64 bf16 rope values and the
row's fp32 scale, a power of two.  The oracle dequantizes exactly (fp64); the GPU path
widens each page to bf16 in LDS, which is exact for such scales, and decodes in bf16,
so the bar is the bf16 tolerance.  Covered: ragged lengths around block boundaries,
causal multi-token queries and 16-token chunks, several row groups, forced splits, a block number outside
the pool and row scales outside the format (status bits, NaN for that sequence only),
every sequence of the full 64 x 8K workload, and bit-for-bit agreement with the bf16 path over a cache that holds the
dequantized rows.
"""

import functools

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I
from oracle import mla_oracle as O

from gpu_util import announce, check, check_every_sequence, run

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


@functools.lru_cache(maxsize=1)
def full_workload():
    """The full 64 x 8K fp8 workload, built once for the tests that use it."""
    return I.make_fp8_workload(I.FP8_WORKLOADS["fp8_b64_l8192"])


def oracle(d, batches=None):
    return O.mla_decode_fp8(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], d["scale"],
                            d["causal"], batches=batches)


SMALL = [
    # heads, s_q, causal, seqlens, workgroups
    (128, 1, False, [1, 63, 64, 65, 777], None),
    (128, 2, True, [2, 130, 1000], 40),          # causal pair, forced splits
    (64, 1, False, [300, 5, 129], 7),            # few workgroups: long ranges
    (48, 3, True, [200, 3, 90], None),           # 144 rows: two row groups
    (128, 16, True, [16, 700, 1500], 24),        # 16-token causal chunks, 16 row groups
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
    """Every sequence of the 64 x 8K fp8 workload against the oracle."""
    w = I.FP8_WORKLOADS["fp8_b64_l8192"]
    d = full_workload()
    announce("fp8 full size")
    out, lse, status = run_fp8(d)
    assert status == 0 and np.isfinite(out).all() and np.isfinite(lse).all()

    def one(b):
        o, l = O.mla_decode_fp8(d["q"][b:b + 1], d["kv_cache"], d["block_table"][b:b + 1],
                                d["seqlens"][b:b + 1], d["scale"], d["causal"])
        return o[0], l[0]
    check_every_sequence(out, lse, one, w.batch, "bf16", what="fp8 full size")


# row scales outside the format: not a power of two, below 2^-117, above 2^119, negative,
# zero, NaN
BAD_SCALES = [0.75, 2.0 ** -118, 2.0 ** 120, -2.0 ** -8, 0.0, float("nan")]


@pytest.mark.parametrize("bad", BAD_SCALES)
@pytest.mark.parametrize("nwg", [None, 9])
def test_fp8_row_scale_outside_the_format(bad, nwg):
    """A row whose scale is not in the format (the oracle rejects such a sequence) sets
    MLA_STATUS_BAD_SCALE and makes that sequence's O and LSE NaN, split or not; the
    other sequences, and a bad scale in a row past a sequence's length, are unaffected."""
    w = I.Workload("fp8scale", 3, 1, 128, 700, "bf16", 192, ragged=True, seed=72)
    d = I.make_fp8_workload(w, seqlens=[700, 300, 130])
    kv = d["kv_cache"]
    # sequence 1, row 200 (page 3); sequence 2, row 140 (past its length 130, page 2)
    kv[d["block_table"][1, 3], 200 - 192, 640:644] = np.array([bad], np.float32).view(np.uint8)
    kv[d["block_table"][2, 2], 140 - 128, 640:644] = np.array([bad], np.float32).view(np.uint8)
    with pytest.raises(ValueError):
        oracle(d, batches=[1])
    announce(f"fp8 bad row scale {bad!r}, nwg={nwg}")
    out, lse, status = run_fp8(d, nwg)
    assert status == B.MLA_STATUS_BAD_SCALE
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref_o, ref_l = oracle(d, batches=[0, 2])
    check(out, lse, ref_o, ref_l, "bf16", batches=[0, 2], what="fp8 sequences without it")


def exact_bf16_cache(kv_fp8, chunk=256):
    """bf16 bit patterns of every dequantized row (the oracle's exact fp64 decoding, in
    chunks of blocks); asserts that bf16 holds each value exactly."""
    bits = np.empty(kv_fp8.shape[:2] + (576,), dtype=np.uint16)
    for i in range(0, kv_fp8.shape[0], chunk):
        x = O.fp8_rows(kv_fp8[i:i + chunk])
        b = I.float32_to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(I.bf16_bits_to_float32(b).astype(np.float64), x)
        bits[i:i + chunk] = b
    return bits


EQUAL = [
    # heads, s_q, causal, seqlens (None: the full workload), workgroups
    (128, 2, True, [2, 130, 1000, 64, 65], 40),
    (128, 1, False, None, None),
]


@pytest.mark.parametrize("heads,s_q,causal,lens,nwg", EQUAL)
def test_fp8_equals_bf16_path_on_widened_cache(heads, s_q, causal, lens, nwg):
    """The widening is exact, so over a bf16 cache holding the dequantized rows the bf16
    path computes on the same values, with the same plan and the same products: O and
    LSE agree bit for bit, for every sequence of the full workload too."""
    if lens is None:
        d = full_workload()
    else:
        w = I.Workload("fp8eq", len(lens), s_q, heads, max(lens), "bf16", 192,
                       causal=causal, ragged=True, seed=90 + s_q)
        d = I.make_fp8_workload(w, seqlens=lens)
    announce(f"fp8 vs bf16 path, H={heads} s_q={s_q} causal={causal} lens={lens} nwg={nwg}")
    d16 = dict(d)
    d16["kv_cache"] = exact_bf16_cache(d["kv_cache"])
    out8, lse8, st8 = run_fp8(d, nwg)
    out16, lse16, st16, _ = run(d16, num_workgroups=nwg)
    assert st8 == 0 and st16 == 0
    assert np.isfinite(out8).all() and np.isfinite(lse8).all()
    assert np.array_equal(out8, out16), float(np.abs(out8 - out16).max())
    assert np.array_equal(lse8, lse16), float(np.abs(lse8 - lse16).max())
