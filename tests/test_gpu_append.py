"""GPU parity of the latent-cache append (mla_kv_append) against the oracle.

The append is a copy, so the bar is bit-exact: the whole cache after the GPU call must
equal the oracle's, bit for bit, in bf16 and fp32, with rows that cross block
boundaries and several new tokens per sequence.  Rows the call cannot place (a
position before the start or past the table, a block number outside the pool) must be
left alone and reported by status bit.  Appending and then decoding on the GPU must
match the oracle's decode of the oracle's appended cache; at the full size of the
s_q = 2 workload (128 sequences of 16K tokens, a 2.4 GB pool) the written rows are read
back and every other row is checked unchanged on the device.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I
from oracle import mla_oracle as O

from gpu_util import announce, check, run, to_device

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _host_bits(t, dtype):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy()


def _new_rows(rng, B_, s_new, dtype):
    x = (rng.standard_normal((B_, s_new, 576)) * 0.5).astype(np.float32)
    return I.float32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("s_new", [1, 2, 3])
def test_append_bit_exact(dtype, s_new):
    lens = [1 + s_new, 64, 65, 128 + s_new, 700]   # new rows straddle block boundaries
    w = I.Workload("append", len(lens), 1, 16, max(lens), dtype, 192, ragged=True,
                   seed=40 + s_new)
    d = I.make_workload(w, seqlens=lens, guard_blocks=2)
    rng = np.random.default_rng(90 + s_new)
    new = _new_rows(rng, len(lens), s_new, dtype)
    announce(f"append {dtype} s_new={s_new} lens={lens}")
    ref, skipped = O.kv_append(d["kv_cache"], d["block_table"], d["seqlens"], new)
    assert skipped == []
    kv = _dev(d["kv_cache"], dtype)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.kv_append(_dev(new, dtype), kv, _dev(d["block_table"], "i32"), _dev(d["seqlens"], "i32"),
                status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = _host_bits(kv, dtype)
    assert np.array_equal(got.view(np.uint8), np.asarray(ref).view(np.uint8))


def test_append_skips_and_reports_unplaceable_rows():
    dtype = "bf16"
    # seq 0: length 1 < s_new (its row 0 would be position -1); seq 1: its last block
    # entry is -1; seq 2: one row past the table, one in a block outside the pool
    kv0 = I.float32_to_bf16_bits((np.random.default_rng(3).standard_normal((4, 64, 576))).astype(np.float32))
    table = np.array([[0, 1], [2, -1], [3, 7]], np.int32)
    lens = np.array([1, 66, 129], np.int32)
    new = _new_rows(np.random.default_rng(4), 3, 2, dtype)
    ref, skipped = O.kv_append(kv0, table, lens, new)
    assert len(skipped) == 5
    kv = _dev(kv0, dtype)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.kv_append(_dev(new, dtype), kv, _dev(table, "i32"), _dev(lens, "i32"), status)
    torch.cuda.synchronize()
    st = int(status.item())
    announce(f"append skip status {st}")
    assert st == (B.MLA_STATUS_BAD_SEQLEN | B.MLA_STATUS_BAD_BLOCK)
    assert np.array_equal(_host_bits(kv, dtype), ref)


def test_append_then_decode_matches_oracle():
    """The decode step as a caller runs it: append the s_q = 2 new rows, then causal decode."""
    old = [0, 63, 64, 300]
    s_q, H = 2, 128
    lens = [L + s_q for L in old]
    w = I.Workload("append_decode", len(lens), s_q, H, max(lens), "bf16", 192, causal=True,
                   ragged=True, seed=77)
    d = I.make_workload(w, seqlens=lens)
    new = _new_rows(np.random.default_rng(78), len(lens), s_q, "bf16")
    kv_ref, skipped = O.kv_append(d["kv_cache"], d["block_table"], d["seqlens"], new)
    assert skipped == []
    ref_o, ref_l = O.mla_decode(d["q"], kv_ref, d["block_table"], d["seqlens"], d["scale"], True)
    t = to_device(d)
    B.kv_append(_dev(new, "bf16"), t["kv"], t["table"], t["lens"])
    out, lse, status, _ = run(d, t=t)
    assert status == 0
    check(out, lse, ref_o, ref_l, "bf16", what="append + causal decode")


def test_append_full_size_spec_workload():
    """128 sequences x 16K tokens, 2 new rows each, into the 2.4 GB pool of the s_q = 2
    workload: the written rows read back exactly; every other row is unchanged."""
    w = I.WORKLOADS["spec_b128_sq2_l16384"]
    d = I.make_workload(w)
    announce("append full size spec_b128_sq2_l16384")
    new = _new_rows(np.random.default_rng(5), w.batch, w.s_q, "bf16")
    kv = _dev(d["kv_cache"], "bf16")
    before = kv.clone()
    table = _dev(d["block_table"], "i32")
    lens = _dev(d["seqlens"], "i32")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.kv_append(_dev(new, "bf16"), kv, table, lens, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # positions L - 2 + t through the table, computed on the host from the drawn inputs
    seq = np.repeat(np.arange(w.batch), w.s_q)
    pos = np.repeat(d["seqlens"].astype(np.int64), w.s_q) - w.s_q + np.tile(np.arange(w.s_q), w.batch)
    blk = d["block_table"][seq, pos // 64].astype(np.int64)
    flat = torch.from_numpy(blk * 64 + pos % 64).cuda()
    kv_rows, before_rows = kv.view(-1, 576), before.view(-1, 576)
    got = kv_rows[flat].view(torch.int16).cpu().numpy()
    assert np.array_equal(got, new.reshape(-1, 576).view(np.int16))
    keep = torch.ones(kv_rows.shape[0], dtype=torch.bool, device="cuda")
    keep[flat] = False
    assert torch.equal(kv_rows[keep].view(torch.int16), before_rows[keep].view(torch.int16))
