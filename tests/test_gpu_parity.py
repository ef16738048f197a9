"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case is compared element by element in full, the full-size workloads too (in
the launch configuration the bench times): the oracle computes their sequences one
by one.
"""

import numpy as np
import pytest
import torch

from mla_decode_attention_flashmla_amd import binding as B
from mla_decode_attention_flashmla_amd import inputs as I
from oracle import mla_oracle as O

from gpu_util import announce, check, check_every_sequence, run, to_device

pytestmark = pytest.mark.gpu


def oracle(d, batches=None):
    w = d["workload"]
    return O.mla_decode(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], d["scale"],
                        d["causal"], dtype=w.dtype, batches=batches)


# ---------------------------------------------------------------- small, full comparison

SMALL = [
    # heads, s_q, causal, seqlens
    (128, 1, False, [1, 63, 64, 65, 777]),
    (128, 2, True, [2, 63, 64, 65, 700]),
    (16, 1, False, [5, 130, 64]),
    (32, 2, False, [129, 1, 300]),
    (64, 2, True, [66, 3, 1000]),
    (48, 3, True, [200, 3, 90]),          # 144 rows: two row groups, ragged second one
]


@pytest.mark.parametrize("heads,s_q,causal,lens", SMALL)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_cases(heads, s_q, causal, lens, dtype):
    w = I.Workload("small", len(lens), s_q, heads, max(lens), dtype, 192, causal=causal,
                   ragged=True, seed=100 + heads + s_q)
    d = I.make_workload(w, seqlens=lens)
    announce(f"small {dtype} H={heads} s_q={s_q} causal={causal} lens={lens}")
    ref_o, ref_l = oracle(d)
    for nwg, minb in ((None, 0), (7, 1), (40, 1)):
        out, lse, status, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
        assert status == 0
        check(out, lse, ref_o, ref_l, dtype, what=f"nwg={nwg} min_split={minb}")


def _random_case(i):
    """Seeded shapes for the sweep below: heads, s_q, causal, lengths (0 and s_q included
    now and then), workgroup count and forced splits."""
    rng = np.random.default_rng(900 + i)
    heads = int(rng.choice([16, 32, 48, 64, 96, 128]))
    s_q = int(rng.integers(1, 5))
    causal = bool(rng.integers(0, 2)) if s_q > 1 else bool(rng.integers(0, 2))
    B = int(rng.integers(1, 4))
    lo = s_q if causal else 0
    lens = [int(x) for x in rng.integers(lo, 800, size=B)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = lo          # a sequence at the shortest valid length
    nwg = int(rng.choice([1, 3, 17, 64, 256]))
    minb = int(rng.choice([0, 0, 1, 2]))
    return heads, s_q, causal, lens, nwg, minb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("i", range(8))
def test_random_shapes(i, dtype):
    """A seeded sweep over shapes, lengths and plans, compared with the oracle in full."""
    heads, s_q, causal, lens, nwg, minb = _random_case(i)
    w = I.Workload("rand", len(lens), s_q, heads, max(max(lens), 1), dtype, 192,
                   causal=causal, ragged=True, seed=950 + i)
    d = I.make_workload(w, seqlens=lens)
    announce(f"random {i} {dtype} H={heads} s_q={s_q} causal={causal} lens={lens} "
             f"nwg={nwg} min_split={minb}")
    ref_o, ref_l = oracle(d)
    out, lse, status, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
    assert status == 0
    check(out, lse, ref_o, ref_l, dtype, what=f"random case {i}")


def test_tiny_fp32_dense_config():
    """The 1 x 16-head x 256-token fp32 config with a dense (identity-table) cache."""
    d = I.make_workload(I.WORKLOADS["tiny_fp32_dense"])
    announce("tiny_fp32_dense")
    ref_o, ref_l = oracle(d)
    out, lse, status, _ = run(d)
    assert status == 0
    check(out, lse, ref_o, ref_l, "f32", what="tiny_fp32_dense")


def test_forced_splits_match_unsplit():
    """Every block its own part (min_split_blocks=1, many workgroups) vs the default plan."""
    w = I.Workload("split", 3, 1, 128, 3000, "bf16", 192, ragged=True, seed=31)
    d = I.make_workload(w, seqlens=[3000, 1, 2049])
    announce("forced splits")
    ref_o, ref_l = oracle(d)
    a = run(d, num_workgroups=256, min_split_blocks=1)
    b = run(d, num_workgroups=1, min_split_blocks=0)
    for out, lse, st, _ in (a, b):
        assert st == 0
        check(out, lse, ref_o, ref_l, "bf16", what="split plan")


def test_stages_equal_fused_call():
    w = I.Workload("st", 4, 1, 128, 2000, "bf16", 192, ragged=True, seed=32)
    d = I.make_workload(w)
    t = to_device(d)
    announce("stage calls vs fused")
    out_a, lse_a, _, plan = run(d, t, num_workgroups=64, min_split_blocks=1)
    out = torch.empty((4, 1, 128, 512), device="cuda")
    lse = torch.empty((4, 1, 128), device="cuda")
    B.decode_main(t["q"], t["kv"], t["table"], t["lens"], float(d["scale"]), out, lse, plan)
    B.decode_combine(t["q"], t["kv"], t["table"], t["lens"], float(d["scale"]), out, lse, plan)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out_a) and np.array_equal(lse.cpu().numpy(), lse_a)


def test_deterministic():
    w = I.Workload("det", 6, 1, 128, 5000, "bf16", 192, ragged=True, seed=33)
    d = I.make_workload(w)
    announce("determinism")
    a = run(d, min_split_blocks=1)
    b = run(d, min_split_blocks=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- definitional pins on device

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_key_returns_that_row(dtype):
    # bf16: the key's weight is exp2 of the scaled score minus the rounded running max,
    # i.e. 1 up to the max's rounding, which is exactly 1 once rounded to bf16 for the
    # products; the row sum adds those rounded weights, so l = 1 and O is the V row
    # exactly (P1 of the definition, bit for bit).  fp32: the weight is exp(0) = 1 and
    # the other keys of the tile are masked to weight 0, so again l = 1 and O = V row.
    w = I.Workload("one", 3, 1, 128, 1, dtype, 192, seed=34)
    d = I.make_workload(w)
    announce(f"single key {dtype}")
    out, lse, st, _ = run(d)
    assert st == 0
    kv = I.bf16_bits_to_float32(d["kv_cache"]) if dtype == "bf16" else d["kv_cache"]
    for b in range(3):
        row = kv[d["block_table"][b, 0], 0, :512]
        assert np.array_equal(out[b, 0], np.broadcast_to(row, (128, 512)))
    ref_o, ref_l = oracle(d)
    assert np.abs(lse - ref_l).max() < 1e-5


def test_uniform_scores_mean_and_log_n():
    w = I.Workload("uni", 2, 1, 128, 1000, "bf16", 192, seed=35)
    d = I.make_workload(w, seqlens=[1000, 77])
    d["q"][:] = 0
    announce("uniform scores")
    out, lse, st, _ = run(d, min_split_blocks=1, num_workgroups=9)
    assert st == 0
    np.testing.assert_allclose(lse[0], np.log(1000.0), atol=2e-6)
    np.testing.assert_allclose(lse[1], np.log(77.0), atol=2e-6)
    ref_o, _ = oracle(d)
    # every weight is exactly 1, so only the split parts' fp16 storage rounds: at most half
    # an fp16 ulp of the part's largest |O| (scaled into [2^14, 2^15)), i.e. 2^-11 of it
    assert np.abs(out - ref_o).max() < 2.0 ** -11 * np.abs(ref_o).max() + 1e-6
    # one workgroup, no split: l is the exact count and only the fp32 accumulation of the
    # products rounds (1000 terms)
    out1, lse1, st1, _ = run(d, num_workgroups=1)
    assert st1 == 0
    np.testing.assert_allclose(lse1[0], np.log(1000.0), atol=2e-6)
    assert np.abs(out1 - ref_o).max() < 1e-5 * np.abs(ref_o).max()


@pytest.mark.parametrize("trend", ["rising", "falling", "alternating"])
def test_score_trends_that_force_rescales(trend):
    """Every head gets the same query q, and key j gets c_j * q / |q|^2 added, so its
    scaled score moves by scale * c_j for all heads.  Rising by 0.1 per token, each 64-key
    page's maximum exceeds the previous page's by 6.4 (9.2 in log2 units, past the
    kernel's slack of 8), so O is rescaled on every page; falling, the first page
    dominates and later weights underflow; alternating +-20 per page, the running maximum
    jumps back and forth.  Forced splits make the combine merge parts whose LSEs differ
    by tens."""
    L = 1000
    w = I.Workload("trend", 2, 1, 128, L, "bf16", 192, seed=47)
    d = I.make_workload(w, seqlens=[L, L - 37])
    q = I.bf16_bits_to_float32(d["q"])
    q[:, :, :, :] = q[:, :, :1, :]                       # one query for all heads
    kv = I.bf16_bits_to_float32(d["kv_cache"])
    scale = float(d["scale"])
    j = np.arange(L)
    shift = {"rising": 0.1 * j, "falling": -0.1 * j,
             "alternating": np.where((j // 64) % 2 == 0, 20.0, -20.0)}[trend] / scale
    for b in range(2):
        qb = q[b, 0, 0].astype(np.float64)
        u = qb / (qb @ qb)                                # q . (c u) = c
        for jj in range(int(d["seqlens"][b])):
            blk, row = d["block_table"][b, jj // 64], jj % 64
            kv[blk, row] = (kv[blk, row] + shift[jj] * u).astype(np.float32)
    d["q"] = I.float32_to_bf16_bits(q)
    d["kv_cache"] = I.float32_to_bf16_bits(kv)
    announce(f"score trend {trend}")
    ref_o, ref_l = oracle(d)
    for nwg, minb in ((None, 0), (16, 1)):
        out, lse, st, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
        assert st == 0
        check(out, lse, ref_o, ref_l, "bf16", what=f"{trend} nwg={nwg}")


def test_causal_reduction_on_device():
    """Token 1 of a causal pair equals a 1-query decode at L; token 0 equals one at L-1."""
    w = I.Workload("cr", 3, 2, 128, 500, "bf16", 192, causal=True, seed=36)
    d = I.make_workload(w, seqlens=[500, 65, 2])
    announce("causal reduction")
    out, lse, st, _ = run(d)
    assert st == 0
    d1 = dict(d, q=np.ascontiguousarray(d["q"][:, 1:2]), causal=False,
              workload=I.Workload("cr1", 3, 1, 128, 500, "bf16", 192, seed=36))
    o1, l1, _, _ = run(d1)
    d0 = dict(d1, q=np.ascontiguousarray(d["q"][:, 0:1]), seqlens=d["seqlens"] - 1)
    o0, l0, _, _ = run(d0)
    assert np.abs(out[:, 1] - o1[:, 0]).max() <= 1e-2 * np.abs(o1).max()
    assert np.abs(out[:, 0] - o0[:, 0]).max() <= 1e-2 * np.abs(o0).max()
    assert np.abs(lse[:, 1] - l1[:, 0]).max() < 2e-3 and np.abs(lse[:, 0] - l0[:, 0]).max() < 2e-3


# ---------------------------------------------------------------- edge cases and failures

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nan_tail_and_guard_blocks_do_not_leak(dtype):
    w = I.Workload("poison", 4, 2, 128, 300, dtype, 192, causal=True, ragged=True, seed=37)
    lens = [300, 65, 2, 129]
    clean = I.make_workload(w, seqlens=lens, guard_blocks=3)
    dirty = I.make_workload(w, seqlens=lens, guard_blocks=3, poison=True)
    announce(f"NaN poison {dtype}")
    a = run(clean, min_split_blocks=1, num_workgroups=16)
    b = run(dirty, min_split_blocks=1, num_workgroups=16)
    assert np.isfinite(b[0]).all() and np.isfinite(b[1]).all()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_length_sequences(dtype):
    w = I.Workload("zero", 4, 1, 128, 200, dtype, 192, ragged=True, seed=38)
    d = I.make_workload(w, seqlens=[0, 200, 0, 64])
    announce(f"zero-length sequences {dtype}")
    ref_o, ref_l = oracle(d)
    for nwg, minb in ((None, 0), (5, 1)):
        out, lse, st, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
        assert st == 0
        assert np.all(out[[0, 2]] == 0) and np.all(np.isneginf(lse[[0, 2]]))
        check(out, lse, ref_o, ref_l, dtype, batches=[1, 3], what="zero-length batch")


def test_all_empty_batch():
    w = I.Workload("empty", 2, 1, 16, 1, "bf16", 192, seed=39)
    d = I.make_workload(w, seqlens=[0, 0])
    announce("all-empty batch")
    out, lse, st, _ = run(d)
    assert st == 0 and np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_invalid_lengths_flag_status_and_nan(dtype):
    w = I.Workload("bad", 3, 2, 128, 128, dtype, 192, causal=True, seed=40)
    d = I.make_workload(w, seqlens=[128, 64, 64])
    d["seqlens"] = np.array([128, -5, 1], np.int32)     # -5 invalid; 1 < s_q invalid (causal)
    announce(f"invalid lengths {dtype}")
    out, lse, st, _ = run(d)
    assert st & B.MLA_STATUS_BAD_SEQLEN
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    assert np.isnan(out[2]).all() and np.isnan(lse[2]).all()
    ref_o, ref_l = O.mla_decode(d["q"][:1], d["kv_cache"], d["block_table"][:1],
                                d["seqlens"][:1], d["scale"], True, dtype=dtype)
    check(out[:1], lse[:1], ref_o, ref_l, dtype, what="valid sequence next to invalid ones")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bad_block_number_flags_status_and_nan(dtype):
    w = I.Workload("blk", 3, 1, 128, 200, dtype, 192, seed=41)
    d = I.make_workload(w)
    d["block_table"] = d["block_table"].copy()
    d["block_table"][1, 2] = d["kv_cache"].shape[0] + 5
    announce(f"bad block number {dtype}")
    out, lse, st, _ = run(d, min_split_blocks=1, num_workgroups=8)
    assert st & B.MLA_STATUS_BAD_BLOCK
    # split over several parts: the merged row is NaN in O and in LSE
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref_o, ref_l = oracle(d, batches=[0, 2])
    check(out, lse, ref_o, ref_l, dtype, batches=[0, 2], what="good sequences")


def test_stale_plan_is_flagged():
    w = I.Workload("stale", 2, 1, 128, 300, "bf16", 192, seed=42)
    d = I.make_workload(w)
    t = to_device(d)
    announce("stale plan")
    _, _, st, plan = run(d, t)
    assert st == 0
    t["lens"] = torch.tensor([300, 200], dtype=torch.int32, device="cuda")
    out = torch.empty((2, 1, 128, 512), device="cuda")
    lse = torch.empty((2, 1, 128), device="cuda")
    B.decode_fwd(t["q"], t["kv"], t["table"], t["lens"], float(d["scale"]), out, lse, plan)
    assert B.read_status(plan) & B.MLA_STATUS_PLAN_MISMATCH
    assert np.isnan(out[1].cpu().numpy()).all() and np.isnan(lse[1].cpu().numpy()).all()


def check_plan(m, nwg, nb, minb):
    """Invariants of a split plan (metadata words m) for block counts nb per segment:
    every block of every segment is covered by exactly one workgroup range, the item
    count and sizes follow the documented rule, part counts and partial slots agree."""
    nseg = int(m[7])
    wg = m[32:32 + 8 * nwg].reshape(nwg, 8)
    seg = m[32 + 8 * nwg:32 + 8 * nwg + 8 * nseg].reshape(nseg, 8)
    assert nseg == len(nb) and m[6] == 0
    T, n, c_al = int(m[9]), int(m[10]), int(m[13])
    assert np.array_equal(seg[:, 0], nb) and T == int(nb.sum())
    c_min = -(-T // nwg)
    if minb == 0 and c_al > 0:
        # segment-aligned: the smallest item size >= c_min whose items fit one per
        # workgroup, at most 4 blocks above c_min
        assert c_min <= c_al <= c_min + 4
        assert n == int((-(-nb // c_al)).sum()) <= nwg
        assert c_al == c_min or int((-(-nb // (c_al - 1))).sum()) > nwg
    elif minb == 0:
        # stream cut: the fewest items whose largest is as short as with one per slot
        assert n == -(-T // c_min), (T, nwg, n)
    else:
        assert n == min(max(T // minb, 1), nwg, T)
    cover = [np.zeros(k, int) for k in seg[:, 0]]
    parts = np.zeros(nseg, int)
    longest = 0
    for r in wg:
        if r[0] < 0:
            continue
        size = 0
        for s in range(r[0], r[2] + 1):
            b0 = r[1] if s == r[0] else 0
            b1 = r[3] if s == r[2] else seg[s, 0]
            if b1 > b0:
                cover[s][b0:b1] += 1
                parts[s] += 1
                size += b1 - b0
        longest = max(longest, size)
    if minb == 0 and c_al > 0:
        assert longest <= c_al
        assert all(r[0] == r[2] for r in wg if r[0] >= 0)    # no range crosses segments
    else:
        assert longest == -(-T // n)
    assert all((c == 1).all() for c in cover)
    assert np.array_equal(parts, seg[:, 3])
    multi = seg[:, 3] > 1
    slots = np.concatenate([np.arange(a, a + k) for a, k in zip(seg[multi, 4], seg[multi, 3])]) \
        if multi.any() else np.zeros(0)
    assert len(set(slots.tolist())) == len(slots) and (slots < nwg + nseg).all()
    return c_al


# (sequences, query tokens): 74 segments (the scheduler's block-wide path), exactly 64
# and 33 (its one-wave path)
@pytest.mark.parametrize("batch,s_q", [(37, 2), (32, 2), (33, 1)])
def test_scheduler_partition_invariants(batch, s_q):
    """Every block of every segment is covered by exactly one workgroup range; part counts
    and partial slots are consistent."""
    groups = s_q  # 128 heads: one 128-row group per query token
    w = I.Workload("sch", batch, s_q, 128, 5000, "bf16", 192, causal=s_q > 1, ragged=True,
                   seed=43)
    d = I.make_workload(w)
    d["seqlens"][5] = 2
    t = to_device(d)
    nb = np.repeat((d["seqlens"] + 63) // 64, groups)
    for nwg, minb in ((256, 0), (256, 1), (13, 3), (1000, 1), (1000, 0), (7, 0), (60, 0),
                      (100, 0)):
        announce(f"scheduler batch={batch} s_q={s_q} nwg={nwg} min_split={minb}")
        plan = B.alloc_plan(batch, s_q, 128, s_q > 1, t["table"].shape[1], nwg)
        B.get_split_metadata(t["lens"], plan, minb)
        torch.cuda.synchronize()
        check_plan(plan.meta.cpu().numpy(), nwg, nb, minb)


def test_scheduler_beyond_lds_segments():
    """More segments than the scheduler keeps in LDS (its per-segment arrays then live in
    the metadata buffer): 5000 sequences, 200 of them 1024 tokens long and the rest
    empty, so the segment-aligned plan (16-block items) is taken and its item column has
    runs of empty segments.  The plan's invariants hold, and every sequence matches the
    oracle (empty ones: O = 0, LSE = -inf)."""
    batch, heads = 5000, 16
    lens = np.zeros(batch, np.int32)
    rng = np.random.default_rng(44)
    lens[np.sort(rng.choice(batch, 200, replace=False))] = 1024
    lens[-1] = 0
    w = I.Workload("manyseg", batch, 1, heads, 1024, "bf16", 192, ragged=True, seed=44)
    d = I.make_workload(w, seqlens=lens)
    t = to_device(d)
    nwg = 256
    nb = (lens + 63) // 64
    for minb in (0, 1):
        announce(f"scheduler with {batch} segments, min_split={minb}")
        plan = B.alloc_plan(batch, 1, heads, False, t["table"].shape[1], nwg)
        B.get_split_metadata(t["lens"], plan, minb)
        torch.cuda.synchronize()
        c_al = check_plan(plan.meta.cpu().numpy(), nwg, nb, minb)
        if minb == 0:
            assert c_al == 16
        out, lse, st, _ = run(d, t, plan=plan)
        assert st == 0
        check_every_sequence(out, lse, oracle_one(d), batch, "bf16",
                             what=f"{batch} segments, min_split={minb}")


def test_plan_for_another_table_width_or_mask_gives_nan():
    """A plan built for another table width or causal flag is flagged, and every output
    row becomes NaN (split segments and whole ones alike)."""
    import dataclasses

    w = I.Workload("width", 3, 2, 128, 600, "bf16", 192, causal=True, ragged=True, seed=45)
    d = I.make_workload(w, seqlens=[600, 70, 200])
    t = to_device(d)
    announce("plan for another table width / causal flag")
    _, _, st, plan = run(d, t, num_workgroups=16, min_split_blocks=2)
    assert st == 0
    wide = torch.full((3, t["table"].shape[1] + 3), -1, dtype=torch.int32, device="cuda")
    wide[:, :t["table"].shape[1]] = t["table"]
    cases = [("table width", dict(t, table=wide), plan),
             ("causal flag", t, dataclasses.replace(plan, causal=0))]
    for what, tt, pl in cases:
        B.get_split_metadata(t["lens"], plan)          # a fresh plan, clean status
        out = torch.zeros((3, 2, 128, 512), device="cuda")
        lse = torch.zeros((3, 2, 128), device="cuda")
        B.decode_fwd(tt["q"], tt["kv"], tt["table"], tt["lens"], float(d["scale"]), out, lse, pl)
        assert B.read_status(plan) & B.MLA_STATUS_PLAN_MISMATCH, what
        assert torch.isnan(out).all().item() and torch.isnan(lse).all().item(), what


# ---------------------------------------------------------------- full-size workloads

FULL = ["tiny_fp32_dense", "paged_b16_l4096", "ragged_b64_l8192", "gate_b64_l8192",
        "spec_b128_sq2_l16384", "long_b4_l131072"]


def oracle_one(d):
    """The oracle on sequence b alone (its own slices of q, table and lengths)."""
    w = d["workload"]

    def one(b):
        o, l = O.mla_decode(d["q"][b:b + 1], d["kv_cache"], d["block_table"][b:b + 1],
                            d["seqlens"][b:b + 1], d["scale"], d["causal"], dtype=w.dtype)
        return o[0], l[0]
    return one


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """Every sequence of every full-size workload, in the bench's launch configuration
    (the device's workgroup count, the default plan)."""
    w = I.WORKLOADS[name]
    announce(f"full-size {name}: generating")
    d = I.make_workload(w)
    announce(f"full-size {name}: GPU run")
    out, lse, st, _ = run(d)
    assert st == 0
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    announce(f"full-size {name}: oracle, {w.batch} sequences")
    check_every_sequence(out, lse, oracle_one(d), w.batch, w.dtype, what=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_rows_per_sequence(dtype):
    """s_q * H at its limit (1024 rows = 8 row groups per sequence), causal, ragged, with
    lengths of exactly s_q (the first query sees one key) up to several pages."""
    heads, s_q = 128, 8
    lens = [8, 9, 70, 1000]
    w = I.Workload("maxrows", len(lens), s_q, heads, max(lens), dtype, 192, causal=True,
                   ragged=True, seed=123)
    d = I.make_workload(w, seqlens=lens)
    announce(f"max rows {dtype} H={heads} s_q={s_q} lens={lens}")
    ref_o, ref_l = oracle(d)
    for nwg, minb in ((None, 0), (13, 1)):
        out, lse, status, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
        assert status == 0
        check(out, lse, ref_o, ref_l, dtype, what=f"max rows nwg={nwg}")


CHUNKED = [
    # heads, s_q, seqlens: many row groups per sequence, each reading the whole cache;
    # lengths from exactly s_q (the first query token sees one key) to several pages
    (128, 16, [16, 17, 200, 1500]),     # 16 row groups, one query token each
    (32, 64, [64, 65, 700]),            # 16 row groups of 4 query tokens x 32 heads
    (128, 128, [128, 300]),             # the largest: 16384 rows, 128 groups
]


@pytest.mark.parametrize("heads,s_q,lens", CHUNKED)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_queries(heads, s_q, lens, dtype):
    """A chunk of s_q new query tokens per sequence under the causal mask: token t of the
    chunk sees the cache up to its own position."""
    w = I.Workload("chunk", len(lens), s_q, heads, max(lens), dtype, 192, causal=True,
                   ragged=True, seed=7 + s_q)
    d = I.make_workload(w, seqlens=lens)
    announce(f"chunked {dtype} H={heads} s_q={s_q} lens={lens}")
    ref_o, ref_l = oracle(d)
    for nwg, minb in ((None, 0), (29, 1)):
        out, lse, status, _ = run(d, num_workgroups=nwg, min_split_blocks=minb)
        assert status == 0
        check(out, lse, ref_o, ref_l, dtype, what=f"chunked nwg={nwg}")


def test_chunked_full_size_workload():
    """64-token chunks of 4 sequences over 8K caches (the chunked bench workload): every
    query token of every sequence."""
    w = I.WORKLOADS["chunk_b4_sq64_l8192"]
    d = I.make_workload(w)
    announce("full-size chunk_b4_sq64_l8192")
    out, lse, st, _ = run(d)
    assert st == 0 and np.isfinite(out).all() and np.isfinite(lse).all()
    check_every_sequence(out, lse, oracle_one(d), w.batch, "bf16", what="chunk full size")


# ---------------------------------------------------------------- strided rows

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nwg,minb", [(None, 0), (40, 1)])
def test_strided_rows_equal_dense(dtype, nwg, minb):
    """mla_decode_fwd_strided with q sliced from a wider buffer (NaN in the gap) and out a
    view of a wider buffer gives the dense call's O and LSE bit for bit, reads nothing
    from q's gaps and writes nothing into out's."""
    lens = [2, 63, 64, 65, 700]   # causal: every length covers the s_q = 2 query tokens
    w = I.Workload("strided", len(lens), 2, 32, max(lens), dtype, 192, causal=True,
                   ragged=True, seed=46)
    d = I.make_workload(w, seqlens=lens)
    announce(f"strided rows {dtype} nwg={nwg} min_split={minb}")
    t = to_device(d)
    out_d, lse_d, st, plan = run(d, t, num_workgroups=nwg, min_split_blocks=minb)
    assert st == 0
    q_rs = 576 + 64
    o_rs = 512 + 8
    qw = torch.full(t["q"].shape[:3] + (q_rs,), float("nan"), dtype=t["q"].dtype, device="cuda")
    qw[..., 32:32 + 576] = t["q"]
    ow = torch.full(t["q"].shape[:3] + (o_rs,), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full(t["q"].shape[:3], 7.0, dtype=torch.float32, device="cuda")
    B.decode_fwd_strided(qw[..., 32:32 + 576], t["kv"], t["table"], t["lens"], float(d["scale"]),
                         ow[..., 4:4 + 512], lse, plan)
    assert B.read_status(plan) == 0
    torch.cuda.synchronize()
    ow = ow.cpu().numpy()
    assert np.array_equal(ow[..., 4:4 + 512], out_d)
    assert np.array_equal(lse.cpu().numpy(), lse_d)
    assert (ow[..., :4] == 7.0).all() and (ow[..., 4 + 512:] == 7.0).all()
