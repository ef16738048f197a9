"""Pins for the CPU oracle: checks against what the definition and mathematics fix.

None of these compare the oracle with itself.  Each targets a plausible mistake:
a wrong softmax normalisation or log base (closed forms, uniform scores), a
wrong gather or block-table order (brute force on dense keys, hand-derived
paged fixture, re-permuted pools), a wrong causal offset (hand-derived causal
fixture, causal reduction), a transposed operand or index (equivariance,
brute force), masking by multiplication (NaN tails), and a wrong merge rule
(split/combine identity).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as O
from mla_decode_attention_flashmla_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _val(v):
    if isinstance(v, (int, float)):
        return float(v)
    if v.startswith("ln"):
        return math.log(float(v[2:]))
    if "/" in v:
        a, b = v.split("/")
        return float(a) / float(b)
    return float(v)


def _load_case(c):
    B, s_q, H = c["batch"], c["s_q"], c["heads"]
    q = np.zeros((B, s_q, H, 576))
    for b, t, h, d, v in c["q"]:
        q[b, t, h, d] = _val(v)
    kv = np.zeros((c["num_blocks"], 64, 576))
    L = c["seqlens"]
    for e in c["kv"]:
        if e[0] == "rows_of_block":
            _, blk, col, _ = e
            kv[blk, :, col] = np.arange(64)
        elif e[0] == "tail_of_block":
            _, blk, col, v = e
            kv[blk, L[0] % 64:, col] = _val(v)
        else:
            blk, row, col, v = e
            kv[blk, row, col] = _val(v)
    return q, kv, np.array(c["block_table"], np.int32), np.array(L, np.int32)


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    q, kv, table, lens = _load_case(case)
    out, lse = O.mla_decode(q, kv, table, lens, case["scale"], case["causal"], dtype="f64")
    exp_out = np.zeros_like(out)
    for b, t, h, col, v in case["expect_out"]:
        exp_out[b, t, h, col] = _val(v)
    exp_lse = np.zeros_like(lse)
    for b, t, h, v in case["expect_lse"]:
        exp_lse[b, t, h] = _val(v)
    np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-12)


def _rand_case(rng, B, s_q, H, lens, causal=False, extra_blocks=0):
    lens = np.asarray(lens, np.int32)
    nblk = (lens + 63) // 64
    total = int(nblk.sum()) + extra_blocks
    perm = rng.permutation(total)
    table = np.full((B, max(1, int(nblk.max()))), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    kv = rng.standard_normal((total, 64, 576))
    q = rng.standard_normal((B, s_q, H, 576))
    return q, kv, table, lens


def _dense_keys(kv, table, lens):
    """Dense per-sequence rows, built with explicit loops (independent of gather_rows)."""
    out = []
    for b, L in enumerate(lens.tolist()):
        rows = []
        for j in range(L):
            rows.append([float(x) for x in kv[table[b][j // 64], j % 64]])
        out.append(rows)
    return out


def test_single_token_returns_that_row():
    """P1: one visible key -> weight 1: O is that V row exactly, LSE is its score."""
    rng = np.random.default_rng(11)
    q, kv, table, lens = _rand_case(rng, 2, 1, 4, [1, 1])
    out, lse = O.mla_decode(q, kv, table, lens, 0.125, dtype="f64")
    for b in range(2):
        row = kv[table[b, 0], 0]
        assert np.array_equal(out[b, 0], np.broadcast_to(row[:512], (4, 512)))
        for h in range(4):
            s0 = 0.125 * math.fsum(q[b, 0, h, d] * row[d] for d in range(576))
            assert abs(lse[b, 0, h] - s0) < 1e-12


def test_uniform_scores_give_mean_and_log_n():
    """P2: q = 0 -> every score 0 -> LSE = ln n, O = arithmetic mean of the V rows."""
    rng = np.random.default_rng(12)
    q, kv, table, lens = _rand_case(rng, 2, 1, 3, [70, 5])
    q[:] = 0.0
    out, lse = O.mla_decode(q, kv, table, lens, 0.3, dtype="f64")
    for b, L in enumerate(lens.tolist()):
        rows = [kv[table[b, j // 64], j % 64] for j in range(L)]
        mean = np.array([math.fsum(r[c] for r in rows) / L for c in range(512)])
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(mean, (3, 512)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b, 0], math.log(L), rtol=0, atol=1e-14)


def test_identical_keys_distinct_values():
    """P2': scores equal because the query only reads rope columns that are equal across rows,
    while the latent (V) columns differ: O = mean of V, LSE = s + ln n."""
    rng = np.random.default_rng(13)
    q, kv, table, lens = _rand_case(rng, 1, 1, 2, [100])
    q[..., :512] = 0.0
    rope = rng.standard_normal(64)
    kv[:, :, 512:] = rope
    scale = 0.07
    out, lse = O.mla_decode(q, kv, table, lens, scale, dtype="f64")
    rows = [kv[table[0, j // 64], j % 64] for j in range(100)]
    mean = np.array([math.fsum(r[c] for r in rows) / 100 for c in range(512)])
    for h in range(2):
        s = scale * math.fsum(q[0, 0, h, 512 + d] * rope[d] for d in range(64))
        np.testing.assert_allclose(out[0, 0, h], mean, rtol=0, atol=1e-13)
        assert abs(lse[0, 0, h] - (s + math.log(100))) < 1e-12


def test_weights_sum_to_one_and_lse_closed_form():
    """P3 + P4: sum of weights is 1; LSE equals ln(fsum(exp(s))) without max shift."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((5, 576))
    keys = rng.standard_normal((300, 576))
    scale = 576 ** -0.5
    p = O.softmax_weights(q, keys, scale)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-14)
    _, lse = O.attend_one(q, keys, scale)
    for h in range(5):
        s = [scale * math.fsum(q[h, d] * keys[j, d] for d in range(576)) for j in range(300)]
        assert abs(lse[h] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-12


def test_weights_depend_on_the_scale_as_the_definition_says():
    """P3': two keys whose raw dot products with q are 0 and 1, scale ln 3: the scaled
    scores are 0 and ln 3, so the weights are exactly 1/4 and 3/4, LSE = ln 4 and
    O = V_0/4 + 3 V_1/4.  A dropped or doubled scale gives other weights (1/(1+e), or
    1/10), so this pins the scale's use, which Sum(p) = 1 and the argmax cannot."""
    q = np.zeros((1, 576))
    q[0, 3] = 1.0
    keys = np.zeros((2, 576))
    keys[1, 3] = 1.0
    keys[0, 10], keys[1, 10] = 8.0, 4.0         # V_0[10] = 8, V_1[10] = 4
    keys[0, 500], keys[1, 500] = -2.0, 6.0
    scale = math.log(3.0)
    p = O.softmax_weights(q, keys, scale)
    np.testing.assert_allclose(p, [[0.25, 0.75]], rtol=0, atol=1e-15)
    o, lse = O.attend_one(q, keys, scale)
    assert abs(lse[0] - math.log(4.0)) < 1e-15
    np.testing.assert_allclose(o[0, 10], 0.25 * 8.0 + 0.75 * 4.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 500], 0.25 * -2.0 + 0.75 * 6.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 3], 0.75, rtol=0, atol=1e-15)   # V_1[3] = 1 (the key)
    assert np.count_nonzero(o[0]) == 3
    # attend_one's O is built from exactly these weights
    np.testing.assert_array_equal(o, p @ keys[:, :512])


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    """P5: pure-Python loops (fsum, math.exp) over dense keys agree to 1e-12."""
    rng = np.random.default_rng(15 + causal)
    lens = [6, 3] if causal else [6, 1]
    q, kv, table, lens = _rand_case(rng, 2, 2, 3, lens, causal=causal, extra_blocks=1)
    scale = 0.2
    out, lse = O.mla_decode(q, kv, table, lens, scale, causal, dtype="f64")
    qb = [[[list(map(float, q[b, t, h])) for h in range(3)] for t in range(2)] for b in range(2)]
    bo, bl = O.brute_force(qb, _dense_keys(kv, table, lens), scale, causal, 2)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_paging_invariance():
    """P6: moving blocks to other pool slots (and rewriting the table) changes nothing."""
    rng = np.random.default_rng(16)
    q, kv, table, lens = _rand_case(rng, 3, 1, 4, [130, 64, 1], extra_blocks=2)
    out1, lse1 = O.mla_decode(q, kv, table, lens, 0.1, dtype="f64")
    p = rng.permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[p] = kv
    table2 = np.where(table >= 0, p[np.maximum(table, 0)], -1).astype(np.int32)
    out2, lse2 = O.mla_decode(q, kv2, table2, lens, 0.1, dtype="f64")
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_split_combine_identity():
    """P7: attending over disjoint key chunks and merging by LSE equals the unsplit result,
    with empty chunks carrying zero weight."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((4, 576))
    keys = rng.standard_normal((500, 576)) * 2.0
    scale = 0.09
    o_ref, l_ref = O.attend_one(q, keys, scale)
    cuts = [0, 0, 17, 64, 64, 300, 499, 500, 500]
    parts = [O.attend_one(q, keys[a:b], scale) for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = O.merge_partials([x[0] for x in parts], [x[1] for x in parts])
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-13)
    # all parts empty
    o0, l0 = O.merge_partials([np.zeros((4, 512))] * 2, [np.full(4, -np.inf)] * 2)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def test_causal_reduction():
    """P8: with 2 causal queries, token 1 equals the 1-query result at length L and
    token 0 equals the 1-query result at length L-1."""
    rng = np.random.default_rng(18)
    q, kv, table, lens = _rand_case(rng, 2, 2, 3, [129, 2], causal=True)
    out, lse = O.mla_decode(q, kv, table, lens, 0.1, True, dtype="f64")
    o1, l1 = O.mla_decode(q[:, 1:2], kv, table, lens, 0.1, False, dtype="f64")
    o0, l0 = O.mla_decode(q[:, 0:1], kv, table, lens - 1, 0.1, False, dtype="f64")
    np.testing.assert_array_equal(out[:, 1], o1[:, 0])
    np.testing.assert_array_equal(lse[:, 1], l1[:, 0])
    np.testing.assert_array_equal(out[:, 0], o0[:, 0])
    np.testing.assert_array_equal(lse[:, 0], l0[:, 0])


def test_equivariance_heads_and_sequences():
    """P9: permuting heads or sequences permutes the outputs the same way."""
    rng = np.random.default_rng(19)
    q, kv, table, lens = _rand_case(rng, 3, 1, 5, [10, 70, 3])
    out, lse = O.mla_decode(q, kv, table, lens, 0.1, dtype="f64")
    ph = rng.permutation(5)
    o2, l2 = O.mla_decode(q[:, :, ph], kv, table, lens, 0.1, dtype="f64")
    np.testing.assert_allclose(o2, out[:, :, ph], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, :, ph], rtol=0, atol=1e-14)
    pb = np.array([2, 0, 1])
    o3, l3 = O.mla_decode(q[pb], kv, table[pb], lens[pb], 0.1, dtype="f64")
    np.testing.assert_allclose(o3, out[pb], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, lse[pb], rtol=0, atol=1e-14)


def test_nan_tail_and_guard_blocks_do_not_leak():
    """P10: NaN rows past each length and NaN unowned blocks leave the result finite and unchanged."""
    w = I.Workload("t", 3, 1, 4, 200, "bf16", 192, ragged=True, seed=21)
    clean = I.make_workload(w, seqlens=[200, 65, 7], guard_blocks=2)
    dirty = I.make_workload(w, seqlens=[200, 65, 7], guard_blocks=2, poison=True)
    assert np.isnan(O.widen(dirty["kv_cache"], "bf16")).any()
    a = O.mla_decode(clean["q"], clean["kv_cache"], clean["block_table"], clean["seqlens"], w.scale)
    b = O.mla_decode(dirty["q"], dirty["kv_cache"], dirty["block_table"], dirty["seqlens"], w.scale)
    assert np.isfinite(b[0]).all() and np.isfinite(b[1]).all()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sharp_peaks_stay_finite_and_dominate():
    """P11: rows scaled x8 produce large scores; LSE stays finite and a peak row that
    holds the largest score carries the largest weight."""
    w = I.Workload("t", 1, 1, 8, 3000, "bf16", 192, peak_rows=4, seed=22)
    d = I.make_workload(w)
    out, lse = O.mla_decode(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], w.scale)
    assert np.isfinite(lse).all() and np.isfinite(out).all()
    keys = O.widen(O.gather_rows(d["kv_cache"], d["block_table"], 0, 3000), "bf16")
    qr = O.widen(d["q"][0, 0], "bf16")
    p = O.softmax_weights(qr, keys, float(w.scale))
    peak_pos = {pos for _, pos in d["peaks"]}
    s = float(w.scale) * (qr @ keys.T)
    for h in range(8):
        if int(np.argmax(s[h])) in peak_pos:
            assert int(np.argmax(p[h])) in peak_pos
    assert any(int(np.argmax(s[h])) in peak_pos for h in range(8))


def test_empty_sequence_convention():
    """A sequence of length 0 has no visible key: O = 0, LSE = -inf."""
    rng = np.random.default_rng(23)
    q, kv, table, lens = _rand_case(rng, 2, 1, 2, [0, 5])
    out, lse = O.mla_decode(q, kv, table, lens, 0.1, dtype="f64")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.isfinite(lse[1]).all()


def test_invalid_lengths_rejected():
    rng = np.random.default_rng(24)
    q, kv, table, lens = _rand_case(rng, 1, 2, 1, [5])
    with pytest.raises(ValueError):
        O.mla_decode(q, kv, table, np.array([65], np.int32), 0.1, dtype="f64")
    with pytest.raises(ValueError):
        O.mla_decode(q, kv, table, np.array([-1], np.int32), 0.1, dtype="f64")
    with pytest.raises(ValueError):
        O.mla_decode(q, kv, table, np.array([1], np.int32), 0.1, causal=True, dtype="f64")


def test_bf16_widening_is_exact():
    """The oracle reads the exact bf16 values: a few hand-checked bit patterns."""
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0000, 0x7F7F], np.uint16)
    vals = O.widen(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[3] == 0.0
    assert vals[2] == 0.333984375           # 0x3EAB = 1.0101011b * 2^-2
    assert vals[4] == 3.3895313892515355e38  # largest finite bf16


# ---------------------------------------------------------------- sparse variant


def _sparse_case(L=300, topk=128, pad=0, seed=7):
    w = I.SparseWorkload("t", 3, 16, L, topk, seed=seed)
    return I.make_sparse_workload(w, pad=pad)


def test_sparse_full_list_equals_dense():
    """Listing every position of a sequence (in any order, padded) selects its whole
    context: the sparse result is the dense one (the gather goes through the same block
    table, so a wrong position-to-row map fails here)."""
    d = _sparse_case(L=100, topk=128)
    ref_o, ref_l = O.mla_decode(d["q"], d["kv_cache"], d["block_table"], d["seqlens"],
                                d["scale"])
    o, l = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"],
                               d["indices"], d["scale"])
    assert (d["indices"] == -1).sum() == 3 * 28
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=1e-12, atol=1e-12)


def test_sparse_order_and_padding_do_not_matter():
    d = _sparse_case(L=500, topk=128, pad=20)
    idx = d["indices"]
    o1, l1 = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], idx,
                                 d["scale"])
    # the same selections, reordered, with the padding squeezed out and re-added
    rng = np.random.default_rng(3)
    idx2 = np.full((3, 200), -1, dtype=np.int32)
    for b in range(3):
        keep = idx[b][(idx[b] >= 0) & (idx[b] < d["seqlens"][b])]
        idx2[b, :keep.size] = rng.permutation(keep)
    o2, l2 = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], idx2,
                                 d["scale"])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_sparse_duplicate_position_counts_twice():
    """Two copies of one key: the weights are 1/2 each, so O is that key's V row and
    LSE is its score plus ln 2 (the single-key result from the dense definition)."""
    d = _sparse_case(L=300, topk=128)
    j = 77
    idx = np.full((3, 128), -1, dtype=np.int32)
    idx[:, 5] = j
    idx[:, 90] = j
    o, l = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], idx,
                               d["scale"])
    one = np.full_like(idx, -1)
    one[:, 0] = j
    o1, l1 = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], one,
                                 d["scale"])
    row = O.widen(d["kv_cache"][d["block_table"][1, j // 64], j % 64, :512], "bf16")
    np.testing.assert_allclose(o1[1, 0], np.broadcast_to(row, (16, 512)), rtol=1e-15)
    np.testing.assert_allclose(o, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, l1 + math.log(2.0), rtol=1e-12)


def test_sparse_nothing_selected_and_brute_force():
    d = _sparse_case(L=40, topk=64)
    idx = np.full((3, 64), -1, dtype=np.int32)
    idx[1, :3] = [40, 41, 1000]                     # at or past the length: padding too
    o, l = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], idx,
                               d["scale"])
    assert np.all(o == 0) and np.all(l == -np.inf)
    # a few selections against pure-Python loops over the selected rows
    idx[2, :4] = [3, 39, 0, 17]
    o, l = O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], idx,
                               d["scale"], batches=[2])
    kv = O.widen(d["kv_cache"], "bf16")
    rows = [list(kv[d["block_table"][2, p // 64], p % 64]) for p in (3, 39, 0, 17)]
    qs = [[list(O.widen(d["q"][2, 0, h], "bf16")) for h in range(2)]]
    bo, bl = O.brute_force([qs], [rows], float(d["scale"]), False, 1)
    np.testing.assert_allclose(o[2, 0, :2], np.array(bo[0][0]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l[2, 0, :2], np.array(bl[0][0]), rtol=1e-12)


# ---------------------------------------------------------------- latent-cache append


def test_append_worked_placement():
    """A hand-worked case: table [[3, 1]], length 66 after appending 3 rows, so the
    new rows are positions 63, 64, 65 = block 3 row 63, block 1 rows 0 and 1."""
    kv = np.arange(5 * 64 * 576, dtype=np.float64).reshape(5, 64, 576)
    table = np.array([[3, 1]], np.int32)
    new = -1.0 - np.arange(3 * 576, dtype=np.float64).reshape(1, 3, 576)
    out, skipped = O.kv_append(kv, table, np.array([66], np.int32), new)
    assert skipped == []
    assert np.array_equal(out[3, 63], new[0, 0])
    assert np.array_equal(out[1, 0], new[0, 1])
    assert np.array_equal(out[1, 1], new[0, 2])
    written = np.zeros((5, 64), bool)
    written[3, 63] = written[1, 0] = written[1, 1] = True
    assert np.array_equal(out[~written], kv[~written])       # nothing else moved
    assert np.array_equal(kv[3, 63], np.arange(576) + (3 * 64 + 63) * 576.0)  # input kept


@pytest.mark.parametrize("s_new", [1, 2])
def test_append_then_causal_decode_equals_dense_attention(s_new):
    """Appending the step's rows and then running causal decode with s_q = s_new equals
    plain attention over the dense concatenation [old rows; new rows], computed with
    pure-Python loops and no paging: query token t sees the old rows and new rows 0..t."""
    rng = np.random.default_rng(11 + s_new)
    old = [5, 63, 64]
    B, H = len(old), 2
    lens = np.array([L + s_new for L in old], np.int32)
    nblk = (lens + 63) // 64
    perm = rng.permutation(int(nblk.sum())).astype(np.int32)
    table = np.full((B, int(nblk.max())), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    kv = rng.standard_normal((int(nblk.sum()), 64, 576)) * 0.5
    old_rows = [[kv[table[b, j // 64], j % 64].tolist() for j in range(old[b])] for b in range(B)]
    new = rng.standard_normal((B, s_new, 576)) * 0.5
    q = rng.standard_normal((B, s_new, H, 576)) * 0.5
    kv2, skipped = O.kv_append(kv, table, lens, new)
    assert skipped == []
    o, l = O.mla_decode(q, kv2, table, lens, 0.07, causal=True, dtype="f64")
    dense = [old_rows[b] + new[b].tolist() for b in range(B)]
    qs = [[[q[b, t, h].tolist() for h in range(H)] for t in range(s_new)] for b in range(B)]
    bo, bl = O.brute_force(qs, dense, 0.07, True, s_new)
    np.testing.assert_allclose(o, np.array(bo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=1e-12)


def test_append_skips_rows_it_cannot_place():
    kv = np.zeros((4, 64, 576))
    table = np.array([[0, 1], [2, -1], [3, 7]], np.int32)
    new = np.ones((3, 2, 576))
    # seq 0: length 1 < s_new, row 0 would be position -1; seq 1: positions 64, 65 fall in
    # table entry -1; seq 2: position 128 is past the table, 127 is in block 7 (outside)
    out, skipped = O.kv_append(kv, table, np.array([1, 66, 129], np.int32), new)
    assert skipped == [(0, 0, "seqlen"), (1, 0, "block"), (1, 1, "block"), (2, 0, "block"),
                       (2, 1, "seqlen")]
    assert np.array_equal(out[0, 0], np.ones(576))           # seq 0 row 1 -> position 0
    assert out.sum() == 576


# ---------------------------------------------------------------- quantized (fp8) cache


def test_e4m3_values_fixed_by_the_format():
    """OCP e4m3: smallest subnormal 2^-9, largest subnormal 7*2^-9, smallest normal 2^-6,
    1.0 = 0x38, largest finite 448 = 0x7E, NaN = 0x7F / 0xFF, signed zero."""
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x40, 0x7E, 0xFE], np.uint8)
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 2.0, 448.0, -448.0]
    got = O.e4m3_value(codes)
    assert list(got) == want
    assert np.signbit(got[1])
    assert np.isnan(O.e4m3_value(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_quantizer_is_nearest_code():
    """The input generator's quantizer picks the nearest finite code (ties to the even
    code), checked by brute force over all 254 finite codes; every code round-trips."""
    grid_codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    grid = O.e4m3_value(grid_codes)
    nz = grid != 0
    assert np.array_equal(I.float_to_e4m3(grid[nz]), grid_codes[nz])
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 30.0, rng.standard_normal(2000) * 0.01,
                        np.array([500.0, -1e4, 0.0])])
    q = O.e4m3_value(I.float_to_e4m3(x))
    err = np.abs(q - np.clip(x, -448, 448))
    best = np.abs(grid[None, :] - np.clip(x, -448, 448)[:, None]).min(axis=1)
    assert np.array_equal(err, best)


def test_fp8_row_layout_worked_example():
    """One 656-byte row by hand: codes 0x38 (1.0) and 0xC0 (-2.0), scale 0.25, rope bf16
    0x3F80 (1.0) and 0xC000 (-2.0)."""
    row = np.zeros(656, np.uint8)
    row[0], row[511] = 0x38, 0xC0
    rope = np.zeros(64, np.uint16)
    rope[0], rope[63] = 0x3F80, 0xC000
    row[512:640] = rope.view(np.uint8)
    row[640:644] = np.array([0.25], np.float32).view(np.uint8)
    v = O.fp8_rows(row)
    assert v.shape == (576,)
    assert v[0] == 0.25 and v[511] == -0.5 and v[512] == 1.0 and v[575] == -2.0
    assert np.count_nonzero(v) == 4


def test_fp8_decode_equals_bf16_decode_when_quantization_is_exact():
    """Latent rows built on the e4m3 grid times a power of two (with 448 * 2^k in each row,
    so the per-row scale max/448 is exactly 2^k) quantize without loss: decode over the
    fp8 cache must then equal decode over the original bf16 cache."""
    w = I.Workload("fp8pin", 3, 2, 4, 150, "bf16", 192, causal=True, ragged=True, seed=17)
    d = I.make_workload(w, seqlens=[150, 2, 64])
    rng = np.random.default_rng(18)
    kv = d["kv_cache"].reshape(-1, 576).copy()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(kv.shape[0], 512))
    k = rng.integers(-8, -1, size=kv.shape[0])
    lat = O.e4m3_value(codes) * np.exp2(k)[:, None]
    lat[:, 7] = 448.0 * np.exp2(k)
    kv[:, :512] = I.float32_to_bf16_bits(lat.astype(np.float32))
    kv = kv.reshape(d["kv_cache"].shape)
    assert np.array_equal(O.widen(kv.reshape(-1, 576)[:, :512], "bf16"), lat)  # exact in bf16
    fp8 = I.quantize_fp8_cache(kv)
    o8, l8 = O.mla_decode_fp8(d["q"], fp8, d["block_table"], d["seqlens"], d["scale"], True)
    ob, lb = O.mla_decode(d["q"], kv, d["block_table"], d["seqlens"], d["scale"], True)
    np.testing.assert_allclose(o8, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l8, lb, rtol=0, atol=1e-13)


def test_fp8_scales_of_the_format():
    """The format's row scales are the powers of two 2^k, -117 <= k <= 119: then every
    code value (2^-9 .. 448 in magnitude) times the scale is a normal bf16 number."""
    ok = [2.0 ** -117, 2.0 ** -8, 0.25, 1.0, 2.0, 2.0 ** 119]
    bad = [2.0 ** -118, 2.0 ** 120, 0.75, 3.0, -1.0, -0.25, 0.0, -0.0, np.nan, np.inf,
           1.0 + 2.0 ** -23, 2.0 ** -126, 2.0 ** 127]
    assert O.fp8_scale_in_format(np.array(ok, np.float32)).all()
    assert not O.fp8_scale_in_format(np.array(bad, np.float32)).any()
    # the bound is where the format stays exact and normal in bf16: smallest subnormal
    # code 2^-9 times 2^-117 is 2^-126, the smallest normal; 448 * 2^119 < 2^128
    assert 2.0 ** -9 * 2.0 ** -117 == 2.0 ** -126 and 448 * 2.0 ** 119 < 2.0 ** 128
    assert 448 * 2.0 ** 120 > float(np.finfo(np.float32).max)


def test_fp8_row_scale_outside_the_format_is_an_invalid_input():
    """A sequence with a row scale outside the format is rejected (as an invalid length
    is); a bad scale in a row past the sequence's length is never read."""
    w = I.Workload("fp8bad", 2, 1, 4, 100, "bf16", 192, seed=19)
    d = I.make_fp8_workload(w, seqlens=[100, 70])
    kv = d["kv_cache"].copy()
    blk = int(d["block_table"][0, 1])
    kv[blk, 36, 640:644] = np.array([0.75], np.float32).view(np.uint8)  # row 100 - 64 = 36: past L
    o, l = O.mla_decode_fp8(d["q"], kv, d["block_table"], d["seqlens"], d["scale"])
    assert np.isfinite(o).all() and np.isfinite(l).all()
    kv[blk, 35, 640:644] = np.array([0.75], np.float32).view(np.uint8)      # row 99: inside
    with pytest.raises(ValueError):
        O.mla_decode_fp8(d["q"], kv, d["block_table"], d["seqlens"], d["scale"])
    o1, l1 = O.mla_decode_fp8(d["q"], kv, d["block_table"], d["seqlens"], d["scale"],
                              batches=[1])
    assert np.isfinite(o1[1]).all() and np.isnan(o1[0]).all()
