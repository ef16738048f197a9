"""Seeded workload generator: determinism, layout and distribution checks (CPU)."""

import numpy as np

from mla_decode_attention_flashmla_amd import inputs as I


def test_deterministic_and_thread_independent(monkeypatch):
    w = I.Workload("t", 3, 2, 8, 300, "bf16", 192, ragged=True, causal=True, seed=7)
    a = I.make_workload(w)
    monkeypatch.setattr(I, "_threads", lambda: 1)
    b = I.make_workload(w)
    for k in ("q", "kv_cache", "block_table", "seqlens"):
        assert np.array_equal(a[k], b[k]), k


def test_block_table_is_a_permutation_of_the_pool():
    w = I.Workload("t", 5, 1, 4, 500, "bf16", 192, ragged=True, seed=8)
    d = I.make_workload(w, guard_blocks=3)
    lens, table = d["seqlens"], d["block_table"]
    nblk = (lens + 63) // 64
    used = np.concatenate([table[b, :nblk[b]] for b in range(5)])
    assert len(set(used.tolist())) == len(used) == int(nblk.sum())
    assert d["kv_cache"].shape[0] == int(nblk.sum()) + 3
    for b in range(5):
        assert np.all(table[b, nblk[b]:] == -1)
    assert lens.min() >= 1 and lens.max() <= 500


def test_dense_config_uses_identity_table():
    d = I.make_workload(I.WORKLOADS["tiny_fp32_dense"])
    assert d["kv_cache"].dtype == np.float32 and d["kv_cache"].shape == (4, 64, 576)
    assert d["block_table"].tolist() == [[0, 1, 2, 3]]
    assert d["q"].shape == (1, 1, 16, 576)
    assert d["scale"] == np.float32(576 ** -0.5)
    # N(0,1): sample moments of 147k draws
    kv = d["kv_cache"].astype(np.float64)
    assert abs(kv.mean()) < 0.02 and abs(kv.std() - 1.0) < 0.02


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    bits = I.float32_to_bf16_bits(x)
    back = I.bf16_bits_to_float32(bits)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); 1+2^-9 rounds down
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]


def test_scaled_normal_draws():
    w = I.WORKLOADS["paged_b16_l4096"]
    x = I._normal_fill(np.random.SeedSequence(1), 1 << 21, 0.5, True)
    v = I.bf16_bits_to_float32(x).astype(np.float64)
    assert abs(v.mean()) < 0.005 and abs(v.std() - 0.5) < 0.005
    assert w.scale == np.float32(192 ** -0.5)


def test_peak_rows_are_scaled_by_eight():
    w = I.Workload("t", 2, 1, 2, 300, "bf16", 192, peak_rows=4, seed=9)
    base = I.Workload("t", 2, 1, 2, 300, "bf16", 192, peak_rows=0, seed=9)
    a, b = I.make_workload(w), I.make_workload(base)
    assert len(a["peaks"]) == 8
    for bb, pos in a["peaks"]:
        blk, row = a["block_table"][bb, pos // 64], pos % 64
        np.testing.assert_array_equal(I.bf16_bits_to_float32(a["kv_cache"][blk, row]),
                                      8 * I.bf16_bits_to_float32(b["kv_cache"][blk, row]))


def test_sample_sequences_include_ends():
    s = I.sample_sequences(64, 6, 5)
    assert s[0] == 0 and s[-1] == 63 and len(s) == 8
