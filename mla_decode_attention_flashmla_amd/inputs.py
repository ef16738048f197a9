"""Seeded synthetic workloads for MLA decode.

This module only draws numbers and lays them out (paged pool, block table,
sequence lengths).  It holds none of the attention arithmetic, so both the
HIP path and the CPU oracle can take their inputs from it.

Layout of one workload (all NumPy, host memory):

* ``q``            [B, s_q, H, 576]  bf16 bits as uint16, or float32
* ``kv_cache``     [num_blocks, 64, 576] same dtype as q (the paged latent pool;
                   columns 0..511 are the latent part that is also V, 512..575 rope)
* ``block_table``  [B, max_blocks] int32, -1 where unused
* ``seqlens``      [B] int32
* ``scale``        float32 softmax scale

Random streams come from ``numpy.random.SeedSequence(seed).spawn(5)`` in a fixed
order: sequence lengths, block permutation, Q, KV pool, sharp-peak rows.  Large
arrays are drawn in fixed 1 Mi-element chunks, each with its own child seed,
so the bytes do not depend on the number of worker threads.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

PAGE = 64          # tokens per KV block
D_QK = 576         # latent (512) + rope (64)
D_V = 512          # V is the first 512 columns of a cache row

_CHUNK = 1 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic MLA decode workload."""

    name: str
    batch: int
    s_q: int
    heads: int
    context: int                  # every sequence length, or the upper bound when ragged
    dtype: str                    # "bf16" or "f32"
    scale_denominator: int        # scale = denominator ** -0.5
    causal: bool = False
    ragged: bool = False          # seqlens uniform in [1, context]
    sigma: float = 0.5            # Q, KV ~ N(0, 1) * sigma
    dense: bool = False           # identity block table over a dense cache
    peak_rows: int = 0            # rows per sequence multiplied by peak_factor
    peak_factor: float = 8.0
    seed: int = 0

    @property
    def scale(self) -> np.float32:
        return np.float32(float(self.scale_denominator) ** -0.5)


# The five workloads the method is exercised on, plus the 8K gate shape.
WORKLOADS = {
    "tiny_fp32_dense": Workload("tiny_fp32_dense", 1, 1, 16, 256, "f32", 576,
                                sigma=1.0, dense=True, seed=0),
    "paged_b16_l4096": Workload("paged_b16_l4096", 16, 1, 128, 4096, "bf16", 192, seed=1),
    "ragged_b64_l8192": Workload("ragged_b64_l8192", 64, 1, 128, 8192, "bf16", 192,
                                 ragged=True, seed=2),
    "spec_b128_sq2_l16384": Workload("spec_b128_sq2_l16384", 128, 2, 128, 16384, "bf16", 192,
                                     causal=True, seed=3),
    "long_b4_l131072": Workload("long_b4_l131072", 4, 1, 128, 131072, "bf16", 192,
                                peak_rows=4, seed=4),
    "gate_b64_l8192": Workload("gate_b64_l8192", 64, 1, 128, 8192, "bf16", 192, seed=5),
    # a chunk of 64 new query tokens per sequence over an 8K cache, causal (chunked
    # queries: each token's 128 heads are one row group)
    "chunk_b4_sq64_l8192": Workload("chunk_b4_sq64_l8192", 4, 64, 128, 8192, "bf16", 192,
                                    causal=True, seed=6),
}


# Quantized latent cache: one 656-byte row per token, 512 latent values as fp8 e4m3 codes
# (OCP 8-bit float: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
# all-ones exponent with all-ones mantissa is NaN; largest finite 448), the 64 rope values
# as bf16, then the row's scale (an fp32 power of two, as in the OCP microscaling
# formats) and 12 bytes of padding.  A latent value is code_value * scale, exact in bf16;
# the rope values are exact.
FP8_ROW_BYTES = 656
FP8_ROPE_OFF = 512
FP8_SCALE_OFF = 640


def float_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code (ties to even, saturating at +-448) of finite float values."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)                       # spacing of the codes at this magnitude
    v = np.minimum(np.round(a / step) * step, 448.0)
    sub = v < 2.0 ** -6
    e2 = np.floor(np.log2(np.where(sub, 1.0, v)))
    man = np.where(sub, v / 2.0 ** -9, (v / np.exp2(e2) - 1.0) * 8.0)
    code = np.where(sub, man, (e2 + 7) * 8 + man).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def quantize_fp8_cache(kv_bits: np.ndarray) -> np.ndarray:
    """The 656-byte-row fp8 cache of a bf16 cache [blocks, 64, 576] (uint16 bits): per row,
    scale = the smallest power of two >= max |latent| / 448 (1 for an all-zero row), codes
    of latent / scale, rope as is."""
    x = bf16_bits_to_float32(kv_bits.reshape(-1, 576))
    lat = x[:, :512].astype(np.float64)
    amax = np.abs(lat).max(axis=1)
    scale = np.where(amax > 0, np.exp2(np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0))),
                     1.0).astype(np.float32)
    codes = float_to_e4m3(lat / scale.astype(np.float64)[:, None])
    out = np.zeros((x.shape[0], FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :512] = codes
    out[:, FP8_ROPE_OFF:FP8_SCALE_OFF] = np.ascontiguousarray(
        kv_bits.reshape(-1, 576)[:, 512:]).view(np.uint8)
    out[:, FP8_SCALE_OFF:FP8_SCALE_OFF + 4] = scale.view(np.uint8).reshape(-1, 4)
    return out.reshape(kv_bits.shape[0], 64, FP8_ROW_BYTES)


def make_fp8_workload(w: "Workload", seqlens: Optional[np.ndarray] = None) -> dict:
    """A paged workload (as make_workload) whose cache is stored as fp8 rows: the bf16
    cache drawn for ``w`` quantized by quantize_fp8_cache (kept under "kv_bf16")."""
    d = make_workload(w, seqlens=seqlens)
    d["kv_bf16"] = d["kv_cache"]
    d["kv_cache"] = quantize_fp8_cache(d["kv_cache"])
    return d


def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Finite inputs only (the generators never produce inf/nan before rounding).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32 (for test helpers and fixtures)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_fill(seed_seq: np.random.SeedSequence, n: int, sigma: float, bf16: bool) -> np.ndarray:
    """n draws of N(0,1)*sigma in fixed chunks (thread-count independent)."""
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seed_seq.spawn(nch)
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    sig = np.float32(sigma)

    def fill(i: int) -> None:
        g = np.random.Generator(np.random.PCG64(kids[i]))
        m = min(_CHUNK, n - i * _CHUNK)
        x = g.standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            x *= sig
        out[i * _CHUNK:i * _CHUNK + m] = float32_to_bf16_bits(x) if bf16 else x

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def make_seqlens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.ragged:
        return rng.integers(1, w.context, size=w.batch, endpoint=True).astype(np.int32)
    return np.full(w.batch, w.context, dtype=np.int32)


def make_workload(w: Workload, seqlens: Optional[np.ndarray] = None, guard_blocks: int = 0,
                  poison: bool = False) -> dict:
    """Draw one workload.

    ``seqlens`` overrides the drawn lengths (edge-case tests).  ``guard_blocks``
    appends pool blocks that no sequence owns; with ``poison`` they, and every
    row at or past a sequence's length inside its last block, are set to NaN
    (a correct kernel never lets them reach the output).
    """
    streams = np.random.SeedSequence(w.seed).spawn(5)
    rng_len = np.random.Generator(np.random.PCG64(streams[0]))
    rng_perm = np.random.Generator(np.random.PCG64(streams[1]))
    rng_peak = np.random.Generator(np.random.PCG64(streams[4]))

    lens = make_seqlens(w, rng_len)
    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32).copy()
    B = int(lens.shape[0])
    nblk = (lens.astype(np.int64) + PAGE - 1) // PAGE
    total = int(nblk.sum())
    max_blocks = max(1, int(nblk.max()) if B else 1)
    num_blocks = total + guard_blocks

    if w.dense:
        perm = np.arange(num_blocks, dtype=np.int32)
    else:
        perm = rng_perm.permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        k = int(nblk[b])
        table[b, :k] = perm[off:off + k]
        off += k

    bf16 = w.dtype == "bf16"
    q = _normal_fill(streams[2], B * w.s_q * w.heads * D_QK, w.sigma, bf16)
    q = q.reshape(B, w.s_q, w.heads, D_QK)
    kv = _normal_fill(streams[3], num_blocks * PAGE * D_QK, w.sigma, bf16)
    kv = kv.reshape(max(num_blocks, 0), PAGE, D_QK)

    peaks = []
    if w.peak_rows:
        for b in range(B):
            L = int(lens[b])
            k = min(w.peak_rows, L)
            pos = np.sort(rng_peak.choice(L, size=k, replace=False)) if k else np.zeros(0, np.int64)
            for p in pos:
                blk, row = int(table[b, p // PAGE]), int(p % PAGE)
                if bf16:
                    vals = bf16_bits_to_float32(kv[blk, row]) * np.float32(w.peak_factor)
                    kv[blk, row] = float32_to_bf16_bits(vals)
                else:
                    kv[blk, row] *= np.float32(w.peak_factor)
                peaks.append((b, int(p)))

    if poison:
        nan = np.uint16(0x7FC0) if bf16 else np.float32(np.nan)
        for b in range(B):
            L = int(lens[b])
            k = int(nblk[b])
            if k and L % PAGE:
                kv[table[b, k - 1], L % PAGE:, :] = nan
        if guard_blocks:
            used = np.zeros(num_blocks, bool)
            used[table[table >= 0]] = True
            kv[~used] = nan

    return {
        "workload": w,
        "q": q,
        "kv_cache": kv,
        "block_table": table,
        "seqlens": lens,
        "scale": w.scale,
        "causal": w.causal,
        "peaks": peaks,
    }


@dataclasses.dataclass(frozen=True)
class SparseWorkload:
    """Shape and distribution of one synthetic sparse MLA decode workload (s_q = 1).

    Each sequence of ``context`` tokens lists ``topk`` selected token positions,
    distinct and in random order; a sequence shorter than ``topk`` lists all of its
    positions and pads with -1.  With ``pool_blocks`` the block table draws its
    entries from a pool of that many blocks (with replacement), so a long logical
    context fits a small pool while the rows read stay scattered; without it every
    block of every sequence is its own.
    """

    name: str
    batch: int
    heads: int
    context: int
    topk: int
    pool_blocks: int = 0
    scale_denominator: int = 192
    sigma: float = 0.5
    ragged: bool = False
    seed: int = 0

    @property
    def scale(self) -> np.float32:
        return np.float32(float(self.scale_denominator) ** -0.5)


# Gate-shaped decode over an fp8 latent cache (64 x 8K, 128 heads)
FP8_WORKLOADS = {
    "fp8_b64_l8192": Workload("fp8_b64_l8192", 64, 1, 128, 8192, "bf16", 192, seed=8),
}


SPARSE_WORKLOADS = {
    # 128K context, 2048 selected tokens per sequence, 64 sequences
    "sparse_b64_l131072_topk2048": SparseWorkload("sparse_b64_l131072_topk2048", 64, 128,
                                                  131072, 2048, pool_blocks=8192, seed=6),
}


def make_sparse_workload(w: SparseWorkload, seqlens: Optional[np.ndarray] = None,
                         pad: int = 0) -> dict:
    """Draw one sparse workload: the paged-decode arrays of ``make_workload`` plus
    ``indices`` [B, topk] int32.  ``pad`` extra -1 entries (and as many positions at or
    past the length) replace list entries, to exercise padding."""
    streams = np.random.SeedSequence(w.seed).spawn(6)
    rng_len = np.random.Generator(np.random.PCG64(streams[0]))
    rng_tab = np.random.Generator(np.random.PCG64(streams[1]))
    rng_idx = np.random.Generator(np.random.PCG64(streams[4]))
    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32).copy()
    elif w.ragged:
        lens = rng_len.integers(1, w.context, size=w.batch, endpoint=True).astype(np.int32)
    else:
        lens = np.full(w.batch, w.context, dtype=np.int32)
    B = int(lens.shape[0])
    nblk = (lens.astype(np.int64) + PAGE - 1) // PAGE
    max_blocks = max(1, int(nblk.max()) if B else 1)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    if w.pool_blocks:
        num_blocks = w.pool_blocks
        for b in range(B):
            table[b, :nblk[b]] = rng_tab.integers(0, num_blocks, size=int(nblk[b]))
    else:
        num_blocks = int(nblk.sum())
        perm = rng_tab.permutation(num_blocks).astype(np.int32)
        off = 0
        for b in range(B):
            k = int(nblk[b])
            table[b, :k] = perm[off:off + k]
            off += k
    idx = np.full((B, w.topk), -1, dtype=np.int32)
    for b in range(B):
        L = int(lens[b])
        k = min(w.topk, L)
        if k:
            idx[b, :k] = rng_idx.choice(L, size=k, replace=False)
        if pad:
            slots = rng_idx.choice(w.topk, size=min(pad, w.topk), replace=False)
            half = len(slots) // 2
            idx[b, slots[:half]] = -1
            idx[b, slots[half:]] = L + rng_idx.integers(0, 1000, size=len(slots) - half)
        idx[b] = idx[b, rng_idx.permutation(w.topk)]
    q = _normal_fill(streams[2], B * w.heads * D_QK, w.sigma, True).reshape(B, 1, w.heads, D_QK)
    kv = _normal_fill(streams[3], num_blocks * PAGE * D_QK, w.sigma, True)
    kv = kv.reshape(num_blocks, PAGE, D_QK)
    return {
        "workload": w,
        "q": q,
        "kv_cache": kv,
        "block_table": table,
        "seqlens": lens,
        "indices": idx,
        "scale": w.scale,
    }


def sample_sequences(batch: int, count: int, seed: int) -> np.ndarray:
    """Indices of sequences checked one by one at full size: first, last and a seeded draw."""
    rng = np.random.default_rng(seed + 1000)
    pick = {0, batch - 1}
    if batch > 2:
        pick.update(int(i) for i in rng.choice(np.arange(1, batch - 1),
                                                size=min(count, batch - 2), replace=False))
    return np.array(sorted(pick), dtype=np.int64)
