"""CPU oracle for MLA decode attention: test infrastructure, not the product.

Only the tests, the smoke check and the bench's CPU-baseline leg use this
module.  It shares no code with the HIP path and imports nothing from it.

What it computes is the plain definition of decode attention over a paged
latent cache, as the DeepSeek-MLA / FlashMLA running example of the TileLang
talk ("What is TileLang?", the DeepSeek MLA kernel and its layout-inference
example) uses it, with the shapes of that example: each cache row holds 576
values (512 latent + 64 rope), every head reads the same rows, K is the whole
row and V is its first 512 values, the softmax is scaled, and the outputs are
O and the natural-log log-sum-exp of the scaled scores.  The tile loop, online
softmax and split/combine of the kernels are ways to reach exactly this
result, so the oracle is the definition written out, in float64:

    rows of sequence b:  R_b[j] = kv_cache[block_table[b, j // 64], j % 64, :]
    visible keys of query token t:  n = L_b            (not causal)
                                    n = L_b - s_q + 1 + t   (causal, the s_q
                                    queries are the last s_q positions)
    s_j        = scale * sum_d q[b,t,h,d] * R_b[j][d]          (j < n)
    LSE[b,t,h] = ln sum_j exp(s_j)
    O[b,t,h,c] = sum_j exp(s_j - LSE) * R_b[j][c]              (c < 512)

A query with no visible key (n = 0) gets O = 0 and LSE = -inf.

``merge_partials`` is the log-sum-exp merge of attention results over
disjoint key sets; it is exercised against the unsplit definition.
``kv_append`` writes a decode step's new latent rows into the pages, where
``gather_rows`` (and so the attention) reads them.  ``mla_decode_fp8`` is the same
definition over a cache of 656-byte quantized rows (fp8 e4m3 latent codes times a
per-row fp32 scale, bf16 rope), each row dequantized exactly before use.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an input array: bf16 bit patterns (uint16) or floats."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def visible_keys(seqlen: int, s_q: int, t: int, causal: bool) -> int:
    """Number of keys query token t of a sequence may attend to."""
    if not causal:
        return seqlen
    return seqlen - s_q + 1 + t


def gather_rows(kv_cache: np.ndarray, block_table: np.ndarray, b: int, seqlen: int) -> np.ndarray:
    """The first ``seqlen`` logical rows of sequence b, read through its block table."""
    if seqlen == 0:
        return kv_cache.reshape(-1, kv_cache.shape[-1])[:0]
    nblk = (seqlen + PAGE - 1) // PAGE
    blocks = np.asarray(block_table[b, :nblk], dtype=np.int64)
    if (blocks < 0).any() or (blocks >= kv_cache.shape[0]).any():
        raise ValueError(f"sequence {b}: block table entry outside the pool")
    return kv_cache[blocks].reshape(nblk * PAGE, kv_cache.shape[-1])[:seqlen]


def check_lengths(seqlens: np.ndarray, block_table: np.ndarray, s_q: int, causal: bool) -> None:
    cap = block_table.shape[1] * PAGE
    for b, L in enumerate(np.asarray(seqlens).tolist()):
        if L < 0 or L > cap:
            raise ValueError(f"sequence {b}: length {L} outside [0, {cap}]")
        if causal and L < s_q:
            raise ValueError(f"sequence {b}: causal length {L} shorter than {s_q} queries")


def weights_and_lse(q_rows: np.ndarray, keys: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Scaled scores s[h, j] = scale * <q_h, K_j> of query rows [H, 576] against keys
    [n, 576] (n >= 1), their log-sum-exp LSE[h] = ln sum_j exp(s[h, j]) (taken as
    m + ln sum_j exp(s - m) with m the row max, so no term overflows), and the weights
    p[h, j] = exp(s[h, j] - LSE[h]).  Returns (p [H, n], LSE [H])."""
    s = scale * (q_rows @ keys.T)                      # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    return np.exp(s - lse[:, None]), lse


def attend_one(q_rows: np.ndarray, keys: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of query rows [H, 576] over keys [n, 576] (V = keys[:, :512]), float64:
    O[h] = sum_j p[h, j] * V_j with the weights of ``weights_and_lse``.

    Returns (O [H, 512], LSE [H]).  n = 0 gives O = 0 and LSE = -inf.
    """
    H = q_rows.shape[0]
    n = keys.shape[0]
    if n == 0:
        return np.zeros((H, D_V)), np.full(H, -np.inf)
    p, lse = weights_and_lse(q_rows, keys, scale)
    return p @ keys[:, :D_V], lse


def mla_decode(q, kv_cache, block_table, seqlens, scale, causal=False, dtype="bf16",
               batches: Iterable[int] | None = None):
    """Float64 O [B, s_q, H, 512] and LSE [B, s_q, H] of MLA decode.

    ``q``/``kv_cache`` hold bf16 bit patterns (dtype "bf16") or floats ("f32",
    "f64").  ``scale`` is used as given (pass the float32 value the kernels see).
    ``batches`` restricts the work to some sequences; the others stay NaN.
    """
    q = np.asarray(q)
    B, s_q, H, D = q.shape
    if D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK):
        raise ValueError("expected q [B,s_q,H,576] and kv_cache [blocks,64,576]")
    seqlens = np.asarray(seqlens)
    check_lengths(seqlens, block_table, s_q, causal)
    scale = float(scale)
    out = np.full((B, s_q, H, D_V), np.nan)
    lse = np.full((B, s_q, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        keys = widen(gather_rows(kv_cache, block_table, b, L), dtype)
        qb = widen(q[b], dtype)                          # [s_q, H, 576]
        for t in range(s_q):
            n = visible_keys(L, s_q, t, causal)
            out[b, t], lse[b, t] = attend_one(qb[t], keys[:n], scale)
    return out, lse


def selected_rows(kv_cache: np.ndarray, block_table: np.ndarray, b: int, seqlen: int,
                  positions: np.ndarray) -> np.ndarray:
    """Rows of sequence b at the listed token positions, in list order.

    Positions outside [0, seqlen) select nothing; a position listed twice is a key twice.
    """
    pos = np.asarray(positions, dtype=np.int64)
    pos = pos[(pos >= 0) & (pos < seqlen)]
    rows = np.empty((pos.shape[0], kv_cache.shape[-1]), dtype=kv_cache.dtype)
    for k, p in enumerate(pos.tolist()):
        blk = int(block_table[b, p // PAGE])
        if blk < 0 or blk >= kv_cache.shape[0]:
            raise ValueError(f"sequence {b}: block table entry outside the pool")
        rows[k] = kv_cache[blk, p % PAGE]
    return rows


def mla_decode_sparse(q, kv_cache, block_table, seqlens, indices, scale, dtype="bf16",
                      batches: Iterable[int] | None = None):
    """Float64 O [B, s_q, H, 512] and LSE [B, s_q, H] of sparse MLA decode.

    The SparseMLA variant of the Triton-TLE talk's performance section (a 128K
    context of which each query reads a selected subset of tokens): every query of
    sequence b attends to the keys at the token positions ``indices[b, :]`` (the
    selected subset, e.g. a top-k list), with the same scores, softmax and outputs
    as ``mla_decode`` over just those keys.  Positions outside [0, L_b) are padding
    and select nothing; a position listed twice counts twice.  No selected key
    gives O = 0 and LSE = -inf.
    """
    q = np.asarray(q)
    B, s_q, H, D = q.shape
    if D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK):
        raise ValueError("expected q [B,s_q,H,576] and kv_cache [blocks,64,576]")
    seqlens = np.asarray(seqlens)
    check_lengths(seqlens, block_table, s_q, False)
    indices = np.asarray(indices)
    if indices.ndim != 2 or indices.shape[0] != B:
        raise ValueError("expected indices [B, topk]")
    scale = float(scale)
    out = np.full((B, s_q, H, D_V), np.nan)
    lse = np.full((B, s_q, H), np.nan)
    for b in (range(B) if batches is None else batches):
        keys = widen(selected_rows(kv_cache, block_table, b, int(seqlens[b]), indices[b]), dtype)
        qb = widen(q[b], dtype)
        for t in range(s_q):
            out[b, t], lse[b, t] = attend_one(qb[t], keys, scale)
    return out, lse


def kv_append(kv_cache, block_table, seqlens, new_kv):
    """The cache after appending each sequence's new latent rows, and the skipped rows.

    The step before decode attention writes the rows that the attention reads:
    row t of ``new_kv[b]`` (0 <= t < s_new) becomes logical row p = L_b - s_new + t
    of sequence b, the lengths already counting the new tokens (the convention under
    which the causal decode gives query token t the keys up to position p).  Logical
    row p lives at ``kv_cache[block_table[b, p // 64], p % 64]``, as in ``gather_rows``.
    A row whose position is outside [0, 64 * table width) or whose block number is
    outside the pool is not written; it is reported as (b, t, "seqlen" or "block").
    Returns (a new cache array, the list of skipped rows).  Exact: values are copied.
    """
    out = np.array(kv_cache, copy=True)
    new_kv = np.asarray(new_kv)
    B, s_new = new_kv.shape[:2]
    cap = block_table.shape[1] * PAGE
    skipped = []
    for b in range(B):
        for t in range(s_new):
            p = int(seqlens[b]) - s_new + t
            if p < 0 or p >= cap:
                skipped.append((b, t, "seqlen"))
                continue
            blk = int(block_table[b, p // PAGE])
            if blk < 0 or blk >= out.shape[0]:
                skipped.append((b, t, "block"))
                continue
            out[blk, p % PAGE] = new_kv[b, t]
    return out, skipped


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Float64 value of fp8 e4m3 codes (OCP 8-bit float): sign bit 7, exponent bits 6..3
    with bias 7, mantissa bits 2..0; exponent 0 is subnormal (mantissa * 2^-9); exponent
    15 with mantissa 7 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 7).astype(np.float64)
    mag = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    mag = np.where((ex == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def fp8_rows(rows: np.ndarray) -> np.ndarray:
    """Float64 [..., 576] rows of a quantized cache stored as 656-byte rows: 512 e4m3
    latent codes times the row's fp32 scale (bytes 640..643; the format takes powers of
    two, but any value is decoded as written), then the 64 bf16 rope values (bytes
    512..639)."""
    r = np.ascontiguousarray(rows, dtype=np.uint8)
    lead = r.shape[:-1]
    r = r.reshape(-1, r.shape[-1])
    scale = r[:, 640:644].copy().view(np.float32)[:, 0].astype(np.float64)
    out = np.empty((r.shape[0], D_QK))
    out[:, :D_V] = e4m3_value(r[:, :512]) * scale[:, None]
    out[:, D_V:] = widen(r[:, 512:640].copy().view(np.uint16), "bf16")
    return out.reshape(*lead, D_QK)


FP8_MIN_SCALE_EXP = -117
FP8_MAX_SCALE_EXP = 119


def fp8_scale_in_format(scales: np.ndarray) -> np.ndarray:
    """True where a row scale belongs to the quantized format: a power of two 2^k with
    -117 <= k <= 119.  Then every e4m3 code value (magnitudes 2^-9 .. 448, or 0) times
    the scale is zero or a normal bf16 number, i.e. the dequantized row is exact in
    bf16; other scales (not a power of two, outside the range, <= 0, NaN, inf) are not
    rows of the format."""
    s = np.asarray(scales, dtype=np.float64)
    ok = np.isfinite(s) & (s > 0)
    man, ex = np.frexp(np.where(ok, s, 1.0))           # s = man * 2^ex, man in [0.5, 1)
    k = ex - 1
    return ok & (man == 0.5) & (k >= FP8_MIN_SCALE_EXP) & (k <= FP8_MAX_SCALE_EXP)


def mla_decode_fp8(q, kv_fp8, block_table, seqlens, scale, causal=False,
                   batches: Iterable[int] | None = None):
    """MLA decode over a quantized latent cache [blocks, 64, 656] bytes: the same
    definition as ``mla_decode`` with every key/value row dequantized exactly (fp64)
    by ``fp8_rows``; q holds bf16 bit patterns.  A sequence one of whose rows [0, L_b)
    has a scale outside the format (``fp8_scale_in_format``) is an invalid input, as an
    invalid length is: ValueError."""
    q = np.asarray(q)
    B, s_q, H, D = q.shape
    if D != D_QK or kv_fp8.shape[1:] != (PAGE, 656):
        raise ValueError("expected q [B,s_q,H,576] and kv_fp8 [blocks,64,656]")
    seqlens = np.asarray(seqlens)
    check_lengths(seqlens, block_table, s_q, causal)
    scale = float(scale)
    out = np.full((B, s_q, H, D_V), np.nan)
    lse = np.full((B, s_q, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        raw = gather_rows(kv_fp8, block_table, b, L)
        row_scales = np.ascontiguousarray(raw[:, 640:644]).view(np.float32)[:, 0]
        if not fp8_scale_in_format(row_scales).all():
            raise ValueError(f"sequence {b}: a row scale outside the quantized format")
        keys = fp8_rows(raw)
        qb = widen(q[b], "bf16")
        for t in range(s_q):
            n = visible_keys(L, s_q, t, causal)
            out[b, t], lse[b, t] = attend_one(qb[t], keys[:n], scale)
    return out, lse


def softmax_weights(q_rows: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """The attention weights p[h, j] = exp(s_j - LSE_h) that ``attend_one`` builds its
    outputs from (the same function, so a pin on them pins the outputs' weights)."""
    return weights_and_lse(q_rows, keys, scale)[0]


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Merge attention results over disjoint key sets into the result over their union.

    With LSE_i the log-sum-exp of part i, the union has LSE = ln sum_i exp(LSE_i)
    and O = sum_i exp(LSE_i - LSE) * O_i.  Parts with no keys (LSE_i = -inf)
    carry zero weight; if every part is empty the result is O = 0, LSE = -inf.
    """
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lses])        # [S, ...]
    o = np.stack([np.asarray(x, dtype=np.float64) for x in outs])          # [S, ..., 512]
    mx = lse.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - safe), 0.0)
    tot = w.sum(axis=0)
    out_lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    return (wn[..., None] * o).sum(axis=0), out_lse


def brute_force(q_list, keys_list, scale: float, causal: bool, s_q: int):
    """Pure-Python loops over dense per-sequence keys, for tiny cases.

    ``q_list[b][t][h]`` is a list of 576 floats; ``keys_list[b]`` a list of rows.
    Sums use math.fsum, exponentials math.exp.  Returns nested lists
    (O[b][t][h][c], LSE[b][t][h]).
    """
    outs, lses = [], []
    for b, rows in enumerate(keys_list):
        ob, lb = [], []
        for t in range(s_q):
            # the causal bound written out (not through visible_keys), so this loop pins it:
            # the s_q queries are the sequence's last s_q positions, t sees keys 0 .. L-s_q+t
            n = len(rows) - s_q + 1 + t if causal else len(rows)
            ot, lt = [], []
            for qh in q_list[b][t]:
                if n == 0:
                    ot.append([0.0] * D_V)
                    lt.append(-math.inf)
                    continue
                s = [scale * math.fsum(qh[d] * rows[j][d] for d in range(D_QK)) for j in range(n)]
                m = max(s)
                z = math.fsum(math.exp(x - m) for x in s)
                L = m + math.log(z)
                p = [math.exp(x - L) for x in s]
                ot.append([math.fsum(p[j] * rows[j][c] for j in range(n)) for c in range(D_V)])
                lt.append(L)
            ob.append(ot)
            lb.append(lt)
        outs.append(ob)
        lses.append(lb)
    return outs, lses
