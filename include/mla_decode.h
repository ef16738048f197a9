/*
 * MLA decode attention on MI355X (gfx950): C ABI of libmla_decode.so.
 *
 * What it computes.  The DeepSeek-MLA decode step that the TileLang talk uses
 * as its running example (section "What is TileLang?": the DeepSeek MLA
 * kernel, its tile configuration, and the layout-inference example in which
 * the score accumulator is reduced to the per-row maximum).  For every
 * sequence b, query token t (0 <= t < s_q) and head h:
 *
 *   R_b[j]  = kv_cache[block_table[b][j / 64]][j % 64][0..575]   (j < L_b)
 *   n       = L_b, or L_b - s_q + 1 + t with the causal mask (the s_q queries
 *             are the last s_q positions of the sequence)
 *   s_j     = scale * sum_d q[b][t][h][d] * R_b[j][d]             (j < n)
 *   lse     = ln sum_j exp(s_j)                 (natural log, scaled scores)
 *   out[c]  = sum_j exp(s_j - lse) * R_b[j][c]                    (c < 512)
 *
 * All heads read the same 576-wide latent rows (512 latent + 64 rope); V is
 * the first 512 values of each row.  A query with no visible key gets
 * out = 0 and lse = -inf.
 *
 * Memory.  Every pointer argument below is a DEVICE pointer except `status`
 * (host) in mla_read_status.  The caller owns all buffers; the library never
 * allocates device memory and keeps no per-call state (mla_decode_fwd_noalloc
 * keeps its plan and partials in the library's static scratch instead).  Inputs
 * are never modified.  All tensors are row-major with dense rows; only
 * mla_decode_fwd_strided lets the (b, t, h) rows of q and out sit a given number of
 * elements apart (q sliced from a wider projection output, out a view of a wider
 * buffer).  Other strided views must be copied to a dense buffer first:
 *
 *   q            [batch][s_q][num_heads][576]        dtype (16-byte aligned)
 *   kv_cache     [num_blocks][64][576]               dtype (16-byte aligned)
 *   block_table  [batch][max_blocks_per_seq]         int32; entries past
 *                ceil(L_b / 64) are never read
 *   seqlens      [batch]                             int32
 *   out          [batch][s_q][num_heads][512]        float32 (16-byte aligned)
 *   lse          [batch][s_q][num_heads]             float32
 *
 * Streams.  Calls only enqueue work on `stream` (a hipStream_t; NULL is the
 * null stream) and return; none synchronizes except mla_read_status.  Kernels
 * launch on the current HIP device: every buffer and `stream` must belong to it
 * (the library cannot check which device a plain pointer names).
 *
 * Errors.  Every entry point returns MLA_OK (0) or a negative MLA_ERR_* code.
 * Arguments are validated on the host before any HIP call; on error nothing
 * is enqueued.  Problems only the device can see (bad lengths or block
 * numbers, a plan built for other lengths) set bits in the plan's status word
 * (MLA_STATUS_*) and turn the affected sequences' out/lse into NaN; read it
 * with mla_read_status.  Nothing throws or aborts across this boundary.
 * Calls on distinct plans/workspaces may run concurrently.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PAGE_SIZE 64
#define MLA_HEAD_DIM 576
#define MLA_V_DIM 512

/* Return codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, misalignment, scale not finite and > 0 */
#define MLA_ERR_UNSUPPORTED (-2) /* unknown dtype, s_q * num_heads above MLA_MAX_ROWS */
#define MLA_ERR_PLAN (-3)        /* metadata or workspace buffer too small for these sizes */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call failed (launch, copy, device query) */
#define MLA_ERR_SCRATCH (-5)     /* mla_decode_fwd_noalloc: sizes need more than its fixed scratch */

/* Element types of q and kv_cache (out/lse are always float32). */
#define MLA_DTYPE_F32 0
#define MLA_DTYPE_BF16 1

/* Largest s_q * num_heads per call (128 query tokens of 128 heads: chunked queries).
 * Every 128 rows of a sequence form one row group that reads the sequence's whole
 * cache, so the cache is read once per row group. */
#define MLA_MAX_ROWS 16384

/* Device status bits (mla_read_status). */
#define MLA_STATUS_BAD_SEQLEN 1     /* L_b < 0, L_b > 64 * max_blocks_per_seq, or causal L_b < s_q */
#define MLA_STATUS_BAD_BLOCK 2      /* a block_table entry read was outside [0, num_blocks) */
#define MLA_STATUS_PLAN_MISMATCH 4  /* plan built for other sizes, seqlens, causal flag or table width */
#define MLA_STATUS_BAD_SCALE 8      /* fp8 cache: a row scale outside 2^-117 .. 2^119 powers of two */

/*
 * Number of workgroups to plan for on `device`: its compute-unit count.
 * One HIP call (device attribute query).  Returns MLA_ERR_HIP without a GPU.
 */
int mla_device_workgroups(int device, int* num_workgroups);

/*
 * Host-only, pure: bytes of the scheduling metadata (`meta`) and of the split
 * workspace that mla_get_split_metadata / mla_decode_fwd need for these sizes.
 * num_workgroups: the persistent grid size (typically mla_device_workgroups).
 */
int mla_plan_size(int batch, int s_q, int num_heads, int num_workgroups,
                  size_t* meta_bytes, size_t* workspace_bytes);

/*
 * Split-KV tile scheduler (one small kernel).  Reads seqlens on the device and
 * writes the work partition into `meta` (device, >= meta_bytes from
 * mla_plan_size): the concatenated stream of 64-token blocks of every
 * (sequence, 128-row group) is cut into near-equal contiguous ranges, one per
 * workgroup; a sequence cut at a range boundary is computed in parts and
 * merged by log-sum-exp.  The stream of T blocks is cut into n ranges:
 * n = T / min_split_blocks for min_split_blocks > 0 (the smallest range a
 * workgroup is given, which bounds the number of parts), or by default
 * (min_split_blocks = 0) the fewest ranges whose longest is as short as with
 * one range per workgroup, n = ceil(T / ceil(T / num_workgroups)); always
 * 1 <= n <= min(T, num_workgroups).
 * The plan is reusable by every mla_decode_fwd with the same sizes and
 * seqlens (e.g. all layers of one decode step).
 */
int mla_get_split_metadata(const int32_t* seqlens, int batch, int s_q, int num_heads,
                           int causal, int max_blocks_per_seq, int num_workgroups,
                           int min_split_blocks, int32_t* meta, size_t meta_bytes,
                           void* stream);

/*
 * MLA decode forward: enqueues the main kernel (paged gather into LDS, scores
 * and PV on MFMA, online softmax) and the log-sum-exp combine of split parts.
 * meta/num_workgroups: from mla_get_split_metadata with the same sizes.
 * workspace: device scratch of >= workspace_bytes (mla_plan_size) for the
 * partial results of split sequences; no zeroing needed.
 * dtype: MLA_DTYPE_BF16 (MFMA path) or MLA_DTYPE_F32 (fp32 path).
 * scale: the softmax scale, finite and > 0 (e.g. 1/sqrt(192)).
 */
int mla_decode_fwd(int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
                   const int32_t* block_table, int max_blocks_per_seq,
                   const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                   float scale, float* out, float* lse,
                   int32_t* meta, size_t meta_bytes, int num_workgroups,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_fwd with strided rows: row (b, t, h) of q starts at
 * q + ((b * s_q + t) * num_heads + h) * q_row_stride and its output row at
 * out + (...) * out_row_stride (elements); every other argument and rule as in
 * mla_decode_fwd (mla_decode_fwd is this call with strides 576 and 512).  The 576
 * (512) values of a row are contiguous and start 16-byte aligned: q_row_stride >= 576
 * and a multiple of 8 (bf16) or 4 (f32), out_row_stride >= 512 and a multiple of 4,
 * both at most 2^40; otherwise MLA_ERR_INVALID_ARG.  lse stays dense.  The rows are
 * only read or written at those addresses: the gaps between them are left untouched.
 */
int mla_decode_fwd_strided(int dtype, const void* q, int64_t q_row_stride,
                           const void* kv_cache, int64_t num_blocks,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seqlens, int batch, int s_q, int num_heads,
                           int causal, float scale, float* out, int64_t out_row_stride,
                           float* lse, int32_t* meta, size_t meta_bytes, int num_workgroups,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of mla_decode_fwd, for callers that time or schedule them
 * apart (same arguments and rules as mla_decode_fwd):
 *   mla_decode_main     the main kernel: every segment computed whole writes
 *                       out/lse; split segments write their parts to workspace;
 *   mla_decode_combine  the log-sum-exp merge of those parts into out/lse, and
 *                       out = 0 / lse = -inf (NaN for invalid lengths) for
 *                       sequences with no key.
 * mla_decode_main followed by mla_decode_combine on one stream equals
 * mla_decode_fwd.
 */
int mla_decode_main(int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
                    const int32_t* block_table, int max_blocks_per_seq,
                    const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                    float scale, float* out, float* lse,
                    int32_t* meta, size_t meta_bytes, int num_workgroups,
                    void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_combine(int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
                       const int32_t* block_table, int max_blocks_per_seq,
                       const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                       float scale, float* out, float* lse,
                       int32_t* meta, size_t meta_bytes, int num_workgroups,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse MLA decode: the SparseMLA variant of the Triton-TLE talk's performance
 * section, in which each query reads only a selected list of token positions out of a
 * long (128K) context.  For every sequence b and head h (one query token, s_q = 1):
 *
 *   sel_b   = [ indices[b][k] for k < topk  if 0 <= indices[b][k] < L_b ]
 *             (other entries, e.g. -1, are padding; a position listed twice counts twice)
 *   s_j     = scale * sum_d q[b][0][h][d] * R_b[j][d]        (j in sel_b)
 *   lse     = ln sum_j exp(s_j),   out[c] = sum_j exp(s_j - lse) * R_b[j][c]
 *
 * with R_b the rows of sequence b through its block table, as in mla_decode_fwd.  No
 * selected key gives out = 0 and lse = -inf.
 *
 * Layouts as in mla_decode_fwd with s_q = 1 and dtype bf16; in addition
 *   indices   [batch][topk] int32 (device), token positions within each sequence.
 * topk is a positive multiple of 64, at most 65536; num_blocks at most 2^25.
 *
 * One call enqueues, on `stream`: one kernel that picks and orders the selected rows
 * (their pool rows, packed lengths and a packed block table, in the workspace), the
 * split scheduler over the packed lengths (it writes `meta`, so no separate
 * mla_get_split_metadata call is made), the main kernel, which reads each selected row
 * straight from the pool, and the combine.  A pool of more than 58254 blocks (past
 * 32-bit byte offsets) instead has its selected rows copied into workspace blocks by
 * one more kernel, which the main kernel then reads as a paged cache.  meta/workspace: device buffers of at
 * least the sizes mla_sparse_plan_size returns for the same batch, num_heads, topk and
 * num_workgroups.  Errors and device status bits as for mla_decode_fwd (a selected
 * position whose block number is outside the pool: MLA_STATUS_BAD_BLOCK and NaN for
 * that sequence; an invalid length: MLA_STATUS_BAD_SEQLEN and NaN).
 */
int mla_sparse_plan_size(int batch, int num_heads, int topk, int num_workgroups,
                         size_t* meta_bytes, size_t* workspace_bytes);
int mla_decode_sparse_fwd(const void* q, const void* kv_cache, int64_t num_blocks,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seqlens, const int32_t* indices, int topk,
                          int batch, int num_heads, float scale, float* out, float* lse,
                          int32_t* meta, size_t meta_bytes, int num_workgroups,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * MLA decode over a quantized latent cache.  The pages name dequantization and
 * mixed-precision layouts among what a kernel compiler must handle (the TileLang talk's
 * "Why a new DSL?" and "What is TileLang?" sections); the row format is this library's
 * own:
 *   kv_fp8  [num_blocks][64][656] bytes (device, 16-byte aligned), one row per token:
 *           bytes 0..511    the 512 latent values as fp8 e4m3 codes (OCP 8-bit float:
 *                           sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 *                           infinities, 0x7F/0xFF NaN, largest finite 448),
 *           bytes 512..639  the 64 rope values as bf16,
 *           bytes 640..643  the row's fp32 scale (latent value = code value * scale),
 *           bytes 644..655  padding.
 * The scale must be a power of two 2^k with -117 <= k <= 119, as in the OCP
 * microscaling formats' shared scales (a power-of-two scale is applied exactly by the
 * hardware conversion, and in this range every code value times the scale is a normal
 * bf16 number or zero, so every latent value is exact in bf16).  The main kernel checks
 * the scale of every row it reads (the rows [0, L_b) of each sequence): a row with any
 * other scale (not a power of two, outside the range, negative, zero, NaN) sets
 * MLA_STATUS_BAD_SCALE and makes that sequence's out and lse NaN.
 * Everything else as mla_decode_fwd with dtype bf16 (q bf16, out/lse fp32, the same
 * definition over the dequantized rows).  One call enqueues the split scheduler (it
 * writes `meta`), the main kernel, which copies each 656-byte-row page into LDS and
 * widens it there to bf16 before the page's products, and the combine.  meta/workspace:
 * device buffers of at least the sizes mla_fp8_plan_size returns (the same as
 * mla_plan_size's).  Errors and status bits as for mla_decode_fwd (a block number
 * outside the pool: MLA_STATUS_BAD_BLOCK and NaN for that sequence; a row scale outside
 * the format: MLA_STATUS_BAD_SCALE and NaN for that sequence).
 */
int mla_fp8_plan_size(int batch, int s_q, int num_heads, int max_blocks_per_seq,
                      int num_workgroups, size_t* meta_bytes, size_t* workspace_bytes);
int mla_decode_fp8_fwd(const void* q, const void* kv_fp8, int64_t num_blocks,
                       const int32_t* block_table, int max_blocks_per_seq,
                       const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                       float scale, float* out, float* lse, int32_t* meta, size_t meta_bytes,
                       int num_workgroups, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Latent-cache append, the step before decode attention (the pages describe only the
 * attention; this call writes the rows it reads, under the same cache layout and the
 * same length convention).  Row t of sequence b (0 <= t < s_new) is written to
 * logical position p = seqlens[b] - s_new + t (seqlens already count the new tokens,
 * as mla_decode_fwd's causal mask reads them), i.e. to
 *   kv_cache[block_table[b][p / 64]][p % 64][0:576].
 * dtype:     MLA_DTYPE_BF16 or MLA_DTYPE_F32, the element type of new_kv and kv_cache.
 * new_kv:    device [batch][s_new][576], contiguous, 16-byte aligned; only read.
 * kv_cache:  device [num_blocks][64][576], 16-byte aligned; the addressed rows are
 *            overwritten, nothing else is touched.
 * block_table [batch][max_blocks_per_seq] int32 and seqlens [batch] int32: device; read.
 * status:    device int32 or NULL.  A row whose position is outside
 *            [0, 64 * max_blocks_per_seq) is skipped and MLA_STATUS_BAD_SEQLEN is OR'ed
 *            in; a row whose block number is outside [0, num_blocks) is skipped with
 *            MLA_STATUS_BAD_BLOCK.  The word is never cleared by the library.
 * Asynchronous on `stream`; allocates nothing.  Rows of different calls, or two rows
 * of one call with the same position, must not overlap in flight: the later write wins
 * only in stream order.  Host-side errors as for mla_decode_fwd.
 */
int mla_kv_append(int dtype, const void* new_kv, void* kv_cache, int64_t num_blocks,
                  const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens,
                  int batch, int s_new, int32_t* status, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mla_get_split_metadata followed by
 * mla_decode_fwd (the default plan, min_split_blocks = 0) in one call, with the plan
 * and the partial results of split sequences kept in the library's own static device
 * scratch of MLA_NOALLOC_SCRATCH_BYTES (80 MiB) per device, instead of caller buffers.
 * The caller still passes inputs and outputs, with the meaning, layout and checks of
 * mla_decode_fwd.  The call allocates nothing (no hipMalloc/hipFree, no allocating
 * library routine); the scratch is part of the loaded library and each device that runs
 * the call holds its own copy until the process ends.  Its address is looked up once
 * per device, on the first call with that device current.
 * Limit: the plan (32 + 8 * (num_workgroups + segments) int32, rounded up to 256 bytes)
 * plus the partials ((num_workgroups + segments) * 128 rows of 1032 bytes for bf16, of
 * 2052 bytes for fp32; segments = batch * ceil(s_q * num_heads / 128)) must fit the
 * scratch, else MLA_ERR_SCRATCH and nothing is enqueued (with 256 workgroups: up to 378
 * segments in bf16, 63 in fp32).
 * Every call on one device shares that device's scratch: calls whose work overlaps on a
 * device (other streams, or other threads, without ordering between them) race and give
 * wrong results; calls ordered on one stream are safe.  The scratch keeps the last
 * call's plan; each call rewrites every word it reads, so nothing is cleared.  Device
 * status bits are not readable here (the plan lives in the scratch): problems only the
 * device can see show as NaN outputs for the affected sequences, as in mla_decode_fwd.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (80u << 20)
int mla_decode_fwd_noalloc(int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seqlens, int batch, int s_q, int num_heads,
                           int causal, float scale, float* out, float* lse,
                           int num_workgroups, void* stream);

/*
 * Synchronizes `stream`, then copies the plan's device status word
 * (MLA_STATUS_* bits, 0 = clean) into *status (host pointer).
 */
int mla_read_status(const int32_t* meta, void* stream, int32_t* status);

/* Static, human-readable text of an MLA_* return code. */
const char* mla_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
