// Sparse MLA decode: the selected rows' packing.
//
// The SparseMLA variant of the Triton-TLE talk's performance section reads, out of a
// long (128K) context, only a selected list of token positions per sequence.  Attention
// does not depend on the order of its keys, so the selected rows of sequence b are
// packed, valid ones first and in list order, into packed blocks of 64:
//
//   mla_sparse_index_kernel   one workgroup per sequence: which list entries select a
//                             key (0 <= position < L_b), their packed order (a block
//                             scan), the pool row of each (the last packed block padded
//                             with its last row), and the packed sequence's length and
//                             block table.
//
// The default path stops there: the scheduler plans over the packed lengths and the bf16
// main kernel reads each packed block as a "gathered page", copying every row straight
// from the pool through these row numbers, so no row is copied twice.  That kernel forms
// a row's byte offset from the pool base in 32 bits, so pools of more than
// kMaxGatherBlocks blocks (4.3 GB) take a copy first: the ABI then also runs
//
//   mla_sparse_gather_kernel  one workgroup per 64 packed rows: copies each row (1152
//                             bytes, 16-byte loads and stores) into packed blocks,
//
// which the paged main kernel then reads like any cache.  A position whose block number
// lies outside the pool turns its packed block's table entry into -1, which the main
// kernel reports as a bad block (status bit, NaN output); an invalid length becomes
// packed length -1, which the scheduler reports.
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void mla_sparse_index_kernel(
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ block_table, int max_blocks,
    int64_t num_blocks, const int32_t* __restrict__ indices, int topk,
    int32_t* __restrict__ src_row, int32_t* __restrict__ packed_len,
    int32_t* __restrict__ packed_table) {
  __shared__ int wave_tot[kThreads / 64];
  __shared__ int bad_chunk[kMaxSparseChunks];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = seqlens[b];
  const bool len_ok = L >= 0 && (int64_t)L <= (int64_t)max_blocks * kPage;
  const int chunks = topk / kPage;
  for (int c = tid; c < chunks; c += kThreads) bad_chunk[c] = 0;

  // thread tid owns list entries [tid*per, tid*per + per)
  const int per = topk / kThreads + (topk % kThreads ? 1 : 0);
  const int e0 = min(topk, tid * per), e1 = min(topk, e0 + per);
  const int32_t* lst = indices + (size_t)b * topk;
  int run = 0;
  for (int e = e0; e < e1; ++e) {
    const int p = lst[e];
    run += (len_ok && p >= 0 && p < L) ? 1 : 0;
  }
  // exclusive block scan of the run lengths
  int x = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += wave_tot[w];
    total += wave_tot[w];
  }
  int pos = before + x - run;
  for (int e = e0; e < e1; ++e) {
    const int p = lst[e];
    if (!(len_ok && p >= 0 && p < L)) continue;
    const int blk = block_table[(size_t)b * max_blocks + p / kPage];
    const bool ok = blk >= 0 && (int64_t)blk < num_blocks;
    src_row[(size_t)b * topk + pos] = ok ? blk * kPage + p % kPage : -1;
    if (!ok) bad_chunk[pos / kPage] = 1;
    ++pos;
  }
  __syncthreads();
  // the rest of the last packed block repeats its last row, so a page read through these
  // lists (the main kernel's gathered pages) only ever addresses real pool rows
  if (total > 0) {
    const int32_t last = src_row[(size_t)b * topk + total - 1];
    const int padded = (total + kPage - 1) / kPage * kPage;
    for (int e = total + tid; e < padded; e += kThreads) src_row[(size_t)b * topk + e] = last;
  }
  if (tid == 0) packed_len[b] = len_ok ? total : -1;
  for (int c = tid; c < chunks; c += kThreads)
    packed_table[(size_t)b * chunks + c] = bad_chunk[c] ? -1 : b * chunks + c;
}

__global__ __launch_bounds__(kThreads) void mla_sparse_gather_kernel(
    const uint4* __restrict__ kv, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ packed_len, int topk, uint4* __restrict__ packed_kv) {
  constexpr int kVec = kDqk * 2 / 16;   // 72 16-byte pieces per row
  const int b = blockIdx.y;
  const int r0 = blockIdx.x * kPage;
  const int n = min(kPage, packed_len[b] - r0);   // rows of this block to copy
  if (n <= 0) return;
  const int32_t* src = src_row + (size_t)b * topk + r0;
  uint4* dst = packed_kv + ((size_t)b * topk + r0) * kVec;
  for (int i = threadIdx.x; i < n * kVec; i += kThreads) {
    const int r = i / kVec, v = i - r * kVec;
    const int s = src[r];
    if (s >= 0) dst[i] = kv[(size_t)s * kVec + v];
  }
}

}  // namespace

hipError_t launch_sparse_pack(const int32_t* seqlens, const int32_t* block_table, int max_blocks,
                              int64_t num_blocks, const int32_t* indices, int topk, int batch,
                              const void* kv, const SparseScratch& s, bool gather,
                              hipStream_t stream) {
  hipLaunchKernelGGL(mla_sparse_index_kernel, dim3(batch), dim3(kThreads), 0, stream, seqlens,
                     block_table, max_blocks, num_blocks, indices, topk, s.src_row, s.packed_len,
                     s.packed_table);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !gather) return e;
  hipLaunchKernelGGL(mla_sparse_gather_kernel, dim3(topk / kPage, batch), dim3(kThreads), 0,
                     stream, (const uint4*)kv, s.src_row, s.packed_len, topk,
                     (uint4*)s.packed_kv);
  return hipGetLastError();
}

}  // namespace mla
