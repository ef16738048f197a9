// Sparse MLA decode: the selected rows' packing.
//
// The SparseMLA variant of the Triton-TLE talk's performance section reads, out of a
// long (128K) context, only a selected list of token positions per sequence.  Attention
// does not depend on the order of its keys, so the selected rows of sequence b are
// packed, valid ones first and in list order, into packed blocks of 64:
//
//   mla_sparse_index_kernel   one workgroup per sequence: which list entries select a
//                             key (0 <= position < L_b), their packed order (counts of
//                             the valid entries before each, from wave ballots), the pool
//                             row of each (the last packed block padded with its last
//                             row), and the packed sequence's length and block table.
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
  // Entries are taken in rounds of 256 (thread t: entry 256 k + t of round k), eight rounds
  // at a time: their list reads, then the block-number reads of the valid ones, all in
  // flight together.  A valid entry's packed position is the number of valid entries before
  // it in list order: the totals of earlier rounds, of earlier waves in its round (wave
  // ballot counts through LDS) and of earlier lanes of its wave (a masked popcount).
  constexpr int kRounds = 8;
  constexpr int kWavesPerWg = kThreads / 64;
  __shared__ int wave_cnt[kRounds][kWavesPerWg];
  __shared__ int bad_chunk[kMaxSparseChunks];
  __shared__ int32_t last_row;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = seqlens[b];
  const bool len_ok = L >= 0 && (int64_t)L <= (int64_t)max_blocks * kPage;
  const int chunks = topk / kPage;
  for (int c = tid; c < chunks; c += kThreads) bad_chunk[c] = 0;
  const int32_t* lst = indices + (size_t)b * topk;
  const int32_t* tab = block_table + (size_t)b * max_blocks;
  int32_t* dst = src_row + (size_t)b * topk;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes before this one
  const int rounds = (topk + kThreads - 1) / kThreads;
  int base = 0;   // valid entries in the rounds already placed
  for (int r0 = 0; r0 < rounds; r0 += kRounds) {
    int p[kRounds], blk[kRounds];
    bool valid[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int e = (r0 + k) * kThreads + tid;
      p[k] = (r0 + k < rounds && e < topk) ? lst[e] : -1;
    }
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      valid[k] = len_ok && p[k] >= 0 && p[k] < L;
      blk[k] = valid[k] ? tab[p[k] / kPage] : 0;
    }
    uint64_t m[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      m[k] = __builtin_amdgcn_ballot_w64(valid[k]);
      if (lane == 0) wave_cnt[k][wave] = __builtin_popcountll(m[k]);
    }
    __syncthreads();
    int run = base;   // valid entries before round r0 + k
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWavesPerWg; ++w) {
        const int c = wave_cnt[k][w];
        before += w < wave ? c : 0;
        total += c;
      }
      if (valid[k]) {
        const int pos = run + before + __builtin_popcountll(m[k] & below);
        const bool ok = blk[k] >= 0 && (int64_t)blk[k] < num_blocks;
        const int32_t row = ok ? blk[k] * kPage + p[k] % kPage : -1;
        dst[pos] = row;
        if (!ok) bad_chunk[pos / kPage] = 1;
        p[k] = pos;     // kept for the padding row below
        blk[k] = row;
      } else {
        p[k] = -1;
      }
      run += total;
    }
    // the entry at position run - 1 is the last valid one so far; a later round with valid
    // entries overwrites it after the barrier below
#pragma unroll
    for (int k = 0; k < kRounds; ++k)
      if (p[k] >= 0 && p[k] == run - 1) last_row = blk[k];
    base = run;
    __syncthreads();   // wave_cnt is reused by the next eight rounds
  }
  const int total = base;
  // the rest of the last packed block repeats its last row, so a page read through these
  // lists (the main kernel's gathered pages) only ever addresses real pool rows
  if (total > 0) {
    const int32_t last = last_row;
    const int padded = (total + kPage - 1) / kPage * kPage;
    for (int e = total + tid; e < padded; e += kThreads) dst[e] = last;
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
