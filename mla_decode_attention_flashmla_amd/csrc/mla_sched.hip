// Split-KV tile scheduler: one workgroup turns seqlens into the work partition.
//
// The decode step's work is a stream of 64-token KV blocks, segment after
// segment, where a segment is one (sequence, 128-row group) pair.  The stream
// is cut into near-equal contiguous ranges, one per persistent workgroup of
// the main kernel; a segment cut by a range boundary is computed in parts
// whose results are merged by log-sum-exp (the "tile configuration" the
// DeepSeek MLA example of the TileLang talk leaves to its author: how many
// blocks, and which work each one takes).
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;

// Exclusive prefix sum of seg[i*kSegWords + src] into seg[i*kSegWords + dst] for i < n,
// by the whole block, in chunks of kThreads.  Returns the total (in every thread).
__device__ int64_t block_exclusive_scan(int32_t* seg, int n, int src, int dst, bool only_multi,
                                        int64_t* lds) {
  int64_t carry = 0;
  const int tid = threadIdx.x;
  for (int base = 0; base < n; base += kThreads) {
    int i = base + tid;
    int64_t v = 0;
    if (i < n) {
      v = seg[(size_t)i * kSegWords + src];
      if (only_multi && v < 2) v = 0;
    }
    lds[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      int64_t add = tid >= off ? lds[tid - off] : 0;
      __syncthreads();
      lds[tid] += add;
      __syncthreads();
    }
    if (i < n) seg[(size_t)i * kSegWords + dst] = (int32_t)(carry + lds[tid] - v);
    int64_t chunk_total = lds[kThreads - 1];
    __syncthreads();
    carry += chunk_total;
  }
  return carry;
}

// Work item holding stream position pos when T blocks are cut into n items
// (item k covers [k*T/n, (k+1)*T/n)).
__device__ inline int item_of(int64_t pos, int64_t T, int64_t n) {
  return (int)(((pos + 1) * n + T - 1) / T - 1);
}

// Last segment whose first block is <= pos (segments with no blocks are skipped over,
// because the next one starts at the same position).
__device__ inline int seg_of(const int32_t* seg, int nseg, int64_t pos) {
  int lo = 0, hi = nseg;  // first index with cum > pos
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)seg[(size_t)mid * kSegWords + S_CUM] > pos) hi = mid; else lo = mid + 1;
  }
  return lo - 1;
}

__global__ __launch_bounds__(kThreads) void mla_sched_kernel(
    const int32_t* __restrict__ seqlens, int batch, int s_q, int heads, int causal,
    int max_blocks, int num_wg, int min_split_blocks, int32_t* __restrict__ meta) {
  __shared__ int64_t lds[kThreads];
  __shared__ int status_lds;
  const int tid = threadIdx.x;
  const int groups = (s_q * heads + kGroupRows - 1) / kGroupRows;
  const int nseg = batch * groups;
  int32_t* wg = meta + kHdrWords;
  int32_t* seg = wg + (size_t)kWgWords * num_wg;

  if (tid == 0) status_lds = 0;
  __syncthreads();

  // 1. per segment: validated length and block count
  const int64_t cap = (int64_t)max_blocks * kPage;
  for (int s = tid; s < nseg; s += kThreads) {
    int b = s / groups;
    int L = seqlens[b];
    bool ok = L >= 0 && (int64_t)L <= cap && (!causal || L >= s_q);
    int32_t* r = seg + (size_t)s * kSegWords;
    r[S_NBLK] = ok ? (L + kPage - 1) / kPage : 0;
    r[S_SEQLEN] = ok ? L : -1;
    if (!ok) atomicOr(&status_lds, 1);
  }
  for (int w = tid; w < num_wg; w += kThreads) {
    int32_t* r = wg + (size_t)w * kWgWords;
    r[W_SEG_BEGIN] = -1;
    r[W_BLK_BEGIN] = r[W_SEG_END] = r[W_BLK_END] = r[W_FIRST_SPLIT] = 0;
  }
  __syncthreads();

  // 2. block offset of every segment in the stream
  const int64_t T = block_exclusive_scan(seg, nseg, S_NBLK, S_CUM, false, lds);
  __syncthreads();

  // 3. cut the stream into n items, spread over the slots
  const int64_t minb = min_split_blocks > 0 ? min_split_blocks : kDefaultMinSplitBlocks;
  int64_t n = T / minb;
  if (n < 1) n = 1;
  if (n > num_wg) n = num_wg;
  if (T == 0) n = 0;
  for (int64_t k = tid; k < n; k += kThreads) {
    int64_t begin = k * T / n, end = (k + 1) * T / n;
    int sb = seg_of(seg, nseg, begin), se = seg_of(seg, nseg, end - 1);
    int slot = (int)(k * num_wg / n);
    int32_t* r = wg + (size_t)slot * kWgWords;
    int64_t cb = seg[(size_t)sb * kSegWords + S_CUM];
    r[W_SEG_BEGIN] = sb;
    r[W_BLK_BEGIN] = (int32_t)(begin - cb);
    r[W_SEG_END] = se;
    r[W_BLK_END] = (int32_t)(end - seg[(size_t)se * kSegWords + S_CUM]);
    r[W_FIRST_SPLIT] = (int32_t)(k - item_of(cb, T, n));
  }
  // 4. parts per segment
  for (int s = tid; s < nseg; s += kThreads) {
    int32_t* r = seg + (size_t)s * kSegWords;
    int nb = r[S_NBLK];
    if (nb == 0) {
      r[S_NSPLIT] = 0;
      r[S_FIRST_ITEM] = -1;
    } else {
      int64_t c = r[S_CUM];
      int first = item_of(c, T, n), last = item_of(c + nb - 1, T, n);
      r[S_NSPLIT] = last - first + 1;
      r[S_FIRST_ITEM] = first;
    }
  }
  __syncthreads();

  // 5. partial slots of segments computed in several parts
  const int64_t slots = block_exclusive_scan(seg, nseg, S_NSPLIT, S_SLOT, true, lds);

  if (tid == 0) {
    meta[H_MAGIC] = kMagic;
    meta[H_BATCH] = batch;
    meta[H_SQ] = s_q;
    meta[H_HEADS] = heads;
    meta[H_CAUSAL] = causal;
    meta[H_NUM_WG] = num_wg;
    meta[H_STATUS] = status_lds;
    meta[H_NUM_SEG] = nseg;
    meta[H_NUM_GROUPS] = groups;
    meta[H_TOTAL_BLOCKS] = (int32_t)T;
    meta[H_NUM_ITEMS] = (int32_t)n;
    meta[H_NUM_SLOTS] = (int32_t)slots;
    meta[H_MAX_BLOCKS] = max_blocks;
  }
}

}  // namespace

hipError_t launch_sched(const int32_t* seqlens, int batch, int s_q, int heads, int causal,
                        int max_blocks, int num_wg, int min_split_blocks, int32_t* meta,
                        hipStream_t stream) {
  hipLaunchKernelGGL(mla_sched_kernel, dim3(1), dim3(kThreads), 0, stream, seqlens, batch, s_q,
                     heads, causal, max_blocks, num_wg, min_split_blocks, meta);
  return hipGetLastError();
}

}  // namespace mla
