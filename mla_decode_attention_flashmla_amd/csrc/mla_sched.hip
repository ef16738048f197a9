// Split-KV tile scheduler: one workgroup turns seqlens into the work partition.
//
// The decode step's work is a stream of 64-token KV blocks, segment after
// segment, where a segment is one (sequence, 128-row group) pair.  The stream
// is cut into near-equal contiguous ranges, one per persistent workgroup of
// the main kernel; a segment cut by a range boundary is computed in parts
// whose results are merged by log-sum-exp (the "tile configuration" the
// DeepSeek MLA example of the TileLang talk leaves to its author: how many
// blocks, and which work each one takes).
//
// By default the plan is segment-aligned when that is cheap: every segment gets
// ceil(nb / c) whole items of at most c blocks, with c the smallest item size for which
// the items fit one per workgroup, so no workgroup's range crosses a segment boundary.
// A range that crosses one costs its workgroup a second part (another Q load at its
// share of the memory bandwidth, another partial written), ~kPartCostBlocks blocks of
// work; so the aligned plan is taken when c exceeds the stream cut's ceil(T / slots) by
// at most that much.  Otherwise, or with a caller-given min_split_blocks, the stream is
// cut into near-equal ranges regardless of segment boundaries.
//
// Up to 64 segments, wave 0 plans them alone (lane s owns segment s) with wave-level
// scans and no workgroup barrier, then all waves write the work table.  Otherwise
// per-segment arrays live in LDS when they fit (up to kLdsSegs segments), larger
// batches keeping them in the metadata buffer itself, and prefix sums are thread-local
// runs plus one wave-shuffle scan of the 256 run totals.  Both paths compute the same
// plan.
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsSegs = 4096;
// Measured cost of one more part in a workgroup's range (Q load and partial write),
// in 64-token blocks of work.
constexpr int kPartCostBlocks = 4;

// Exclusive prefix sum over the block of one value per thread; returns the total.
__device__ int64_t block_scan_exclusive(int64_t v, int64_t& total, int64_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += wave_tot[w];
    all += wave_tot[w];
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// floor(a / b) for 0 <= a < 2^53, b > 0, through one correctly rounded fp64 division:
// the quotient's rounding error, at most a * 2^-53 / b, is below the 1 / b gap between
// a non-integer quotient and the next integer, so the floor is exact (and a 64-bit
// integer division is a long serial instruction sequence on this GPU).
__device__ inline int64_t floordiv(int64_t a, int64_t b) {
  return (int64_t)__builtin_floor((double)a / (double)b);
}

// Work item holding stream position pos when T blocks are cut into n items
// (item k covers [k*T/n, (k+1)*T/n)).  pos < T < 2^31, n <= 65535: every operand of the
// divisions stays below 2^47.
__device__ inline int item_of(int64_t pos, int64_t T, int64_t n) {
  return (int)(floordiv((pos + 1) * n + T - 1, T) - 1);
}

template <class Arr>
__device__ inline int seg_of(const Arr& cum, int nseg, int64_t pos) {
  // last segment whose first block is <= pos (segments with no blocks share the next
  // one's offset, so the last such index always has blocks)
  int lo = 0, hi = nseg;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cum(mid) > pos) hi = mid; else lo = mid + 1;
  }
  return lo - 1;
}

// Exclusive prefix sum over one wave; *total receives the wave's sum.
__device__ inline int64_t wave_scan_exclusive(int64_t v, int64_t* total) {
  const int lane = threadIdx.x & 63;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

__device__ inline int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Segments of at most one wave: lane s < nseg owns segment s.
constexpr int kWaveSegs = 64;

__global__ __launch_bounds__(kThreads) void mla_sched_kernel(
    const int32_t* __restrict__ seqlens, int batch, int s_q, int heads, int causal,
    int max_blocks, int num_wg, int min_split_blocks, int32_t* __restrict__ meta) {
  __shared__ int32_t l_nblk[kLdsSegs], l_cum[kLdsSegs], l_item[kLdsSegs], l_len[kLdsSegs];
  __shared__ int64_t wave_tot[kThreads / 64];
  __shared__ int status_lds;
  const int tid = threadIdx.x;
  const int groups = (s_q * heads + kGroupRows - 1) / kGroupRows;
  const int nseg = batch * groups;
  const bool in_lds = nseg <= kLdsSegs;
  int32_t* wg = meta + kHdrWords;
  int32_t* seg = wg + (size_t)kWgWords * num_wg;
  auto NB = [&](int s) -> int32_t& { return in_lds ? l_nblk[s] : seg[(size_t)s * kSegWords + S_NBLK]; };
  auto CUM = [&](int s) -> int32_t& { return in_lds ? l_cum[s] : seg[(size_t)s * kSegWords + S_CUM]; };
  // first item of a segment (segment-aligned plans), defined for every segment: an empty
  // one holds the next segment's, so the column never decreases.  Outside LDS it has a
  // word of its own: S_FIRST_ITEM is rewritten with -1 for empty segments in step 6,
  // while step 7 still searches this column.
  auto ITEM = [&](int s) -> int32_t& {
    return in_lds ? l_item[s] : seg[(size_t)s * kSegWords + S_AL_ITEM];
  };

  __shared__ int64_t sh_plan[4];  // T, n, c_al, slots when one wave plans the segments
  if (tid == 0) status_lds = 0;
  __syncthreads();

  const int64_t cap = (int64_t)max_blocks * kPage;
  int64_t T = 0, n = 0, c_al = 0, slots = 0;
  // parts of segment s and its first item, for block counts nb and first block c
  // (aligned plans: its first item `item`)
  auto parts_for = [&](int nb, int64_t c, int item, int& first) -> int {
    if (!nb || n == 0) {
      first = -1;
      return 0;
    }
    if (c_al > 0) {
      first = item;
      return (int)floordiv(nb + c_al - 1, c_al);
    }
    first = item_of(c, T, n);
    return item_of(c + nb - 1, T, n) - first + 1;
  };

  if (nseg <= kWaveSegs) {
    // Few segments: wave 0 plans them alone (lane s owns segment s), with wave-level
    // scans and no workgroup barrier; the same steps as the general path below.
    if (tid < 64) {
      const int sg = tid;
      const bool has = sg < nseg;
      int nb = 0;
      bool bad = false;
      if (has) {
        const int b = sg / groups;
        const int L = seqlens[b];
        const bool ok = L >= 0 && (int64_t)L <= cap && (!causal || L >= s_q);
        nb = ok ? (L + kPage - 1) / kPage : 0;
        l_nblk[sg] = nb;
        l_len[sg] = ok ? L : -1;
        int32_t* r = seg + (size_t)sg * kSegWords;
        r[S_NBLK] = nb;
        r[S_SEQLEN] = ok ? L : -1;
        bad = !ok;
      }
      const int64_t cum = wave_scan_exclusive(nb, &T);
      if (has) {
        l_cum[sg] = (int32_t)cum;
        seg[(size_t)sg * kSegWords + S_CUM] = (int32_t)cum;
      }
      const int64_t c_min = T > 0 ? floordiv(T + num_wg - 1, num_wg) : 1;
      if (min_split_blocks == 0 && T > 0 && T <= 0x7fffffffLL) {
        auto items_for = [&](int64_t c) { return wave_sum(has ? floordiv(nb + c - 1, c) : 0); };
        if (items_for(c_min) <= num_wg) {
          c_al = c_min;
        } else {
          const int64_t nonempty = wave_sum(has && nb > 0 ? 1 : 0);
          if (nonempty < num_wg) {
            int64_t lo = c_min, hi = floordiv(T + (num_wg - nonempty) - 1, num_wg - nonempty);
            if (hi > c_min + kPartCostBlocks) hi = c_min + kPartCostBlocks + 1;
            while (lo < hi) {
              const int64_t mid = (lo + hi) >> 1;
              if (items_for(mid) <= num_wg) hi = mid; else lo = mid + 1;
            }
            if (lo <= c_min + kPartCostBlocks && items_for(lo) <= num_wg) c_al = lo;
          }
        }
      }
      int item = 0;
      if (c_al > 0) {
        item = (int)wave_scan_exclusive(has ? floordiv(nb + c_al - 1, c_al) : 0, &n);
        if (has) l_item[sg] = item;
      } else {
        n = min_split_blocks > 0 ? floordiv(T, min_split_blocks)
                                 : (c_min > 0 ? floordiv(T + c_min - 1, c_min) : 1);
        if (n > T) n = T;
        if (n < 1) n = 1;
        if (n > num_wg) n = num_wg;
      }
      if (T == 0 || T > 0x7fffffffLL) n = 0;
      int first = -1;
      const int ns = has ? parts_for(nb, cum, item, first) : 0;
      const int64_t slot = wave_scan_exclusive(ns > 1 ? ns : 0, &slots);
      if (has) {
        int32_t* r = seg + (size_t)sg * kSegWords;
        r[S_NSPLIT] = ns;
        r[S_FIRST_ITEM] = first;
        r[S_SLOT] = (int32_t)slot;
      }
      const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
      if (tid == 0) {
        if (any_bad || T > 0x7fffffffLL) status_lds |= MLA_STATUS_BAD_SEQLEN;
        sh_plan[0] = T;
        sh_plan[1] = n;
        sh_plan[2] = c_al;
        sh_plan[3] = slots;
      }
    }
    __syncthreads();
    T = sh_plan[0];
    n = sh_plan[1];
    c_al = sh_plan[2];
    slots = sh_plan[3];
  } else {
    // 1. validated length and block count of every segment
    for (int s = tid; s < nseg; s += kThreads) {
      const int b = s / groups;
      const int L = seqlens[b];
      const bool ok = L >= 0 && (int64_t)L <= cap && (!causal || L >= s_q);
      const int nb = ok ? (L + kPage - 1) / kPage : 0;
      NB(s) = nb;
      if (in_lds) l_len[s] = ok ? L : -1;
      int32_t* r = seg + (size_t)s * kSegWords;
      r[S_NBLK] = nb;
      r[S_SEQLEN] = ok ? L : -1;
      if (!ok) atomicOr(&status_lds, MLA_STATUS_BAD_SEQLEN);
    }
    __syncthreads();

    // 2. block offset of every segment in the stream (thread-local runs + block scan)
    const int per = (nseg + kThreads - 1) / kThreads;
    const int r0 = min(nseg, tid * per), r1 = min(nseg, r0 + per);
    int64_t run = 0;
    for (int s = r0; s < r1; ++s) run += NB(s);
    int64_t acc = block_scan_exclusive(run, T, wave_tot);
    for (int s = r0; s < r1; ++s) {
      const int nb = NB(s);
      CUM(s) = (int32_t)acc;
      seg[(size_t)s * kSegWords + S_CUM] = (int32_t)acc;
      acc += nb;
    }
    __syncthreads();

    // 3. the item size of a segment-aligned plan, if one is taken (see the top of the file)
    const int64_t c_min = T > 0 ? floordiv(T + num_wg - 1, num_wg) : 1;
    if (min_split_blocks == 0 && T > 0 && T <= 0x7fffffffLL) {
      // items of at most c blocks, one per workgroup: sum over segments of ceil(nb / c)
      auto items_for = [&](int64_t c) {
        int64_t v = 0;
        for (int s = r0; s < r1; ++s) v += floordiv(NB(s) + c - 1, c);
        int64_t tot;
        block_scan_exclusive(v, tot, wave_tot);
        return tot;
      };
      if (items_for(c_min) <= num_wg) {
        c_al = c_min;
      } else {
        int64_t ne_run = 0;
        for (int s = r0; s < r1; ++s) ne_run += NB(s) > 0 ? 1 : 0;
        int64_t nonempty;
        block_scan_exclusive(ne_run, nonempty, wave_tot);
        if (nonempty < num_wg) {
          // sum ceil(nb / c) <= T / c + nonempty, so c = ceil(T / (slots - nonempty)) fits;
          // search [c_min, that] for the smallest size that fits
          int64_t lo = c_min, hi = floordiv(T + (num_wg - nonempty) - 1, num_wg - nonempty);
          if (hi > c_min + kPartCostBlocks) hi = c_min + kPartCostBlocks + 1;
          while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (items_for(mid) <= num_wg) hi = mid; else lo = mid + 1;
          }
          if (lo <= c_min + kPartCostBlocks && items_for(lo) <= num_wg) c_al = lo;
        }
      }
    }

    // 4. the items and their count n.  Aligned: segment s holds items [ITEM(s),
    // ITEM(s) + parts), its blocks split near-evenly among them.  Stream cut: n near-equal
    // ranges; by default the fewest items whose largest one is as short as with one item
    // per slot, n = ceil(T / c_min) (each part costs a partial result written and read
    // back); a caller-given min_split_blocks sets n = T / min_split_blocks instead.  Either
    // way 1 <= n <= min(T, slots).
    if (c_al > 0) {
      int64_t v = 0;
      for (int s = r0; s < r1; ++s) v += floordiv(NB(s) + c_al - 1, c_al);
      int64_t a0 = block_scan_exclusive(v, n, wave_tot);
      for (int s = r0; s < r1; ++s) {
        ITEM(s) = (int32_t)a0;
        a0 += floordiv(NB(s) + c_al - 1, c_al);
      }
      __syncthreads();
    } else {
      if (min_split_blocks > 0) {
        n = floordiv(T, min_split_blocks);
      } else {
        n = c_min > 0 ? floordiv(T + c_min - 1, c_min) : 1;
      }
      if (n > T) n = T;
      if (n < 1) n = 1;
      if (n > num_wg) n = num_wg;
    }
    // the plan stores block offsets in 32 bits: a longer stream gets no work and a status bit
    if (T == 0 || T > 0x7fffffffLL) n = 0;
    if (T > 0x7fffffffLL && tid == 0) atomicOr(&status_lds, MLA_STATUS_BAD_SEQLEN);

    // 5. parts per segment, 6. partial slots of segments computed in several parts
    run = 0;
    for (int s = r0; s < r1; ++s) {
      int first;
      const int ns = parts_for(NB(s), CUM(s), c_al > 0 ? ITEM(s) : 0, first);
      if (ns > 1) run += ns;
    }
    acc = block_scan_exclusive(run, slots, wave_tot);
    for (int s = r0; s < r1; ++s) {
      int32_t* r = seg + (size_t)s * kSegWords;
      int first;
      const int ns = parts_for(NB(s), CUM(s), c_al > 0 ? ITEM(s) : 0, first);
      r[S_NSPLIT] = ns;
      r[S_FIRST_ITEM] = first;
      r[S_SLOT] = (int32_t)acc;
      if (ns > 1) acc += ns;
    }
    __syncthreads();
  }

  // 7. one work-table row per workgroup slot
  const bool aligned = c_al > 0;
  // parts of segment s in an aligned plan
  auto parts_al = [&](int s) -> int { return (int)floordiv(NB(s) + c_al - 1, c_al); };
  auto cum_at = [&](int s) { return CUM(s); };
  auto item_at = [&](int s) { return ITEM(s); };
  // validated length of segment s: from LDS when the segment arrays live there (a read
  // of the row this kernel just wrote would wait a global round trip)
  auto len_of = [&](int s) -> int32_t {
    return in_lds ? l_len[s] : seg[(size_t)s * kSegWords + S_SEQLEN];
  };
  for (int w = tid; w < num_wg; w += kThreads) {
    int32_t* r = wg + (size_t)w * kWgWords;
    // slot w holds item k iff k*num_wg/n == w for some k
    int k = -1;
    if (n > 0) {
      const int64_t kk = floordiv((int64_t)w * n + num_wg - 1, num_wg);  // smallest k with k*W/n >= w
      if (kk < n && floordiv(kk * num_wg, n) == w) k = (int)kk;
    }
    if (k < 0) {
      r[W_SEG_BEGIN] = -1;
      r[W_BLK_BEGIN] = r[W_SEG_END] = r[W_BLK_END] = r[W_FIRST_SPLIT] = 0;
      r[W_NBLK0] = r[W_SEQLEN0] = 0;
      continue;
    }
    if (aligned) {
      // the segment holding item k (segments without blocks share the next one's first
      // item, so the last segment whose first item is <= k has blocks)
      const int sb = seg_of(item_at, nseg, k);
      const int j = k - ITEM(sb);
      const int64_t nb = NB(sb), ps = parts_al(sb);
      r[W_SEG_BEGIN] = sb;
      r[W_BLK_BEGIN] = (int32_t)floordiv((int64_t)j * nb, ps);
      r[W_SEG_END] = sb;
      r[W_BLK_END] = (int32_t)floordiv((int64_t)(j + 1) * nb, ps);
      r[W_FIRST_SPLIT] = j;
      r[W_NBLK0] = (int32_t)nb;
      r[W_SEQLEN0] = len_of(sb);
      continue;
    }
    const int64_t begin = floordiv((int64_t)k * T, n), end = floordiv((int64_t)(k + 1) * T, n);
    const int sb = seg_of(cum_at, nseg, begin), se = seg_of(cum_at, nseg, end - 1);
    const int64_t cb = CUM(sb);
    r[W_SEG_BEGIN] = sb;
    r[W_BLK_BEGIN] = (int32_t)(begin - cb);
    r[W_SEG_END] = se;
    r[W_BLK_END] = (int32_t)(end - CUM(se));
    r[W_FIRST_SPLIT] = (int32_t)(k - item_of(cb, T, n));
    r[W_NBLK0] = NB(sb);
    r[W_SEQLEN0] = len_of(sb);
  }

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
    meta[H_ALIGNED] = aligned ? (int32_t)c_al : 0;
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
