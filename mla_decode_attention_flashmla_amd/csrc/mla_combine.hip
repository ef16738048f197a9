// Log-sum-exp combine of split parts.
//
// A segment (sequence, 128-row group) whose blocks were spread over several
// workgroups left one partial (O_i normalised over its own keys, LSE_i) per
// part.  Over the union of the parts' keys:
//   LSE = M + ln sum_i exp(LSE_i - M),  M = max_i LSE_i
//   O   = sum_i exp(LSE_i - LSE) * O_i
// Parts with no visible key (LSE_i = -inf) carry weight 0.  Segments with no
// part at all (length 0, or an invalid length) are written here too: O = 0 and
// LSE = -inf, or NaN for invalid lengths.  Long contexts (the 128K sparse-MLA
// case of the Triton-TLE talk's performance section) are what make splitting,
// and so this merge, necessary when few sequences must fill all compute units.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRowsPerBlock = 4;  // 64 threads per row, 8 columns per thread
constexpr int kThreads = 64 * kRowsPerBlock;
constexpr int kMaxSplitsLds = 1024;

// kHalf: the partial O values are fp16 under a power-of-two scale per (part, row),
// folded here into the part's weight; otherwise fp32.
template <bool kHalf>
__global__ __launch_bounds__(kThreads) void mla_combine_kernel(
    int batch, int s_q, int heads, int causal, int max_blocks, int nwg, float* __restrict__ out,
    float* __restrict__ lse_out,
    const int32_t* __restrict__ meta, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, const float* __restrict__ part_scale, int64_t o_rs) {
  __shared__ float w_s[kRowsPerBlock][kMaxSplitsLds];
  __shared__ float lse_s[kRowsPerBlock];
  // parts whose O loads are in flight together: one round trip merges a row of up to 16
  // fp16 parts (the 128-row groups of a 16-sequence batch) where 4 at a time took four
  constexpr int kBatch = kHalf ? 16 : 8;
  const int seg = blockIdx.x;
  // The header words and this segment's row are all read before any of them is tested,
  // so they arrive in one round trip: the row lies inside the buffer the host validated
  // for these sizes, and nothing read from it is used before the header check.
  const int32_t* sr = meta + kHdrWords + (size_t)kWgWords * nwg + (size_t)seg * kSegWords;
  const int h_magic = meta[H_MAGIC], h_batch = meta[H_BATCH], h_sq = meta[H_SQ];
  const int h_heads = meta[H_HEADS], h_nwg = meta[H_NUM_WG], h_groups = meta[H_NUM_GROUPS];
  const int h_causal = meta[H_CAUSAL], h_maxb = meta[H_MAX_BLOCKS];
  const int nsplit = sr[S_NSPLIT], s_len = sr[S_SEQLEN], s_slot = sr[S_SLOT];
  // all of them loaded here, before the first test (kept from being sunk past it)
  asm volatile("" ::"s"(h_magic), "s"(h_batch), "s"(h_sq), "s"(h_heads), "s"(h_nwg),
               "s"(h_groups), "s"(h_causal), "s"(h_maxb), "s"(nsplit), "s"(s_len),
               "s"(s_slot));
  // the row this thread writes, from the call's own sizes (the grid covers every row)
  const int M = s_q * heads;
  const int groups = (M + kGroupRows - 1) / kGroupRows;
  const int b = seg / groups, rg = seg - b * groups;
  const int rows_in_group = min(kGroupRows, M - rg * kGroupRows);
  const int rl = threadIdx.x >> 6;            // row within this block
  const int lane = threadIdx.x & 63;
  const int row_in_group = blockIdx.y * kRowsPerBlock + rl;
  const bool row_ok = row_in_group < rows_in_group;
  const int row = rg * kGroupRows + row_in_group;
  const int t = row / heads, hd = row - t * heads;
  const size_t ri = ((size_t)b * s_q + t) * heads + hd;
  // A plan made for another call (other sizes, causal flag or table width) was flagged
  // by the main kernel, which then wrote nothing: every row of the output becomes NaN,
  // whether its segment was split or not.
  const bool plan_ok = (h_magic == kMagic) & (h_batch == batch) & (h_sq == s_q) &
                       (h_heads == heads) & (h_nwg == nwg) & (h_groups == groups) &
                       (h_causal == causal) & (h_maxb == max_blocks);
  if (!plan_ok) {
    if (!row_ok) return;
    const float nan = __builtin_nanf("");
    float4* o = (float4*)(out + ri * o_rs) + 2 * lane;
    o[0] = make_float4(nan, nan, nan, nan);
    o[1] = make_float4(nan, nan, nan, nan);
    if (lane == 0) lse_out[ri] = nan;
    return;
  }
  if (nsplit == 1) return;

  if (nsplit == 0) {
    if (!row_ok) return;
    const float fill = s_len < 0 ? __builtin_nanf("") : 0.f;
    float4 v = make_float4(fill, fill, fill, fill);
    float4* o = (float4*)(out + ri * o_rs) + 2 * lane;
    o[0] = v;
    o[1] = v;
    if (lane == 0) lse_out[ri] = s_len < 0 ? __builtin_nanf("") : -INFINITY;
    return;
  }

  const size_t slot0 = (size_t)s_slot;
  // the parts must lie inside the workspace sized for this call (nwg + segments slots)
  if (s_slot < 0 || slot0 + (size_t)nsplit > (size_t)nwg + (size_t)gridDim.x) return;
  // this thread's 8 columns of part j's row: 32 bytes of fp32 or 16 bytes of fp16
  const size_t pstride = (size_t)kGroupRows * kDv;  // elements from one part's row to the next's
  const size_t pbase = (slot0 * kGroupRows + row_in_group) * kDv + 8 * lane;
  // fp16 parts stay packed (4 registers each) until they are added
  uint4 raw[kHalf ? kBatch : 1];
  float4 pa[kHalf ? 1 : kBatch], pc[kHalf ? 1 : kBatch];
  auto load_part = [&](int jslot, int i) {
    if constexpr (kHalf) {
      raw[jslot] = *(const uint4*)((const _Float16*)part_o + pbase + i * pstride);
    } else {
      pa[jslot] = *(const float4*)(part_o + pbase + i * pstride);
      pc[jslot] = *(const float4*)(part_o + pbase + i * pstride + 4);
    }
  };
  // The first kBatch parts' O values are requested before the weights are known, so
  // their latency overlaps the LSE reads (every load below is independent).
  if (row_ok) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (j < nsplit) load_part(j, j);
  }

  // weights exp(LSE_i - LSE) for this row, computed by its 64 threads; lane i keeps part
  // i's LSE and scale from the max pass for the sum pass (parts past 64 are read again)
  float mx = -INFINITY;
  bool nan = false;
  float l0 = -INFINITY, sc0 = 1.f;
  if (row_ok && lane < nsplit) {
    l0 = part_lse[(slot0 + lane) * kGroupRows + row_in_group];
    if constexpr (kHalf) sc0 = part_scale[(slot0 + lane) * kGroupRows + row_in_group];
    nan = __builtin_isnan(l0);
    mx = fmaxf(mx, l0);
  }
  if (row_ok)
    for (int i = lane + 64; i < nsplit; i += 64) {
      const float l = part_lse[(slot0 + i) * kGroupRows + row_in_group];
      nan = nan || __builtin_isnan(l);
      mx = fmaxf(mx, l);
    }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  // one row is one wave: any lane that read a NaN part flags the row
  nan = __builtin_amdgcn_ballot_w64(nan) != 0;
  const float base = mx == -INFINITY ? 0.f : mx;
  float sum = 0.f;
  if (row_ok && lane < nsplit) {
    const float w = l0 == -INFINITY ? 0.f : expf(l0 - base);
    w_s[rl][lane] = w * sc0;
    sum = w;
  }
  if (row_ok)
    for (int i = lane + 64; i < nsplit; i += 64) {
      const float l = part_lse[(slot0 + i) * kGroupRows + row_in_group];
      const float w = l == -INFINITY ? 0.f : expf(l - base);
      const float sc = kHalf ? part_scale[(slot0 + i) * kGroupRows + row_in_group] : 1.f;
      if (i < kMaxSplitsLds) w_s[rl][i] = w * sc;
      sum += w;
    }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  // a part flagged bad (NaN) makes the whole row NaN, O and LSE alike
  const float inv = nan ? __builtin_nanf("") : (sum > 0.f ? 1.f / sum : 0.f);
  if (lane == 0)
    lse_s[rl] = nan ? __builtin_nanf("") : (sum > 0.f ? base + logf(sum) : -INFINITY);
  __syncthreads();
  if (!row_ok) return;

  // weight of part i's stored values: exp(LSE_i - M), times its scale for fp16 partials
  auto weight = [&](int i) {
    if (i < kMaxSplitsLds) return w_s[rl][i];
    const float l = part_lse[(slot0 + i) * kGroupRows + row_in_group];
    const float sc = kHalf ? part_scale[(slot0 + i) * kGroupRows + row_in_group] : 1.f;
    return l == -INFINITY ? 0.f : expf(l - base) * sc;
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add4 = [&](float w, const float4& a, const float4& c) {
    acc[0] = fmaf(w, a.x, acc[0]);
    acc[1] = fmaf(w, a.y, acc[1]);
    acc[2] = fmaf(w, a.z, acc[2]);
    acc[3] = fmaf(w, a.w, acc[3]);
    acc[4] = fmaf(w, c.x, acc[4]);
    acc[5] = fmaf(w, c.y, acc[5]);
    acc[6] = fmaf(w, c.z, acc[6]);
    acc[7] = fmaf(w, c.w, acc[7]);
  };
  auto add = [&](float w, int jslot) {
    if constexpr (kHalf) {
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      const uint4 r = raw[jslot];
      const f16x2 a = __builtin_bit_cast(f16x2, r.x), b2 = __builtin_bit_cast(f16x2, r.y);
      const f16x2 c = __builtin_bit_cast(f16x2, r.z), d = __builtin_bit_cast(f16x2, r.w);
      add4(w, make_float4((float)a[0], (float)a[1], (float)b2[0], (float)b2[1]),
           make_float4((float)c[0], (float)c[1], (float)d[0], (float)d[1]));
    } else {
      add4(w, pa[jslot], pc[jslot]);
    }
  };
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (j < nsplit) add(weight(j), j);
  // further parts, kBatch at a time with all their loads issued first
  for (int i0 = kBatch; i0 < nsplit; i0 += kBatch) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (i0 + j < nsplit) load_part(j, i0 + j);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (i0 + j < nsplit) add(weight(i0 + j), j);
  }
  float4* o = (float4*)(out + ri * o_rs) + 2 * lane;
  o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (lane == 0) lse_out[ri] = lse_s[rl];
}

}  // namespace

hipError_t launch_combine(const Problem& p, hipStream_t stream) {
  const int groups = num_groups(p.s_q, p.heads);
  const int nseg = p.batch * groups;
  if (nseg == 0) return hipSuccess;
  dim3 grid(nseg, kGroupRows / kRowsPerBlock);
  if (p.part_half)
    hipLaunchKernelGGL(mla_combine_kernel<true>, grid, dim3(kThreads), 0, stream, p.batch, p.s_q,
                       p.heads, p.causal, p.max_blocks, p.num_wg, p.out, p.lse, p.meta,
                       p.part_o, p.part_lse, p.part_scale, p.o_rs);
  else
    hipLaunchKernelGGL(mla_combine_kernel<false>, grid, dim3(kThreads), 0, stream, p.batch,
                       p.s_q, p.heads, p.causal, p.max_blocks, p.num_wg, p.out, p.lse, p.meta,
                       p.part_o, p.part_lse, p.part_scale, p.o_rs);
  return hipGetLastError();
}

}  // namespace mla
