// MLA decode main kernel for float32 inputs (vector ALU, exact fp32 arithmetic).
//
// Same work partition, output and partial conventions as the bf16 MFMA kernel;
// used where inputs are fp32 and must not be rounded to bf16.  One workgroup
// walks its block range once per 16-row slice of its 128-row group:
//   stage 32 keys (fp32, 576 wide) in LDS -> 16 x 32 scaled scores -> online
//   softmax per row -> O[16 x 512] += P . V with V = the first 512 key columns.
// Rows past a sequence's length are never read (zero-filled in LDS).
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;        // rows per slice
constexpr int kTok = 32;         // keys per LDS tile
constexpr int kLd = kDqk + 1;    // padded LDS row (fp32 words)

__global__ __launch_bounds__(kThreads) void mla_main_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, int64_t num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seqlens,
    int batch, int s_q, int heads, int causal, float scale, float* __restrict__ out,
    float* __restrict__ lse_out, int32_t* __restrict__ meta, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  __shared__ float qs[kRows * kLd];
  __shared__ float ks[kTok * kLd];
  __shared__ float ps[kRows * kTok];
  __shared__ float alpha_s[kRows], m_s[kRows], l_s[kRows];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  const int nwg = gridDim.x;
  int slot = blockIdx.x;
  if ((nwg & 7) == 0) slot = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (meta[H_MAGIC] != kMagic || meta[H_BATCH] != batch || meta[H_SQ] != s_q ||
      meta[H_HEADS] != heads || meta[H_CAUSAL] != causal || meta[H_NUM_WG] != nwg ||
      meta[H_MAX_BLOCKS] != max_blocks) {
    if (tid == 0) atomicOr(&meta[H_STATUS], MLA_STATUS_PLAN_MISMATCH);
    return;
  }
  const int32_t* wrow = meta + kHdrWords + (size_t)slot * kWgWords;
  const int32_t* segt = meta + kHdrWords + (size_t)kWgWords * nwg;
  const int seg_first = wrow[W_SEG_BEGIN];
  if (seg_first < 0) return;
  const int blk_first = wrow[W_BLK_BEGIN];
  const int seg_last = wrow[W_SEG_END];
  const int blk_last_end = wrow[W_BLK_END];
  const int split_first = wrow[W_FIRST_SPLIT];
  const int groups = meta[H_NUM_GROUPS];
  const int M = s_q * heads;
  // ranges read from the plan stay inside this call's tables even if the plan is corrupt
  const int nseg = batch * ((M + kGroupRows - 1) / kGroupRows);
  if (groups != (M + kGroupRows - 1) / kGroupRows || seg_first >= nseg || seg_last < seg_first ||
      seg_last >= nseg || blk_first < 0 || blk_last_end > max_blocks) {
    if (tid == 0) atomicOr(&meta[H_STATUS], MLA_STATUS_PLAN_MISMATCH);
    return;
  }

  for (int seg = seg_first; seg <= seg_last; ++seg) {
    const int32_t* sr = segt + (size_t)seg * kSegWords;
    const int nb = min(max(sr[S_NBLK], 0), max_blocks);
    if (nb == 0) continue;
    const int L = sr[S_SEQLEN];
    const int b = seg / groups;
    const int rg = seg - b * groups;
    const int kb = seg == seg_first ? blk_first : 0;
    const int ke = seg == seg_last ? blk_last_end : nb;
    const bool mismatch = seqlens[b] != L;
    const int rows_in_group = min(kGroupRows, M - rg * kGroupRows);
    const int tok_begin = kb * kPage, tok_end = min(ke * kPage, L);

    for (int r0 = 0; r0 < rows_in_group; r0 += kRows) {
      // Q slice -> LDS (rows past M are zero)
      for (int i = tid; i < kRows * kDqk; i += kThreads) {
        const int r = i / kDqk, d = i - r * kDqk;
        const int row = rg * kGroupRows + r0 + r;
        float v = 0.f;
        if (r0 + r < rows_in_group) {
          const int t = row / heads, hd = row - t * heads;
          v = q[(((size_t)b * s_q + t) * heads + hd) * kDqk + d];
        }
        qs[r * kLd + d] = v;
      }
      if (tid < kRows) { m_s[tid] = -INFINITY; l_s[tid] = 0.f; }
      if (tid == 0) bad_s = 0;
      float acc[kRows][2];
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r][0] = acc[r][1] = 0.f;
      __syncthreads();

      // Keys of a 32-token tile, read into registers one tile ahead (18 float4 per
      // thread, all in flight at once).  A tile starts on a multiple of 32 tokens, so it
      // lies in one block: one block number, then 32 consecutive rows of it, one
      // contiguous run.  Rows at or past the length are zero.
      constexpr int kVec = kTok * kDqk / 4 / kThreads;
      static_assert(kVec * 4 * kThreads == kTok * kDqk, "tile split");
      float4 kreg[kVec];
      auto load_tile = [&](int t0) {
        const int id = block_table[(size_t)b * max_blocks + t0 / kPage];
        const bool ok = id >= 0 && (int64_t)id < num_blocks;
        if (!ok && tid == 0) bad_s = 1;
        const float4* src =
            (const float4*)(kv + ((size_t)(ok ? id : 0) * kPage + (t0 % kPage)) * kDqk);
        const int n_in = ok ? min(kTok, tok_end - t0) * kDqk / 4 : 0;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int i = tid + kThreads * k;
          kreg[k] = i < n_in ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      };
      if (tok_begin < tok_end) load_tile(tok_begin);
      for (int tok0 = tok_begin; tok0 < tok_end; tok0 += kTok) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int i = 4 * (tid + kThreads * k);
          const int j = i / kDqk, d = i - j * kDqk;
          float* dst = ks + j * kLd + d;
          dst[0] = kreg[k].x;
          dst[1] = kreg[k].y;
          dst[2] = kreg[k].z;
          dst[3] = kreg[k].w;
        }
        if (tok0 + kTok < tok_end) load_tile(tok0 + kTok);
        __syncthreads();
        // scores: thread -> key j, rows r and r + 8
        {
          // four independent partial sums per row keep the LDS reads and FMAs pipelined
          const int j = tid & 31, r = tid >> 5;
          float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
          for (int d = 0; d < kDqk; d += 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float kd = ks[j * kLd + d + e];
              a0[e] = fmaf(qs[r * kLd + d + e], kd, a0[e]);
              a1[e] = fmaf(qs[(r + 8) * kLd + d + e], kd, a1[e]);
            }
          }
          const float s0 = (a0[0] + a0[1]) + (a0[2] + a0[3]);
          const float s1 = (a1[0] + a1[1]) + (a1[2] + a1[3]);
          const int tok = tok0 + j;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int rr = r + 8 * u;
            const int row = rg * kGroupRows + r0 + rr;
            const int t = row / heads;
            const int n = causal ? L - s_q + 1 + t : L;
            const float sv = (u ? s1 : s0) * scale;
            ps[rr * kTok + j] = (tok < n && tok < tok_end) ? sv : -INFINITY;
          }
        }
        __syncthreads();
        // online softmax, one thread per row
        if (tid < kRows) {
          const float m_old = m_s[tid];
          float mx = -INFINITY;
          for (int j = 0; j < kTok; ++j) mx = fmaxf(mx, ps[tid * kTok + j]);
          const float m_new = fmaxf(m_old, mx);
          float alpha = 1.f, sum = 0.f;
          if (m_new != -INFINITY) {
            alpha = m_old == -INFINITY ? 0.f : expf(m_old - m_new);
            for (int j = 0; j < kTok; ++j) {
              const float p = expf(ps[tid * kTok + j] - m_new);
              ps[tid * kTok + j] = p;
              sum += p;
            }
          } else {
            for (int j = 0; j < kTok; ++j) ps[tid * kTok + j] = 0.f;
          }
          m_s[tid] = m_new;
          l_s[tid] = l_s[tid] * alpha + sum;
          alpha_s[tid] = alpha;
        }
        __syncthreads();
        // O += P . V, thread -> columns 2*tid, 2*tid+1
        {
          const int c = 2 * tid;
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            const float a = alpha_s[r];
            float o0 = acc[r][0] * a, o1 = acc[r][1] * a;
            for (int j = 0; j < kTok; ++j) {
              const float p = ps[r * kTok + j];
              o0 = fmaf(p, ks[j * kLd + c], o0);
              o1 = fmaf(p, ks[j * kLd + c + 1], o1);
            }
            acc[r][0] = o0;
            acc[r][1] = o1;
          }
        }
        __syncthreads();
      }

      // epilogue
      const int nsplit = sr[S_NSPLIT];
      const bool bad = mismatch || bad_s;
      const int split = seg == seg_first ? split_first : 0;
      const size_t slot_i = (size_t)sr[S_SLOT] + split;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if (r0 + r >= rows_in_group) break;
        const int row_in_group = r0 + r;
        const int row = rg * kGroupRows + row_in_group;
        const int t = row / heads, hd = row - t * heads;
        const float l = l_s[r];
        float o0, o1, lv;
        if (bad) {
          o0 = o1 = lv = __builtin_nanf("");
        } else if (l > 0.f) {
          o0 = acc[r][0] / l;
          o1 = acc[r][1] / l;
          lv = m_s[r] + logf(l);
        } else {
          o0 = o1 = 0.f;
          lv = -INFINITY;
        }
        float* orow;
        float* lrow;
        if (nsplit == 1) {
          const size_t ri = ((size_t)b * s_q + t) * heads + hd;
          orow = out + ri * kDv;
          lrow = lse_out + ri;
        } else {
          orow = part_o + (slot_i * kGroupRows + row_in_group) * kDv;
          lrow = part_lse + slot_i * kGroupRows + row_in_group;
        }
        orow[2 * tid] = o0;
        orow[2 * tid + 1] = o1;
        if (tid == 0) *lrow = lv;
      }
      if (tid == 0 && bad)
        atomicOr(&meta[H_STATUS], (bad_s ? MLA_STATUS_BAD_BLOCK : 0) |
                                      (mismatch ? MLA_STATUS_PLAN_MISMATCH : 0));
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_main_f32(const Problem& p, hipStream_t stream) {
  hipLaunchKernelGGL(mla_main_f32_kernel, dim3(p.num_wg), dim3(kThreads), 0, stream,
                     (const float*)p.q, (const float*)p.kv, p.num_blocks, p.block_table,
                     p.max_blocks, p.seqlens, p.batch, p.s_q, p.heads, p.causal, p.scale, p.out,
                     p.lse, p.meta, p.part_o, p.part_lse);
  return hipGetLastError();
}

}  // namespace mla
