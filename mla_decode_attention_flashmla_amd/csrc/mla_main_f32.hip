// MLA decode main kernel for float32 inputs (fp32 matrix cores, no rounding of inputs).
//
// Same work partition, output and partial conventions as the bf16 MFMA kernel;
// used where inputs are fp32 and must not be rounded to bf16.  One workgroup
// walks its block range once per 16-row slice of its 128-row group:
//   stage 32 keys (fp32, 576 wide) in LDS -> 16 x 32 scaled scores -> online
//   softmax per row -> O[16 x 512] += P . V with V = the first 512 key columns.
// Rows past a sequence's length are never read (zero-filled in LDS).
//
// Both products run on v_mfma_f32_16x16x4f32 (fp32 operands, fp32 accumulation).  For
// a 16 x 16 tile, lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16], and holds
// D[4 (l / 16) + v][l % 16] in its four accumulators.  Scores: wave w sums dims
// 144w .. 144w + 143 (lane group g = l / 16 takes 36 consecutive dims of them), and the
// four partial 16 x 32 score blocks are added through LDS.  P . V: wave w owns output
// columns 128w .. 128w + 127 (8 tiles), lane group g taking keys 8g .. 8g + 7.
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 16;        // rows per slice
constexpr int kTok = 32;         // keys per LDS tile
constexpr int kLd = kDqk + 4;    // padded LDS row (fp32 words): 16-byte rows, rows j and
                                 // j+1 four banks apart for 16-byte reads

// kStrided: q and out rows q_rs / o_rs elements apart; the dense instantiation reads the
// Q slice as one contiguous run and takes the row widths as constants.
template <bool kStrided>
__global__ __launch_bounds__(kThreads) void mla_main_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, int64_t num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seqlens,
    int batch, int s_q, int heads, int causal, float scale, float* __restrict__ out,
    float* __restrict__ lse_out, int32_t* __restrict__ meta, float* __restrict__ part_o,
    float* __restrict__ part_lse, int64_t q_rs_arg, int64_t o_rs_arg) {
  const int64_t q_rs = kStrided ? q_rs_arg : (int64_t)kDqk;
  const int64_t o_rs = kStrided ? o_rs_arg : (int64_t)kDv;
  __shared__ __attribute__((aligned(16))) float qs[kRows * kLd];
  __shared__ __attribute__((aligned(16))) float ks[kTok * kLd];
  __shared__ __attribute__((aligned(16))) float ps[kRows * kTok];   // read as float4
  __shared__ float sp[4][kRows][kTok];   // each wave's partial scores
  __shared__ float alpha_s[kRows], m_s[kRows], l_s[kRows];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;   // MFMA lane: row/column index, k group
  const int nwg = gridDim.x;
  int slot = blockIdx.x;
  if ((nwg & 7) == 0) slot = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  // The header and this slot's row are read together (one round trip): the row lies
  // inside the buffer the host validated for these sizes, and nothing read from it is
  // used before the header check.
  const int32_t* wrow = meta + kHdrWords + (size_t)slot * kWgWords;
  const int32_t* segt = meta + kHdrWords + (size_t)kWgWords * nwg;
  const int h_magic = meta[H_MAGIC], h_batch = meta[H_BATCH], h_sq = meta[H_SQ];
  const int h_heads = meta[H_HEADS], h_causal = meta[H_CAUSAL], h_nwg = meta[H_NUM_WG];
  const int h_maxb = meta[H_MAX_BLOCKS], groups = meta[H_NUM_GROUPS];
  const int seg_first = wrow[W_SEG_BEGIN], blk_first = wrow[W_BLK_BEGIN];
  const int seg_last = wrow[W_SEG_END], blk_last_end = wrow[W_BLK_END];
  const int split_first = wrow[W_FIRST_SPLIT];
  // all of them loaded here, before the first test (kept from being sunk past it)
  asm volatile("" ::"s"(h_magic), "s"(h_batch), "s"(h_sq), "s"(h_heads), "s"(h_causal),
               "s"(h_nwg), "s"(h_maxb), "s"(groups), "s"(seg_first), "s"(blk_first),
               "s"(seg_last), "s"(blk_last_end), "s"(split_first));
  const bool plan_ok = (h_magic == kMagic) & (h_batch == batch) & (h_sq == s_q) &
                       (h_heads == heads) & (h_causal == causal) & (h_nwg == nwg) &
                       (h_maxb == max_blocks);
  if (!plan_ok) {
    if (tid == 0) atomicOr(&meta[H_STATUS], MLA_STATUS_PLAN_MISMATCH);
    return;
  }
  if (seg_first < 0) return;
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
      // Q slice -> LDS (rows past M are zero).  Row (t, h) of sequence b is q row
      // b*M + t*heads + h, q_rs elements after the previous one: dense rows make the
      // slice one contiguous run.
      {
        const float* qsrc = q + ((size_t)b * M + rg * kGroupRows + r0) * q_rs;
        const int n_rows = min(kRows, rows_in_group - r0);
        constexpr int kQVec = kRows * kDqk / 4 / kThreads;
        static_assert(kQVec * 4 * kThreads == kRows * kDqk, "slice split");
        float4 qv[kQVec];
#pragma unroll
        for (int k = 0; k < kQVec; ++k) {
          const int i = tid + kThreads * k;
          if constexpr (kStrided) {
            const int r = i / (kDqk / 4), c = i - r * (kDqk / 4);
            qv[k] = r < n_rows ? *(const float4*)(qsrc + (size_t)r * q_rs + 4 * c)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
          } else {
            qv[k] = i < n_rows * (kDqk / 4) ? ((const float4*)qsrc)[i]
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
        // the first key tile's loads go out before the Q slice is stored, so the two
        // reads overlap (bad_s is cleared by the one thread that sets it, before it can)
        if (tid == 0) bad_s = 0;
        if (tok_begin < tok_end) load_tile(tok_begin);
#pragma unroll
        for (int k = 0; k < kQVec; ++k) {
          const int i = 4 * (tid + kThreads * k);
          const int r = i / kDqk, d = i - r * kDqk;
          *(float4*)(qs + r * kLd + d) = qv[k];
        }
      }
      if (tid < kRows) { m_s[tid] = -INFINITY; l_s[tid] = 0.f; }
      // O[4 lg + v][128 wave + 16 ct + li] of this slice
      floatx4 oacc[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) oacc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();

      for (int tok0 = tok_begin; tok0 < tok_end; tok0 += kTok) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int i = 4 * (tid + kThreads * k);
          const int j = i / kDqk, d = i - j * kDqk;
          *(float4*)(ks + j * kLd + d) = kreg[k];
        }
        if (tok0 + kTok < tok_end) load_tile(tok0 + kTok);
        __syncthreads();
        // this wave's partial scores over dims 144 wave + 36 lg + (0 .. 35): keys li and
        // 16 + li against row li (rows 16 floats apart in LDS are 4 banks apart, so the
        // 16-byte reads of 16 lanes are conflict-free)
        {
          const float* qa = qs + li * kLd + 144 * wave + 36 * lg;
          const float* kb = ks + li * kLd + 144 * wave + 36 * lg;
          floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 9; ++c) {
            const float4 a = *(const float4*)(qa + 4 * c);
            const float4 k0 = *(const float4*)(kb + 4 * c);
            const float4 k1 = *(const float4*)(kb + 16 * kLd + 4 * c);
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, k0.x, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, k1.x, s1, 0, 0, 0);
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, k0.y, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, k1.y, s1, 0, 0, 0);
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, k0.z, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, k1.z, s1, 0, 0, 0);
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, k0.w, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, k1.w, s1, 0, 0, 0);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            sp[wave][4 * lg + v][li] = s0[v];
            sp[wave][4 * lg + v][16 + li] = s1[v];
          }
        }
        __syncthreads();
        // online softmax: thread -> key j, rows r and r + 8, each score the sum of the four
        // waves' parts; a row's 32 keys sit in 32 consecutive lanes of one wave, so its max
        // and sum are shuffle reductions over those lanes
        {
          const int j = tid & 31, r = tid >> 5;
          const int tok = tok0 + j;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int rr = r + 8 * u;
            const int row = rg * kGroupRows + r0 + rr;
            const int t = row / heads;
            const int n = causal ? L - s_q + 1 + t : L;
            const float dot = ((sp[0][rr][j] + sp[1][rr][j]) + sp[2][rr][j]) + sp[3][rr][j];
            const float sv = (tok < n && tok < tok_end) ? dot * scale : -INFINITY;
            float mx = sv;
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
            const float m_old = m_s[rr];
            const float m_new = fmaxf(m_old, mx);
            float alpha = 1.f, p = 0.f;
            if (m_new != -INFINITY) {
              alpha = m_old == -INFINITY ? 0.f : expf(m_old - m_new);
              p = expf(sv - m_new);
            }
            float sum = p;
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 32);
            ps[rr * kTok + j] = p;
            if (j == 0) {
              m_s[rr] = m_new;
              l_s[rr] = l_s[rr] * alpha + sum;
              alpha_s[rr] = alpha;
            }
          }
        }
        __syncthreads();
        // O = alpha O + P . V over this wave's 8 column tiles.  MFMA s of a tile takes keys
        // 16 (s / 4) + 4 lg + s % 4 in lane group lg: P's as two 16-byte reads, and V's
        // rows for the four groups 4 rows (16 banks) apart, so the reads are conflict-free.
        {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = alpha_s[4 * lg + v];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) oacc[ct][v] *= a;
          }
          const float4 pa = *(const float4*)(ps + li * kTok + 4 * lg);
          const float4 pb = *(const float4*)(ps + li * kTok + 16 + 4 * lg);
          const float pk[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
          const float* vb = ks + (4 * lg) * kLd + 128 * wave + li;
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8)
              oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  pk[s8], vb[(16 * (s8 >> 2) + (s8 & 3)) * kLd + 16 * ct], oacc[ct], 0, 0, 0);
        }
        __syncthreads();
      }

      // epilogue: lane (li, lg) of wave w writes rows 4 lg + v, columns 128 w + 16 ct + li
      const int nsplit = sr[S_NSPLIT];
      const bool bad = mismatch || bad_s;
      const int split = seg == seg_first ? split_first : 0;
      const size_t slot_i = (size_t)sr[S_SLOT] + split;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * lg + v;
        if (r0 + r >= rows_in_group) continue;
        const int row_in_group = r0 + r;
        const int row = rg * kGroupRows + row_in_group;
        const int t = row / heads, hd = row - t * heads;
        const float l = l_s[r];
        float lv;
        if (bad) lv = __builtin_nanf("");
        else if (l > 0.f) lv = m_s[r] + logf(l);
        else lv = -INFINITY;
        float* orow;
        float* lrow;
        if (nsplit == 1) {
          const size_t ri = ((size_t)b * s_q + t) * heads + hd;
          orow = out + ri * o_rs;
          lrow = lse_out + ri;
        } else {
          orow = part_o + (slot_i * kGroupRows + row_in_group) * kDv;
          lrow = part_lse + slot_i * kGroupRows + row_in_group;
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          float o;
          if (bad) o = __builtin_nanf("");
          else if (l > 0.f) o = oacc[ct][v] / l;
          else o = 0.f;
          orow[128 * wave + 16 * ct + li] = o;
        }
        if (wave == 0 && li == 0) *lrow = lv;
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
  if (p.q_rs != kDqk || p.o_rs != kDv)
    hipLaunchKernelGGL(mla_main_f32_kernel<true>, dim3(p.num_wg), dim3(kThreads), 0, stream,
                       (const float*)p.q, (const float*)p.kv, p.num_blocks, p.block_table,
                       p.max_blocks, p.seqlens, p.batch, p.s_q, p.heads, p.causal, p.scale,
                       p.out, p.lse, p.meta, p.part_o, p.part_lse, p.q_rs, p.o_rs);
  else
    hipLaunchKernelGGL(mla_main_f32_kernel<false>, dim3(p.num_wg), dim3(kThreads), 0, stream,
                       (const float*)p.q, (const float*)p.kv, p.num_blocks, p.block_table,
                       p.max_blocks, p.seqlens, p.batch, p.s_q, p.heads, p.causal, p.scale,
                       p.out, p.lse, p.meta, p.part_o, p.part_lse, p.q_rs, p.o_rs);
  return hipGetLastError();
}

}  // namespace mla
