// Latent-cache append: the step that precedes decode attention.
//
// Decode attention reads, for each sequence, the latent rows of every token so far
// (576 values: 512 latent + 64 rope, the shapes of the DeepSeek-MLA example of the
// TileLang talk, section "What is TileLang?").  Before the attention of a decode step,
// the rows of the step's new tokens are written into the sequence's pages: row t of
// sequence b (0 <= t < s_new) goes to logical position p = L_b - s_new + t, where the
// lengths L_b already count the new tokens (the same convention under which the
// causal decode lets query token t see positions up to p), i.e. to
//   kv_cache[block_table[b][p / 64]][p % 64][0:576].
// A row whose position is outside [0, 64 * max_blocks) is skipped with the bad-length
// status bit, one whose block number lies outside the pool with the bad-block bit.
//
// One wave per row: 16-byte loads and stores (bf16: 72 per row, fp32: 144), so a row is
// read and written as whole cache lines.
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kWavesPerBlock) void mla_append_kernel(
    const u32x4* __restrict__ new_kv, u32x4* __restrict__ kv_cache, int64_t num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seqlens,
    int batch, int s_new, int chunks_per_row, int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= (int64_t)batch * s_new) return;
  const int b = (int)(row / s_new), t = (int)(row - (int64_t)b * s_new);
  const int L = seqlens[b];
  const int64_t p = (int64_t)L - s_new + t;
  if (p < 0 || p >= (int64_t)max_blocks * kPage) {
    if (lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_SEQLEN);
    return;
  }
  const int id = block_table[(size_t)b * max_blocks + p / kPage];
  if (id < 0 || (int64_t)id >= num_blocks) {
    if (lane == 0 && status) atomicOr(status, MLA_STATUS_BAD_BLOCK);
    return;
  }
  const u32x4* src = new_kv + row * chunks_per_row;
  u32x4* dst = kv_cache + ((int64_t)id * kPage + p % kPage) * chunks_per_row;
  for (int c = lane; c < chunks_per_row; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_append(const void* new_kv, void* kv_cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                         int batch, int s_new, int elem_bytes, int32_t* status,
                         hipStream_t stream) {
  const int64_t rows = (int64_t)batch * s_new;
  if (rows == 0) return hipSuccess;
  const int chunks = kDqk * elem_bytes / 16;
  const int64_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(mla_append_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, (const u32x4*)new_kv, (u32x4*)kv_cache, num_blocks, block_table,
                     max_blocks, seqlens, batch, s_new, chunks, status);
  return hipGetLastError();
}

}  // namespace mla
