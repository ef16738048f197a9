// Quantized latent cache, first form: dequantize the blocks a batch reads, then decode.
//
// The quantized cache keeps one 656-byte row per token: the 512 latent values as fp8
// e4m3 codes (OCP 8-bit float: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities; exponent and mantissa all ones is NaN), the 64 rope values as bf16, the
// row's fp32 scale at byte 640 and 12 bytes of padding.  A latent value is
// code_value * scale.  (The pages name dequantization and mixed precision as compiler
// concerns, the TileLang talk's "Why a new DSL?" and "What is TileLang?" sections; the
// row format is this library's own.)
//
// mla_fp8_dequant_kernel: one workgroup per (sequence, block of its length) turns the
// block's 64 rows into bf16 rows of 576 in a workspace pool (value * scale rounded to
// nearest even) and writes the packed block table; a block number outside the pool
// gives table entry -1, which the main kernel reports (status bit, NaN for that
// sequence).  The paged decode then runs on the workspace pool unchanged.
#include "mla_internal.h"
#include "mla_decode.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 656;
constexpr int kRopeOff = 512;
constexpr int kScaleOff = 640;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  float mag = ex == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)ex - 7);
  if (ex == 15u && m == 7u) mag = __builtin_nanf("");
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads) void mla_fp8_dequant_kernel(
    const uint8_t* __restrict__ kv8, int64_t num_blocks, const int32_t* __restrict__ block_table,
    int max_blocks, const int32_t* __restrict__ seqlens, uint16_t* __restrict__ pool,
    int32_t* __restrict__ packed_table) {
  const int k = blockIdx.x, b = blockIdx.y;
  const int L = seqlens[b];
  const int64_t cap = (int64_t)max_blocks * kPage;
  if (L <= 0 || (int64_t)L > cap || (int64_t)k * kPage >= L) return;  // block not read
  const size_t slot = (size_t)b * max_blocks + k;
  const int id = block_table[(size_t)b * max_blocks + k];
  if (id < 0 || (int64_t)id >= num_blocks) {
    if (threadIdx.x == 0) packed_table[slot] = -1;
    return;
  }
  if (threadIdx.x == 0) packed_table[slot] = (int32_t)slot;
  const uint8_t* src = kv8 + (size_t)id * kPage * kRowBytes;
  uint16_t* dst = pool + slot * kPage * kDqk;
  const int lane = threadIdx.x & 63, rsub = threadIdx.x >> 6;
  for (int r = rsub; r < kPage; r += kThreads / 64) {
    const uint8_t* row = src + (size_t)r * kRowBytes;
    const float sc = *(const float*)(row + kScaleOff);
    // latent: 8 codes per lane -> 8 bf16 (16 bytes)
    const u32x2 c = *(const u32x2*)(row + 8 * lane);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = e4m3_value((c[0] >> (8 * i)) & 0xFFu) * sc;
      v[4 + i] = e4m3_value((c[1] >> (8 * i)) & 0xFFu) * sc;
    }
    const u32x4 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                     pack_bf16(v[6], v[7])};
    *(u32x4*)(dst + (size_t)r * kDqk + 8 * lane) = o;
    // rope: 128 bytes copied by 8 lanes
    if (lane < 8)
      *(u32x4*)(dst + (size_t)r * kDqk + 512 + 8 * lane) =
          *(const u32x4*)(row + kRopeOff + 16 * lane);
  }
}

}  // namespace

hipError_t launch_fp8_dequant(const void* kv8, int64_t num_blocks, const int32_t* block_table,
                              int max_blocks, const int32_t* seqlens, int batch, void* pool,
                              int32_t* packed_table, hipStream_t stream) {
  if (batch == 0 || max_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_fp8_dequant_kernel, dim3(max_blocks, batch), dim3(kThreads), 0, stream,
                     (const uint8_t*)kv8, num_blocks, block_table, max_blocks, seqlens,
                     (uint16_t*)pool, packed_table);
  return hipGetLastError();
}

}  // namespace mla
