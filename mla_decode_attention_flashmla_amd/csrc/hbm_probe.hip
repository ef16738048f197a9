// Read-bandwidth probes for the roofline measurement (libmla_probe.so).
//
// The decode's main kernel is bound by HBM reads at s_q = 1.  The datasheet's 8 TB/s
// is not what any kernel reaches; these probes measure what reads alone reach on the
// device, so the main kernel's fraction can be read against an achievable ceiling:
//   stream      every thread reads 16-byte words in a grid-stride loop, eight loads in
//               flight (optionally with the non-temporal hint), many workgroups per CU;
//   pages       the main kernel's copy structure without its compute: one workgroup of
//               4 waves per CU walks its share of a permuted list of `unit`-byte blocks,
//               copying each into LDS with 16-byte direct-to-LDS loads, NBUF buffers
//               (NBUF - 1 blocks in flight), one wait and barrier per block.
// Nothing here is on the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kNt>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (kNt)
        v[k] = __builtin_nontemporal_load(p + i + k * stride);
      else
        v[k] = p[i + k * stride];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  // never true for the probe's data; keeps the loads live
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u)
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.z;
}

// 16 bytes per lane from sbase + voff into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  sbase = (const void*)(uintptr_t)((hi << 32) | lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(sbase)
      : "memory");
}

// kUnit bytes per block (a multiple of 4 KiB: each of the 4 waves copies kUnit / 4 bytes,
// 1 KiB per instruction), kBuf LDS buffers.
template <int kUnit, int kBuf>
__global__ __launch_bounds__(256, 1) void page_read_kernel(const char* __restrict__ base,
                                                           const int32_t* __restrict__ order,
                                                           int nunits, uint32_t* __restrict__ sink) {
  static_assert(kUnit % 4096 == 0 && kUnit * kBuf <= 160 * 1024, "LDS");
  constexpr int kPerWave = kUnit / 4096;  // instructions per wave per block
  __shared__ __attribute__((aligned(16))) char lds[kUnit * kBuf];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = (int)((int64_t)blockIdx.x * nunits / gridDim.x);
  const int u1 = (int)((int64_t)(blockIdx.x + 1) * nunits / gridDim.x);
  const int n = u1 - u0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  auto issue = [&](int k) {
    const char* src = base + (size_t)(uint32_t)order[u0 + k] * kUnit + wave * (kUnit / 4);
    const uint32_t dst = lds0 + (k % kBuf) * kUnit + wave * (kUnit / 4);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) dma16(src + i * 1024, (uint32_t)lane * 16u, dst + i * 1024);
  };
  for (int k = 0; k < kBuf - 1 && k < n; ++k) issue(k);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int k = 0; k < n; ++k) {
    if (k + kBuf - 1 < n) {
      issue(k + kBuf - 1);
      // blocks k .. k + kBuf - 1 in flight: wait for block k only
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kBuf - 1) * kPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const char* buf = lds + (k % kBuf) * kUnit;
    acc ^= *(const u32x4*)(buf + (threadIdx.x * 16) % kUnit);
    // every wave is done with this buffer before a later block is copied into it
    __syncthreads();
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc.z;
}

}  // namespace

extern "C" {

int mla_probe_stream_read(const void* buf, size_t bytes, int nontemporal, int workgroups,
                          uint32_t* sink, void* stream) {
  if (!buf || !sink || workgroups < 1 || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
  const size_t n16 = bytes / 16;
  hipStream_t st = (hipStream_t)stream;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(256), 0, st,
                       (const u32x4*)buf, n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(256), 0, st,
                       (const u32x4*)buf, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_probe_page_read(const void* buf, int unit_bytes, int nbuf, const int32_t* order,
                        int nunits, int workgroups, uint32_t* sink, void* stream) {
  if (!buf || !order || !sink || nunits < 1 || workgroups < 1 || ((uintptr_t)buf & 15))
    return -1;
  hipStream_t st = (hipStream_t)stream;
  const char* b = (const char*)buf;
  if (unit_bytes == 73728 && nbuf == 2)
    hipLaunchKernelGGL((page_read_kernel<73728, 2>), dim3(workgroups), dim3(256), 0, st, b, order,
                       nunits, sink);
  else if (unit_bytes == 36864 && nbuf == 4)
    hipLaunchKernelGGL((page_read_kernel<36864, 4>), dim3(workgroups), dim3(256), 0, st, b, order,
                       nunits, sink);
  else if (unit_bytes == 36864 && nbuf == 3)
    hipLaunchKernelGGL((page_read_kernel<36864, 3>), dim3(workgroups), dim3(256), 0, st, b, order,
                       nunits, sink);
  else if (unit_bytes == 16384 && nbuf == 8)
    hipLaunchKernelGGL((page_read_kernel<16384, 8>), dim3(workgroups), dim3(256), 0, st, b, order,
                       nunits, sink);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
