// C ABI of libmla_decode.so: host-side validation, plan sizing and launches.
//
// Every argument check happens before the first HIP call, so a rejected call
// enqueues nothing and needs no GPU.  The library allocates no device memory: callers
// pass every buffer, except for mla_decode_fwd_noalloc, whose scratch is static device
// data of the library.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "mla_decode.h"
#include "mla_internal.h"

using namespace mla;

// Scratch of mla_decode_fwd_noalloc: the split plan, then the partial results of split
// segments.  Each device that runs the call holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, not the device memory:
// only the address hipGetSymbolAddress returns (kept per device below) is handed to
// kernels.
static __device__ __attribute__((aligned(256))) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_sizes(int batch, int s_q, int heads, int num_wg) {
  if (batch < 0 || s_q < 1 || heads < 1 || num_wg < 1) return MLA_ERR_INVALID_ARG;
  if ((int64_t)s_q * heads > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
  if (num_wg > 65535) return MLA_ERR_UNSUPPORTED;
  // segment count and table sizes must stay within int32 device indexing
  if ((int64_t)batch * num_groups(s_q, heads) > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

namespace mla {
// mla_append.hip
hipError_t launch_append(const void* new_kv, void* kv_cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                         int batch, int s_new, int elem_bytes, int32_t* status,
                         hipStream_t stream);
}  // namespace mla

extern "C" {

int mla_device_workgroups(int device, int* num_workgroups) {
  if (!num_workgroups) return MLA_ERR_INVALID_ARG;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return MLA_ERR_HIP;
  *num_workgroups = cus;
  return MLA_OK;
}

int mla_plan_size(int batch, int s_q, int num_heads, int num_workgroups, size_t* meta_bytes,
                  size_t* workspace_bytes) {
  if (!meta_bytes || !workspace_bytes) return MLA_ERR_INVALID_ARG;
  int rc = check_sizes(batch, s_q, num_heads, num_workgroups);
  if (rc) return rc;
  *meta_bytes = meta_words(batch, s_q, num_heads, num_workgroups) * sizeof(int32_t);
  *workspace_bytes = mla::workspace_bytes(batch, s_q, num_heads, num_workgroups);
  return MLA_OK;
}

int mla_get_split_metadata(const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                           int max_blocks_per_seq, int num_workgroups, int min_split_blocks,
                           int32_t* meta, size_t meta_bytes, void* stream) {
  int rc = check_sizes(batch, s_q, num_heads, num_workgroups);
  if (rc) return rc;
  if (!meta || (batch > 0 && !seqlens)) return MLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (max_blocks_per_seq < 0 || min_split_blocks < 0) return MLA_ERR_INVALID_ARG;
  if (meta_bytes < meta_words(batch, s_q, num_heads, num_workgroups) * sizeof(int32_t))
    return MLA_ERR_PLAN;
  if (launch_sched(seqlens, batch, s_q, num_heads, causal, max_blocks_per_seq, num_workgroups,
                   min_split_blocks, meta, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"

namespace {

enum Stage { kStageMain = 1, kStageCombine = 2 };

int decode(int stages, int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
           const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens,
           int batch, int s_q, int num_heads, int causal, float scale, float* out, float* lse,
           int32_t* meta, size_t meta_bytes, int num_workgroups, void* workspace,
           size_t workspace_bytes, void* stream, int64_t q_row_stride = kDqk,
           int64_t out_row_stride = kDv) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  // rows of q and out may be strided (q sliced from a wider projection output, out a view
  // of a wider buffer); every row must start 16-byte aligned
  const int64_t q_align = dtype == MLA_DTYPE_BF16 ? 8 : 4;
  if (q_row_stride < kDqk || q_row_stride % q_align != 0 || q_row_stride > ((int64_t)1 << 40) ||
      out_row_stride < kDv || out_row_stride % 4 != 0 || out_row_stride > ((int64_t)1 << 40))
    return MLA_ERR_INVALID_ARG;
  int rc = check_sizes(batch, s_q, num_heads, num_workgroups);
  if (rc) return rc;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (num_blocks < 0 || max_blocks_per_seq < 0) return MLA_ERR_INVALID_ARG;
  if (!meta) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!q || !out || !lse || !seqlens || !block_table) return MLA_ERR_INVALID_ARG;
  if (num_blocks > 0 && !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (kv_cache && !aligned16(kv_cache)))
    return MLA_ERR_INVALID_ARG;
  if (meta_bytes < meta_words(batch, s_q, num_heads, num_workgroups) * sizeof(int32_t))
    return MLA_ERR_PLAN;
  const size_t ws_need = mla::workspace_bytes(batch, s_q, num_heads, num_workgroups);
  if (workspace_bytes < ws_need) return MLA_ERR_PLAN;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARG;

  Problem p;
  p.q = q;
  p.kv = kv_cache;
  p.num_blocks = num_blocks;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.seqlens = seqlens;
  p.batch = batch;
  p.s_q = s_q;
  p.heads = num_heads;
  p.causal = causal;
  p.scale = scale;
  p.out = out;
  p.lse = lse;
  p.q_rs = q_row_stride;
  p.o_rs = out_row_stride;
  p.meta = meta;
  p.num_wg = num_workgroups;
  const size_t slots = num_slots(batch, s_q, num_heads, num_workgroups);
  p.part_o = (float*)workspace;
  p.part_lse = p.part_o + slots * kGroupRows * kDv;
  p.part_half = dtype == MLA_DTYPE_BF16;
  p.src_row = nullptr;
  p.fp8 = false;
  p.part_scale = p.part_half ? part_scale_ptr(p.part_o, slots) : nullptr;

  hipStream_t st = (hipStream_t)stream;
  if (stages & kStageMain) {
    hipError_t e = dtype == MLA_DTYPE_BF16 ? launch_main_bf16(p, st) : launch_main_f32(p, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  if (stages & kStageCombine) {
    if (launch_combine(p, st) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

#define MLA_DECODE_ARGS                                                                      \
  int dtype, const void *q, const void *kv_cache, int64_t num_blocks,                       \
      const int32_t *block_table, int max_blocks_per_seq, const int32_t *seqlens, int batch, \
      int s_q, int num_heads, int causal, float scale, float *out, float *lse,               \
      int32_t *meta, size_t meta_bytes, int num_workgroups, void *workspace,                 \
      size_t workspace_bytes, void *stream
#define MLA_DECODE_PASS                                                                      \
  dtype, q, kv_cache, num_blocks, block_table, max_blocks_per_seq, seqlens, batch, s_q,     \
      num_heads, causal, scale, out, lse, meta, meta_bytes, num_workgroups, workspace,       \
      workspace_bytes, stream

int mla_decode_fwd(MLA_DECODE_ARGS) {
  return decode(kStageMain | kStageCombine, MLA_DECODE_PASS);
}
int mla_decode_fwd_strided(int dtype, const void* q, int64_t q_row_stride, const void* kv_cache,
                           int64_t num_blocks, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q,
                           int num_heads, int causal, float scale, float* out,
                           int64_t out_row_stride, float* lse, int32_t* meta, size_t meta_bytes,
                           int num_workgroups, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode(kStageMain | kStageCombine, MLA_DECODE_PASS, q_row_stride, out_row_stride);
}
int mla_decode_main(MLA_DECODE_ARGS) { return decode(kStageMain, MLA_DECODE_PASS); }
int mla_decode_combine(MLA_DECODE_ARGS) { return decode(kStageCombine, MLA_DECODE_PASS); }

int mla_read_status(const int32_t* meta, void* stream, int32_t* status) {
  if (!meta || !status) return MLA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, meta + H_STATUS, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess)
    return MLA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MLA_ERR_HIP;
  *status = v;
  return MLA_OK;
}

int mla_sparse_plan_size(int batch, int num_heads, int topk, int num_workgroups,
                         size_t* meta_bytes, size_t* workspace_bytes) {
  if (!meta_bytes || !workspace_bytes) return MLA_ERR_INVALID_ARG;
  int rc = check_sizes(batch, 1, num_heads, num_workgroups);
  if (rc) return rc;
  if (topk < kPage || topk % kPage != 0) return MLA_ERR_INVALID_ARG;
  if (topk > kMaxSparseTopk) return MLA_ERR_UNSUPPORTED;
  *meta_bytes = meta_words(batch, 1, num_heads, num_workgroups) * sizeof(int32_t);
  *workspace_bytes = align256(mla::workspace_bytes(batch, 1, num_heads, num_workgroups)) +
                     sparse_scratch_bytes(batch, topk);
  return MLA_OK;
}

int mla_decode_sparse_fwd(const void* q, const void* kv_cache, int64_t num_blocks,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seqlens, const int32_t* indices, int topk, int batch,
                          int num_heads, float scale, float* out, float* lse, int32_t* meta,
                          size_t meta_bytes, int num_workgroups, void* workspace,
                          size_t workspace_bytes, void* stream) {
  size_t need_meta = 0, need_ws = 0;
  int rc = mla_sparse_plan_size(batch, num_heads, topk, num_workgroups, &need_meta, &need_ws);
  if (rc) return rc;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MLA_ERR_INVALID_ARG;
  // pool rows are addressed with 32-bit row numbers
  if (num_blocks < 0 || num_blocks > ((int64_t)1 << 25) || max_blocks_per_seq < 0)
    return MLA_ERR_INVALID_ARG;
  if (!meta) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!q || !out || !lse || !seqlens || !block_table || !indices) return MLA_ERR_INVALID_ARG;
  if (num_blocks > 0 && !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (kv_cache && !aligned16(kv_cache)))
    return MLA_ERR_INVALID_ARG;
  if (meta_bytes < need_meta || workspace_bytes < need_ws) return MLA_ERR_PLAN;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARG;

  hipStream_t st = (hipStream_t)stream;
  const size_t dense_ws = align256(mla::workspace_bytes(batch, 1, num_heads, num_workgroups));
  const SparseScratch sc = sparse_scratch((char*)workspace + dense_ws, batch, topk);
  // Pools addressable by 32-bit byte offsets: the main kernel gathers the selected rows
  // straight from the pool.  Larger pools: the rows are first copied into packed blocks.
  const bool fused = num_blocks <= kMaxGatherBlocks;
  if (launch_sparse_pack(seqlens, block_table, max_blocks_per_seq, num_blocks, indices, topk,
                         batch, kv_cache, sc, !fused, st) != hipSuccess)
    return MLA_ERR_HIP;
  const int chunks = topk / kPage;
  if (launch_sched(sc.packed_len, batch, 1, num_heads, 0, chunks, num_workgroups, 0, meta,
                   st) != hipSuccess)
    return MLA_ERR_HIP;
  Problem p;
  p.q = q;
  p.kv = fused ? kv_cache : sc.packed_kv;
  p.src_row = fused ? sc.src_row : nullptr;
  p.fp8 = false;
  p.num_blocks = (int64_t)batch * chunks;
  p.block_table = sc.packed_table;
  p.max_blocks = chunks;
  p.seqlens = sc.packed_len;
  p.batch = batch;
  p.s_q = 1;
  p.heads = num_heads;
  p.causal = 0;
  p.scale = scale;
  p.out = out;
  p.lse = lse;
  p.meta = meta;
  p.num_wg = num_workgroups;
  const size_t slots = num_slots(batch, 1, num_heads, num_workgroups);
  p.part_o = (float*)workspace;
  p.part_lse = p.part_o + slots * kGroupRows * kDv;
  p.part_half = true;
  p.part_scale = part_scale_ptr(p.part_o, slots);
  if (launch_main_bf16(p, st) != hipSuccess) return MLA_ERR_HIP;
  if (launch_combine(p, st) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_fp8_plan_size(int batch, int s_q, int num_heads, int max_blocks_per_seq,
                      int num_workgroups, size_t* meta_bytes, size_t* workspace_bytes) {
  if (!meta_bytes || !workspace_bytes) return MLA_ERR_INVALID_ARG;
  int rc = check_sizes(batch, s_q, num_heads, num_workgroups);
  if (rc) return rc;
  if (max_blocks_per_seq < 0) return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * max_blocks_per_seq > (int64_t)1 << 25) return MLA_ERR_UNSUPPORTED;
  *meta_bytes = meta_words(batch, s_q, num_heads, num_workgroups) * sizeof(int32_t);
  *workspace_bytes = mla::workspace_bytes(batch, s_q, num_heads, num_workgroups);
  return MLA_OK;
}

int mla_decode_fp8_fwd(const void* q, const void* kv_fp8, int64_t num_blocks,
                       const int32_t* block_table, int max_blocks_per_seq,
                       const int32_t* seqlens, int batch, int s_q, int num_heads, int causal,
                       float scale, float* out, float* lse, int32_t* meta, size_t meta_bytes,
                       int num_workgroups, void* workspace, size_t workspace_bytes,
                       void* stream) {
  size_t need_meta = 0, need_ws = 0;
  int rc = mla_fp8_plan_size(batch, s_q, num_heads, max_blocks_per_seq, num_workgroups,
                             &need_meta, &need_ws);
  if (rc) return rc;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (num_blocks < 0 || num_blocks > ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARG;
  if (!meta) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!q || !out || !lse || !seqlens || (max_blocks_per_seq > 0 && !block_table))
    return MLA_ERR_INVALID_ARG;
  if (num_blocks > 0 && !kv_fp8) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (kv_fp8 && !aligned16(kv_fp8)))
    return MLA_ERR_INVALID_ARG;
  if (meta_bytes < need_meta || workspace_bytes < need_ws) return MLA_ERR_PLAN;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARG;

  hipStream_t st = (hipStream_t)stream;
  if (launch_sched(seqlens, batch, s_q, num_heads, causal, max_blocks_per_seq, num_workgroups, 0,
                   meta, st) != hipSuccess)
    return MLA_ERR_HIP;
  Problem p;
  p.q = q;
  p.kv = kv_fp8;
  p.num_blocks = num_blocks;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.seqlens = seqlens;
  p.batch = batch;
  p.s_q = s_q;
  p.heads = num_heads;
  p.causal = causal;
  p.scale = scale;
  p.out = out;
  p.lse = lse;
  p.meta = meta;
  p.num_wg = num_workgroups;
  const size_t slots = num_slots(batch, s_q, num_heads, num_workgroups);
  p.part_o = (float*)workspace;
  p.part_lse = p.part_o + slots * kGroupRows * kDv;
  p.part_half = true;
  p.part_scale = part_scale_ptr(p.part_o, slots);
  p.src_row = nullptr;
  p.fp8 = true;
  if (launch_main_bf16(p, st) != hipSuccess) return MLA_ERR_HIP;
  if (launch_combine(p, st) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_kv_append(int dtype, const void* new_kv, void* kv_cache, int64_t num_blocks,
                  const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens,
                  int batch, int s_new, int32_t* status, void* stream) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || s_new < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * s_new == 0) return MLA_OK;
  if ((int64_t)batch * s_new > ((int64_t)1 << 31) - 64) return MLA_ERR_UNSUPPORTED;
  if (!new_kv || !seqlens || (max_blocks_per_seq > 0 && !block_table)) return MLA_ERR_INVALID_ARG;
  if (num_blocks > 0 && !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(new_kv) || (kv_cache && !aligned16(kv_cache))) return MLA_ERR_INVALID_ARG;
  if (status && ((uintptr_t)status & 3u)) return MLA_ERR_INVALID_ARG;
  if (launch_append(new_kv, kv_cache, num_blocks, block_table, max_blocks_per_seq, seqlens,
                    batch, s_new, dtype == MLA_DTYPE_BF16 ? 2 : 4, status,
                    (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept; nullptr if the lookup fails.
char* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = (char*)addr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Compact partial-result layout of the no-allocation call, for `slots` part slots:
// fp16 O [slots][128][512], then the per-row scales and LSEs [slots][128] (bf16
// inputs), or fp32 O then the LSEs (fp32 inputs).
size_t noalloc_partial_bytes(bool half, size_t slots) {
  const size_t rows = slots * kGroupRows;
  return half ? rows * (kDv * 2 + 4 + 4) : rows * (kDv * 4 + 4);
}

}  // namespace

extern "C" {

int mla_decode_fwd_noalloc(int dtype, const void* q, const void* kv_cache, int64_t num_blocks,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seqlens, int batch, int s_q, int num_heads,
                           int causal, float scale, float* out, float* lse,
                           int num_workgroups, void* stream) {
  // the same host checks as mla_get_split_metadata + mla_decode_fwd, before any HIP call
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  int rc = check_sizes(batch, s_q, num_heads, num_workgroups);
  if (rc) return rc;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (num_blocks < 0 || max_blocks_per_seq < 0) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!q || !out || !lse || !seqlens || !block_table) return MLA_ERR_INVALID_ARG;
  if (num_blocks > 0 && !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (kv_cache && !aligned16(kv_cache)))
    return MLA_ERR_INVALID_ARG;
  const bool half = dtype == MLA_DTYPE_BF16;
  const size_t meta_b = align256(meta_words(batch, s_q, num_heads, num_workgroups) * 4);
  const size_t slots = num_slots(batch, s_q, num_heads, num_workgroups);
  if (meta_b + noalloc_partial_bytes(half, slots) > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_SCRATCH;

  char* base = scratch_on_current_device();
  if (!base) return MLA_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  int32_t* meta = (int32_t*)base;
  // the scheduler writes every plan word the other kernels read (status included), and
  // each partial is written before it is read: nothing needs clearing between calls
  if (launch_sched(seqlens, batch, s_q, num_heads, causal, max_blocks_per_seq, num_workgroups,
                   0, meta, st) != hipSuccess)
    return MLA_ERR_HIP;
  Problem p;
  p.q = q;
  p.kv = kv_cache;
  p.num_blocks = num_blocks;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.seqlens = seqlens;
  p.batch = batch;
  p.s_q = s_q;
  p.heads = num_heads;
  p.causal = causal;
  p.scale = scale;
  p.out = out;
  p.lse = lse;
  p.meta = meta;
  p.num_wg = num_workgroups;
  char* part = base + meta_b;
  const size_t rows = slots * kGroupRows;
  p.part_o = (float*)part;
  p.part_half = half;
  p.part_scale = half ? (float*)(part + rows * kDv * 2) : nullptr;
  p.part_lse = half ? (float*)(part + rows * (kDv * 2 + 4)) : (float*)(part + rows * kDv * 4);
  p.src_row = nullptr;
  p.fp8 = false;
  hipError_t e = half ? launch_main_bf16(p, st) : launch_main_f32(p, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (launch_combine(p, st) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

const char* mla_status_string(int code) {
  switch (code) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case MLA_ERR_PLAN: return "metadata or workspace buffer too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_SCRATCH: return "plan and partial results exceed the fixed scratch of the "
                                 "no-allocation call";
    default: return "unknown status code";
  }
}

}  // extern "C"
