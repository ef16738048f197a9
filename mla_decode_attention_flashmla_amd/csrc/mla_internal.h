// Internal layout shared by the host library and the kernels of libmla_decode.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;        // tokens per KV block
constexpr int kDqk = 576;        // latent 512 + rope 64
constexpr int kDv = 512;         // V = first 512 columns
constexpr int kGroupRows = 128;  // query rows (t, h) per row group, one workgroup's rows

// Scheduling metadata, int32 words.
//   header      kHdrWords
//   work table  num_workgroups x kWgWords   (one row per persistent workgroup slot)
//   seg table   num_segments   x kSegWords  (one row per (sequence, row group))
constexpr int kHdrWords = 32;
constexpr int kWgWords = 8;
constexpr int kSegWords = 8;
// identifies the plan layout below; changes whenever the layout does, so a plan written
// under another layout is rejected instead of misread
constexpr int32_t kMagic = 0x4D4C4132;

enum Hdr {
  H_MAGIC = 0, H_BATCH, H_SQ, H_HEADS, H_CAUSAL, H_NUM_WG, H_STATUS, H_NUM_SEG,
  H_NUM_GROUPS, H_TOTAL_BLOCKS, H_NUM_ITEMS, H_NUM_SLOTS, H_MAX_BLOCKS,
  H_ALIGNED,  // item size of a segment-aligned plan, 0 for a stream cut
};
// work-table row: first segment, first block in it, last segment, end block in it (exclusive),
// split index of the first segment, and that segment's block count and length (so a
// workgroup can start its first page without another dependent read).  seg_begin < 0:
// the slot has no work.
enum Wg { W_SEG_BEGIN = 0, W_BLK_BEGIN, W_SEG_END, W_BLK_END, W_FIRST_SPLIT, W_NBLK0, W_SEQLEN0 };
// segment row: blocks, validated length (-1: invalid), block offset in the stream,
// number of parts (0: no keys or invalid, 1: computed whole), first partial slot, first
// work item (-1 for a segment with no blocks), and the scheduler's own running item
// count of a segment-aligned plan (non-decreasing over segments, empty ones included:
// the column the work-table rows search; batches beyond its LDS arrays keep it here).
enum Seg { S_NBLK = 0, S_SEQLEN, S_CUM, S_NSPLIT, S_SLOT, S_FIRST_ITEM, S_AL_ITEM };

inline int num_groups(int s_q, int heads) { return (s_q * heads + kGroupRows - 1) / kGroupRows; }

inline size_t meta_words(int batch, int s_q, int heads, int num_wg) {
  return (size_t)kHdrWords + (size_t)kWgWords * num_wg +
         (size_t)kSegWords * batch * num_groups(s_q, heads);
}
inline size_t num_slots(int batch, int s_q, int heads, int num_wg) {
  return (size_t)num_wg + (size_t)batch * num_groups(s_q, heads);
}
// workspace: partial O [slots][128][512] fp32 (or fp16 + per-row scales), then partial
// LSE [slots][128] fp32
inline size_t workspace_bytes(int batch, int s_q, int heads, int num_wg) {
  return num_slots(batch, s_q, heads, num_wg) * kGroupRows * (kDv + 1) * sizeof(float);
}

struct Problem {
  const void* q;
  const void* kv;
  int64_t num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seqlens;
  int batch, s_q, heads, causal;
  float scale;
  float* out;
  float* lse;
  // elements from one (b, t, h) row of q / out to the next (dense: 576 / 512)
  int64_t q_rs = kDqk;
  int64_t o_rs = kDv;
  int32_t* meta;
  int num_wg;
  float* part_o;    // [slots][128][512] fp32, or fp16 (part_half) in the first half
  float* part_lse;  // [slots][128]
  float* part_scale;  // [slots][128], fp16 partials only: each row's power-of-two scale
  bool part_half;     // partial O stored as scaled fp16 (bf16 path) instead of fp32
  // gathered pages (bf16 path): block_table entry id names rows src_row[64*id .. +63] of
  // the pool `kv` instead of block id; nullptr for a paged cache
  const int32_t* src_row;
  // fp8 pages (bf16 path): kv holds 656-byte rows (e4m3 latent codes, bf16 rope, a
  // power-of-two fp32 scale), widened to bf16 in LDS by the main kernel
  bool fp8;
};
// Gathered pages address pool rows by 32-bit byte offsets: pools up to this many blocks.
constexpr int64_t kMaxGatherBlocks = 0xffffffffLL / (kPage * kDqk * 2);
// With fp16 partials the per-row scales sit in the unused second half of the O region.
inline float* part_scale_ptr(float* part_o, size_t slots) {
  return (float*)((char*)part_o + slots * kGroupRows * kDv * 2);
}

// Sparse decode scratch, carved from the caller's workspace after the partial results:
// the packed rows [batch * topk][576] bf16, the pool row of each packed row, the packed
// block table [batch][topk / 64] and the packed lengths [batch].
constexpr int kMaxSparseTopk = 65536;
constexpr int kMaxSparseChunks = kMaxSparseTopk / kPage;
struct SparseScratch {
  void* packed_kv;
  int32_t* src_row;
  int32_t* packed_table;
  int32_t* packed_len;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t sparse_scratch_bytes(int batch, int topk) {
  const size_t rows = (size_t)batch * topk;
  return align256(rows * kDqk * 2) + align256(rows * 4) + align256(rows / kPage * 4) +
         align256((size_t)batch * 4);
}
inline SparseScratch sparse_scratch(void* base, int batch, int topk) {
  const size_t rows = (size_t)batch * topk;
  char* p = (char*)base;
  SparseScratch s;
  s.packed_kv = p;
  p += align256(rows * kDqk * 2);
  s.src_row = (int32_t*)p;
  p += align256(rows * 4);
  s.packed_table = (int32_t*)p;
  p += align256(rows / kPage * 4);
  s.packed_len = (int32_t*)p;
  return s;
}

hipError_t launch_sched(const int32_t* seqlens, int batch, int s_q, int heads, int causal,
                        int max_blocks, int num_wg, int min_split_blocks, int32_t* meta,
                        hipStream_t stream);
hipError_t launch_main_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_main_f32(const Problem& p, hipStream_t stream);
hipError_t launch_combine(const Problem& p, hipStream_t stream);
// gather: also copy the selected rows into packed blocks (the two-pass form); without
// it only the pool-row lists, packed lengths and packed block table are written, for
// the main kernel's gathered pages
hipError_t launch_sparse_pack(const int32_t* seqlens, const int32_t* block_table, int max_blocks,
                              int64_t num_blocks, const int32_t* indices, int topk, int batch,
                              const void* kv, const SparseScratch& s, bool gather,
                              hipStream_t stream);

}  // namespace mla
