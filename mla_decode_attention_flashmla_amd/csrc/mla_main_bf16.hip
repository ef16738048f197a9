// MLA decode main kernel, bf16 inputs, gfx950 MFMA.
//
// One persistent workgroup (4 waves, one per SIMD) walks its range of 64-token
// KV blocks.  Each block ("page") is copied once from HBM into LDS with 16-byte
// direct-to-LDS loads and then serves as both K (all 576 columns) and V (the
// first 512): the "each cache tile into shared memory" placement the TileLang
// talk recommends for MLA (section "Future work").  The copy of page k+1 is in
// flight while page k is computed: copy is its own pipeline stage, as the
// talk's num_stages pipelining derives (section "What is TileLang?", pipeline
// inference).
//
// Each wave owns 32 query rows (row = (token, head)).  Per page it computes
//   S^T[token, row] = K . Q^T     on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q in VGPRs)
// so that, in the accumulator layout, a lane holds one row and 16 tokens: the
// row max and row sum are in-lane plus one permlane32 swap (the reduce from the
// score accumulator to the per-row max whose layout follows from the GEMM's,
// the middle step of the talk's layout inference).  Then
//   O^T[col, row] = alpha * O^T + V^T . P^T   on the same MFMA
// with V^T read from the same LDS page by ds_read_b64_tr_b16 and P^T taken
// straight from the score registers (the token order of the V read matches the
// accumulator layout, so P needs no shuffle).
//
// Registers: O^T (32 rows x 512 fp32 = 256 per lane) lives in the AGPRs
// a0..a255 for a whole segment and only inline asm touches them (MFMA, zero,
// rescale, read-out); the compiler works in VGPRs only (Q fragments, scores,
// P, LDS fragments).  The score MFMAs are asm too, to keep their accumulators
// in VGPRs.  Wait states the hardware needs around these MFMAs are written
// into the asm: after the last score MFMA of a page (before VALU reads of the
// scores), before the first PV MFMA (after VALU writes of P and O), and before
// the epilogue reads O^T (a rescale reads it only after the next page's score
// MFMAs, so the PV loop ends without them).  Inside the PV loop the later chunks
// of P are written by VALU at least 4 MFMAs before the first MFMA that reads them.
//
// The running max is allowed to lag the true row max by up to 8 (log2 units):
// O is only rescaled when a page raises some row's max by more than that, so
// exp2 arguments stay <= 8 and the rescale (three VALU ops per O element) is rare.
//
// Page sources (template parameters, one instantiation each):
//   paged     a 64-token block of the bf16 cache, named by the block table;
//   kGather   64 rows read one by one from the bf16 pool by their pool row numbers (the
//             rows a sparse selection picked, listed by the index kernel);
//   kFp8      a block of 656-byte rows (e4m3 latent codes, bf16 rope, a power-of-two
//             scale), copied as is and widened to the bf16 layout below in LDS before
//             the page's scores.
// Every source ends in the same LDS layout, so the products, the softmax and the
// epilogue are shared.  A fourth instantiation, kStrided, is the paged one with q and
// out rows at strides given at run time instead of the dense 576 / 512.
//
// LDS page layout (77824 bytes, two pages double-buffered), for 64 banks of 4 bytes:
//   main region  columns 0..511 of row r (1024 bytes) at 1088*r + 16*((r>>2)&3).
//                Row starts are 64*(r&3) + 16*((r>>2)&3) modulo 256 bytes, so the
//                16 rows of a K read (ds_read_b128, same column) hit 16 different
//                4-bank groups, and the 4 rows x 64 bytes of a transposed V read
//                (ds_read_b64_tr_b16) hit 4 disjoint 16-bank ranges.
//   tail region  columns 512..575 at 69632 + 128*r: 8 16-byte chunks, chunk t of
//                row r at position t ^ ((r>>1)&7) (16 rows of one chunk: 16 groups)
#include <type_traits>

#include "mla_internal.h"
#include "mla_decode.h"
#include "mla_oacc_asm.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowPitch = 1088;               // main-region row r starts at 1088*r + 16*((r>>2)&3)
constexpr int kMainBytes = 69632;             // 64 rows
constexpr int kTailStride = 128;
constexpr int kBufBytes = kMainBytes + kPage * kTailStride;
constexpr int kKDepth = 3;                    // K fragments read this many k-steps ahead
constexpr int kVDepth = 4;                    // V fragments read this many MFMAs ahead

__host__ __device__ constexpr int main_row(int r) { return kRowPitch * r + 16 * ((r >> 2) & 3); }
static_assert(main_row(63) + 1024 <= kMainBytes, "main region");
static_assert(main_row(16) == 17408 && main_row(12) - main_row(4) == 8736, "row offsets");
constexpr int kKSteps = kDqk / 16;           // 36 MFMA k-steps over the 576 columns
constexpr int kCTiles = kDv / 32;            // 16 column tiles of O^T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleSlack = 8.0f;        // log2 units the running max may lag the true max
constexpr float kNegBig = -1.0e30f;          // finite "no key yet" running max

// f(integral_constant<int, I>) for I = B .. E-1: every index is a compile-time constant,
// so the O^T tile an asm MFMA names is always resolved at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// 16 bytes per lane from global (SGPR base + VGPR offset) straight into LDS at
// m0 + 16 * lane.  Issued through asm so the compiler does not wait for it before
// unrelated LDS reads; completion is awaited explicitly with vmcnt(0).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // both are wave-uniform by construction; readfirstlane keeps them in SGPRs.  It
  // returns a signed int: each half goes through uint32_t so the low word is never
  // sign-extended into the high one.
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t au = (hi << 32) | lo;
  sbase = (const void*)(uintptr_t)au;
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

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The page copies of bf16 pages set M0 once per window of LDS destinations: a write of
// M0 stalls the wave while its LDS reads are in flight (~40 cycles in the score loop,
// measured), so one write per copy cost ~750 cycles per page.  The copy instruction's
// offset is added to both its LDS address (M0 + offset + 16 * lane) and its global
// address, so a copy names its LDS destination by a constant offset from the window's
// M0 and lowers its global base by the same amount.  Nothing between set_m0 and the
// window's copies writes M0 (the compiler has no use for it in this kernel; the other
// copy helpers restore it).
__device__ __forceinline__ void set_m0(uint32_t lds_addr) {
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds_addr) : "memory", "m0");
}
// 16 bytes per lane from sbase + voff into LDS at M0 + kOff + 16 * lane
template <int kOff>
__device__ __forceinline__ void dma16_at(const void* sbase, uint32_t voff) {
  static_assert(kOff >= -4096 && kOff <= 4095 && kOff % 16 == 0, "instruction offset");
  const uint64_t a = (uint64_t)(uintptr_t)sbase - (uint64_t)(int64_t)kOff;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const void* base = (const void*)(uintptr_t)((hi << 32) | lo);
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2 nt" ::"v"(voff), "s"(base), "n"(kOff)
               : "memory");
}
// Windows of a wave's 18 copies (rows r0 = 16 * wave ..): main rows r0 .. r0+7 and
// r0+8 .. r0+15, each window's M0 placed so that the rows' offsets main_row(r) - M0 fall
// in [-3552, 4080]; then the two tail copies, 1 KiB apart.
constexpr int kWinCenter = 3552;
__host__ __device__ constexpr int win_off(int i) {   // row r0 + i relative to its window's M0
  return 1088 * i + 16 * ((i >> 2) & 3) - (i < 8 ? 0 : 8736) - kWinCenter;
}
static_assert(win_off(0) == -3552 && win_off(7) == 4080 && win_off(8) == -3552 &&
              win_off(15) == 4080, "window offsets");

// 4 bytes per lane from global into LDS at m0 + 4 * lane (the fp8 rows' scales)
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
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
      "global_load_lds_dword %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(sbase)
      : "memory");
}

__device__ __forceinline__ float swap_halves_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- score MFMAs, accumulator in VGPRs ----
__device__ __forceinline__ void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(acc) : "v"(a), "v"(b));
}

// ---- O^T tiles in AGPRs (tile ct = a[16ct .. 16ct+15]); ct is a compile-time constant ----
#define MLA_FOR_TILES(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15)

__device__ __forceinline__ void o_pv(int ct, const bf16x8& a, const bf16x8& b) {
  switch (ct) {
#define X(n)                                                                                  \
  case n:                                                                                     \
    asm volatile("v_mfma_f32_32x32x16_bf16 " MLA_OT##n ", %0, %1, " MLA_OT##n ::"v"(a), "v"(b) \
                 : MLA_OT##n##_CLOBBER);                                                      \
    break;
    MLA_FOR_TILES(X)
#undef X
  }
}
__device__ __forceinline__ void o_zero() {
#define X(n) asm volatile(MLA_OT##n##_ZERO ::: MLA_OT##n##_CLOBBER);
  MLA_FOR_TILES(X)
#undef X
}
__device__ __forceinline__ void o_scale(float alpha) {
  float t0, t1, t2, t3;
#define X(n)                                                                         \
  asm volatile(MLA_OT##n##_SCALE : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3) : "v"(alpha) \
               : MLA_OT##n##_CLOBBER);
  MLA_FOR_TILES(X)
#undef X
}
__device__ __forceinline__ void o_read(int ct, float (&v)[16]) {
  switch (ct) {
#define X(n)                                                                                 \
  case n:                                                                                    \
    asm volatile(MLA_OT##n##_READ                                                            \
                 : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]),    \
                   "=v"(v[6]), "=v"(v[7]), "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), \
                   "=v"(v[12]), "=v"(v[13]), "=v"(v[14]), "=v"(v[15]));                      \
    break;
    MLA_FOR_TILES(X)
#undef X
  }
}

__device__ __forceinline__ int M_rows(int s_q, int heads) { return s_q * heads; }

__device__ __forceinline__ int sload(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*p);
}

struct PageSrc {
  const char* base;     // block start in global memory (gathered pages: the pool's start)
  const int32_t* rows;  // gathered pages: the pool row of each of the page's 64 rows
  int valid_rows;       // rows [0, valid_rows) are real keys; later rows re-read the last one
  int load;             // 0: bad block number, nothing is read
};

// One of this wave's 18 loads of a page (72 per page in all) into the LDS buffer at
// lds_addr: i = 0..15 copies main row 16*wave + i (1 KiB, the LDS row offset is a
// compile-time constant), i = 16, 17 copy the tail chunks of rows 16*wave + 8*(i-16)
// .. +7.  Rows at or past valid_rows re-read the last valid row.  Spreading the 18
// loads over the score loop keeps the copy's LDS writes from arriving in one burst.
//
// Gathered pages (kGather): row r of the page is pool row src.rows[r], a row of its own
// anywhere in the pool.  g.ridx holds this wave's 16 of them (rows 16*wave ..), read as
// scalars when the page's source is known, and g.tail[t] each lane's row of tail load t.
// Every entry is a real pool row (the packing pass pads a sequence's last block with its
// last row), so no clamp is needed.  The tail loads address each lane's row by a 32-bit
// byte offset from the pool's start, which the host guarantees by the pool's size.
struct GatherRows {
  int ridx[16];
  int tail[2];
};

//
// fp8 pages (kFp8): rows of 656 bytes (512 e4m3 codes, 64 bf16 rope values, the fp32
// power-of-two scale).  Parts 0..7 copy the codes of row pairs (2p, 2p+1), p = 8*wave +
// i, into the main slot of row 2p (row 2p's codes, then row 2p+1's); parts 8, 9 copy the
// rope values into the tail region as for bf16 pages; part 10 copies the wave's 16
// scales to the scale area.  fp8_convert() then widens the codes in place to the bf16
// main layout before the page's scores.
constexpr int kFp8RowBytes = 656;
constexpr int kFp8Parts = 11;
// per-lane byte offsets of the fp8 copies of a full page, relative to the first row of
// each part: codes (lane -> row (lane/32), 16 bytes at 16*(lane%32)), the two rope parts
// (lane -> row lane/8, the swizzled rope chunk) and the scales (lane -> row lane%16)
struct Fp8Lanes {
  uint32_t codes, tail[2], scale;
};

template <bool kGather, bool kFp8, int i>
__device__ __forceinline__ void issue_page_part(const PageSrc& src, uint32_t lds_addr,
                                                int wave, int lane,
                                                const uint32_t (&tail_lane_off)[2],
                                                const GatherRows& g, uint32_t scale_lds,
                                                const Fp8Lanes& f) {
  if (!src.load) return;
  const int vmax = src.valid_rows - 1;
  const int r0 = 16 * wave;
  if constexpr (kFp8) {
    // fp8 pages reach here only full (a segment's partial last page goes through
    // issue_fp8_partial): a scalar base per part, one per-lane offset per kind
    if (i < 8) {
      const int p = 8 * wave + i;
      dma16(src.base + 2 * p * kFp8RowBytes, f.codes, lds_addr + main_row(2 * p));
    } else if (i < 10) {
      const int t = i - 8;
      dma16(src.base + (r0 + 8 * t) * kFp8RowBytes, f.tail[t],
            lds_addr + kMainBytes + (r0 + 8 * t) * kTailStride);
    } else if (i == 10) {
      dma4(src.base + r0 * kFp8RowBytes, f.scale, scale_lds + wave * 256);
    }
    return;
  }
  const uint32_t lw = lds_addr + (uint32_t)main_row(r0);
  if constexpr (i == 0) set_m0(lw + kWinCenter);
  if constexpr (i == 8) set_m0(lw + 8736 + kWinCenter);
  if constexpr (i == 16) set_m0(lds_addr + kMainBytes + r0 * kTailStride);
  if constexpr (i < 16) {
    const char* rsrc;
    if constexpr (kGather) {
      rsrc = src.base + (size_t)(uint32_t)g.ridx[i] * (kDqk * 2);
    } else {
      const int rs = r0 + i < vmax ? r0 + i : vmax;
      rsrc = src.base + rs * (kDqk * 2);
    }
    dma16_at<win_off(i)>(rsrc, (uint32_t)lane * 16u);
  } else {
    constexpr int t = i - 16;
    uint32_t voff;
    if constexpr (kGather) {
      voff = (uint32_t)g.tail[t] * (uint32_t)(kDqk * 2) + tail_lane_off[t];
    } else {
      int row = r0 + 8 * t + (lane >> 3);
      row = row < vmax ? row : vmax;
      voff = (uint32_t)row * (kDqk * 2) + tail_lane_off[t];
    }
    dma16_at<kTailStride * 8 * t>(src.base, voff);
  }
}
constexpr int kPageParts = 18;

// fp8: all 11 parts of a partial page (a segment's last), rows at or past its length
// re-reading the last valid row; issued at once where the page's source is known
__device__ __forceinline__ void issue_fp8_partial(const PageSrc& src, uint32_t lds_addr,
                                                  int wave, int lane, uint32_t scale_lds,
                                                  const Fp8Lanes& f) {
  if (!src.load) return;
  const int vmax = src.valid_rows - 1;
  const int r0 = 16 * wave;
  // lane values computed here (not hoisted to the kernel's start and kept live)
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = 8 * wave + i;
    int row = 2 * p + (lane >> 5);
    row = row < vmax ? row : vmax;
    dma16(src.base, (uint32_t)row * kFp8RowBytes + (uint32_t)(lane & 31) * 16u,
          lds_addr + main_row(2 * p));
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int row = r0 + 8 * t + (lane >> 3);
    row = row < vmax ? row : vmax;
    dma16(src.base, (uint32_t)row * kFp8RowBytes + f.tail[t] - (uint32_t)(lane >> 3) * kFp8RowBytes,
          lds_addr + kMainBytes + (r0 + 8 * t) * kTailStride);
  }
  int row = r0 + (lane & 15);
  row = row < vmax ? row : vmax;
  dma4(src.base, (uint32_t)row * kFp8RowBytes + 640u, scale_lds + wave * 256);
}

template <bool kGather, bool kFp8>
__device__ __forceinline__ void issue_page(const PageSrc& src, uint32_t lds_addr, int wave,
                                           int lane, const uint32_t (&tail_lane_off)[2],
                                           const GatherRows& g, uint32_t scale_lds,
                                           const Fp8Lanes& f) {
  if constexpr (kFp8) {
    if (src.valid_rows < kPage) {
      issue_fp8_partial(src, lds_addr, wave, lane, scale_lds, f);
      return;
    }
  }
  auto part = [&](auto I) __attribute__((always_inline)) {
    issue_page_part<kGather, kFp8, decltype(I)::value>(src, lds_addr, wave, lane, tail_lane_off, g,
                                                       scale_lds, f);
  };
  static_for<0, (kFp8 ? kFp8Parts : kPageParts)>(part);
}

// fp8 pages: widen this wave's 8 row pairs from e4m3 codes to the bf16 main layout in
// place.  Lane l works on row 2p + l/32: with i = l%32 it reads codes 8i..8i+7 and
// 256+8i..256+8i+7 (two 8-byte reads) and writes their bf16 values at columns 8i and
// 256+8i, so every read and write is contiguous across the lanes of a row (no LDS bank
// conflicts).  Every pair's codes and scale are read before any lane writes, so row
// 2p's bf16 may overwrite the pair's codes and the reads are not serialized behind the
// writes.  A wave touches only the rows and the scale area its own copies filled.  The
// hardware conversion applies the row's scale exactly when it is a power of two 2^k with
// -117 <= k <= 119: then every code value times the scale is a normal bf16 number (or
// zero).  Returns true in a lane that met a scale outside that set (the row is then not
// in the format: the caller flags the segment and makes its result NaN).
__device__ __forceinline__ bool fp8_convert(uint32_t page_lds, uint32_t scale_lds, int wave,
                                            int lane) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) float lds_f32;
  const uint32_t half = (uint32_t)(lane >> 5), il = (uint32_t)(lane & 31);
  u32x2 lo[8], hi[8];
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = 8 * wave + i;
    const int row = 2 * p + (int)half;
    const uint32_t src = page_lds + main_row(2 * p) + 512u * half + 8u * il;
    lo[i] = *(const lds_u32x2*)(uintptr_t)src;
    hi[i] = *(const lds_u32x2*)(uintptr_t)(src + 256);
    sc[i] = *(const lds_f32*)(uintptr_t)(scale_lds + (row >> 4) * 256 + (row & 15) * 4);
  }
  auto widen8 = [](u32x2 c, float s) __attribute__((always_inline)) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      o[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[k], s, false));
      o[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[k], s, true));
    }
    return o;
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = 8 * wave + i;
    const int row = 2 * p + (int)half;
    const uint32_t dst = page_lds + main_row(row) + 16u * il;
    *(lds_u32x4*)(uintptr_t)dst = widen8(lo[i], sc[i]);
    *(lds_u32x4*)(uintptr_t)(dst + 512) = widen8(hi[i], sc[i]);
  }
  // sign 0, mantissa 0, biased exponent 10..246 (2^-117 .. 2^119)
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = __float_as_uint(sc[i]);
    bad = bad || (bits & 0x807fffffu) != 0 || (bits >> 23) - 10u > 236u;
  }
  return bad;
}

template <bool kGather, bool kFp8, bool kStrided>
__global__ __launch_bounds__(kThreads, 1) void mla_main_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv,
    const int32_t* __restrict__ src_row, int64_t num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seqlens,
    int batch, int s_q, int heads, int causal, float scale, float* __restrict__ out,
    float* __restrict__ lse_out, int32_t* __restrict__ meta, const int32_t* __restrict__ plan,
    _Float16* __restrict__ part_o, float* __restrict__ part_lse, float* __restrict__ part_scale,
    int64_t q_rs_arg, int64_t o_rs_arg) {
  static_assert(!kStrided || (!kGather && !kFp8), "strided rows: paged bf16 pages only");
  // rows of q and out q_rs / o_rs elements apart.  The dense instantiations take the row
  // widths as constants: two more 64-bit values live through the page loop cost scalar
  // registers there.
  const int64_t q_rs = kStrided ? q_rs_arg : (int64_t)kDqk;
  const int64_t o_rs = kStrided ? o_rs_arg : (int64_t)kDv;
  // two page buffers; fp8 pages add 1 KiB of row scales
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes + (kFp8 ? 1024 : 0)];
  // fp8 pages: the last segment in which some wave met a row scale outside the format,
  // one slot per segment parity (a wave may start the next segment's first page while
  // another still reads the flag of the previous segment in its epilogue)
  __shared__ int bad_scale_seg[2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;     // which half of the wave (token/column sub-block)
  const int l32 = lane & 31;   // row within the wave's 32 rows

  // blockIdx -> slot: consecutive slots on the same XCD (blocks go round-robin over 8 XCDs)
  const int nwg = gridDim.x;
  int slot = blockIdx.x;
  if ((nwg & 7) == 0) slot = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);

  // The header and this slot's row are read together (one round trip): the row lies
  // inside the buffer the host validated for these sizes, and nothing read from it is
  // used before the header check.
  // `plan` is the same buffer as `meta`, read-only: this kernel writes only the status
  // word (through `meta`), which it never reads, so every plan word it reads is loaded
  // with scalar loads (through `meta` the compiler must use vector loads, each followed by
  // a wait for every vector memory operation in flight, page copies included).
  const int32_t* wrow = plan + kHdrWords + (size_t)slot * kWgWords;
  const int32_t* segt = plan + kHdrWords + (size_t)kWgWords * nwg;
  const int h_magic = sload(plan + H_MAGIC), h_batch = sload(plan + H_BATCH);
  const int h_sq = sload(plan + H_SQ), h_heads = sload(plan + H_HEADS);
  const int h_causal = sload(plan + H_CAUSAL), h_nwg = sload(plan + H_NUM_WG);
  const int h_maxb = sload(plan + H_MAX_BLOCKS), groups = sload(plan + H_NUM_GROUPS);
  const int seg_first = sload(wrow + W_SEG_BEGIN);
  const int blk_first = sload(wrow + W_BLK_BEGIN);
  const int seg_last = sload(wrow + W_SEG_END);
  const int blk_last_end = sload(wrow + W_BLK_END);
  const int split_first = sload(wrow + W_FIRST_SPLIT);
  const int nblk_first = sload(wrow + W_NBLK0);
  const int seqlen_first = sload(wrow + W_SEQLEN0);
  if (h_magic != kMagic || h_batch != batch || h_sq != s_q || h_heads != heads ||
      h_causal != causal || h_nwg != nwg || h_maxb != max_blocks) {
    if (threadIdx.x == 0) atomicOr(&meta[H_STATUS], MLA_STATUS_PLAN_MISMATCH);
    return;
  }
  if (seg_first < 0) return;
  // ranges read from the plan stay inside this call's tables even if the plan is corrupt
  const int nseg = batch * ((M_rows(s_q, heads) + kGroupRows - 1) / kGroupRows);
  if (groups != (M_rows(s_q, heads) + kGroupRows - 1) / kGroupRows || seg_first >= nseg || seg_last < seg_first || seg_last >= nseg || blk_first < 0 ||
      nblk_first < 0 || nblk_first > max_blocks || blk_last_end > max_blocks) {
    if (threadIdx.x == 0) atomicOr(&meta[H_STATUS], MLA_STATUS_PLAN_MISMATCH);
    return;
  }
  const int M = s_q * heads;

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  const uint32_t scale_lds = lds0 + 2 * kBufBytes;  // fp8 pages: the page's 64 row scales
  // tail loads of rows 16*wave + 8i .. +7: lane -> row 8g + lane/8 (g = 2*wave + i), LDS
  // position lane%8, which holds chunk (lane%8) ^ ((row>>1)&7) = (lane%8) ^ ((4i + lane/16) & 7)
  uint32_t tail_lane_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    tail_lane_off[i] = (uint32_t)((64 + ((lane & 7) ^ ((4 * i + (lane >> 4)) & 7))) * 16);
  const float scale_log2 = scale * kLog2e;
  Fp8Lanes f8l;
  if constexpr (kFp8) {
    // the tail offset's chunk part is tail_lane_off minus the bf16 row's 1024-byte main part
    f8l.codes = (uint32_t)(lane >> 5) * kFp8RowBytes + (uint32_t)(lane & 31) * 16u;
    f8l.tail[0] = (uint32_t)(lane >> 3) * kFp8RowBytes + tail_lane_off[0] - 512u;
    f8l.tail[1] = (uint32_t)(lane >> 3) * kFp8RowBytes + tail_lane_off[1] - 512u;
    f8l.scale = (uint32_t)(lane & 15) * kFp8RowBytes + 640u;
  } else {
    f8l.codes = f8l.tail[0] = f8l.tail[1] = f8l.scale = 0;
  }

  // per-lane LDS byte offsets of the K (row-wise) and V (transposed) reads
  //   K: row l32 (+32 per token tile), 16-byte chunk 2s + h
  //   V: row 4h + (lane%16)/4 (+16 per k-chunk, +8 for the second read), columns
  //      32ct + 16*((lane/16)&1) + 4*(lane%4)
  const uint32_t k_off = (uint32_t)(main_row(l32) + h * 16);
  const uint32_t v_off = (uint32_t)(main_row(4 * h + ((lane & 15) >> 2)) +
                                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);

  auto seg_nblk = [&](int s) {
    const int v = sload(segt + (size_t)s * kSegWords + S_NBLK);
    return v < 0 ? 0 : (v > max_blocks ? max_blocks : v);
  };
  // Source of a page with `rows` valid rows (1..64) in block `id`; ps.load is 0 for a
  // block number outside the pool, which the caller records as a bad block.  All of it
  // is wave-uniform scalar work (one unsigned compare against the pool size clamped to
  // 31 bits), done once per page.
  const uint32_t pool_blocks = num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)num_blocks;
  auto page_src_id = [&](int rows, int id) -> PageSrc {
    PageSrc ps;
    ps.load = (uint32_t)id < pool_blocks ? 1 : 0;
    if constexpr (kGather) {
      ps.base = (const char*)kv;
      ps.rows = src_row + (size_t)(ps.load ? (uint32_t)id : 0u) * kPage;
    } else if constexpr (kFp8) {
      ps.base = (const char*)kv + (size_t)(ps.load ? (uint32_t)id : 0u) * (kPage * kFp8RowBytes);
      ps.rows = nullptr;
    } else {
      ps.base = (const char*)kv + (size_t)(ps.load ? (uint32_t)id : 0u) * (kPage * kDqk * 2);
      ps.rows = nullptr;
    }
    ps.valid_rows = rows;
    return ps;
  };
  // gathered pages: this wave's 16 pool rows of a page (scalar loads), and each lane's
  // row of the two tail loads (lane l: row 8t + l/8 of the wave's 16), handed from the
  // scalars to the lanes through one VGPR (lane j holds row j) and a lane permute
  GatherRows grows;
  auto set_rows = [&]() __attribute__((always_inline)) {
    int all = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      asm("v_writelane_b32 %0, %1, %2" : "+v"(all) : "s"(grows.ridx[j]), "i"(j));
#pragma unroll
    for (int t = 0; t < 2; ++t)
      grows.tail[t] = __builtin_amdgcn_ds_bpermute((8 * t + (lane >> 3)) * 4, all);
  };
  // rows j0.. of this wave's 16 for page source ps
  auto load_ridx = [&](const PageSrc& ps, int j0) __attribute__((always_inline)) {
    if constexpr (kGather) {
      if (ps.load) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j >= j0) grows.ridx[j] = sload(ps.rows + 16 * wave + j);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < 16; ++j) grows.ridx[j] = 0;
  grows.tail[0] = grows.tail[1] = 0;
  // gathered pages: the first 8 of the wave's rows of page pf_blk of the current
  // segment, read one page early (at the start of the PV loop, once that page's block
  // number has arrived), so the page's first copies never wait for a scalar load; the
  // other 8 are read when the page starts and first used half-way through its scores
  constexpr int kPfRows = 8;
  int pf_ridx[kPfRows];
  int pf_blk = -1;
#pragma unroll
  for (int j = 0; j < kPfRows; ++j) pf_ridx[j] = 0;
  // valid rows of page blk of a sequence of length L, clamped to 1..64 whatever the plan says
  auto page_rows = [](int L, int blk) {
    const int rem = L - blk * kPage;
    return rem < 1 ? 1 : (rem < kPage ? rem : kPage);
  };
  auto page_src = [&](int s, int L, int blk) -> PageSrc {
    return page_src_id(page_rows(L, blk),
                       sload(block_table + (size_t)(s / groups) * max_blocks + blk));
  };
  // block number of page pre_blk of the current segment, read one page early (during
  // the softmax, where no LDS read waits behind the scalar load)
  int pre_id = 0, pre_blk = -1;

  if constexpr (kFp8) {
    // cleared before any wave can flag its first page
    if (threadIdx.x < 2) bad_scale_seg[threadIdx.x] = -1;
    __syncthreads();
  }
  int seg = seg_first;
  int blk = blk_first;
  int buf = 0;
  bool bad_block_next = false;  // a page of the next segment had a bad block number
  bool first_seg = true;

  while (true) {
    const int nb = first_seg ? nblk_first : seg_nblk(seg);
    const int blk_end = seg == seg_last ? blk_last_end : nb;
    const int b = seg / groups;
    const int rg = seg - b * groups;
    const int L = first_seg ? seqlen_first : sload(segt + (size_t)seg * kSegWords + S_SEQLEN);
    const int last_rows = page_rows(L, nb - 1);
    bool bad_block = bad_block_next;
    bad_block_next = false;
    const bool mismatch = sload(seqlens + b) != L;
    // read now, used by the epilogue: the loads complete while the pages run
    const int seg_nsplit = sload(segt + (size_t)seg * kSegWords + S_NSPLIT);
    const int seg_slot = sload(segt + (size_t)seg * kSegWords + S_SLOT);

    // this lane's query row
    const int row_in_group = wave * 32 + l32;
    const int row = rg * kGroupRows + row_in_group;
    const bool row_ok = row < M;
    const int t = row_ok ? row / heads : 0;
    const int hd = row_ok ? row - t * heads : 0;
    const int n_row = causal ? L - s_q + 1 + t : L;
    const int n_min = causal ? L - s_q + 1 : L;
    const bool wave_active = rg * kGroupRows + wave * 32 < M;

    // Q fragments: B operand of the score MFMA, k = 16*s + 8*h + j, column = row.  For the
    // first segment they are requested before the first page copy, so waiting for them
    // does not wait for the copy (loads complete in order).
    // Lanes of rows past the group's end (row_ok false) load row (t, hd) = (0, 0) of the
    // sequence instead: their scores and outputs are never stored, and the loads need no
    // per-load branch.
    bf16x8 qf[kKSteps];
    {
      // row (t, hd) of sequence b is row b*M + row of q, q_rs elements apart
      const __bf16* qrow = q + ((size_t)b * M + (row_ok ? row : 0)) * q_rs + 8 * h;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) qf[s] = *(const bf16x8*)(qrow + 16 * s);
    }
    if (first_seg) {
      PageSrc ps = page_src(seg, L, blk);
      bad_block = bad_block || ps.load == 0;
      if constexpr (kGather) {
        load_ridx(ps, 0);
        if (ps.load) set_rows();
      }
      issue_page<kGather, kFp8>(ps, lds0, wave, lane, tail_lane_off, grows, scale_lds, f8l);
      first_seg = false;
    }
    // The compiler waits for the Q loads here, not at their uses in the score loop:
    // it cannot see the page copies (issued from asm), so a wait it placed there (for
    // "all but the later Q loads") would also wait for copies in flight.  Here the
    // first page's copies are in flight anyway and the page wait follows.
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) asm volatile("" : "+v"(qf[s]));
    o_zero();
    // Q fragments and O (zeroed by VALU) are read by asm MFMAs only after
    // this fence and its wait states
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7" ::: "memory");
    float m_run = kNegBig, l_run = 0.f;
    pre_blk = -1;
    pf_blk = -1;
    bool first_page = true;

    for (; blk < blk_end; ++blk) {
      // where the next page comes from (this segment, or the next one with blocks)
      int nseg = seg, nblk = blk + 1;
      bool has_next = true;
      if (nblk >= blk_end) {
        nseg = seg + 1;
        nblk = 0;
        while (nseg <= seg_last && seg_nblk(nseg) == 0) ++nseg;
        has_next = nseg <= seg_last;
      }
      wait_dma();
      if constexpr (kFp8) {
        // each wave widens the rows its own copies filled (no barrier needed before), and
        // the barrier after it publishes the page (and any bad-scale flag) and ends every
        // wave's previous page
        if (__builtin_amdgcn_ballot_w64(fp8_convert(lds0 + buf * kBufBytes, scale_lds, wave,
                                                    lane)) != 0) {
          if (lane == 0) bad_scale_seg[seg & 1] = seg;
        }
      }
      __syncthreads();
      PageSrc nps;
      nps.load = 0;
      if (has_next) {
        if (nseg == seg) {
          // every page but the segment's last is full; its block number was prefetched
          nps = nblk == pre_blk ? page_src_id(nblk + 1 == nb ? last_rows : kPage, pre_id)
                                : page_src(nseg, L, nblk);
          bad_block = bad_block || nps.load == 0;
        } else {
          nps = page_src(nseg, sload(segt + (size_t)nseg * kSegWords + S_SEQLEN), nblk);
          bad_block_next = bad_block_next || nps.load == 0;
        }
      }
      const uint32_t next_lds = lds0 + (buf ^ 1) * kBufBytes;
      if constexpr (kFp8) {
        // a partial next page is copied here, whole; the score loop copies full pages
        if (nps.load && nps.valid_rows < kPage) {
          issue_fp8_partial(nps, next_lds, wave, lane, scale_lds, f8l);
          nps.load = 0;
        }
      }
      if constexpr (kGather) {
        if (nps.load && nseg == seg && nblk == pf_blk) {
#pragma unroll
          for (int j = 0; j < kPfRows; ++j) grows.ridx[j] = pf_ridx[j];
          load_ridx(nps, kPfRows);
        } else {
          load_ridx(nps, 0);
        }
      }
      if (!wave_active) {
        if constexpr (kGather) {
          if (nps.load) set_rows();
        }
        issue_page<kGather, kFp8>(nps, next_lds, wave, lane, tail_lane_off, grows, scale_lds, f8l);
        buf ^= 1;
        continue;
      }

      const lds_char* page = (const lds_char*)(uintptr_t)(lds0 + buf * kBufBytes);
      // ---- scores S^T = K . Q^T, two 32-token tiles ----
      // K fragments are read one k-step ahead of the MFMAs that use them; the
      // scheduling fences keep the compiler from hoisting every read (and its
      // registers) to the top.
      f32x16 sacc[2];
      auto kfrag = [&](int s, int T) -> bf16x8 {
        const lds_char* a;
        if (s < 32) {
          a = page + k_off + (main_row(32) * T) + s * 32;
        } else {
          const int c = (2 * (s - 32) + h) ^ ((l32 >> 1) & 7);
          a = page + kMainBytes + (T * 32 + l32) * kTailStride + c * 16;
        }
        return *(const bf16x8*)a;
      };
      bf16x8 kf[kKDepth + 1][2];
#pragma unroll
      for (int s = 0; s < kKDepth; ++s) {
        kf[s][0] = kfrag(s, 0);
        kf[s][1] = kfrag(s, 1);
      }
      auto score_step = [&](auto S_) __attribute__((always_inline)) {
        constexpr int s = decltype(S_)::value;
        if constexpr (s + kKDepth < kKSteps) {
          kf[(s + kKDepth) % (kKDepth + 1)][0] = kfrag(s + kKDepth, 0);
          kf[(s + kKDepth) % (kKDepth + 1)][1] = kfrag(s + kKDepth, 1);
        }
        const bf16x8& a0 = kf[s % (kKDepth + 1)][0];
        const bf16x8& a1 = kf[s % (kKDepth + 1)][1];
        // One copy instruction every other k-step, issued right after the step's first
        // MFMA: a vector-memory issue that stalls (the memory system is busy streaming
        // the cache) then overlaps that MFMA instead of delaying the LDS reads and MFMAs
        // behind it (~1,100 cycles per page less than issuing it first).
        // (gathered pages: the two tail copies follow the loop)
        constexpr bool part = (s & 1) == 0 && s / 2 < (kGather ? 16 : (kFp8 ? kFp8Parts : kPageParts));
        if constexpr (s == 0)
          mfma_s_first(sacc[0], a0, qf[s]);
        else
          mfma_s(sacc[0], a0, qf[s]);
        if constexpr (part)
          issue_page_part<kGather, kFp8, s / 2>(nps, next_lds, wave, lane, tail_lane_off, grows,
                                                scale_lds, f8l);
        if constexpr (s == 0)
          mfma_s_first(sacc[1], a1, qf[s]);
        else if constexpr (s + 1 < kKSteps)
          mfma_s(sacc[1], a1, qf[s]);
        else
          mfma_s_last(sacc[1], a1, qf[s]);
        __builtin_amdgcn_sched_barrier(0);
      };
      static_for<0, kKSteps>(score_step);
      if constexpr (kGather) {
        // each lane's rows for the two tail copies, now that all 16 row numbers are in
        if (nps.load) {
          set_rows();
          issue_page_part<kGather, kFp8, 16>(nps, next_lds, wave, lane, tail_lane_off, grows, scale_lds, f8l);
          issue_page_part<kGather, kFp8, 17>(nps, next_lds, wave, lane, tail_lane_off, grows, scale_lds, f8l);
        }
      }
      if (blk + 2 < blk_end) {
        pre_blk = blk + 2;
        pre_id = sload(block_table + (size_t)b * max_blocks + pre_blk);
      }
      // ---- causal / length mask, only for pages that reach past the shortest row's end ----
      const int tok0 = blk * kPage;
      if (tok0 + kPage > n_min) {
        asm volatile("");  // keeps this a branch rather than selects on every page
#pragma unroll
        for (int T = 0; T < 2; ++T) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = tok0 + 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
            if (tok >= n_row) sacc[T][r] = -INFINITY;
          }
        }
      }
      // ---- online softmax (log2 domain) ----
      // the max is taken on raw scores (the scale is positive) and the scale is folded
      // into the exponent's FMA
      float mx = -INFINITY;
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[T][r]);
      }
      mx = swap_halves_max(mx) * scale_log2;
      const float m_new = fmaxf(m_run, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack) != 0) {
        if (!first_page) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          o_scale(alpha);
        }
        m_run = m_new;
      }
      first_page = false;
      // P^T in bf16, one 16-token chunk per PV k-step (chunk 2T + g holds tile T's
      // accumulator values 8g .. 8g + 7).  Chunk 0 is computed here; each later chunk is
      // computed inside the PV loop, during the 16 MFMAs of the chunk before it, where
      // its VALU work runs beside the matrix unit instead of before it.
      u32x4 pk[4];
      float ev[8];
      auto p_exp = [&](int kc, int j) __attribute__((always_inline)) {
        ev[j] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(sacc[kc >> 1][8 * (kc & 1) + j], scale_log2, -m_run));
      };
      // The row sum adds the weights as the PV MFMAs use them, rounded to bf16 (each
      // packed half widened back to fp32 by a shift or a mask), so the normalisation
      // divides by the sum of exactly the weights the products applied: a single visible
      // key gets weight 1 and O equals its V row.
      auto p_pack = [&](int kc, int q) __attribute__((always_inline)) {
        uint32_t t = pack_bf16(ev[2 * q], ev[2 * q + 1]);
        asm volatile("" : "+v"(t));  // converted here, not merged with the chunk's others
        pk[kc][q] = t;
        l_run += __uint_as_float(t << 16) + __uint_as_float(t & 0xffff0000u);
      };
#pragma unroll
      for (int j = 0; j < 8; ++j) p_exp(0, j);
#pragma unroll
      for (int q = 0; q < 4; ++q) p_pack(0, q);
      // ---- O^T += V^T . P^T ----
      auto vfrag = [&](int i) -> bf16x8 {
        const int kc = i / kCTiles, ct = i % kCTiles;
        const lds_char* a = page + v_off + kc * main_row(16) + ct * 64;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3)))*)a);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3)))*)(a + (main_row(12) - main_row(4))));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // P and (after a rescale or zeroing) O were just written by VALU: fence the
      // scheduler, then wait states before the first MFMA reads them
      if constexpr (kGather) {
        // rows of the page after next (its block number was read during the softmax)
        if (pre_blk == blk + 2 && (uint32_t)pre_id < pool_blocks) {
          const int32_t* r = src_row + (size_t)pre_id * kPage + 16 * wave;
#pragma unroll
          for (int j = 0; j < kPfRows; ++j) pf_ridx[j] = sload(r + j);
          pf_blk = pre_blk;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7" ::: "memory");
      constexpr int kPv = 4 * kCTiles;
      bf16x8 vf[kVDepth + 1];
#pragma unroll
      for (int i = 0; i < kVDepth; ++i) vf[i] = vfrag(i);
      auto pv_step = [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        constexpr int kc = i / kCTiles, ct = i % kCTiles;
        if constexpr (i + kVDepth < kPv) vf[(i + kVDepth) % (kVDepth + 1)] = vfrag(i + kVDepth);
        // no wait states after the page's last PV MFMA: O^T is next read by VALU or
        // AGPR moves only at a rescale (after the next page's score MFMAs) or in the
        // epilogue, which waits for it
        o_pv(ct, vf[i % (kVDepth + 1)], __builtin_bit_cast(bf16x8, pk[kc]));
        // the next chunk's weights behind this MFMA: exponentials on the chunk's first 8
        // MFMAs, packing and row sums on the next 4, so at least 4 MFMAs separate the
        // last write of a chunk's P^T from the first MFMA that reads it
        if constexpr (kc < 3 && ct < 12) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (ct < 8)
            p_exp(kc + 1, ct);
          else
            p_pack(kc + 1, ct - 8);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      static_for<0, kPv>(pv_step);
      buf ^= 1;
    }

    // ---- epilogue: this segment's rows, whole or as one part ----
    // wait states for the last PV MFMA's O^T before it is read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    bool bad_scale = false;
    if constexpr (kFp8) bad_scale = bad_scale_seg[seg & 1] == seg;
    const bool bad = bad_block || mismatch || bad_scale;
    const bool whole = seg_nsplit == 1;
    const float l_tot = swap_halves_sum(l_run);
    float inv, lse_v;
    if (bad) {
      inv = __builtin_nanf("");
      lse_v = __builtin_nanf("");
    } else if (l_tot > 0.f) {
      inv = 1.0f / l_tot;
      lse_v = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    } else {
      inv = 0.f;
      lse_v = -INFINITY;
    }
    // One part of a split segment stores O_i in fp16 under a power-of-two scale per row
    // that puts the row's largest |O_i| in [2^14, 2^15), so every value keeps fp16's 11
    // significant bits and none overflows; the combine multiplies the scale back.  Half
    // the bytes of fp32 partials, written here and read again by the combine.
    int pe = 0;
    float inv_s = inv;
    if (wave_active && !whole) {
      float amax = 0.f;
#pragma unroll
      for (int ct = 0; ct < kCTiles; ++ct) {
        float v[16];
        o_read(ct, v);
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
      }
      amax = swap_halves_max(amax) * inv;
      pe = __builtin_amdgcn_frexp_expf(amax);   // amax in [2^(pe-1), 2^pe)
      pe = pe < -100 ? -100 : (pe > 100 ? 100 : pe);
      inv_s = inv * __builtin_ldexpf(1.f, 15 - pe);
    }
    // The rows are written through LDS so that every store covers whole rows: in the
    // accumulator layout a lane holds one row and a store instruction would touch 32
    // rows with 16 bytes each.  The last page's buffer is free once every wave is done
    // with its products (the next segment's first page, if any, is in flight into the
    // other buffer); each wave stages its own 32 rows in a quarter of it, in passes of
    // 512 bytes per row (256 fp16 or 128 fp32 columns).
    __syncthreads();
    if (wave_active) {
      constexpr int kStagePitch = 528;   // 512 bytes + 16: rows start 4 banks apart
      static_assert(4 * 32 * kStagePitch <= kBufBytes, "epilogue staging");
      typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
      typedef __attribute__((address_space(3))) f16x4 lds_f16x4;
      typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
      // lane values computed here, not hoisted to the kernel's start and kept live
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      const uint32_t stage = lds0 + (buf ^ 1) * kBufBytes + wave * 32 * kStagePitch;
      const uint32_t w_off = stage + (lane_e & 31) * kStagePitch + 8 * (lane_e >> 5);
      const int rr = lane_e >> 5, cl = lane_e & 31;              // read-back: row 2i + rr, chunk cl
      const int row_base = rg * kGroupRows + wave * 32;          // first row of this wave
      if (whole) {
        float* obase = out + ((size_t)b * M + row_base) * o_rs;
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int ct = 4 * pass + c4;
            float v[16];
            o_read(ct, v);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 o4 = {v[4 * g] * inv, v[4 * g + 1] * inv, v[4 * g + 2] * inv, v[4 * g + 3] * inv};
              *(lds_f32x4*)(uintptr_t)(w_off + (32 * c4 + 8 * g) * 4 + 8 * h) = o4;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            u32x4 x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              x[k] = *(const lds_u32x4*)(uintptr_t)(stage + (2 * (i + k) + rr) * kStagePitch + cl * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int r = 2 * (i + k) + rr;
              if (row_base + r < M) *(u32x4*)(obase + (size_t)r * o_rs + 128 * pass + 4 * cl) = x[k];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (row_ok && h == 0) lse_out[(size_t)b * M + row] = lse_v;
      } else {
        const int split = seg == seg_first ? split_first : 0;
        const size_t slot_i = (size_t)seg_slot + split;
        _Float16* obase = part_o + (slot_i * kGroupRows + wave * 32) * kDv;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8) {
            const int ct = 8 * pass + c8;
            float v[16];
            o_read(ct, v);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f16x4 o4 = {(_Float16)(v[4 * g] * inv_s), (_Float16)(v[4 * g + 1] * inv_s),
                          (_Float16)(v[4 * g + 2] * inv_s), (_Float16)(v[4 * g + 3] * inv_s)};
              *(lds_f16x4*)(uintptr_t)(w_off + (32 * c8 + 8 * g) * 2) = o4;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            u32x4 x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              x[k] = *(const lds_u32x4*)(uintptr_t)(stage + (2 * (i + k) + rr) * kStagePitch + cl * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int r = 2 * (i + k) + rr;
              if (row_base + r < M) *(u32x4*)(obase + (size_t)r * kDv + 256 * pass + 8 * cl) = x[k];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (row_ok && h == 0) {
          part_lse[slot_i * kGroupRows + row_in_group] = lse_v;
          part_scale[slot_i * kGroupRows + row_in_group] = __builtin_ldexpf(1.f, pe - 15);
        }
      }
    }
    if (bad && threadIdx.x == 0)
      atomicOr(&meta[H_STATUS], (bad_block ? MLA_STATUS_BAD_BLOCK : 0) |
                                    (mismatch ? MLA_STATUS_PLAN_MISMATCH : 0) |
                                    (bad_scale ? MLA_STATUS_BAD_SCALE : 0));

    // next segment with blocks
    int nseg = seg + 1;
    while (nseg <= seg_last && seg_nblk(nseg) == 0) ++nseg;
    if (nseg > seg_last) break;
    seg = nseg;
    blk = 0;
  }
}

}  // namespace

hipError_t launch_main_bf16(const Problem& p, hipStream_t stream) {
  const bool strided = p.q_rs != kDqk || p.o_rs != kDv;
  if (strided && (p.fp8 || p.src_row)) return hipErrorInvalidValue;
  if (p.fp8) {
    hipLaunchKernelGGL((mla_main_bf16_kernel<false, true, false>), dim3(p.num_wg), dim3(kThreads), 0,
                       stream, (const __bf16*)p.q, (const __bf16*)p.kv, nullptr, p.num_blocks,
                       p.block_table, p.max_blocks, p.seqlens, p.batch, p.s_q, p.heads, p.causal,
                       p.scale, p.out, p.lse, p.meta, p.meta, (_Float16*)p.part_o, p.part_lse,
                       p.part_scale, p.q_rs, p.o_rs);
  } else if (p.src_row) {
    hipLaunchKernelGGL((mla_main_bf16_kernel<true, false, false>), dim3(p.num_wg), dim3(kThreads), 0,
                       stream, (const __bf16*)p.q, (const __bf16*)p.kv, p.src_row, p.num_blocks,
                       p.block_table, p.max_blocks, p.seqlens, p.batch, p.s_q, p.heads, p.causal,
                       p.scale, p.out, p.lse, p.meta, p.meta, (_Float16*)p.part_o, p.part_lse,
                       p.part_scale, p.q_rs, p.o_rs);
  } else if (strided) {
    hipLaunchKernelGGL((mla_main_bf16_kernel<false, false, true>), dim3(p.num_wg),
                       dim3(kThreads), 0, stream, (const __bf16*)p.q, (const __bf16*)p.kv,
                       nullptr, p.num_blocks, p.block_table, p.max_blocks, p.seqlens, p.batch,
                       p.s_q, p.heads, p.causal, p.scale, p.out, p.lse, p.meta, p.meta,
                       (_Float16*)p.part_o, p.part_lse, p.part_scale, p.q_rs, p.o_rs);
  } else {
    hipLaunchKernelGGL((mla_main_bf16_kernel<false, false, false>), dim3(p.num_wg),
                       dim3(kThreads), 0, stream, (const __bf16*)p.q, (const __bf16*)p.kv,
                       nullptr, p.num_blocks, p.block_table, p.max_blocks, p.seqlens, p.batch,
                       p.s_q, p.heads, p.causal, p.scale, p.out, p.lse, p.meta, p.meta,
                       (_Float16*)p.part_o, p.part_lse, p.part_scale, p.q_rs, p.o_rs);
  }
  return hipGetLastError();
}

}  // namespace mla
