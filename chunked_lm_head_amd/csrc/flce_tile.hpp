// flce_tile.hpp - the bf16 MFMA tile engine shared by every contraction of the
// chunked LM-head + cross-entropy path on gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// 256 x 256 fp32 tile C[m][n] = sum_k A(m, k) B(n, k) with
// v_mfma_f32_16x16x32_bf16; each wave owns 128 x 128 of it as 8 x 8 MFMA blocks
// (256 fp32 accumulators per lane, held in AGPRs).  On MI355X this shape
// sustains about 16% more bf16 throughput than 32x32x16 under the clock the
// chip holds at full load, which is why it is used although it needs the
// same LDS traffic per FLOP.
//
// Pipeline: K advances 64 at a time (two MFMA steps of 32) through a 2-stage
// LDS ring (2 x 64 KiB, A and B 32 KiB each); the next stage is in flight
// while the current one is multiplied.  Every operand moves global -> LDS by
// the direct-to-LDS form of buffer_load_dwordx4 (no registers, no VALU), from
// a buffer descriptor that covers exactly the valid bytes; masked lanes use an
// offset past its end, so ragged edges read zeros and no load can leave its
// tensor.  One barrier per stage, placed between the MFMAs of B blocks 0..3
// and 4..7 of its second step, so that the fragment reads of the next stage
// overlap the MFMAs of the current one.
//
// Two operand layouts in global memory, two layouts in LDS:
//  * K-contiguous ([mn][k], e.g. H and W in the logit GEMM): LDS rows of 64 k
//    (128 B); chunk c of row r sits at chunk c ^ k_swizzle(r).  Fragments are
//    ds_read_b128.
//  * MN-contiguous ([k][mn], e.g. W in dH = G W, G in dW = G^T H): LDS
//    rows of 256 mn (512 B) per k; 16-byte chunk c of row k sits at
//    c ^ mn_swizzle(k).  Fragments are two ds_read_b64_tr_b16, which transpose
//    4 x 4 blocks of 16-bit values across lanes: within each group of 16
//    lanes, lane i receives element i % 4 of the 8-byte chunks addressed by
//    lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group.
// Both swizzles make the fragment reads of a wave conflict-free across the
// LDS banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;

constexpr int kTile = 256;                                   // macro tile (rows = cols)
constexpr int kKS = 32;                                      // K per MFMA step
constexpr int kBK = 64;                                      // K per pipeline stage (2 steps)
constexpr int kStages = 2;                                   // LDS ring depth
constexpr int kThreads = 256;                                // 4 wave64s
constexpr int kOperandStageBytes = kTile * kBK * 2;          // 32 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;          // A + B
constexpr int kPipeBytes = kStages * kStageBytes;            // 128 KiB
constexpr uint32_t kOOB = 0x80000000u;                       // offset past every descriptor
constexpr int kRsrcWord3 = 0x00020000;                       // gfx9 raw buffer, 32-bit data

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                           kRsrcWord3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The same descriptor as 4 scalar dwords, for the inline-asm loads below.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = kRsrcWord3;
  return r;
}

// One direct-to-LDS load: every lane copies 16 bytes from rsrc + voff to LDS
// address lds + 16 * lane.  Written in assembly so that the compiler does not
// order later LDS reads of *other* ring stages behind it (it cannot tell the
// stages apart and would wait for every such load); the K loop orders them
// itself with explicit vmcnt waits and barriers.  M0 is saved and restored.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t voff, const lds_t *lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(m0));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Bytes left past an advance, kept in a scalar register so that the buffer
// descriptor stays scalar (a VALU saturating subtract would force a
// readfirstlane loop around every load).
__device__ __forceinline__ uint32_t remaining(uint32_t nbytes, uint32_t adv) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(adv < nbytes ? nbytes - adv : 0u));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with the vector-memory and LDS counters constrained (gfx9 encoding).
template <int VM, int LG>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LG << 8));
}

// Workgroup id -> logical tile id such that each XCD (ids are dealt to the 8
// XCDs round-robin) receives one contiguous range of logical ids.
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  const int xcd = bid & 7, pos = bid >> 3, q = n >> 3, r = n & 7;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + pos;
}

// Logical id -> (tm, tn) walking groups of `gm` tile rows column by column, so
// that workgroups running together share A tiles and B tiles.
__device__ __forceinline__ void grouped_tile(int L, int tiles_m, int tiles_n, int gm, int &tm,
                                             int &tn) {
  const int per_group = gm * tiles_n;
  const int g = L / per_group;
  const int first = g * gm;
  const int rows = min(tiles_m - first, gm);
  const int in = L - g * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

// ---------------------------------------------------------------------------
// Operands.  Each wave issues 8 DMA instructions per operand per stage.
// ---------------------------------------------------------------------------

// Chunk swizzle of the K-major LDS layout (rows of eight 16-byte chunks, one
// 128-byte line of global memory each): a fragment read takes chunk c of 16
// consecutive rows in each 16-lane group; folding the low three row bits into
// the chunk index spreads them over all banks (measured conflict-free with
// the LDS bank-conflict counter at every 2 KiB offset, for both K halves of a
// stage, where an unswizzled layout costs twelve extra cycles per read).
__device__ __forceinline__ int k_swizzle(int r) { return r & 7; }

// One stage's K slice of an operand: its buffer descriptor (scalar), first k,
// and whether the whole slice lies inside the valid K extent.
struct DmaSlice {
  i32x4 rs;
  int k0;
  bool full;
};

// Row-major [mn][k]: element (r, k) at byte (r * ld + k) * 2 from base.
// A stage holds 256 rows of 64 k (128 bytes); each wave loads 64 rows, one
// full row per 8 lanes, in 8 loads of 8 rows.
struct OperandK {
  static constexpr int kReads = 1;  // LDS reads per MFMA fragment
  static constexpr bool kGrouped = false;
  const char *base;  // tile origin (row 0, k 0)
  uint32_t nbytes;   // valid bytes from base
  int kext;          // valid K extent (multiple of 8)
  int kc;            // per lane: k offset of its chunk within a stage (the same in every load)
  uint32_t voff[8];  // per lane and load: row/chunk offset, kOOB for rows past the tile

  __device__ __forceinline__ void init(const uint16_t *base_, int ld, int rows, int kext_,
                                       int wave, int lane) {
    base = (const char *)base_;
    rows = rows < 0 ? 0 : rows;
    kext = kext_ < 0 ? 0 : kext_;
    nbytes = (rows > 0 && kext > 0) ? (uint32_t)((rows - 1) * ld + kext) * 2u : 0u;
    // rows of one load start at a multiple of 8, so the swizzle is lane-only
    const int c = (lane & 7) ^ k_swizzle(lane >> 3);
    kc = c * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (lane >> 3);
      voff[i] = r < rows ? (uint32_t)(r * ld + c * 8) * 2u : kOOB;
    }
  }

  // Descriptor of the K slice [k0, k0 + kBK) of every row.
  __device__ __forceinline__ DmaSlice prep(int k0) const {
    const uint32_t adv = (uint32_t)k0 * 2u;
    return DmaSlice{rsrc_words(base + adv, remaining(nbytes, adv)), k0, k0 + kBK <= kext};
  }
  // Load i (0..7) of this wave's share of a stage.
  __device__ __forceinline__ void issue_one(const DmaSlice &d, lds_t *stage, int i,
                                            int wave) const {
    const uint32_t off = (d.full || d.k0 + kc < kext) ? voff[i] : kOOB;
    dma16(d.rs, off, stage + (wave * 64 + i * 8) * (kBK * 2));
  }
  __device__ __forceinline__ void issue(lds_t *stage, int k0, int wave) const {
    const DmaSlice d = prep(k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(d, stage, i, wave);
  }

  // Rows row0 .. row0+15 (one per lane % 16), k = 32 kk + 8 (lane / 16) .. +7.
  __device__ __forceinline__ static bf16x8 frag(const lds_t *stage, int row0, int kk, int lane) {
    const int r = row0 + (lane & 15);
    const int c = 4 * kk + (lane >> 4);
    const int phys = c ^ k_swizzle(r);
    return *(const lds_bf16x8 *)(stage + r * (kBK * 2) + phys * 16);
  }
};

// Chunk swizzle of the MN-major LDS layout: rows k and k + 8 of a stage must
// differ so that the two 16-lane groups of one transpose read (same columns,
// k 8 apart) fall into different banks, and rows k .. k+3 so that the four
// k rows one read gathers do.
__device__ __forceinline__ int mn_swizzle(int k) { return 4 * (k & 3) + 2 * ((k >> 3) & 1); }

// Row-major [k][mn]: element (c, k) at byte (k * ld + c) * 2 from base.
// A stage holds 64 k rows of 256 columns (512 bytes); each wave loads 16 of
// them, two per load.
struct OperandMN {
  static constexpr int kReads = 2;  // LDS reads per MFMA fragment
  static constexpr bool kGrouped = false;
  const char *base;   // tile origin (k 0, column 0)
  uint32_t nbytes;    // valid bytes from base
  uint32_t row_bytes; // ld * 2
  int kext;           // valid K extent
  int kr0;            // per lane: k row of its chunk in load 0 (load i: kr0 + 2 i)
  uint32_t voff[8];   // per lane and load: k-row/chunk offset, kOOB past the columns

  __device__ __forceinline__ void init(const uint16_t *base_, int ld, int cols, int kext_,
                                       int wave, int lane) {
    base = (const char *)base_;
    cols = cols < 0 ? 0 : cols;
    kext = kext_ < 0 ? 0 : kext_;
    row_bytes = (uint32_t)ld * 2u;
    nbytes = (cols > 0 && kext > 0) ? (uint32_t)((kext - 1) * ld + cols) * 2u : 0u;
    kr0 = wave * 16 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kr0 + 2 * i;
      const int c = (lane & 31) ^ mn_swizzle(k);
      voff[i] = c * 8 < cols ? (uint32_t)(k * ld + c * 8) * 2u : kOOB;
    }
  }

  // Descriptor of the k rows [k0, k0 + kBK).
  __device__ __forceinline__ DmaSlice prep(int k0) const {
    const uint32_t adv = (uint32_t)k0 * row_bytes;
    return DmaSlice{rsrc_words(base + adv, remaining(nbytes, adv)), k0, k0 + kBK <= kext};
  }
  // Load i (0..7) of this wave's share of a stage.
  __device__ __forceinline__ void issue_one(const DmaSlice &d, lds_t *stage, int i,
                                            int wave) const {
    const uint32_t off = (d.full || d.k0 + kr0 + 2 * i < kext) ? voff[i] : kOOB;
    dma16(d.rs, off, stage + (wave * 16 + i * 2) * (kTile * 2));
  }
  __device__ __forceinline__ void issue(lds_t *stage, int k0, int wave) const {
    const DmaSlice d = prep(k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(d, stage, i, wave);
  }

  // Columns mn0 .. mn0+15 (one per lane % 16), k = 32 kk + 8 (lane / 16) ..
  // +7.  Lane j of a 16-lane group addresses 4 columns mn0 + 4 (j % 4) .. +3
  // of k row 32 kk + 8 g + 4 half + j / 4; the transpose hands lane i column
  // mn0 + i of the four k rows.
  __device__ __forceinline__ static bf16x8 frag(const lds_t *stage, int mn0, int kk, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int c = (mn0 >> 3) + ((j & 3) >> 1);
    const int sub = 8 * (j & 1);
    s16x4 h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = 32 * kk + 8 * g + 4 * half + (j >> 2);
      const int phys = c ^ mn_swizzle(k);
      h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(stage + k * (kTile * 2) + phys * 16 + sub));
    }
    const s16x4 lo = h[0], hi = h[1];
    const short v8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3],
                                                           hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }
};

// A bf16 block written in place of an fp32 block of the same shape: each
// 128-column group of a row keeps its values in the first half of the group's
// 512 bytes, so logical column k sits at bf16 position k + (k & ~127) of the
// row (every group followed by 128 unused positions).
__device__ __forceinline__ int grouped_col(int k) { return k + (k & ~127); }

// OperandK over such a grouped block: K (the columns) starts at logical
// column kbase, a multiple of kBK, so each stage's 64 columns lie inside one
// group and are contiguous.  `base` is the row origin (logical column 0).
struct OperandKG : OperandK {
  static constexpr bool kGrouped = true;
  int kbase;

  __device__ __forceinline__ void init(const uint16_t *row_base, int ld, int rows, int kbase_,
                                       int kext_, int wave, int lane) {
    OperandK::init(row_base, ld, rows, kext_, wave, lane);
    kbase = kbase_;
    nbytes = (rows > 0 && kext > 0)
                 ? (uint32_t)((rows - 1) * ld + grouped_col(kbase + kext - 1) + 1) * 2u
                 : 0u;
  }
  __device__ __forceinline__ DmaSlice prep(int k0) const {
    const uint32_t adv = (uint32_t)grouped_col(kbase + k0) * 2u;
    return DmaSlice{rsrc_words(base + adv, remaining(nbytes, adv)), k0, k0 + kBK <= kext};
  }
  __device__ __forceinline__ void issue(lds_t *stage, int k0, int wave) const {
    const DmaSlice d = prep(k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(d, stage, i, wave);
  }
};

// OperandMN over a grouped block: a tile of 256 logical columns starting at a
// multiple of 256 spans two groups; `base` is the tile's first column (its
// physical position, twice the logical one).  Only the per-lane column offsets
// differ from OperandMN.
struct OperandMNG : OperandMN {
  static constexpr bool kGrouped = true;
  __device__ __forceinline__ void init(const uint16_t *base_, int ld, int cols, int kext_,
                                       int wave, int lane) {
    base = (const char *)base_;
    cols = cols < 0 ? 0 : cols;
    kext = kext_ < 0 ? 0 : kext_;
    row_bytes = (uint32_t)ld * 2u;
    nbytes = (cols > 0 && kext > 0) ? (uint32_t)((kext - 1) * ld + grouped_col(cols - 1) + 1) * 2u
                                    : 0u;
    kr0 = wave * 16 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kr0 + 2 * i;
      const int c = (lane & 31) ^ mn_swizzle(k);
      voff[i] = c * 8 < cols ? (uint32_t)(k * ld + grouped_col(c * 8)) * 2u : kOOB;
    }
  }
};

// Row (within the wave's 128) of accumulator register r of block mb, for this
// lane; the column within the block is lane % 16.
__device__ __forceinline__ int acc_row(int mb, int r, int lane) {
  return mb * 16 + ((lane >> 4) << 2) + r;
}

struct Acc {
  f32x4 v[8][8];  // [mb][nb]: rows mb*16.., cols nb*16.. of the wave's 128 x 128
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][j][r] = 0.f;
  }
  // Zero, except rows >= rows_valid (wave-relative) start at -inf.  Their
  // operand rows read as zeros, so they end the K loop at exactly -inf, which
  // the log-sum-exp and softmax epilogues treat as absent without masking.
  __device__ __forceinline__ void init_rows(int rows_valid, int lane) {
    if (rows_valid >= 128) {
      zero();
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = acc_row(i, r, lane) < rows_valid ? 0.f : -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j][r] = x;
      }
  }
};

// Fragments of one K step: the wave's 8 A blocks, and 4 of its 8 B blocks.
struct FragA {
  bf16x8 a[8];
};
struct FragB {
  bf16x8 b[4];
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment q (0..11) of K step kk of a stage, in the order the first half
// step consumes them: A block 0, B blocks 0..3, A blocks 1..7.
template <class OA, class OB>
__device__ __forceinline__ void load_next_one(int q, FragA &fa, FragB &fb, const lds_t *stage,
                                              int kk, int wm, int wn, int lane) {
  if (q == 0)
    fa.a[0] = OA::frag(stage, wm * 128, kk, lane);
  else if (q < 5)
    fb.b[q - 1] = OB::frag(stage + kOperandStageBytes, wn * 128 + (q - 1) * 16, kk, lane);
  else
    fa.a[q - 4] = OA::frag(stage, wm * 128 + (q - 4) * 16, kk, lane);
}

template <class OA, class OB>
__device__ __forceinline__ void load_next(FragA &fa, FragB &fb, const lds_t *stage, int kk,
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int q = 0; q < 12; ++q) load_next_one<OA, OB>(q, fa, fb, stage, kk, wm, wn, lane);
}

// B block 4 + j of K step kk of a stage.
template <class OB>
__device__ __forceinline__ void load_bhi_one(int j, FragB &fb, const lds_t *stage, int kk,
                                             int wn, int lane) {
  fb.b[j] = OB::frag(stage + kOperandStageBytes, wn * 128 + 64 + j * 16, kk, lane);
}

// acc[mb][4 h + j] += A_mb B_(4 h + j) for the 32 blocks of half h.
template <int H>
__device__ __forceinline__ void mma_half(const FragA &fa, const FragB &fb, Acc &acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][4 * H + j] = mfma16(fa.a[i], fb.b[j], acc.v[i][4 * H + j]);
}

// Issues both stages of a tile's K loop (after a barrier that frees the LDS
// ring, with no other vector-memory operation in flight).  Stages past the
// end of K are issued too, as loads from an empty range that zero-fill ring
// slots; the counts in pipe_run rely on it.
template <class OA, class OB>
__device__ __forceinline__ void pipe_prologue(const OA &A, const OB &B, lds_t *smem, int wave) {
#pragma unroll
  for (int s = 0; s < kStages; ++s) {
    A.issue(smem + s * kStageBytes, s * kBK, wave);
    B.issue(smem + s * kStageBytes + kOperandStageBytes, s * kBK, wave);
  }
}

__device__ __forceinline__ lds_t *stage_of(lds_t *smem, int kt) {
  return smem + ((kt >> 1) & (kStages - 1)) * kStageBytes;
}

// How a K step takes part in refilling the ring.
enum StepLoads {
  kNoLoads,   // first step of a tile: the prologue filled both slots
  kPublish,   // second step of a stage: barrier, then the first 8 loads of the refill
  kFinish,    // first step of a later stage: the last 8 loads of the refill
};

// One K step kt (32 wide) that is not the last, scheduled by hand in groups
// of four MFMAs (A block g against four B blocks); no instruction crosses a
// group boundary, so the memory work stays spread over the matrix work:
//  * first half (B blocks 0..3): groups 0..3 each read one of B blocks 4..7
//    of this step; on kFinish steps each group also issues one load (B);
//  * on kPublish steps: wait until the next stage has landed, barrier; this
//    stage's slot is then refilled with the stage after next, one load (A)
//    per group of the second half and one per group of the next step's
//    first half, so that the load unit (about 64 bytes per clock per CU,
//    half of which a full-rate stage needs) is never handed a burst;
//  * second half (B blocks 4..7): groups 0..5 read two fragments each of
//    step kt+1 into `nxt` and `blo`.
// The ring holds the stage being multiplied and the next one, so each
// barrier covers a stage (two K steps); the last load of a refill still has
// a full K step to land.
//
// The barrier carries no memory fence of its own: the wait just before it
// covers what it must order (the next stage's loads landed, every read of
// this stage, whose slot the loads issued after it overwrite, returned).
template <StepLoads kLoads, class OA, class OB>
__device__ __forceinline__ void pipe_step(const OA &A, const OB &B, int kt, lds_t *smem,
                                          Acc &acc, const FragA &cur, FragA &nxt, FragB &blo,
                                          FragB &bhi, DmaSlice &da, DmaSlice &db, int wave,
                                          int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  lds_t *cst = stage_of(smem, kt);
  lds_t *fill = stage_of(smem, kt - 1);  // the slot a kFinish step refills
#pragma unroll
  for (int g = 0; g < 8; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[g][j] = mfma16(cur.a[g], blo.b[j], acc.v[g][j]);
    if (g < 4) load_bhi_one<OB>(g, bhi, cst, kt & 1, wn, lane);
    if constexpr (kLoads == kFinish) B.issue_one(db, fill + kOperandStageBytes, g, wave);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kLoads == kPublish) {
    // All loads landed (nothing newer is in flight) and every LDS read of this
    // wave returned, the B block reads of this step among them.
    wait_vm_lgkm<0, 0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = ((kt >> 1) + kStages) * kBK;
    da = A.prep(k0);
    db = B.prep(k0);
  }
  const lds_t *nst = stage_of(smem, kt + 1);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[g][4 + j] = mfma16(cur.a[g], bhi.b[j], acc.v[g][4 + j]);
    if constexpr (kLoads == kPublish) A.issue_one(da, cst, g, wave);
    if (g < 6) {
      load_next_one<OA, OB>(2 * g, nxt, blo, nst, (kt + 1) & 1, wm, wn, lane);
      load_next_one<OA, OB>(2 * g + 1, nxt, blo, nst, (kt + 1) & 1, wm, wn, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The last K step: no further stage to publish or load.
template <class OB>
__device__ __forceinline__ void pipe_last(int kt, lds_t *smem, Acc &acc, const FragA &cur,
                                          FragB &blo, FragB &bhi, int wave, int lane) {
  const int wn = wave & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) load_bhi_one<OB>(j, bhi, stage_of(smem, kt), kt & 1, wn, lane);
  mma_half<0>(cur, blo, acc);
  mma_half<1>(cur, bhi, acc);
}

// acc += A_tile * B_tile^T over nk >= 1 K steps of 32, with the prologue
// already issued and its loads the only vector-memory operations in flight.
// The loop runs one stage (two steps, the second publishing) per iteration,
// so that the two A fragment sets swap roles without register copies.  The
// step count is rounded up to whole stages, at least 2: the extra steps read
// k past the end, which the loads zero-fill, and add exact zeros.  The first
// stage runs before the loop, so that every value the loop carries comes out
// of an MFMA: equal starting values (all zeros) entering the loop would be
// merged into one register, and the accumulators shuffled between registers
// on every pass.  Ends with all loads landed and a barrier, so the caller may
// reuse the LDS ring afterwards.
template <class OA, class OB>
__device__ __forceinline__ void pipe_run(const OA &A, const OB &B, int nk, lds_t *smem, Acc &acc,
                                         int wave, int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  const int n2 = nk <= 4 ? 4 : (nk + 1) & ~1;
  wait_vmcnt<8 + 8>();  // own loads of stage 0 landed; stage 1's 16 may be in flight
  __syncthreads();
  FragA f0, f1;
  FragB blo, bhi;
  DmaSlice da, db;
  load_next<OA, OB>(f0, blo, smem, 0, wm, wn, lane);
  pipe_step<kNoLoads>(A, B, 0, smem, acc, f0, f1, blo, bhi, da, db, wave, lane);
  pipe_step<kPublish>(A, B, 1, smem, acc, f1, f0, blo, bhi, da, db, wave, lane);
  for (int kt = 2; kt < n2 - 2; kt += 2) {
    pipe_step<kFinish>(A, B, kt, smem, acc, f0, f1, blo, bhi, da, db, wave, lane);
    pipe_step<kPublish>(A, B, kt + 1, smem, acc, f1, f0, blo, bhi, da, db, wave, lane);
  }
  pipe_step<kFinish>(A, B, n2 - 2, smem, acc, f0, f1, blo, bhi, da, db, wave, lane);
  pipe_last<OB>(n2 - 1, smem, acc, f1, blo, bhi, wave, lane);
  wait_vmcnt<0>();  // loads past the end still write LDS: let them land
  __syncthreads();
}

// acc += A_tile * B_tile^T over nk K steps of 32.  Starts and ends with a
// barrier, so the caller may use the LDS area before and after.
template <class OA, class OB>
__device__ __forceinline__ void tile_mainloop(const OA &A, const OB &B, int nk, lds_t *smem,
                                              Acc &acc, int wave, int lane) {
  wait_vmcnt<0>();  // no older vector-memory operation may hide in the counts below
  __syncthreads();
  if (nk <= 0) return;
  pipe_prologue(A, B, smem, wave);
  pipe_run(A, B, nk, smem, acc, wave, lane);
}

}  // namespace flce
