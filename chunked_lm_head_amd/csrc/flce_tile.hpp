// flce_tile.hpp - the bf16 MFMA tile engine shared by every contraction of the
// chunked LM-head + cross-entropy path on gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// 256 x 256 fp32 tile C[m][n] = sum_k A(m, k) B(n, k) with
// v_mfma_f32_32x32x16_bf16; each wave owns 128 x 128 of it as 4 x 4 MFMA blocks
// (256 fp32 accumulators per lane, held in AGPRs).
//
// Pipeline: K advances 32 at a time through a 4-stage LDS ring (4 x 32 KiB);
// stage k + 3 is in flight while stage k is multiplied.  Every operand moves
// global -> LDS by the direct-to-LDS form of buffer_load_dwordx4 (no
// registers, no VALU), from a buffer descriptor that covers exactly the valid
// bytes; masked lanes use an offset past its end, so ragged edges read zeros
// and no load can leave its tensor.  One barrier per K step, placed between
// the two 16-wide halves of the step so that the fragment reads of the next
// stage overlap the MFMAs of the current one.
//
// Two operand layouts in global memory, two layouts in LDS:
//  * K-contiguous ([mn][k], e.g. H and W in the logit GEMM): LDS rows of 32 k
//    (64 B); chunk c of row r sits at chunk c ^ ((r >> 2) & 3).  Fragments are
//    ds_read_b128.
//  * MN-contiguous ([k][mn], e.g. W in dH = G W, H and G in dW = G^T H): LDS
//    rows of 256 mn (512 B) per k; 16-byte chunk c of row k sits at
//    c ^ (4 * (k & 3)).  Fragments are two ds_read_b64_tr_b16, which transpose
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
constexpr int kBK = 32;                                      // K per pipeline stage
constexpr int kStages = 4;                                   // LDS ring depth
constexpr int kThreads = 256;                                // 4 wave64s
constexpr int kOperandStageBytes = kTile * kBK * 2;          // 16 KiB
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
// Operands.  Each wave issues 4 DMA instructions per operand per stage.
// ---------------------------------------------------------------------------

// Row-major [mn][k]: element (r, k) at byte (r * ld + k) * 2 from base.
struct OperandK {
  static constexpr int kReads = 1;  // LDS reads per MFMA fragment
  const char *base;  // tile origin (row 0, k 0)
  uint32_t nbytes;   // valid bytes from base
  int kext;          // valid K extent (multiple of 8)
  uint32_t voff[4];  // per lane: row/chunk offset within a stage, kOOB for rows past the tile
  int kc[4];         // per lane: k offset of its chunk within a stage

  __device__ __forceinline__ void init(const uint16_t *base_, int ld, int rows, int kext_,
                                       int wave, int lane) {
    base = (const char *)base_;
    rows = rows < 0 ? 0 : rows;
    kext = kext_ < 0 ? 0 : kext_;
    nbytes = (rows > 0 && kext > 0) ? (uint32_t)((rows - 1) * ld + kext) * 2u : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 64 + i * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      kc[i] = c * 8;
      voff[i] = r < rows ? (uint32_t)(r * ld + c * 8) * 2u : kOOB;
    }
  }

  __device__ __forceinline__ void issue(lds_t *stage, int k0, int wave) const {
    const uint32_t adv = (uint32_t)k0 * 2u;
    const i32x4 rs = rsrc_words(base + adv, remaining(nbytes, adv));
    const bool full = k0 + kBK <= kext;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (full || k0 + kc[i] < kext) ? voff[i] : kOOB;
      dma16(rs, off, stage + (wave * 64 + i * 16) * (kBK * 2));
    }
  }

  // Rows row0 .. row0+31, k = 16 ks + 8 (lane / 32) .. +7.
  __device__ __forceinline__ static bf16x8 frag(const lds_t *stage, int row0, int ks, int lane) {
    const int r = row0 + (lane & 31);
    const int c = ks * 2 + (lane >> 5);
    const int phys = c ^ ((r >> 2) & 3);
    return *(const lds_bf16x8 *)(stage + r * (kBK * 2) + phys * 16);
  }
};

// Row-major [k][mn]: element (c, k) at byte (k * ld + c) * 2 from base.
struct OperandMN {
  static constexpr int kReads = 2;  // LDS reads per MFMA fragment
  const char *base;   // tile origin (k 0, column 0)
  uint32_t nbytes;    // valid bytes from base
  uint32_t row_bytes; // ld * 2
  int kext;           // valid K extent
  uint32_t voff[4];   // per lane: k-row/chunk offset within a stage, kOOB past the columns
  int kr[4];          // per lane: k row of its chunk within a stage

  __device__ __forceinline__ void init(const uint16_t *base_, int ld, int cols, int kext_,
                                       int wave, int lane) {
    base = (const char *)base_;
    cols = cols < 0 ? 0 : cols;
    kext = kext_ < 0 ? 0 : kext_;
    row_bytes = (uint32_t)ld * 2u;
    nbytes = (cols > 0 && kext > 0) ? (uint32_t)((kext - 1) * ld + cols) * 2u : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = wave * 8 + i * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (k & 3));
      kr[i] = k;
      voff[i] = c * 8 < cols ? (uint32_t)(k * ld + c * 8) * 2u : kOOB;
    }
  }

  __device__ __forceinline__ void issue(lds_t *stage, int k0, int wave) const {
    const uint32_t adv = (uint32_t)k0 * row_bytes;
    const i32x4 rs = rsrc_words(base + adv, remaining(nbytes, adv));
    const bool full = k0 + kBK <= kext;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (full || k0 + kr[i] < kext) ? voff[i] : kOOB;
      dma16(rs, off, stage + (wave * 8 + i * 2) * (kTile * 2));
    }
  }

  // Columns mn0 .. mn0+31 (one per lane % 32), k = 16 ks + 8 (lane / 32) .. +7.
  __device__ __forceinline__ static bf16x8 frag(const lds_t *stage, int mn0, int ks, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int c = (mn0 >> 3) + 2 * (g & 1) + ((j & 3) >> 1);
    const int sub = 8 * (j & 1);
    s16x4 h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = ks * 16 + 8 * (g >> 1) + 4 * half + (j >> 2);
      const int phys = c ^ (4 * (k & 3));
      h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(stage + k * (kTile * 2) + phys * 16 + sub));
    }
    const s16x4 lo = h[0], hi = h[1];
    const short v8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3],
                                                           hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }
};

// Row (within the wave's 128) of accumulator register r of block mb, for this lane.
__device__ __forceinline__ int acc_row(int mb, int r, int lane) {
  return mb * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

struct Acc {
  f32x16 v[4][4];  // [mb][nb]: rows mb*32.., cols nb*32.. of the wave's 128 x 128
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
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
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = acc_row(i, r, lane) < rows_valid ? 0.f : -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j][r] = x;
      }
  }
};

struct Frags {
  bf16x8 a[4], b[4];
};

// Scheduling pattern for one half step: the 16 MFMAs alternate with the NR LDS
// fragment reads of the other half and NV global->LDS loads, spread evenly, so
// that neither the matrix pipe nor the LDS queue sees a long burst (issue is in
// order per wave).
template <int NR, int NV, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < 16) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int nread = ((I + 1) * NR) / 16 - (I * NR) / 16;
    if constexpr (nread > 0) __builtin_amdgcn_sched_group_barrier(0x100, nread, 0);  // DS reads
    constexpr int nvmem = ((I + 1) * NV) / 16 - (I * NV) / 16;
    if constexpr (nvmem > 0) __builtin_amdgcn_sched_group_barrier(0x020, nvmem, 0);  // loads
    interleave<NR, NV, I + 1>();
  }
}

template <class OA, class OB>
__device__ __forceinline__ void load_frags(Frags &f, const lds_t *stage, int ks, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = OA::frag(stage, wm * 128 + i * 32, ks, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = OB::frag(stage + kOperandStageBytes, wn * 128 + j * 32, ks, lane);
}

__device__ __forceinline__ void mma(const Frags &f, Acc &acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.v[i][j], 0, 0, 0);
}

// Issues the first kStages-1 stages of a tile's K loop (after a barrier that
// frees the LDS ring, with no other vector-memory operation in flight).
// Stages past the end of K are issued too, as loads from an empty range that
// zero-fill ring slots nobody reads; the counts in pipe_run rely on it.
template <class OA, class OB>
__device__ __forceinline__ void pipe_prologue(const OA &A, const OB &B, lds_t *smem, int wave) {
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    A.issue(smem + s * kStageBytes, s * kBK, wave);
    B.issue(smem + s * kStageBytes + kOperandStageBytes, s * kBK, wave);
  }
}

// acc += A_tile * B_tile^T over nk >= 1 K-steps of 32, with the prologue
// already issued and its loads the only vector-memory operations in flight.
// Each step: MFMAs of the first 16-wide half (the second half's fragments
// loading in between), publish the next stage (wait for own loads, barrier),
// issue the stage three ahead, MFMAs of the second half (the next stage's
// first fragments and the new loads in between).  The last step is peeled so
// that the loop body has no branch.  Ends with all loads landed and a barrier,
// so the caller may reuse the LDS ring afterwards.
template <class OA, class OB>
__device__ __forceinline__ void pipe_run(const OA &A, const OB &B, int nk, lds_t *smem, Acc &acc,
                                         int wave, int lane) {
  constexpr int kReads = OA::kReads * 4 + OB::kReads * 4;  // LDS reads per half step
  const int wm = wave >> 1, wn = wave & 1;
  wait_vmcnt<16>();  // own loads of stage 0 landed; stages 1 and 2 may be in flight
  __syncthreads();
  Frags f0, f1;
  load_frags<OA, OB>(f0, smem, 0, wm, wn, lane);
  for (int kt = 0; kt < nk - 1; ++kt) {
    const lds_t *cur = smem + (kt & (kStages - 1)) * kStageBytes;
    load_frags<OA, OB>(f1, cur, 1, wm, wn, lane);
    mma(f0, acc);
    interleave<kReads, 0>();
    wait_vmcnt<8>();  // own loads of stage kt+1 landed (kt+2 may be in flight)
    __syncthreads();  // ... and everyone's; everyone is done with stage kt-1
    lds_t *st = smem + ((kt + 3) & (kStages - 1)) * kStageBytes;
    A.issue(st, (kt + 3) * kBK, wave);
    B.issue(st + kOperandStageBytes, (kt + 3) * kBK, wave);
    load_frags<OA, OB>(f0, smem + ((kt + 1) & (kStages - 1)) * kStageBytes, 0, wm, wn, lane);
    mma(f1, acc);
    interleave<kReads, 8>();
  }
  load_frags<OA, OB>(f1, smem + ((nk - 1) & (kStages - 1)) * kStageBytes, 1, wm, wn, lane);
  mma(f0, acc);
  mma(f1, acc);
  wait_vmcnt<0>();  // loads past the end still write LDS: let them land
  __syncthreads();
}

// acc += A_tile * B_tile^T over nk K-steps of 32.  Starts and ends with a
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
