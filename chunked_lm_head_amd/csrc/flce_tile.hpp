// flce_tile.hpp - the bf16 MFMA tile engine shared by every contraction of the
// chunked LM-head + cross-entropy path on gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// 256 x 256 fp32 tile C[m][n] = sum_k A[m][k] B[n][k] with
// v_mfma_f32_32x32x16_bf16; each wave owns 128 x 128 of it as 4 x 4 MFMA blocks
// (256 fp32 accumulators per lane).  K advances 64 at a time through a
// double-buffered LDS pipeline (2 stages x (A + B) x 32 KiB = 128 KiB of the
// 160 KiB LDS).
//
// Operands are read with buffer loads whose descriptor covers exactly the
// valid bytes, and masked lanes use an offset past the descriptor's range, so
// ragged edges read zeros and no load can leave its tensor.  Two operand
// kinds exist:
//   * K-contiguous (row-major [mn][k], e.g. H and W in the logit GEMM): copied
//     global -> LDS with the direct-to-LDS form of buffer_load_dwordx4, no
//     registers involved;
//   * MN-contiguous (row-major [k][mn], e.g. W in dH = G W and H in
//     dW = G^T H): each thread loads an 8 x 8 block of bf16 into registers,
//     transposes it with v_perm_b32 and writes 8 k-contiguous rows to LDS.
// Both land in the same LDS layout: 256 rows of 64 bf16 (128 B), the 16-byte
// chunk c of row r stored at chunk c ^ ((r >> 1) & 7), so that the MFMA
// fragment reads (32 consecutive rows, one chunk) spread over all banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;

constexpr int kTile = 256;                                   // macro tile (rows = cols)
constexpr int kBK = 64;                                      // K per pipeline stage
constexpr int kThreads = 256;                                // 4 wave64s
constexpr int kOperandStageBytes = kTile * kBK * 2;          // 32 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;          // A + B
constexpr int kPipeBytes = 2 * kStageBytes;                  // 128 KiB, double buffered
constexpr uint32_t kOOB = 0x80000000u;                       // offset past every descriptor
constexpr int kRsrcWord3 = 0x00020000;                       // gfx9 raw buffer, 32-bit data

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                           kRsrcWord3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
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
// Operands.
// ---------------------------------------------------------------------------

// Row-major [mn][k]: element (r, k) at byte (r * ld + k) * 2 from the base.
struct OperandK {
  __amdgpu_buffer_rsrc_t rs;
  int ld;    // elements between rows
  int rows;  // valid rows of this tile (0..256)
  int kext;  // valid K extent (multiple of 8)
  struct Stage {};

  __device__ __forceinline__ void init(const uint16_t *base, int ld_, int rows_, int kext_) {
    ld = ld_;
    rows = rows_ < 0 ? 0 : rows_;
    kext = kext_ < 0 ? 0 : kext_;
    const uint32_t nbytes =
        (rows > 0 && kext > 0) ? (uint32_t)(((rows - 1) * ld + kext) * 2) : 0u;
    rs = make_rsrc(base, nbytes);
  }

  // Each wave copies 64 rows (8 instructions of 8 rows x 128 B) straight into LDS.
  __device__ __forceinline__ void prefetch(lds_t *stage, int k0, int wave, int lane, Stage &) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rbase = wave * 64 + i * 8;
      const int r = rbase + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);   // logical chunk stored at lane's slot
      const int k = k0 + c * 8;
      const bool ok = (r < rows) && (k < kext);
      const uint32_t voff = ok ? (uint32_t)(r * ld + k) * 2u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(stage + rbase * 128), 16, voff,
                                               0, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(lds_t *, int, Stage &) const {}
};

// Row-major [k][mn]: element (c, k) at byte (k * ld + c) * 2 from the base.
struct OperandMN {
  __amdgpu_buffer_rsrc_t rs;
  int ld;    // elements between k rows
  int cols;  // valid mn columns of this tile (0..256, multiple of 8)
  int kext;  // valid K extent
  struct Stage {
    u32x4 v[8];
  };

  __device__ __forceinline__ void init(const uint16_t *base, int ld_, int cols_, int kext_) {
    ld = ld_;
    cols = cols_ < 0 ? 0 : cols_;
    kext = kext_ < 0 ? 0 : kext_;
    const uint32_t nbytes =
        (cols > 0 && kext > 0) ? (uint32_t)(((kext - 1) * ld + cols) * 2) : 0u;
    rs = make_rsrc(base, nbytes);
  }

  // Thread (kb = tid % 8, cb = tid / 8) loads k rows kb*8 .. kb*8+7 of columns cb*8 .. cb*8+7.
  __device__ __forceinline__ void prefetch(lds_t *, int k0, int wave, int lane, Stage &st) const {
    const int tid = wave * 64 + lane;
    const int kb = tid & 7, c = (tid >> 3) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + kb * 8 + i;
      const bool ok = (k < kext) && (c < cols);
      const uint32_t voff = ok ? (uint32_t)(k * ld + c) * 2u : kOOB;
      st.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
    }
  }

  // Transpose the 8 x 8 block and store column j as LDS row cb*8 + j (8 consecutive k).
  __device__ __forceinline__ void commit(lds_t *stage, int tid, Stage &st) const {
    const int kb = tid & 7, cb = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = st.v[2 * e][j >> 1], b = st.v[2 * e + 1][j >> 1];
        o[e] = (j & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                       : __builtin_amdgcn_perm(b, a, 0x05040100u);
      }
      const int r = cb * 8 + j;
      const int phys = kb ^ ((r >> 1) & 7);
      *(lds_u32x4 *)(stage + r * 128 + phys * 16) = o;
    }
  }
};

// MFMA fragment: rows row0 .. row0+31 of a staged tile, k = 16*ks + 8*(lane/32) .. +7.
__device__ __forceinline__ bf16x8 read_frag(const lds_t *tile, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  const int c = ks * 2 + (lane >> 5);
  const int phys = c ^ ((r >> 1) & 7);
  return *(const lds_bf16x8 *)(tile + r * 128 + phys * 16);
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
};

// Row (within the wave's 128) of accumulator register r of block mb, for this lane.
__device__ __forceinline__ int acc_row(int mb, int r, int lane) {
  return mb * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

__device__ __forceinline__ void mma_stage(const lds_t *sA, const lds_t *sB, Acc &acc, int wm,
                                          int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = read_frag(sA, wm * 128 + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = read_frag(sB, wn * 128 + j * 32, ks, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
  }
}

// acc += A_tile * B_tile^T over nk K-steps of 64.  Ends with a barrier, so the
// caller may reuse the LDS pipeline area afterwards.
template <class OA, class OB>
__device__ __forceinline__ void tile_mainloop(const OA &A, const OB &B, int nk, lds_t *smem,
                                              Acc &acc, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  typename OA::Stage stA;
  typename OB::Stage stB;
  if (nk <= 0) return;
  A.prefetch(smem, 0, wave, lane, stA);
  B.prefetch(smem + kOperandStageBytes, 0, wave, lane, stB);
  A.commit(smem, tid, stA);
  B.commit(smem + kOperandStageBytes, tid, stB);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    lds_t *cur = smem + (kt & 1) * kStageBytes;
    lds_t *nxt = smem + ((kt & 1) ^ 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      A.prefetch(nxt, (kt + 1) * kBK, wave, lane, stA);
      B.prefetch(nxt + kOperandStageBytes, (kt + 1) * kBK, wave, lane, stB);
    }
    mma_stage(cur, cur + kOperandStageBytes, acc, wm, wn, lane);
    if (more) {
      A.commit(nxt, tid, stA);
      B.commit(nxt + kOperandStageBytes, tid, stB);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

}  // namespace flce
