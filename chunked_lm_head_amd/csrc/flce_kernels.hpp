// flce_kernels.hpp - HIP kernels of the chunked LM-head + cross-entropy path.
//
// Forward (Unsloth GRPO long-context page, section "Chunking der abgeflachten
// Sequenzlaenge": chunked logits kept in fp32, selective log-softmax; TRL v1.13
// article, section on the four hurdles: chunked NLL):
//   fwd_lse     one launch over (256-token tile, vocabulary split) pairs.  Each
//               workgroup walks the 256-row vocabulary tiles of its split,
//               computing the logit tile z^T = W_tile H_tile^T on MFMA and
//               folding it at once into a running (max, sum exp) per token, in
//               base 2; it also picks out the label's logit.  Logits never
//               leave registers.  Output: per-(split, token) partials.
//   fwd_combine merges the splits -> lse, per-token NLL / log-prob.
//   fwd_mean    fixed-order sum over tokens -> mean over non-ignored tokens.
// Backward (same page, section "Auslagern von Aktivierungen fuer Log-Softmax":
// recompute, then back-propagate the per-token grad_output):
//   bwd_prep    per-token scale c_t and lse_t * log2(e).
//   bwd_grad    recomputes one logit tile and writes
//               G = c_t (softmax - onehot) as bf16 into a bounded block of the
//               workspace ([rows of a row block] x [vocabulary chunk]).
//   bwd_dh      fp32 partial sums of G W for the row block (split over K).
//   bwd_dw      dW (+)= G^T H for the vocabulary chunk.
//   bwd_dh_out  sums the K splits and rounds grad_hidden to bf16.
//
// Accumulators are read in the epilogues through acc_read(), one register at a
// time where it is consumed, so that they stay in AGPRs and the epilogue needs
// few VGPRs.
#pragma once

#include "flce_tile.hpp"

namespace flce {

constexpr float kInf = __builtin_inff();

// One accumulator value out of its AGPR, at the point of use.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

__device__ __forceinline__ void store_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), rs, off, 0, 0);
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

// Per lane and token column: which accumulator register (4 mb + r) of the
// wave's 128 rows holds vocabulary row `rel` (-1 if none): row = 16 mb +
// 4 (lane / 16) + r.
__device__ __forceinline__ int label_reg(int rel, int lane) {
  if ((unsigned)rel >= 128u) return -1;
  if (((rel >> 2) & 3) != (lane >> 4)) return -1;
  return (rel >> 4) * 4 + (rel & 3);
}

// Per-logit transform before the log-softmax (the chunked call's
// logit_scale_multiply / logit_scale_divide / logit_softcapping / temperature
// on the Unsloth GRPO page, section "Chunking der abgeflachten
// Sequenzlaenge"), in the order multiply, divide, cap * tanh(. / cap),
// divide by temperature.  Without a cap the whole transform is one positive
// scale, folded into the base-2 prescale of the exponentials; with a cap
// (kCap kernels) it is applied per logit.  Every factor is positive, so the
// transform is increasing and the running maximum stays a maximum.
struct Xform {
  float zscale;    // no cap: the whole transform (z' = z * zscale); cap: multiply / divide
  float cap;       // cap kernels only
  float inv_cap;
  float inv_temp;
};

// tanh through the hardware base-2 exponential: 1 - 2 / (1 + e^(2u)); exact
// limits +-1 for large |u|, absolute error about 1e-7 near 0.
__device__ __forceinline__ float tanh_exp2(float u) {
  const float e = fast_exp2(u * (2.f * kLog2e));
  return 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e);
}

// Capped transform of one raw logit; -inf (rows past the vocabulary) stays -inf.
__device__ __forceinline__ float xform_cap(float z, const Xform &x, float &t) {
  t = tanh_exp2(z * x.zscale * x.inv_cap);
  return z == -kInf ? -kInf : x.cap * t * x.inv_temp;
}

// Merges two (max, sum of 2^(x - max)) pairs of the base-2 log-sum-exp.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  float S = 0.f;
  if (M != -kInf)
    S = (m == -kInf ? 0.f : s * fast_exp2(m - M)) + (m2 == -kInf ? 0.f : s2 * fast_exp2(m2 - M));
  m = M;
  s = S;
}

// ---------------------------------------------------------------------------
// Forward: fused logit GEMM + online log-sum-exp + label gather.
// ---------------------------------------------------------------------------
struct FwdLseParams {
  const uint16_t *hidden;   // [T, D] bf16
  const uint16_t *weight;   // [V, D] bf16
  const int64_t *labels;    // [T], or null: no label logits (zlab is not written)
  int64_t ignore_index;
  int T, D, V;
  int n_tt, n_vt, splits, T_pad;
  Xform xf;                 // logit transform (z below is the transformed logit)
  float *part_m;            // [splits, T_pad] running max of z*log2(e)
  float *part_s;            // [splits, T_pad] sum of 2^(z*log2(e) - max)
  float *zlab;              // [T_pad] logit of the label
  const int *act_list;      // token tiles to compute (fwd_skip_prep_kernel), or null: all
  const int *n_act;         // their count
  const int *splits_eff;    // with a list: the vocabulary splits to use (<= splits)
};

constexpr int kLdsFwd = kPipeBytes;  // the partial-merge exchange reuses the ring

template <bool kCap>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) fwd_lse_kernel(FwdLseParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kLdsFwd];
  lds_t *smem = (lds_t *)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // With a tile list, the first n_act * splits workgroups take the listed tiles, spread
  // over the XCDs as the whole grid would be (a workgroup's XCD is its index mod 8),
  // and the rest exit: the work stays balanced whichever tiles drop out.
  int n_rows = p.n_tt, n_wg = (int)gridDim.x, splits = p.splits;
  if (p.act_list) {
    n_rows = *p.n_act;
    splits = *p.splits_eff;
    n_wg = n_rows * splits;
    if ((int)blockIdx.x >= n_wg) return;
  }
  int tt, sp;
  grouped_tile(xcd_contiguous(blockIdx.x, n_wg), n_rows, splits, 8, tt, sp);
  if (p.act_list) tt = p.act_list[tt];
  const int vt0 = (int)((int64_t)sp * p.n_vt / splits);
  const int vt1 = (int)((int64_t)(sp + 1) * p.n_vt / splits);
  const int t0 = tt * kTile;

  OperandK B;
  B.init(p.hidden + (size_t)t0 * p.D, p.D, min(kTile, p.T - t0), p.D, wave, lane);
  const int nk = (p.D + kKS - 1) / kKS;

  int lab[8];
  float mrun[8], srun[8], zl[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int t = t0 + wn * 128 + nb * 16 + (lane & 15);
    int y = -1;
    if (p.labels && t < p.T) {  // no labels: log-sum-exp only
      const int64_t yy = p.labels[t];
      if (yy != p.ignore_index && yy >= 0 && yy < p.V) y = (int)yy;
    }
    lab[nb] = y;
    mrun[nb] = -kInf;
    srun[nb] = 0.f;
    zl[nb] = 0.f;
  }
  unsigned have = 0;  // bit nb: this lane captured the label logit of token column nb
  const float ks = p.xf.zscale * kLog2e;  // base-2 prescale of the uncapped transform

  // The next vocabulary tile's first stages are issued before the current
  // tile's epilogue, which touches neither LDS nor memory.
  OperandK A;
  A.init(p.weight + (size_t)vt0 * kTile * p.D, p.D, min(kTile, p.V - vt0 * kTile), p.D, wave,
         lane);
  wait_vmcnt<0>();
  __syncthreads();
  pipe_prologue(A, B, smem, wave);
  Acc acc;
  for (int vt = vt0; vt < vt1; ++vt) {
    const int v0 = vt * kTile;
    const int vw = v0 + wm * 128;  // first vocabulary row of this wave's half
    acc.init_rows(p.V - vw, lane);  // rows past the vocabulary end at -inf
    pipe_run(A, B, nk, smem, acc, wave, lane);
    if (vt + 1 < vt1) {
      A.init(p.weight + (size_t)(v0 + kTile) * p.D, p.D, min(kTile, p.V - v0 - kTile), p.D,
             wave, lane);
      pipe_prologue(A, B, smem, wave);
    }

#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      // label logit: exactly one (tile, wave, lane, register) holds it
      const int lr = label_reg(lab[nb] - vw, lane);
      if (__builtin_amdgcn_ballot_w64(lr >= 0)) {
#pragma unroll
        for (int q = 0; q < 32; ++q)
          if (lr == q) zl[nb] = acc_read(acc.v[q >> 2][nb][q & 3]);
        if (lr >= 0) have |= 1u << nb;
      }
      float zmax = -kInf;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) zmax = fmaxf(zmax, acc_read(acc.v[mb][nb][r]));
      const float mold = mrun[nb];
      float t;
      const float mnew =
          fmaxf(mold, kCap ? xform_cap(zmax, p.xf, t) * kLog2e : zmax * ks);  // increasing
      if (mnew != -kInf) {
        float s = 0.f;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc_read(acc.v[mb][nb][r]);
            if constexpr (kCap)
              s += fast_exp2(__builtin_fmaf(xform_cap(z, p.xf, t), kLog2e, -mnew));
            else
              s += fast_exp2(__builtin_fmaf(z, ks, -mnew));
          }
        srun[nb] = (mold == -kInf ? 0.f : srun[nb] * fast_exp2(mold - mnew)) + s;
        mrun[nb] = mnew;
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    if (have & (1u << nb)) {
      float t;
      p.zlab[t0 + wn * 128 + nb * 16 + (lane & 15)] =
          kCap ? xform_cap(zl[nb], p.xf, t) : zl[nb] * p.xf.zscale;
    }
  }

  // Merge the four lanes holding one token (l, l ^ 16, l ^ 32, l ^ 48), then
  // the two waves (wm).
  lds_f32x2 *xch = (lds_f32x2 *)smem;  // [wn][nb][16], in the (idle) ring
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    lse_merge(mrun[nb], srun[nb], __shfl_xor(mrun[nb], 16), __shfl_xor(srun[nb], 16));
    lse_merge(mrun[nb], srun[nb], __shfl_xor(mrun[nb], 32), __shfl_xor(srun[nb], 32));
    if (wm == 1 && lane < 16) xch[(wn * 8 + nb) * 16 + lane] = f32x2{mrun[nb], srun[nb]};
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const f32x2 o = xch[(wn * 8 + nb) * 16 + lane];
      float M = mrun[nb], S = srun[nb];
      lse_merge(M, S, o[0], o[1]);
      const int t = t0 + wn * 128 + nb * 16 + lane;
      p.part_m[(size_t)sp * p.T_pad + t] = M;
      p.part_s[(size_t)sp * p.T_pad + t] = S;
    }
  }
}

constexpr int kCuCount = 256;  // compute units of an MI355X (8 XCDs of 32)

// The token tiles holding at least one token whose label is not ignore_index, in
// order, for a forward that leaves the others out: act_list[0, *n_act) and a flag per
// tile.  One block; a wave tests a tile (four labels per lane), then a block-wide scan
// numbers the active tiles of each group of 1024.  It also picks the forward's
// vocabulary splits for that many tiles (*splits_eff, at most max_splits, the partial
// buffers' capacity): the s that minimises ceil(n_act * s / 256) * ceil(n_vt / s), the
// rounds of one workgroup per CU times the vocabulary tiles each walks (ties: the
// larger s).
struct FwdSkipPrepParams {
  const int64_t *labels;
  int64_t ignore_index;
  int T, n_tt, n_vt, max_splits;
  uint8_t *tile_act;  // [n_tt]
  int *act_list;      // [n_tt]
  int *n_act;
  int *splits_eff;
};

// Numbers the flagged tiles (flags[0, n) of 0 / 1, written by this block before the
// call) in order: list[0, *count) by a block-wide scan over groups of 1024 flags, and
// returns the count to every thread.  For a block of 1024 threads; scan is 1024 ints of
// LDS.
__device__ __forceinline__ int list_flagged(const uint8_t *flags, int n, int *list, int *count,
                                            int *scan) {
  __syncthreads();  // the block's flag stores are visible to it
  int base = 0;
  for (int g = 0; g < n; g += 1024) {
    const int tt = g + (int)threadIdx.x;
    const int f = tt < n ? flags[tt] : 0;
    scan[threadIdx.x] = f;
    __syncthreads();
    for (int w = 1; w < 1024; w <<= 1) {  // inclusive Hillis-Steele scan
      const int v = (int)threadIdx.x >= w ? scan[threadIdx.x - w] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    if (f) list[base + scan[threadIdx.x] - 1] = tt;
    base += scan[1023];
    __syncthreads();  // scan[1023] read by all before the next group overwrites it
  }
  if (threadIdx.x == 0) *count = base;
  return base;
}

__global__ void __launch_bounds__(1024) fwd_skip_prep_kernel(FwdSkipPrepParams p) {
  __shared__ int scan[1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int tt = wave; tt < p.n_tt; tt += 1024 / 64) {
    int any = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tt * kTile + lane * 4 + j;
      if (t < p.T) any |= p.labels[t] != p.ignore_index;
    }
    const bool act = __builtin_amdgcn_ballot_w64(any) != 0;
    if (lane == 0) p.tile_act[tt] = act;
  }
  const int n = max(list_flagged(p.tile_act, p.n_tt, p.act_list, p.n_act, scan), 1);
  if (threadIdx.x == 0) {
    int best = 1;
    int64_t best_cost = (int64_t)((n + kCuCount - 1) / kCuCount) * p.n_vt;
    for (int s = 2; s <= min(p.max_splits, p.n_vt); ++s) {
      const int64_t cost = (((int64_t)n * s + kCuCount - 1) / kCuCount) * ((p.n_vt + s - 1) / s);
      if (cost <= best_cost) {
        best = s;
        best_cost = cost;
      }
    }
    *p.splits_eff = best;
  }
}

struct FwdCombineParams {
  const float *part_m, *part_s, *zlab;
  const uint8_t *tile_act;  // token tiles the forward computed, or null: all
  const int *splits_eff;    // the forward's split count when it took a tile list, or null
  const int64_t *labels;
  int64_t ignore_index;
  int T, V, splits, T_pad, mode;
  int lanes;  // lanes merging one token's split partials: a power of two <= 64
  float *out, *lse;
  double *blk_sum;
  int *blk_cnt;
};

// Per token: merge the splits' (max, sum) partials into lse, then out and the
// block's share of the mean.  `lanes` lanes of one wave merge one token's
// partials (lane j takes splits j, j + lanes, ...) and a fixed shuffle tree
// combines them; a block takes 256 / lanes tokens.  So many splits (small T,
// large V) spread over many blocks instead of serialising on one thread, and
// the result is the same on every run.
__global__ void __launch_bounds__(256) fwd_combine_kernel(FwdCombineParams p) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  const int L = p.lanes, g = threadIdx.x / L, j = threadIdx.x % L, per = 256 / L;
  const int splits = p.splits_eff ? *p.splits_eff : p.splits;
  double contrib = 0.0;
  int cnt = 0;
  {
    const int t = blockIdx.x * per + g;
    float M = -kInf, S = 0.f;  // a tile left out keeps the empty sum: lse -inf
    if (t < p.T && (!p.tile_act || p.tile_act[t / kTile])) {
      for (int s = j; s < splits; s += L)
        lse_merge(M, S, p.part_m[(size_t)s * p.T_pad + t], p.part_s[(size_t)s * p.T_pad + t]);
    }
    for (int w = 1; w < L; w <<= 1) {  // lanes of a group stay within one wave
      const float m2 = __shfl_xor(M, w), s2 = __shfl_xor(S, w);
      lse_merge(M, S, m2, s2);
    }
    if (j == 0 && t < p.T) {
      const float lse = (M + fast_log2(S)) * kLn2;
      const int64_t y = p.labels[t];
      float o;
      if (y == p.ignore_index) {
        o = 0.f;
      } else if (y < 0 || y >= p.V) {
        o = __builtin_nanf("");
        contrib += (double)o;
        ++cnt;
      } else {
        const float nll = lse - p.zlab[t];
        o = p.mode == 0 ? nll : -nll;
        contrib += (double)o;
        ++cnt;
      }
      p.out[t] = o;
      p.lse[t] = lse;
    }
  }
  ssum[threadIdx.x] = contrib;
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ssum[threadIdx.x] += ssum[threadIdx.x + w];
      scnt[threadIdx.x] += scnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    p.blk_sum[blockIdx.x] = ssum[0];
    p.blk_cnt[blockIdx.x] = scnt[0];
  }
}

__global__ void __launch_bounds__(256)
    fwd_mean_kernel(const double *blk_sum, const int *blk_cnt, int nblk, float *mean_out) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  double s = 0.0;
  int c = 0;
  for (int i = threadIdx.x; i < nblk; i += 256) {
    s += blk_sum[i];
    c += blk_cnt[i];
  }
  ssum[threadIdx.x] = s;
  scnt[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ssum[threadIdx.x] += ssum[threadIdx.x + w];
      scnt[threadIdx.x] += scnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean_out[0] = scnt[0] ? (float)(ssum[0] / (double)scnt[0]) : 0.f;
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------
// Token rows of a backward row block.  Without a list, row r of the block is token
// 256 tile0 + r.  With one (the token tiles that hold a token with a gradient, in order,
// from bwd_prep_kernel), the block holds list entries [tile0, tile0 + tiles_rb) and row r
// is token 256 list[tile0 + r / 256] + r % 256: tiles without gradient are left out and
// the others packed into the leading row blocks.  When every tile that holds a token is
// listed (*count == n_real) that is the same as no list.
struct RowMap {
  const int *list;   // or null
  const int *count;  // number of listed tiles
  int n_real;        // tiles that hold tokens: ceil(T / 256)
  int tile0;         // first tile (no list) or list entry of the block
  int tiles_rb;      // tiles per row block
};

// Tiles of the block to compute: `fallback` (the count as laid out) unless a list leaves
// tiles out; `ident` tells whether rows are laid out as without a list.  `cnt` is *count
// (read early by the caller, so that its latency overlaps other work), unused without a
// list.
__device__ __forceinline__ int rowmap_tiles(const RowMap &m, int cnt, int fallback, bool &ident) {
  ident = !m.list || cnt == m.n_real;
  return ident ? fallback : min(max(cnt - m.tile0, 0), m.tiles_rb);
}
__device__ __forceinline__ int rowmap_count(const RowMap &m) { return m.list ? *m.count : 0; }
// Token tile of the block's tile i.
__device__ __forceinline__ int rowmap_tile(const RowMap &m, bool ident, int i) {
  return ident ? m.tile0 + i : m.list[m.tile0 + i];
}


// Split layout of a row block's dH partial sums in the [splits, R, D] buffer: `s_eff` K
// splits whose sums lie `stride` rows apart.  As planned (splits, R apart) unless the block
// holds a list of tiles_m tiles, fewer than the planned splits can spread over the CUs:
// then as many splits as keep one round of workgroups, stacked tiles_m * 256 rows apart so
// that they fit the same buffer.  The dH kernel and bwd_dh_out_kernel both use it, and it
// depends on the block alone, so every chunk of the block lays its sums out alike.
__device__ __forceinline__ void dh_layout(bool ident, int tiles_m, int tiles_n, int splits,
                                          int tiles_rb, int R, int &s_eff, int &stride) {
  s_eff = splits;
  stride = R;
  if (ident || tiles_m <= 0) return;
  const int s2 = min(kCuCount / (tiles_m * tiles_n), splits * tiles_rb / tiles_m);
  if (s2 > splits) {
    s_eff = s2;
    stride = tiles_m * kTile;
  }
}

struct BwdPrepParams {
  const int64_t *labels;
  const float *lse;
  const float *grad_out;   // [T] or null
  const float *grad_mean;  // scalar or null
  int64_t ignore_index;
  int T, V, T_pad, mode;
  float *c;     // [T_pad] per-token scale (0 where the row has no gradient)
  float *lse2;  // [T_pad] lse * log2(e); +inf where c == 0 so softmax terms vanish
  int n_real;          // tiles that hold tokens: ceil(T / 256)
  uint8_t *tile_act;   // [n_real]: the tile holds a token with c != 0
  int *act_list;       // [n_real]: those tiles in order, *n_act of them
  int *n_act;
};

__global__ void __launch_bounds__(1024) bwd_prep_kernel(BwdPrepParams p) {
  __shared__ int scnt[1024];
  int cnt = 0;
  for (int t = threadIdx.x; t < p.T; t += 1024) cnt += (p.labels[t] != p.ignore_index);
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) scnt[threadIdx.x] += scnt[threadIdx.x + w];
    __syncthreads();
  }
  const int n_valid = scnt[0];
  const float sign = p.mode == 0 ? 1.f : -1.f;
  float gm = 0.f;
  if (!p.grad_out && n_valid > 0) gm = p.grad_mean[0] / (float)n_valid;
  for (int t = threadIdx.x; t < p.T_pad; t += 1024) {
    float c = 0.f, l2 = kInf;
    if (t < p.T) {
      const int64_t y = p.labels[t];
      if (y != p.ignore_index && y >= 0 && y < p.V) {
        c = sign * (p.grad_out ? p.grad_out[t] : gm);
        if (c != 0.f) l2 = p.lse[t] * kLog2e;
      }
    }
    if (c == 0.f) l2 = kInf;
    p.c[t] = c;
    p.lse2[t] = l2;
  }
  // Which token tiles carry any gradient, and their list: the backward GEMMs take only
  // those (G rows of the others are zero, so their dH rows are zero and they add
  // nothing to dW).  One wave per tile: each lane tests four of its 256 values.
  __syncthreads();  // the block's writes of c are visible to it
  const int lane = threadIdx.x & 63;
  for (int tt = threadIdx.x >> 6; tt < p.n_real; tt += 1024 / 64) {
    const f32x4 v = *(const f32x4 *)(p.c + (size_t)tt * kTile + lane * 4);
    const bool nz = (v[0] != 0.f) | (v[1] != 0.f) | (v[2] != 0.f) | (v[3] != 0.f);
    const bool act = __builtin_amdgcn_ballot_w64(nz) != 0;
    if (lane == 0) p.tile_act[tt] = act;
  }
  list_flagged(p.tile_act, p.n_real, p.act_list, p.n_act, scnt);
}

// dH rows of the token tiles without gradient are zero.  A block per tile.
__global__ void __launch_bounds__(256) bwd_zero_rows_kernel(const uint8_t *tile_act, int T,
                                                            int D, uint16_t *dH) {
  const int tt = blockIdx.x;
  if (tile_act[tt]) return;
  const int t0 = tt * kTile, rows = min(kTile, T - t0), per_row = D >> 3;
  for (int i = threadIdx.x; i < rows * per_row; i += 256) {
    const int r = i / per_row, c8 = (i - r * per_row) * 8;
    *(u32x4 *)(dH + (size_t)(t0 + r) * D + c8) = u32x4{0u, 0u, 0u, 0u};
  }
}

struct BwdGradParams {
  const uint16_t *hidden, *weight;
  const int64_t *labels;
  const float *c, *lse2;
  int64_t ignore_index;
  int T, D, V;
  int vc0;               // first vocabulary row of this chunk
  int n_vt;              // vocabulary tiles of the chunk that hold rows < V
  int tiles_n;           // token tiles of the row block as laid out
  RowMap map;            // the row block's token tiles
  Xform xf;              // logit transform; G is the gradient with respect to the raw logits
  uint16_t *G;           // [R, Gp] bf16, row = row of the block, col = vocab - vc0
  int Gp;
};

// G tiles of one row block and vocabulary chunk.  A workgroup keeps one
// token tile (the B operand, H rows) and walks a contiguous range of the
// chunk's vocabulary tiles, as the forward does: the next tile's first stages
// are issued before the current tile's epilogue, which writes its G values
// straight from registers (8 bytes per lane: four consecutive vocabulary
// entries of one token), so the load ring stays busy across tiles.  Token
// tiles past T and vocabulary tiles past V are skipped: no consumer reads
// those G rows, and the columns of a partial tile past V come out as exact
// zeros (their logits are -inf).
template <bool kCap>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_grad_kernel(BwdGradParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  lds_t *smem = (lds_t *)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // At most one workgroup per CU: n_here token tiles x vs vocabulary ranges with
  // n_here * vs <= 256 (so that no workgroup waits for a second round), spread over the
  // XCDs as a grid of exactly that size would be; the rest of the grid exits.
  bool ident;
  const int n_here = rowmap_tiles(p.map, rowmap_count(p.map), p.tiles_n, ident);
  const int vs = min(p.n_vt, max(1, kCuCount / max(n_here, 1)));
  const int n_wg = n_here * vs;
  if ((int)blockIdx.x >= n_wg) return;
  int tn, sp;
  grouped_tile(xcd_contiguous(blockIdx.x, n_wg), n_here, vs, 8, tn, sp);
  const int vt0 = (int)((int64_t)sp * p.n_vt / vs);
  const int vt1 = (int)((int64_t)(sp + 1) * p.n_vt / vs);
  const int t0 = rowmap_tile(p.map, ident, tn) * kTile;
  if (t0 >= p.T || vt0 >= vt1) return;

  // Per-token values of this lane's 8 token columns, loaded before any DMA.
  float cc[8], l2[8];
  int yy[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int t = t0 + wn * 128 + nb * 16 + (lane & 15);  // < rb0 + R <= T_pad
    cc[nb] = p.c[t];
    l2[nb] = p.lse2[t];
    yy[nb] = -1;
    if (cc[nb] != 0.f) yy[nb] = (int)p.labels[t];  // c != 0 implies 0 <= y < V
  }
  // uncapped: G = c s (P - onehot), P = 2^(z s log2 e - l2), s the whole scale
  const float ks = p.xf.zscale * kLog2e;
  // capped: G = c (P - onehot) dz'/dz, dz'/dz = scale (1 - t^2) / temperature
  const float dscale = p.xf.zscale * p.xf.inv_temp;

  OperandK B;
  B.init(p.hidden + (size_t)t0 * p.D, p.D, min(kTile, p.T - t0), p.D, wave, lane);
  const int nk = (p.D + kKS - 1) / kKS;
  OperandK A;
  int v0 = p.vc0 + vt0 * kTile;
  A.init(p.weight + (size_t)v0 * p.D, p.D, min(kTile, p.V - v0), p.D, wave, lane);
  wait_vmcnt<0>();
  __syncthreads();
  pipe_prologue(A, B, smem, wave);
  Acc acc;
  for (int vt = vt0; vt < vt1; ++vt) {
    v0 = p.vc0 + vt * kTile;
    const int vw = v0 + wm * 128;    // first vocabulary row of this wave's half
    acc.init_rows(p.V - vw, lane);  // rows past the vocabulary end at -inf, i.e. G = 0
    pipe_run(A, B, nk, smem, acc, wave, lane);
    if (vt + 1 < vt1) {
      A.init(p.weight + (size_t)(v0 + kTile) * p.D, p.D, min(kTile, p.V - v0 - kTile), p.D,
             wave, lane);
      pipe_prologue(A, B, smem, wave);
    }
    uint16_t *gcol = p.G + (vw - p.vc0);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int tl = tn * kTile + wn * 128 + nb * 16 + (lane & 15);  // row of G
      const float c = cc[nb];
      const int lr = label_reg(yy[nb] - vw, lane);
      const bool any_label = __builtin_amdgcn_ballot_w64(lr >= 0) != 0;
      const float cs = c * p.xf.zscale;
      uint16_t *grow = gcol + (size_t)tl * p.Gp;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        float g[4], d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = acc_read(acc.v[mb][nb][e]);
          if constexpr (kCap) {
            float tt;
            const float zt = xform_cap(z, p.xf, tt);
            g[e] = fast_exp2(__builtin_fmaf(zt, kLog2e, -l2[nb]));
            d[e] = c * dscale * (1.f - tt * tt);
          } else {
            g[e] = cs * fast_exp2(__builtin_fmaf(z, ks, -l2[nb]));
          }
        }
        if (any_label) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (lr == mb * 4 + e) g[e] -= kCap ? 1.f : cs;
        }
        if constexpr (kCap) {
#pragma unroll
          for (int e = 0; e < 4; ++e) g[e] *= d[e];
        }
        u32x2 w;
        w[0] = pack_bf16(g[0], g[1]);
        w[1] = pack_bf16(g[2], g[3]);
        *(u32x2 *)(grow + acc_row(mb, 0, lane)) = w;  // 4 consecutive vocabulary rows
      }
    }
  }
}

// Writes (or adds) a wave's 128 x 128 fp32 accumulator block to row-major
// memory through a buffer descriptor; lanes whose column lies past `cols`
// and rows past the descriptor's range are dropped by the hardware.  When
// adding, the old values of two 16-column blocks (64 per lane) are loaded
// together before any is consumed: after the K loop the fragment registers
// are free, and four round trips per tile instead of sixteen keep the
// epilogue short.
template <int kNb>
__device__ __forceinline__ void add_acc_cols(const Acc &acc, __amdgpu_buffer_rsrc_t rs, int ld,
                                             int row0, int col0, int cols, int nb0, int lane) {
  uint32_t off[kNb][32];
  float old[kNb][32];
#pragma unroll
  for (int j = 0; j < kNb; ++j) {
    const int col = col0 + (nb0 + j) * 16 + (lane & 15);
    const bool col_ok = col < cols;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      off[j][q] = col_ok ? (uint32_t)((row0 + acc_row(q >> 2, q & 3, lane)) * ld + col) * 4u : kOOB;
      old[j][q] = load_f32(rs, off[j][q]);
    }
  }
#pragma unroll
  for (int j = 0; j < kNb; ++j)
#pragma unroll
    for (int q = 0; q < 32; ++q)
      store_f32(rs, off[j][q], acc_read(acc.v[q >> 2][nb0 + j][q & 3]) + old[j][q]);
}

__device__ __forceinline__ void store_acc_block(const Acc &acc, __amdgpu_buffer_rsrc_t rs,
                                                int ld, int row0, int col0, int cols,
                                                bool accumulate, int lane) {
  if (accumulate) {
#pragma unroll
    for (int nb = 0; nb < 8; nb += 2) add_acc_cols<2>(acc, rs, ld, row0, col0, cols, nb, lane);
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int col = col0 + nb * 16 + (lane & 15);
      const bool col_ok = col < cols;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t off =
              col_ok ? (uint32_t)((row0 + acc_row(mb, r, lane)) * ld + col) * 4u : kOOB;
          store_f32(rs, off, acc_read(acc.v[mb][nb][r]));
        }
    }
  }
}

struct BwdDhParams {
  const uint16_t *G;
  const uint16_t *weight;
  int Gp, D, V;
  int vc0, vcount;       // vocabulary rows [vc0, vc0 + vcount) of this chunk exist
  int Kc;                // K extent of the chunk (columns of G)
  int R;                 // rows of the row block (multiple of 256)
  int tiles_m, tiles_n, splits;
  float *acc;            // [splits, R, D] fp32
  int accumulate;
  RowMap map;            // the row block's token tiles (tiles_m of them as laid out)
};

// One dH tile (split s of K): A = G rows, plain (OperandK) or grouped in
// place of an fp32 block (OperandKG, the distillation's layout).
template <class OA>
__device__ __forceinline__ void dh_tile(const BwdDhParams &p, lds_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  bool ident;
  const int tiles_m = rowmap_tiles(p.map, rowmap_count(p.map), p.tiles_m, ident);
  int splits, stride;
  dh_layout(ident, tiles_m, p.tiles_n, p.splits, p.map.tiles_rb, p.R, splits, stride);
  const int per_split = tiles_m * p.tiles_n;
  const int n_wg = per_split * splits;  // the rest of the grid exits
  if ((int)blockIdx.x >= n_wg) return;
  const int L = xcd_contiguous(blockIdx.x, n_wg);
  const int s = L / per_split;
  int tm, tn;
  grouped_tile(L - s * per_split, tiles_m, p.tiles_n, 8, tm, tn);
  const int ktiles = (p.Kc + kBK - 1) / kBK;
  const int kbeg = (int)((int64_t)s * ktiles / splits) * kBK;
  const int kend = min(p.Kc, (int)((int64_t)(s + 1) * ktiles / splits) * kBK);
  const int h0 = tn * kTile;

  OA A;            // G rows of this tile, K = vocabulary (contiguous)
  if constexpr (OA::kGrouped)
    A.init(p.G + (size_t)(tm * kTile) * p.Gp, p.Gp, kTile, kbeg, kend - kbeg, wave, lane);
  else
    A.init(p.G + (size_t)(tm * kTile) * p.Gp + kbeg, p.Gp, kTile, kend - kbeg, wave, lane);
  OperandMN B;     // W[vc0 + k][h0 + n]: K = vocabulary rows
  B.init(p.weight + (size_t)(p.vc0 + kbeg) * p.D + h0, p.D, min(kTile, p.D - h0),
         min(kend, p.vcount) - kbeg, wave, lane);
  Acc acc;
  acc.zero();
  tile_mainloop(A, B, (kend - kbeg + kKS - 1) / kKS, smem, acc, wave, lane);

  // rows [tm*256, tm*256 + 256) of split s, all inside the buffer
  const float *tile = p.acc + ((size_t)s * stride + (size_t)tm * kTile) * p.D;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile, (uint32_t)kTile * (uint32_t)p.D * 4u);
  store_acc_block(acc, rs, p.D, wm * 128, h0 + wn * 128, p.D, p.accumulate != 0, lane);
}

__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_dh_kernel(BwdDhParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  dh_tile<OperandK>(p, (lds_t *)smem_raw);
}

// H^T of a row block: ht[d][t] = hidden[rb0 + t][d] for t < rcount, zeros for
// rcount <= t < round_up(rcount, 64); rows of R tokens (K-contiguous for dW).
// 64 x 64 tiles through LDS, 16-byte loads and stores.
struct BwdHtParams {
  const uint16_t *hidden;  // [T, D]
  uint16_t *ht;            // [D, R]
  int T, D, R, rb0, rcount;
  int tiles_id;            // token tiles of the block as laid out
  RowMap map;              // the row block's token tiles
};

__global__ void __launch_bounds__(256) bwd_ht_kernel(BwdHtParams p) {
  __shared__ uint16_t tile[64][72];  // [d][t]; 8 columns of padding
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const int r8 = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;
  // Rows [t0, t0 + 64) lie in one token tile: as laid out, tokens rb0 + t (t < rcount);
  // from a list, that tile's tokens (rows of tiles past the list are not needed).
  bool ident;
  const int n_here = rowmap_tiles(p.map, rowmap_count(p.map), p.tiles_id, ident);
  int src0 = p.rb0 + t0, nsrc = p.rcount - t0;
  if (!ident) {
    const int i = t0 / kTile;
    if (i >= n_here) return;
    src0 = rowmap_tile(p.map, false, i) * kTile + t0 % kTile;
    nsrc = p.T - src0;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tr = r8 + 32 * j, d = d0 + c8;  // d % 8 == 0 and D % 8 == 0
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tr < nsrc && d < p.D) v = *(const u32x4 *)(p.hidden + (size_t)(src0 + tr) * p.D + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[c8 + 2 * e][tr] = (uint16_t)(v[e] & 0xffffu);
      tile[c8 + 2 * e + 1][tr] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int dr = r8 + 32 * j, d = d0 + dr, t = t0 + c8;  // t % 8 == 0 and R % 256 == 0
    if (d < p.D && t < p.R) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)tile[dr][c8 + 2 * e] | ((uint32_t)tile[dr][c8 + 2 * e + 1] << 16);
      *(u32x4 *)(p.ht + (size_t)d * p.R + t) = v;
    }
  }
}

struct BwdDwParams {
  const uint16_t *G;
  const uint16_t *ht;    // [D, R] H^T of the row block (bwd_ht_kernel)
  int Gp, D, V, R;
  int rcount;            // tokens [0, rcount) of this row block exist
  int vc0;
  int tiles_m, tiles_n;
  float *dW;             // [V, D] fp32
  int accumulate;
  RowMap map;            // the row block's token tiles
};

// One dW tile: A = G^T, plain (OperandMN) or grouped (OperandMNG).
template <class OA>
__device__ __forceinline__ void dw_tile(const BwdDwParams &p, lds_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, 8, tm, tn);
  const int v0 = p.vc0 + tm * kTile;
  if (v0 >= p.V) return;  // the whole tile lies past the vocabulary
  const int h0 = tn * kTile;
  const int cnt = rowmap_count(p.map);  // used after the first stages are issued

  // G^T: G[k = row][m = vocabulary]; H^T[h0 + n][k = row], K-contiguous, zeros past
  // rcount.  K (rows of the block) starts as laid out, [0, rcount).
  const uint16_t *g_col = p.G + (OA::kGrouped ? grouped_col(tm * kTile) : tm * kTile);
  const uint16_t *ht_row = p.ht + (size_t)h0 * p.R;
  const int hrows = min(kTile, p.D - h0);
  OA A;
  A.init(g_col, p.Gp, kTile, p.rcount, wave, lane);
  OperandK B;
  B.init(ht_row, p.R, hrows, (p.rcount + 7) & ~7, wave, lane);
  Acc acc;
  acc.zero();
  int nk = (p.rcount + kKS - 1) / kKS;
  if (nk > 0) pipe_prologue(A, B, smem, wave);
  // A list that leaves tiles out packs the others into whole tiles of rows: K is then
  // 256 rows per tile of the block.  The count is looked at after the first stages are
  // issued, so that its read overlaps their loads; another K drains them and starts again.
  bool ident;
  const int n_here = rowmap_tiles(p.map, cnt, 0, ident);
  if (!ident && n_here * kTile != p.rcount) {
    const int kend = n_here * kTile;
    wait_vmcnt<0>();  // the issued loads still write LDS: let them land first
    __syncthreads();
    nk = (kend + kKS - 1) / kKS;
    if (nk <= 0 && p.accumulate) return;  // nothing to add to dW
    if (nk > 0) {
      A.init(g_col, p.Gp, kTile, kend, wave, lane);
      B.init(ht_row, p.R, hrows, kend, wave, lane);
      pipe_prologue(A, B, smem, wave);
    }
  }
  if (nk > 0) pipe_run(A, B, nk, smem, acc, wave, lane);

  // rows [v0, min(V, v0 + 256)) of dW
  const uint32_t rows = (uint32_t)min(kTile, p.V - v0);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.dW + (size_t)v0 * p.D, rows * (uint32_t)p.D * 4u);
  store_acc_block(acc, rs, p.D, wm * 128, h0 + wn * 128, p.D, p.accumulate != 0, lane);
}

__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_dw_kernel(BwdDwParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  dw_tile<OperandMN>(p, (lds_t *)smem_raw);
}

struct BwdDhOutParams {
  const float *acc;   // [splits, R, D]
  uint16_t *dH;       // [T, D] bf16
  int T, D, R, splits, rb0, rcount;
  RowMap map;         // the row block's token tiles
};

__global__ void __launch_bounds__(256) bwd_dh_out_kernel(BwdDhOutParams p) {
  bool ident;
  const int n_here = rowmap_tiles(p.map, rowmap_count(p.map), 0, ident);
  int splits, stride;
  dh_layout(ident, n_here, (p.D + kTile - 1) / kTile, p.splits, p.map.tiles_rb, p.R, splits,
            stride);
  const int per_row = p.D >> 3;
  const int64_t n = (int64_t)(ident ? p.rcount : n_here * kTile) * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int row = (int)(i / per_row), c8 = (int)(i - (int64_t)row * per_row) * 8;
    // token of the row: rb0 + row as laid out (row < rcount), else through the list
    // (rows of the batch's last tile may lie past T)
    int tok = p.rb0 + row;
    if (!ident) {
      tok = rowmap_tile(p.map, false, row / kTile) * kTile + row % kTile;
      if (tok >= p.T) continue;
    }
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const float *src = p.acc + ((size_t)s * stride + row) * p.D + c8;
      lo += *(const f32x4 *)src;
      hi += *(const f32x4 *)(src + 4);
    }
    u32x4 o;
    o[0] = pack_bf16(lo[0], lo[1]);
    o[1] = pack_bf16(lo[2], lo[3]);
    o[2] = pack_bf16(hi[0], hi[1]);
    o[3] = pack_bf16(hi[2], hi[3]);
    *(u32x4 *)(p.dH + (size_t)tok * p.D + c8) = o;
  }
}

__global__ void __launch_bounds__(256) fill_f32_kernel(float *dst, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = value;
}

}  // namespace flce
