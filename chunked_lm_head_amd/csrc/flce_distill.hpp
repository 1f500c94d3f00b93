// flce_distill.hpp - chunked distillation through two LM heads (student,
// teacher) over one vocabulary: per token the forward Kullback-Leibler
// divergence KL(p_t || p_s) of the student's softmax from the teacher's, and
// the student's gradients.
//
// The TRL v1.13 article (speed section) applies the chunked bf16 loss to the
// distillation trainer, which computes every chunk twice, once with the
// student's hidden states and lm_head and once with the teacher's; it gives no
// divergence, and the forward KL is the textbook distillation loss.  Per token
//     KL = sum_v p_t (z_t' - lse_t) - sum_v p_t (z_s' - lse_s)
//        = A - lse_t - B + lse_s,   A = sum_v p_t z_t',  B = sum_v p_t z_s',
// and dKL/dz_s' = p_s - p_t, so the student's backward is the cross-entropy
// backward with the one-hot target replaced by p_t.
//
// The generalized Jensen-Shannon divergence (the same article names a fused
// linear JSD loss), with weight beta and M = beta p_t + (1 - beta) p_s:
//     JSD = beta KL(p_t || M) + (1 - beta) KL(p_s || M),
//     dJSD/dz_s' = p_s (g - gbar),  g = (1 - beta) log(p_s / M),  gbar = sum_v p_s g,
// needs the row sum gbar before any gradient value exists, so its schedule
// has one more block pass: per row block, teacher + student passes over every
// vocabulary chunk form the divergence and gbar (as partial sums), then
// teacher + student passes write G for the dH and dW kernels.
//
// Schedule (one call): the two log-sum-exps come from the fused forward
// kernel without labels; then, per block of rows and vocabulary chunk, the
// teacher kernel recomputes its logits and writes p_t in fp32 (with partial
// sums of A), and the student kernel recomputes its logits, reads p_t, adds
// partial sums of B and writes G = c (p_s - p_t) dz_s'/dz_s in bf16 over p_t,
// in place (each 128-column group's bf16 values in the first half of its fp32
// bytes), for the dH and dW kernels, which read that grouped layout.  The
// block, 4 bytes per element, stays within the fp32 logits of one chunk of
// chunk_rows rows.
#pragma once

#include "flce_kernels.hpp"

namespace flce {

// lse (natural log) and lse * log2(e) of every token from the forward
// kernel's per-split partials; rows T <= t < n get lse2 = +inf so their
// softmax terms vanish.  As in the forward combine, `lanes` lanes merge one
// token's partials and a fixed shuffle tree combines them; a block takes
// 256 / lanes tokens.
struct DstLseParams {
  const float *part_m, *part_s;
  int T, splits, T_pad, n;
  int lanes;     // power of two <= 64
  float *lse;    // [n]
  float *lse2;   // [n]
};

__global__ void __launch_bounds__(256) dst_lse_kernel(DstLseParams p) {
  const int L = p.lanes, g = threadIdx.x / L, j = threadIdx.x % L, per = 256 / L;
  {
    const int t = blockIdx.x * per + g;
    float M = -kInf, S = 0.f;
    if (t < p.T) {
      for (int s = j; s < p.splits; s += L)
        lse_merge(M, S, p.part_m[(size_t)s * p.T_pad + t], p.part_s[(size_t)s * p.T_pad + t]);
    }
    for (int w = 1; w < L; w <<= 1) {
      const float m2 = __shfl_xor(M, w), s2 = __shfl_xor(S, w);
      lse_merge(M, S, m2, s2);
    }
    if (j == 0 && t < p.n) {
      if (t < p.T) {
        const float l2 = M + fast_log2(S);
        p.lse[t] = l2 * kLn2;
        p.lse2[t] = l2;
      } else {
        p.lse[t] = 0.f;
        p.lse2[t] = kInf;
      }
    }
  }
}

// Upstream scale c_t of each token (0 for masked tokens and rows past T).
struct DstPrepParams {
  const int64_t *labels;   // mask: tokens whose label is ignore_index are left out; null = none
  const float *grad_out;   // [T] dL/d kl_t, or null
  const float *grad_mean;  // dL/d mean (device scalar), used when grad_out is null
  int64_t ignore_index;
  int T, n;
  float *c;                // [n]
};

__global__ void __launch_bounds__(1024) dst_prep_kernel(DstPrepParams p) {
  __shared__ int scnt[1024];
  int cnt = 0;
  for (int t = threadIdx.x; t < p.T; t += 1024)
    cnt += !p.labels || p.labels[t] != p.ignore_index;
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) scnt[threadIdx.x] += scnt[threadIdx.x + w];
    __syncthreads();
  }
  const int n_valid = scnt[0];
  float gm = 0.f;
  if (!p.grad_out && n_valid > 0) gm = p.grad_mean[0] / (float)n_valid;
  for (int t = threadIdx.x; t < p.n; t += 1024) {
    float c = 0.f;
    if (t < p.T && (!p.labels || p.labels[t] != p.ignore_index))
      c = p.grad_out ? p.grad_out[t] : gm;
    p.c[t] = c;
  }
}

// What a block pass of dst_tile_kernel computes.
enum DstRole {
  kRoleTeacher = 0,   // p_t -> P, partial sums of p_t z_t'
  kRoleStudentKL = 1, // partial sums of p_t z_s', G = c (p_s - p_t) dz'/dz over P
  kRoleJsdStats = 2,  // partial sums of the JSD terms and of p_s g (gbar)
  kRoleJsdGrad = 3,   // G = c p_s (g - gbar) dz'/dz over P
};

struct DstTileParams {
  const uint16_t *hidden, *weight;  // this head's [T, D] and [V, D], bf16
  const float *lse2;                // [Tb] this head's lse * log2(e), +inf past T
  const float *c;                   // [Tb] student: upstream scale (0: no gradient)
  const float *gbar2;               // [Tb] JSD gradient pass: gbar / ln 2 per token
  float beta;                       // JSD weight of the teacher in M
  int T, D, V;
  int rb0, vc0;                     // first token / vocabulary row of this block
  int n_vt;                         // vocabulary tiles of the chunk that hold rows < V
  int tiles_n, vsplits;             // token tiles of the row block; vocabulary ranges
  int R;                            // rows of the row block
  Xform xf;
  float *P;                         // [R, Pp] teacher probabilities, fp32
  int Pp;
  uint16_t *G;                      // student gradient, bf16 (zeros when c = 0), written over
  int Gp;                           // P: the same bytes, Gp = 2 Pp, grouped columns
  float *part;                      // [vsplits, R] this launch's per-token partial sums
  float *part2;                     // JSD statistics pass: partial sums of p_s g / ln 2
};

// One head's logit tiles of a block, walking vocabulary tiles per token tile
// as the recompute kernel of the cross-entropy backward does.
//   teacher:           P = p_t = 2^(z_t' log2 e - lse2_t) -> fp32 block,
//                      partial sums of p_t z_t' (A);
//   student, KL:       reads p_t, partial sums of p_t z_s' (B), and
//                      G = c (p_s - p_t) dz_s'/dz_s -> bf16, over p_t;
//   student, JSD:      reads p_t; in log2 units (l = log2 of a probability),
//                      g2 = (1 - beta) (l_s - l_M); statistics pass: partial
//                      sums of beta p_t (l_t - l_M) + p_s g2 (the divergence /
//                      ln 2) and of p_s g2 (gbar / ln 2); gradient pass:
//                      G = c ln2 p_s (g2 - gbar2) dz_s'/dz_s over p_t.
//                      Probabilities below FLT_MIN count as 0 (their terms
//                      vanish; the hardware logarithm flushes denormals).
// A student wave reads the p_t values of one token row (its 128 columns) and
// then writes that row's G into the first half of the same bytes: each G store
// overlaps only p_t values of the same or earlier blocks of the row, which the
// store's own data already waited for; no other wave touches those bytes.
// Rows past the vocabulary have z = -inf: p = 0 there and the products are
// taken as 0.  Every workgroup writes its partial-sum slot (zeros when its
// vocabulary range is empty), so the reduction reads no stale values.
template <int kRole, bool kCap>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) dst_tile_kernel(DstTileParams p) {
  constexpr bool kTeacher = kRole == kRoleTeacher;
  constexpr bool kJsd = kRole == kRoleJsdStats || kRole == kRoleJsdGrad;
  constexpr bool kWritesG = kRole == kRoleStudentKL || kRole == kRoleJsdGrad;
  constexpr bool kSums = kRole != kRoleJsdGrad;  // writes per-token partial sums
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  lds_t *smem = (lds_t *)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tn, sp;
  grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), p.tiles_n, p.vsplits, 8, tn, sp);
  const int vt0 = (int)((int64_t)sp * p.n_vt / p.vsplits);
  const int vt1 = (int)((int64_t)(sp + 1) * p.n_vt / p.vsplits);
  const int t0 = p.rb0 + tn * kTile;

  float psum[8], psum2[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) psum[nb] = psum2[nb] = 0.f;

  if (t0 < p.T && vt0 < vt1) {
    float l2[8], cc[8], gb[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int t = t0 + wn * 128 + nb * 16 + (lane & 15);  // < rb0 + R <= Tb
      l2[nb] = p.lse2[t];
      cc[nb] = kWritesG ? p.c[t] : 0.f;
      gb[nb] = kRole == kRoleJsdGrad ? p.gbar2[t] : 0.f;
    }
    const float beta = p.beta, nbeta = 1.f - p.beta;
    constexpr float kFltMin = 1.17549435e-38f;
    const float dscale = p.xf.zscale * p.xf.inv_temp;  // capped: dz'/dz = dscale (1 - t^2)

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
      const int vw = v0 + wm * 128;
      acc.init_rows(p.V - vw, lane);
      pipe_run(A, B, nk, smem, acc, wave, lane);
      if (vt + 1 < vt1) {
        A.init(p.weight + (size_t)(v0 + kTile) * p.D, p.D, min(kTile, p.V - v0 - kTile), p.D,
               wave, lane);
        pipe_prologue(A, B, smem, wave);
      }
      const int col = vw - p.vc0;  // column of this wave's first vocabulary row in the block
      const int tl0 = t0 - p.rb0 + wn * 128 + (lane & 15);  // row nb = 0 in the block
      // Students read p_t one token row (nb) ahead: row nb + 1 is in flight while
      // row nb is processed.
      f32x4 ptb[2][8];
      if constexpr (!kTeacher) {
        const float *prow0 = p.P + (size_t)tl0 * p.Pp + col;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) ptb[0][mb] = *(const f32x4 *)(prow0 + acc_row(mb, 0, lane));
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int tl = tl0 + nb * 16;  // row in the block
        float *prow = p.P + (size_t)tl * p.Pp + col;
        f32x4 *pt = ptb[nb & 1];
        if constexpr (!kTeacher) {
          if (nb + 1 < 8) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
              ptb[(nb + 1) & 1][mb] = *(const f32x4 *)(prow + 16 * p.Pp + acc_row(mb, 0, lane));
          }
          // G of row nb is written over that row's p_t below: every read of rows nb
          // and nb + 1 is issued first
          __asm__ volatile("" ::: "memory");
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          float zp[4], pr[4], d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc_read(acc.v[mb][nb][e]);
            if constexpr (kCap) {
              float tt;
              zp[e] = xform_cap(z, p.xf, tt);
              d[e] = dscale * (1.f - tt * tt);
            } else {
              zp[e] = z * p.xf.zscale;
              d[e] = p.xf.zscale;
            }
            const float lq2 = __builtin_fmaf(zp[e], kLog2e, -l2[nb]);
            pr[e] = fast_exp2(lq2);
            if constexpr (!kJsd) {
              // p z' with p = 0 (and z' = -inf) past the vocabulary taken as 0
              const float w = kTeacher ? pr[e] : pt[mb][e];
              psum[nb] += z == -kInf ? 0.f : w * zp[e];
            } else {
              const float pv = pt[mb][e];
              const bool qn = pr[e] > kFltMin, pn = pv > kFltMin;
              const float lm2 = fast_log2(beta * pv + nbeta * pr[e]);  // finite if qn or pn
              const float g2 = nbeta * (lq2 - lm2);
              if constexpr (kRole == kRoleJsdStats) {
                const float qg = qn ? pr[e] * g2 : 0.f;
                psum[nb] += (pn ? beta * pv * (fast_log2(pv) - lm2) : 0.f) + qg;
                psum2[nb] += qg;
              } else {
                pr[e] = qn ? pr[e] * (g2 - gb[nb]) : 0.f;  // p_s (g2 - gbar2)
              }
            }
          }
          if constexpr (kTeacher) {
            *(f32x4 *)(prow + acc_row(mb, 0, lane)) = f32x4{pr[0], pr[1], pr[2], pr[3]};
          } else if constexpr (kWritesG) {
            float g[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              g[e] = kJsd ? cc[nb] * kLn2 * pr[e] * d[e] : cc[nb] * (pr[e] - pt[mb][e]) * d[e];
            u32x2 w;
            w[0] = pack_bf16(g[0], g[1]);
            w[1] = pack_bf16(g[2], g[3]);
            *(u32x2 *)(p.G + (size_t)tl * p.Gp + grouped_col(col + acc_row(mb, 0, lane))) = w;
          }
        }
      }
    }
  }

  if constexpr (kSums) {
    // Sum the four lanes holding one token (l, l ^ 16, l ^ 32, l ^ 48), then the
    // two waves (wm), in the (idle) ring; one value per token of the tile.
    float *xch = (float *)smem_raw;  // [2 sums][wn][nb][16]
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      psum[nb] += __shfl_xor(psum[nb], 16);
      psum[nb] += __shfl_xor(psum[nb], 32);
      if (wm == 1 && lane < 16) xch[(wn * 8 + nb) * 16 + lane] = psum[nb];
      if constexpr (kRole == kRoleJsdStats) {
        psum2[nb] += __shfl_xor(psum2[nb], 16);
        psum2[nb] += __shfl_xor(psum2[nb], 32);
        if (wm == 1 && lane < 16) xch[256 + (wn * 8 + nb) * 16 + lane] = psum2[nb];
      }
    }
    __syncthreads();
    if (wm == 0 && lane < 16) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int tl = tn * kTile + wn * 128 + nb * 16 + lane;
        p.part[(size_t)sp * p.R + tl] = psum[nb] + xch[(wn * 8 + nb) * 16 + lane];
        if constexpr (kRole == kRoleJsdStats)
          p.part2[(size_t)sp * p.R + tl] = psum2[nb] + xch[256 + (wn * 8 + nb) * 16 + lane];
      }
    }
  }
}

// dH and dW of the student from its G block in the grouped layout above.
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) dst_dh_kernel(BwdDhParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  dh_tile<OperandKG>(p, (lds_t *)smem_raw);
}

__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(1, 1))) dst_dw_kernel(BwdDwParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPipeBytes];
  dw_tile<OperandMNG>(p, (lds_t *)smem_raw);
}

// out[rb0 + t] = sum over the nparts slots of part[slot, t], t < rcount, in a
// fixed order (the same bits on every run).  A block takes 64 tokens; its
// four waves each sum every fourth slot with eight independent loads in
// flight, and the four sums are added in wave order.
__global__ void __launch_bounds__(256)
    dst_reduce_kernel(const float *part, int nparts, int R, int rb0, int rcount, float *out) {
  __shared__ float ssum[4][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (t < rcount) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = g;
    for (; j + 28 < nparts; j += 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += part[(size_t)(j + 4 * u) * R + t];
    }
    for (int u = 0; j < nparts; j += 4, ++u) acc[u & 7] += part[(size_t)j * R + t];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += acc[u];
  }
  ssum[g][lane] = s;
  __syncthreads();
  if (g == 0 && t < rcount) out[rb0 + t] = ((ssum[0][lane] + ssum[1][lane]) + ssum[2][lane]) + ssum[3][lane];
}

// kl_t = A - lse_t - B + lse_s (JSD: ln 2 * A) for kept tokens, 0 for masked
// ones; block sums for the mean (fwd_mean_kernel finishes it).
struct DstCombineParams {
  const float *A, *B, *lse_s, *lse_t;
  int jsd;                // 1: kl_t = ln 2 * A_t (A holds the JSD sum / ln 2)
  const int64_t *labels;  // mask, or null
  int64_t ignore_index;
  int T;
  float *kl;              // [T], or null
  double *blk_sum;
  int *blk_cnt;
};

__global__ void __launch_bounds__(256) dst_combine_kernel(DstCombineParams p) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  const int t = blockIdx.x * 256 + threadIdx.x;
  double contrib = 0.0;
  int cnt = 0;
  if (t < p.T) {
    float k = 0.f;
    if (!p.labels || p.labels[t] != p.ignore_index) {
      k = p.jsd ? kLn2 * p.A[t] : (p.A[t] - p.lse_t[t]) - (p.B[t] - p.lse_s[t]);
      contrib = (double)k;
      cnt = 1;
    }
    if (p.kl) p.kl[t] = k;
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

}  // namespace flce
