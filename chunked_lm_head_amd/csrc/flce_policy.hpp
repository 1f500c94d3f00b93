// flce_policy.hpp - policy-optimisation losses (GRPO, DPO, KTO) on the
// per-token log-probs of the chunked selective log-softmax.
//
// The TRL v1.13 article (section on the other v1.13 changes) names fused
// linear GRPO, DPO and KTO losses built on the chunked LM head without
// defining them; the Unsloth GRPO long-context page feeds the chunked
// selective log-softmax into GRPO.  These kernels compute the published
// objectives from the log-probs that the fused forward kernel writes:
//   GRPO (DeepSeekMath's group relative policy optimisation, with its
//   unbiased KL estimator): r = exp(logp - old), s = min(r A, clip(r, 1 - el,
//   1 + eh) A), k = exp(ref - logp) - (ref - logp) - 1,
//   L = -(1/B') sum_b (1/n_b) sum_{t in b} (s - beta k);
//   DPO: pi_b = sum_{t in b} logp, Delta_i = beta ((pi_i - ref_i) -
//   (pi_{P+i} - ref_{P+i})), L = (1/P) sum_i softplus(-Delta_i);
//   KTO: r_b = pi_b - ref_b, z0 = max(kl_ref, 0), v_b = lD sigmoid(beta (r_b -
//   z0)) (desirable) or lU sigmoid(beta (z0 - r_b)), L = (1/B) sum_b (l_b - v_b).
// Sequence b is the rows [b S, (b + 1) S) of the flattened batch; tokens
// whose label is ignore_index are not completion tokens.  The loss's gradient
// in each log-prob, times the upstream scalar, becomes the per-token upstream
// gradient of the log-prob backward, so dH and dW come from the same
// recompute + GEMM kernels as the cross-entropy path.
//
// Three small launches: a block per sequence reduces its tokens (in double,
// a fixed order); one block forms the loss and a per-sequence factor; a
// thread per token writes dL/dlogp.
#pragma once

#include "flce_kernels.hpp"

namespace flce {

enum PolicyKind { kPolicyGrpo = 0, kPolicyDpo = 1, kPolicyKto = 2 };

struct PolicyParams {
  const int64_t *labels;
  int64_t ignore_index;
  int T, n_seq, S;
  const float *logp;        // [T] from the forward (0 off the completions)
  const float *advantages;  // GRPO [n_seq]
  const float *old_logp;    // GRPO [T] or null (old = logp)
  const float *ref_logp;    // GRPO [T] or null (no KL term)
  const float *ref_seq;     // DPO, KTO [n_seq]
  const uint8_t *desirable; // KTO [n_seq]
  const float *kl_ref;      // KTO device scalar or null (0)
  const float *grad_loss;   // upstream scalar, or null (no gradient)
  float beta, eps_low, eps_high, w_des, w_und;
  double *seq_val;          // [n_seq] GRPO: sum of s - beta k; DPO, KTO: pi_b
  int *seq_n;               // [n_seq] completion tokens
  float *seq_g;             // [n_seq] dL/d(per-sequence value) times the upstream scalar
  float *loss;              // device scalar
  float *c;                 // [T] dL/dlogp times the upstream scalar (the backward's grad_out)
};

// GRPO's per-token objective s - beta k and its derivative in logp (fp32; the
// clipped branch has no gradient, the unclipped one r A; at a tie, r A).
__device__ __forceinline__ void grpo_token(float lp, float old, bool has_old, float ref,
                                           bool has_ref, float A, const PolicyParams &p,
                                           float &obj, float &dobj) {
  const float r = has_old ? expf(lp - old) : 1.f;
  const float un = r * A;
  const float cl = fminf(fmaxf(r, 1.f - p.eps_low), 1.f + p.eps_high) * A;
  float s = fminf(un, cl), ds = un <= cl ? un : 0.f;
  float k = 0.f, dk = 0.f;
  if (has_ref) {  // k = e^d - d - 1 through expm1, which keeps k's relative accuracy at small d
    const float d = ref - lp;
    const float em1 = expm1f(d);
    k = em1 - d;
    dk = -em1;
  }
  obj = s - p.beta * k;
  dobj = ds - p.beta * dk;
}

// One block per sequence: completion-token count and the sequence's sum (GRPO:
// the objective; DPO and KTO: the log-prob), each thread over a stride of the
// sequence, then a fixed tree over the block.
template <int kKind>
__global__ void __launch_bounds__(256) pol_seq_kernel(PolicyParams p) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  const int b = blockIdx.x;
  const size_t base = (size_t)b * p.S;
  double acc = 0.0;
  int cnt = 0;
  for (int i = threadIdx.x; i < p.S; i += 256) {
    const size_t t = base + i;
    if (p.labels[t] == p.ignore_index) continue;
    ++cnt;
    const float lp = p.logp[t];
    if constexpr (kKind == kPolicyGrpo) {
      float obj, dobj;
      grpo_token(lp, p.old_logp ? p.old_logp[t] : 0.f, p.old_logp != nullptr,
                 p.ref_logp ? p.ref_logp[t] : 0.f, p.ref_logp != nullptr, p.advantages[b], p,
                 obj, dobj);
      acc += (double)obj;
    } else {
      acc += (double)lp;
    }
  }
  ssum[threadIdx.x] = acc;
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
    p.seq_val[b] = ssum[0];
    p.seq_n[b] = scnt[0];
  }
}

__device__ __forceinline__ double sigmoid_d(double x) {
  const double e = exp(-fabs(x));
  return x >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

__device__ __forceinline__ double softplus_d(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

// One block: the loss (a fixed-order double sum over sequences) and each
// sequence's gradient factor times the upstream scalar.
template <int kKind>
__global__ void __launch_bounds__(1024) pol_loss_kernel(PolicyParams p) {
  __shared__ double ssum[1024];
  __shared__ int scnt[1024];
  const double gl = p.grad_loss ? (double)p.grad_loss[0] : 0.0;
  const int tid = threadIdx.x;
  // GRPO's B' (sequences with a completion token) first.
  int used = 0;
  if constexpr (kKind == kPolicyGrpo) {
    for (int b = tid; b < p.n_seq; b += 1024) used += p.seq_n[b] > 0;
    scnt[tid] = used;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w) scnt[tid] += scnt[tid + w];
      __syncthreads();
    }
    used = scnt[0];
    __syncthreads();
  }
  const double z0 = (kKind == kPolicyKto && p.kl_ref) ? fmax((double)p.kl_ref[0], 0.0) : 0.0;
  const int P = p.n_seq / 2;
  const int items = kKind == kPolicyDpo ? P : p.n_seq;
  double acc = 0.0;
  for (int i = tid; i < items; i += 1024) {
    if constexpr (kKind == kPolicyGrpo) {
      const int n = p.seq_n[i];
      double g = 0.0;
      if (n > 0) {
        acc += p.seq_val[i] / n;
        g = -gl / ((double)used * n);
      }
      p.seq_g[i] = (float)g;
    } else if constexpr (kKind == kPolicyDpo) {
      const double delta = (double)p.beta * ((p.seq_val[i] - (double)p.ref_seq[i]) -
                                             (p.seq_val[P + i] - (double)p.ref_seq[P + i]));
      acc += softplus_d(-delta);
      const double g = gl * (double)p.beta * sigmoid_d(-delta) / P;
      p.seq_g[i] = (float)-g;
      p.seq_g[P + i] = (float)g;
    } else {
      const bool des = p.desirable[i] != 0;
      const double r = p.seq_val[i] - (double)p.ref_seq[i];
      const double x = des ? (double)p.beta * (r - z0) : (double)p.beta * (z0 - r);
      const double lam = des ? (double)p.w_des : (double)p.w_und;
      const double sx = sigmoid_d(x);
      acc += lam - lam * sx;
      p.seq_g[i] = (float)(-gl * lam * sx * (1.0 - sx) * (des ? p.beta : -p.beta) / p.n_seq);
    }
  }
  ssum[tid] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) ssum[tid] += ssum[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    double loss;
    if constexpr (kKind == kPolicyGrpo)
      loss = used > 0 ? -ssum[0] / used : 0.0;
    else if constexpr (kKind == kPolicyDpo)
      loss = P > 0 ? ssum[0] / P : 0.0;
    else
      loss = p.n_seq > 0 ? ssum[0] / p.n_seq : 0.0;
    p.loss[0] = (float)loss;
  }
}

// c_t = dL/dlogp_t times the upstream scalar; 0 off the completions.
template <int kKind>
__global__ void __launch_bounds__(256) pol_grad_kernel(PolicyParams p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.T) return;
  float c = 0.f;
  if (p.labels[t] != p.ignore_index) {
    const int b = t / p.S;
    const float g = p.seq_g[b];
    if constexpr (kKind == kPolicyGrpo) {
      float obj, dobj;
      grpo_token(p.logp[t], p.old_logp ? p.old_logp[t] : 0.f, p.old_logp != nullptr,
                 p.ref_logp ? p.ref_logp[t] : 0.f, p.ref_logp != nullptr, p.advantages[b], p,
                 obj, dobj);
      c = g * dobj;
    } else {
      c = g;
    }
  }
  p.c[t] = c;
}

}  // namespace flce
