// flce_api.hip - host side of the C ABI declared in include/flce.h: argument
// checks, the schedule for a shape, the workspace layout and the launches.
//
// Schedule (all tiles are 256 x 256, K steps of 64):
//  * Forward: one fused launch over (token tile, vocabulary split).  The number
//    of splits is chosen so that about 2048 workgroups exist (8 per CU); each
//    walks ~n_vt/splits vocabulary tiles keeping a running log-sum-exp, so the
//    workspace holds only splits x T partials.
//  * Backward: rows are taken in blocks of R tokens (R <= 8192) and the
//    vocabulary in chunks of Vc rows, with R * Vc bf16 gradient values no more
//    than the fp32 logits of one chunk of chunk_rows rows (chunk_rows * V * 4
//    bytes), the bound the pages' Equation 3 describes.  Per row block: H^T
//    (the dW kernel's K-contiguous operand); per (row block, vocabulary
//    chunk): recompute + G, dH partial sums, dW update.
//  * Distillation: both log-sum-exps by the forward kernel, then per block the
//    teacher's probabilities (fp32) and the student's G (bf16) written over
//    them, 4 bytes per element within the same bound, and the student's dH
//    and dW.
//  * Host policy: rows per chunk from the chunk multiplier, and the choice of
//    mini-batches and chunk size for a memory budget (no device call).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "flce.h"
#include "flce_distill.hpp"
#include "flce_policy.hpp"

namespace {

using namespace flce;

thread_local char g_last_error[512] = "";

flce_status fail(flce_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
flce_status fail(flce_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

constexpr int64_t kMaxD = 1 << 16;
constexpr int64_t kMaxTV = (int64_t)1 << 30;  // T and V each
constexpr int64_t kRowBlockMax = 8192;
// Forward workgroups: token tiles x vocabulary splits, at most this many (8 per CU), so
// that no launch ends with a ninth round of a few workgroups.
constexpr int64_t kFwdTargetWG = 2048;
constexpr int64_t kCUs = 256;  // compute units of an MI355X (8 XCDs of 32)
constexpr int64_t kDhPartialCap = (int64_t)128 << 20;  // bytes of split-K partial sums

constexpr int64_t kI32Bytes = ((int64_t)1 << 31) - 1;
constexpr size_t kScratchBytes = FLCE_FORWARD_SCRATCH_BYTES;  // flce_forward_noalloc's array

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// dH split-K count for a row block of `tiles` output tiles, at most `sp_max`.  A launch
// lasts about ceil(tiles * s / 256) / s of a whole K walk: the rounds of one workgroup per
// CU, each over 1/s of K.  Where a row block has fewer dH tiles than CUs (short token
// shares, one-tile batches), splits fill the chip: the most that keep one round, and more
// (several rounds) only for a gain of 10% or more, since every split adds partial sums for
// bwd_dh_out to read.  A split count that leaves a few workgroups for a second round
// costs a whole round.
int64_t dh_split_count(int64_t tiles, int64_t sp_max) {
  int64_t best = std::max<int64_t>(1, std::min(kCUs / tiles, sp_max));
  for (int64_t s = best + 1; s <= sp_max; ++s)
    if (cdiv(tiles * s, kCUs) * best * 10 <= cdiv(tiles * best, kCUs) * s * 9) best = s;
  return best;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int64_t T, D, V, chunk_rows;
  int64_t n_tt, n_vt, splits, T_pad;          // forward
  int64_t R, n_rb, Vc, n_vc, dh_splits, Tb;   // backward; Tb = n_rb * R
  int64_t comb_lanes, n_cblk;  // forward combine: lanes per token, blocks
  size_t off_pm, off_ps, off_zl, off_bs, off_bc, fwd_bytes;
  size_t off_c, off_l2, off_list, off_G, off_dh, off_ht, bwd_bytes;
  size_t gtile_bytes, chunk_bound;
  size_t total;
};

flce_status check_shape(int64_t T, int64_t D, int64_t V, int64_t chunk_rows) {
  if (T < 0) return fail(FLCE_ERR_SHAPE, "T = %lld must be >= 0", (long long)T);
  if (D < 1 || V < 1 || chunk_rows < 1)
    return fail(FLCE_ERR_SHAPE, "D = %lld, V = %lld, chunk_rows = %lld must be >= 1",
                (long long)D, (long long)V, (long long)chunk_rows);
  if (D % 8) return fail(FLCE_ERR_UNSUPPORTED, "D = %lld is not a multiple of 8", (long long)D);
  if (D > kMaxD || T > kMaxTV || V > kMaxTV)
    return fail(FLCE_ERR_SHAPE, "sizes out of range (D <= %lld, T and V <= %lld)",
                (long long)kMaxD, (long long)kMaxTV);
  return FLCE_OK;
}

// Row block R (tokens) and vocabulary chunk (tiles) of a staged block of
// elem_bytes bytes per (token, vocabulary) element, bounded by the fp32 logits
// of one chunk of chunk_rows rows, chunk_rows * V * 4 bytes (at least one tile);
// the widest array of the block must stay below 2 GiB (32-bit tile addressing),
// as must the lm_head rows of one chunk (D bf16 values each).
void block_shape(int64_t n_tt, int64_t n_vt, int64_t D, int64_t V, int64_t chunk_rows,
                 int64_t elem_bytes, int64_t widest_bytes, int64_t &R, int64_t &tiles_per_chunk,
                 int64_t &n_vc) {
  if (chunk_rows > kMaxTV) chunk_rows = kMaxTV;
  const int64_t cap = std::max<int64_t>(chunk_rows * V * 4 / elem_bytes, (int64_t)kTile * kTile);
  const int64_t vc_lim = std::max<int64_t>(kTile, (kI32Bytes / (2 * D)) / kTile * kTile);
  R = std::min<int64_t>(kRowBlockMax, n_tt * kTile);
  int64_t n_rb = cdiv(n_tt * kTile, R);
  R = cdiv(n_tt, n_rb) * kTile;
  int64_t vc_max = cap / R / kTile * kTile;
  if (vc_max < kTile) {
    R = std::max<int64_t>(kTile, cap / kTile / kTile * kTile);
    n_rb = cdiv(n_tt * kTile, R);
    R = cdiv(n_tt, n_rb) * kTile;
    vc_max = kTile;
  }
  vc_max = std::min(vc_max, vc_lim);
  vc_max = std::min(vc_max,
                    std::max<int64_t>(kTile, (kI32Bytes / (widest_bytes * R)) / kTile * kTile));
  // Chunks of a multiple of 16 vocabulary tiles keep the dW grid (chunk tiles x
  // 16 hidden tiles at D = 4096) a multiple of the 256 CUs.
  tiles_per_chunk = vc_max / kTile;
  if (tiles_per_chunk >= 16 && (tiles_per_chunk / 16 * 16) * 20 >= tiles_per_chunk * 17)
    tiles_per_chunk = tiles_per_chunk / 16 * 16;
  tiles_per_chunk = std::min(tiles_per_chunk, n_vt);
  n_vc = cdiv(n_vt, tiles_per_chunk);
}

// Backward time of a plan, in microseconds, from a model fitted to 72 measured kernel
// times of 24 plans on MI355X (hidden sizes 1,024 to 5,120, 2,048 to 20,480 tokens): a
// round of 256 workgroups over a 256 x 256 x 256 tile takes kModelTile us (the recompute,
// which also writes G, kModelGrad times that), a partly filled round (f of the CUs busy)
// 0.8 + 0.2 f of a full one (its CUs hold a higher clock), the dH and dW epilogues'
// read-modify-writes move kModelBwDh and kModelBwDw bytes per us, and a launch costs
// kModelLaunch us.  r: token tiles per row block (the last one may be shorter), t:
// vocabulary tiles per chunk, s: dH split count, D: the hidden size of dH and dW, and
// pass_units: the per-tile work of the passes that walk the vocabulary tiles of a
// (row block, chunk), in 256-deep K tiles weighted by their epilogues (the recompute:
// D / 256 x kModelGrad).
constexpr double kModelTile = 6.0, kModelGrad = 1.12, kModelBwDh = 9.0e6, kModelBwDw = 4.5e6,
                 kModelLaunch = 20.0;
// The distillation's block passes relative to a plain K walk, from the measured rates of
// its teacher (p_t written in fp32) and KL student (p_t read, G written) passes against
// the recompute's at distill_qwen3.
constexpr double kModelTeacher = 1.15, kModelStudent = 1.29;

double model_rounds(int64_t wgs, double k) {
  const int64_t full = wgs / kCUs, rem = wgs % kCUs;
  return (double)full * k + (rem ? (0.8 + 0.2 * (double)rem / kCUs) * k : 0.0);
}

double model_bwd(int64_t n_tt, int64_t n_vt, int64_t D, int64_t r, int64_t t, int64_t s,
                 double pass_units) {
  const int64_t Dt = cdiv(D, kTile);
  const int64_t n_rb = cdiv(n_tt, r), n_vc = cdiv(n_vt, t);
  const int64_t rs[2] = {r, n_tt - (n_rb - 1) * r}, rn[2] = {n_rb - 1, 1};
  const int64_t ts[2] = {t, n_vt - (n_vc - 1) * t}, tn[2] = {n_vc - 1, 1};
  double us = 0.0;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      const double n = (double)(rn[i] * tn[j]);
      if (n == 0.0) continue;
      const int64_t ri = rs[i], tc = ts[j];
      const int64_t vs = std::min<int64_t>(tc, std::max<int64_t>(1, kCUs / ri));
      const double grad = (double)cdiv(tc, vs) * pass_units * kModelTile;
      const double dh = model_rounds(ri * Dt * s, (double)tc / (double)s) * kModelTile;
      const double dw = model_rounds(tc * Dt, (double)ri) * kModelTile;
      us += n * (grad + dh + dw + 3.0 * kModelLaunch);  // (one more launch per pass aside)
    }
  const double tile_bytes = (double)kTile * (double)D * 4.0;
  us += (double)n_tt * tile_bytes * (double)s * (double)(2 * n_vc - 1) / kModelBwDh;  // dH sums
  us += (double)n_vt * tile_bytes * (double)(2 * n_rb - 1) / kModelBwDw;              // dW
  us += (double)n_tt * tile_bytes * ((double)s + 0.5) / kModelBwDh;                   // dh_out
  us += 2.0 * (double)n_rb * kModelLaunch;
  return us;
}

int64_t dh_splits_for(int64_t r, int64_t t, int64_t D) {
  const int64_t cap = std::max<int64_t>(1, kDhPartialCap / (r * kTile * D * 4));
  return dh_split_count(r * cdiv(D, kTile), std::min(cap, cdiv(t * kTile, kBK)));
}

// The backward's row block and chunk: where the model puts another choice at least 5%
// below the one the budget rules make (partial rounds of 256 workgroups in dH or dW, or a
// last chunk or row block that fills the chip poorly), that choice, among row blocks of
// [half, all] of R (equalised over the tokens) and chunks of [half, all] of the widest the
// budget allows for them.  The budget is block_shape's: elem_bytes per staged element
// within chunk_rows * V * 4 bytes, widest_bytes per element of the widest array and the
// lm_head rows of a chunk (D_max bf16 values each) below 2 GiB.
void fit_backward(int64_t n_tt, int64_t n_vt, int64_t D, int64_t D_max, int64_t V,
                  int64_t chunk_rows, int64_t elem_bytes, int64_t widest_bytes,
                  double pass_units, int64_t &R, int64_t &tiles_per_chunk, int64_t &n_vc) {
  const int64_t r0 = R / kTile, t0 = tiles_per_chunk;
  const double base =
      model_bwd(n_tt, n_vt, D, r0, t0, dh_splits_for(r0, t0, D), pass_units);
  double best = base;
  int64_t br = r0, bt = t0;
  if (chunk_rows > kMaxTV) chunk_rows = kMaxTV;
  const int64_t cap = std::max<int64_t>(chunk_rows * V * 4 / elem_bytes, (int64_t)kTile * kTile);
  int64_t last_r = 0;
  for (int64_t rc = (r0 + 1) / 2; rc <= r0; ++rc) {
    const int64_t r = cdiv(n_tt, cdiv(n_tt, rc));
    if (r == last_r) continue;
    last_r = r;
    int64_t tm = cap / (r * kTile) / kTile;
    tm = std::min(tm, (kI32Bytes / (2 * D_max)) / kTile);
    tm = std::min(tm, (kI32Bytes / (widest_bytes * r * kTile)) / kTile);
    tm = std::min(tm, n_vt);
    for (int64_t t = std::max<int64_t>(1, tm / 2); t <= tm; ++t) {
      const double c = model_bwd(n_tt, n_vt, D, r, t, dh_splits_for(r, t, D), pass_units);
      if (c < best) {
        best = c;
        br = r;
        bt = t;
      }
    }
  }
  if (best < 0.95 * base) {
    R = br * kTile;
    tiles_per_chunk = bt;
    n_vc = cdiv(n_vt, bt);
  }
}

// Lanes that merge one token's split partials: the power of two covering the
// splits, at most a wave.  A 256-thread block then takes 256 / lanes tokens.
int64_t combine_lanes(int64_t splits) {
  int64_t l = 1;
  while (l < 64 && l < splits) l <<= 1;
  return l;
}

flce_status make_plan(int64_t T, int64_t D, int64_t V, int64_t chunk_rows, Plan &p) {
  flce_status st = check_shape(T, D, V, chunk_rows);
  if (st != FLCE_OK) return st;
  memset(&p, 0, sizeof(p));
  p.T = T;
  p.D = D;
  p.V = V;
  p.chunk_rows = chunk_rows;
  const int64_t Tn = std::max<int64_t>(T, 1);
  p.n_tt = cdiv(Tn, kTile);
  p.n_vt = cdiv(V, kTile);
  p.T_pad = p.n_tt * kTile;
  p.splits = std::min<int64_t>(std::max<int64_t>(kFwdTargetWG / p.n_tt, 1), p.n_vt);
  p.comb_lanes = combine_lanes(p.splits);
  p.n_cblk = cdiv(Tn, 256 / p.comb_lanes);

  // Backward blocking: bf16 gradient values, 2 bytes each.
  int64_t R, n_vc, tiles_per_chunk;
  block_shape(p.n_tt, p.n_vt, D, V, chunk_rows, 2, 2, R, tiles_per_chunk, n_vc);
  fit_backward(p.n_tt, p.n_vt, D, D, V, chunk_rows, 2, 2,
               (double)cdiv(D, kTile) * kModelGrad, R, tiles_per_chunk, n_vc);
  p.R = R;
  p.n_rb = cdiv(p.n_tt * kTile, R);
  p.Tb = p.n_rb * R;
  p.Vc = tiles_per_chunk * kTile;
  p.n_vc = n_vc;
  const int64_t dh_tiles = (R / kTile) * cdiv(D, kTile);
  p.dh_splits = dh_split_count(
      dh_tiles, std::min(std::max<int64_t>(1, kDhPartialCap / (R * D * 4)), cdiv(p.Vc, kBK)));

  size_t off = 0;
  p.off_pm = off; off = align256(off + (size_t)p.splits * p.T_pad * 4);
  p.off_ps = off; off = align256(off + (size_t)p.splits * p.T_pad * 4);
  p.off_zl = off; off = align256(off + (size_t)p.T_pad * 4);
  p.off_bs = off; off = align256(off + (size_t)p.n_cblk * 8);
  p.off_bc = off; off = align256(off + (size_t)p.n_cblk * 4);
  p.fwd_bytes = off;
  off = 0;
  p.off_c = off;  off = align256(off + (size_t)p.Tb * 4);
  p.off_l2 = off; off = align256(off + (size_t)p.Tb * 4);
  p.off_list = off; off = align256(off + 4 + (size_t)p.Tb / kTile * 5);  // count, list, flags
  p.off_G = off;  off = align256(off + (size_t)p.R * p.Vc * 2);
  p.off_dh = off; off = align256(off + (size_t)p.dh_splits * p.R * p.D * 4);
  p.off_ht = off; off = align256(off + (size_t)p.R * p.D * 2);
  p.bwd_bytes = off;
  p.gtile_bytes = (size_t)p.R * p.Vc * 2;
  p.chunk_bound = (size_t)p.chunk_rows * p.V * 4;
  p.total = std::max(p.fwd_bytes, p.bwd_bytes);
  return FLCE_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Schedule of the distillation call: the forward layout for the two
// log-sum-exps, and blocks of R rows x Vc vocabulary entries holding the
// teacher's fp32 probabilities, then the student's bf16 gradient over them (4
// bytes per element), within the fp32 logits of one chunk of chunk_rows rows.
struct DistillPlan {
  int64_t T, Ds, Dt, V, chunk_rows;
  int64_t n_tt, n_vt, splits, T_pad, n_cblk;
  int64_t R, n_rb, Tb, Vc, n_vc, vsplits, dh_splits;
  size_t off_pm, off_ps, off_zl, off_bs, off_bc;
  size_t off_lse_s, off_lse_t, off_l2s, off_l2t, off_c, off_A, off_B;
  size_t off_P, off_pa, off_pb, off_dh, off_ht;
  size_t total;
};

flce_status make_distill_plan(int64_t T, int64_t Ds, int64_t Dt, int64_t V, int64_t chunk_rows,
                              DistillPlan &p) {
  flce_status st = check_shape(T, Ds, V, chunk_rows);
  if (st != FLCE_OK) return st;
  st = check_shape(T, Dt, V, chunk_rows);
  if (st != FLCE_OK) return st;
  memset(&p, 0, sizeof(p));
  p.T = T;
  p.Ds = Ds;
  p.Dt = Dt;
  p.V = V;
  p.chunk_rows = chunk_rows;
  const int64_t Tn = std::max<int64_t>(T, 1);
  p.n_tt = cdiv(Tn, kTile);
  p.n_vt = cdiv(V, kTile);
  p.T_pad = p.n_tt * kTile;
  p.splits = std::min<int64_t>(std::max<int64_t>(kFwdTargetWG / p.n_tt, 1), p.n_vt);
  p.n_cblk = cdiv(Tn, 256);
  int64_t R, tiles_per_chunk, n_vc;
  block_shape(p.n_tt, p.n_vt, std::max(Ds, Dt), V, chunk_rows, 4, 4, R, tiles_per_chunk, n_vc);
  // Prefer chunks of a multiple of 16 vocabulary tiles (whole-wave dW grids and
  // tile launches): halve the row block while that makes room for them.
  const int64_t cap = std::max<int64_t>(std::min<int64_t>(chunk_rows, kMaxTV) * V,
                                        (int64_t)kTile * kTile);
  const int64_t vc_lim = std::max<int64_t>(kTile, (kI32Bytes / (2 * std::max(Ds, Dt))) / kTile * kTile);
  while (tiles_per_chunk < 16 && tiles_per_chunk < p.n_vt && R >= 4 * kTile) {
    const int64_t half = R / 2 / kTile * kTile;
    int64_t vc = std::min<int64_t>(cap / half / kTile * kTile, vc_lim);
    vc = std::min<int64_t>(vc, (kI32Bytes / (4 * half)) / kTile * kTile);
    int64_t tiles = std::min<int64_t>(vc / kTile, p.n_vt);
    if (tiles >= 16) tiles = tiles / 16 * 16;
    if (tiles <= tiles_per_chunk) break;
    R = half;
    tiles_per_chunk = tiles;
    n_vc = cdiv(p.n_vt, tiles);
  }
  // per (row block, chunk): the teacher's block pass over Dt and the student's over Ds
  fit_backward(p.n_tt, p.n_vt, Ds, std::max(Ds, Dt), V, chunk_rows, 4, 4,
               (double)cdiv(Dt, kTile) * kModelTeacher + (double)cdiv(Ds, kTile) * kModelStudent,
               R, tiles_per_chunk, n_vc);
  p.R = R;
  p.n_rb = cdiv(p.n_tt * kTile, R);
  p.Tb = p.n_rb * R;
  p.Vc = tiles_per_chunk * kTile;
  p.n_vc = n_vc;
  // at most one workgroup per CU (a second round would double the launch)
  p.vsplits = std::min<int64_t>(tiles_per_chunk, std::max<int64_t>(1, kCUs / (R / kTile)));
  // dH: one workgroup per output tile once the tiles fill the chip (split-K
  // would add a read-modify-write of the partial sums per chunk).
  const int64_t dh_tiles = (R / kTile) * cdiv(Ds, kTile);
  p.dh_splits = dh_split_count(
      dh_tiles, std::min(std::max<int64_t>(1, kDhPartialCap / (R * Ds * 4)), cdiv(p.Vc, kBK)));

  size_t off = 0;
  p.off_pm = off;    off = align256(off + (size_t)p.splits * p.T_pad * 4);
  p.off_ps = off;    off = align256(off + (size_t)p.splits * p.T_pad * 4);
  p.off_zl = off;    off = align256(off + (size_t)p.T_pad * 4);
  p.off_bs = off;    off = align256(off + (size_t)p.n_cblk * 8);
  p.off_bc = off;    off = align256(off + (size_t)p.n_cblk * 4);
  p.off_lse_s = off; off = align256(off + (size_t)p.Tb * 4);
  p.off_lse_t = off; off = align256(off + (size_t)p.Tb * 4);
  p.off_l2s = off;   off = align256(off + (size_t)p.Tb * 4);
  p.off_l2t = off;   off = align256(off + (size_t)p.Tb * 4);
  p.off_c = off;     off = align256(off + (size_t)p.Tb * 4);
  p.off_A = off;     off = align256(off + (size_t)p.Tb * 4);
  p.off_B = off;     off = align256(off + (size_t)p.Tb * 4);
  p.off_P = off;     off = align256(off + (size_t)p.R * p.Vc * 4);  // p_t, then G over it
  p.off_pa = off;    off = align256(off + (size_t)p.n_vc * p.vsplits * p.R * 4);
  p.off_pb = off;    off = align256(off + (size_t)p.n_vc * p.vsplits * p.R * 4);
  p.off_dh = off;    off = align256(off + (size_t)p.dh_splits * p.R * p.Ds * 4);
  p.off_ht = off;    off = align256(off + (size_t)p.R * p.Ds * 2);
  p.total = off;
  return FLCE_OK;
}

// The current device must be a gfx950.  The answer is cached per device; calls
// from several threads may fill the cache at once and store the same value.
flce_status check_device() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FLCE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(FLCE_ERR_UNSUPPORTED, "device index %d", dev);
  int known = cache[dev].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(FLCE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(known, std::memory_order_relaxed);
  }
  if (known != 1) return fail(FLCE_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  return FLCE_OK;
}

const char *kernel_name(int id) {
  static const char *const names[FLCE_KERNEL_COUNT] = {
      "?",           "fwd_lse",     "fwd_combine", "fwd_mean",    "bwd_prep",
      "bwd_ht",      "bwd_grad",    "bwd_dh",      "bwd_dw",      "bwd_dh_out",
      "fill",        "dst_lse",     "dst_prep",    "dst_teacher", "dst_student",
      "dst_reduce",  "dst_dh",      "dst_dw",      "dst_combine", "policy",
      "fwd_skip_prep", "bwd_zero_rows"};
  return id > 0 && id < FLCE_KERNEL_COUNT ? names[id] : "?";
}

// Per-launch timing (flce_timing_begin / flce_timing_end): while on, an event
// is recorded on the launching stream after every kernel (tagged with its
// code) and before each entry point's first launch (tag 0).  The flag is read
// without the lock on every launch; the marks are taken under it.
struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;
  std::vector<hipStream_t> st;
  std::vector<int32_t> id;
  int32_t used = 0, dropped = 0;
};

Timing &timing() {
  static Timing t;
  return t;
}

void timing_mark(int32_t id, hipStream_t s) {
  Timing &t = timing();
  if (!t.on.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on.load(std::memory_order_relaxed)) return;
  if (t.used >= (int32_t)t.ev.size()) {
    ++t.dropped;
    return;
  }
  if (hipEventRecord(t.ev[t.used], s) != hipSuccess) {
    (void)hipGetLastError();  // a lost mark must not read as the next launch's failure
    ++t.dropped;
    return;
  }
  t.st[t.used] = s;
  t.id[t.used] = id;
  ++t.used;
}

// Marks the start of an entry point's launches on s.
void timing_start(hipStream_t s) { timing_mark(0, s); }

// Checks a launch of kernel `id` on s and, with timing on, marks its end.
flce_status launched(int32_t id, hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FLCE_ERR_HIP, "%s launch: %s", kernel_name(id), hipGetErrorString(e));
  timing_mark(id, s);
  return FLCE_OK;
}

#define FLCE_TRY(x)                      \
  do {                                   \
    flce_status s_ = (x);                \
    if (s_ != FLCE_OK) return s_;        \
  } while (0)

// Folds the logit transform into the kernels' parameters.  Without a cap the
// transform is the single scale (multiply / divide) / temperature; with one,
// the kernels apply cap * tanh(z * scale / cap) / temperature per logit.
flce_status make_xform(const flce_logit_transform *t, Xform &x, bool &cap) {
  x.zscale = 1.f;
  x.cap = 0.f;
  x.inv_cap = 0.f;
  x.inv_temp = 1.f;
  cap = false;
  if (!t) return FLCE_OK;
  const float mul = t->scale_multiply, div = t->scale_divide, sc = t->softcap,
              temp = t->temperature;
  if (!std::isfinite(mul) || !std::isfinite(div) || !std::isfinite(sc) ||
      !std::isfinite(temp) || mul < 0.f || div < 0.f || sc < 0.f || !(temp > 0.f))
    return fail(FLCE_ERR_ARG,
                "logit transform (multiply %g, divide %g, softcap %g, temperature %g): the "
                "first three must be finite and >= 0, temperature finite and > 0",
                mul, div, sc, temp);
  const double s1 = (mul != 0.f ? (double)mul : 1.0) / (div != 0.f ? (double)div : 1.0);
  const double inv_temp = 1.0 / (double)temp;
  cap = sc != 0.f;
  const double zscale = cap ? s1 : s1 * inv_temp;
  const double inv_cap = cap ? 1.0 / (double)sc : 0.0;
  const double lim = 3.0e38, tiny = 1.0e-37;
  if (!(zscale <= lim && zscale >= tiny) || !(inv_temp <= lim && inv_temp >= tiny) ||
      !(inv_cap <= lim) || (cap && inv_cap < tiny))
    return fail(FLCE_ERR_ARG, "logit transform factors are out of the fp32 range");
  x.zscale = (float)zscale;
  x.cap = sc;
  x.inv_cap = (float)inv_cap;
  x.inv_temp = cap ? (float)inv_temp : 1.f;
  return FLCE_OK;
}

// Every kernel parameter block below is value-initialised ({}), so a field that a
// launch does not set is zero (null pointers, flags off).

// H^T of a row block for the dW kernel's K-contiguous operand.
// With a list in `map` the rows are its tiles' (T: the token count).
flce_status launch_ht(const void *hidden, uint16_t *ht, int64_t D, int64_t R, int64_t rb0,
                      int64_t rcount, hipStream_t s, const RowMap &map = RowMap{},
                      int64_t T = 0) {
  BwdHtParams t{};
  t.hidden = (const uint16_t *)hidden;
  t.ht = ht;
  t.T = (int)T;
  t.D = (int)D;
  t.R = (int)R;
  t.rb0 = (int)rb0;
  t.rcount = (int)rcount;
  t.tiles_id = (int)cdiv(rcount, kTile);
  t.map = map;
  // a list never holds more tiles for a block than it has as laid out
  const int64_t rows = map.list ? t.tiles_id * kTile : rcount;
  bwd_ht_kernel<<<dim3((unsigned)cdiv(rows, 64), (unsigned)cdiv(D, 64)), 256, 0, s>>>(t);
  return launched(FLCE_KERNEL_BWD_HT, s);
}

// dH partial sums and the dW update of one (row block, vocabulary chunk) from
// its bf16 gradient block G: token rows of pitch Gp, gcols vocabulary columns
// (a multiple of 256), plain or grouped (written over an fp32 block: Gp =
// 2 gcols, each 128-column group in the first half of its fp32 bytes).  A
// NULL dhacc skips dH, a NULL grad_weight skips dW.  `map` gives the row block's
// token tiles (no list: as laid out).
flce_status launch_dh_dw(const uint16_t *G, int Gp, int64_t gcols, bool grouped,
                         const void *weight, const uint16_t *ht, int64_t D, int64_t V, int64_t R,
                         int64_t rcount, int64_t vc0, int64_t vcount, int64_t dh_splits,
                         float *dhacc, float *grad_weight, bool acc_dh, bool acc_dw,
                         const RowMap &map, hipStream_t s) {
  const int tiles_h = (int)cdiv(D, kTile);
  BwdDhParams h{};
  h.G = G;
  h.weight = (const uint16_t *)weight;
  h.Gp = Gp;
  h.D = (int)D;
  h.V = (int)V;
  h.vc0 = (int)vc0;
  h.vcount = (int)vcount;
  h.Kc = (int)std::min<int64_t>(gcols, cdiv(vcount, kBK) * kBK);  // G is zero past vcount
  h.R = (int)R;
  h.tiles_m = (int)(R / kTile);
  h.tiles_n = tiles_h;
  h.splits = (int)dh_splits;
  h.acc = dhacc;
  h.accumulate = acc_dh ? 1 : 0;
  h.map = map;
  const unsigned dh_grid = (unsigned)(h.tiles_m * h.tiles_n * h.splits);
  if (dhacc) {
    if (grouped)
      dst_dh_kernel<<<dh_grid, kThreads, 0, s>>>(h);
    else
      bwd_dh_kernel<<<dh_grid, kThreads, 0, s>>>(h);
    FLCE_TRY(launched(grouped ? FLCE_KERNEL_DST_DH : FLCE_KERNEL_BWD_DH, s));
  }
  if (!grad_weight) return FLCE_OK;

  BwdDwParams w{};
  w.G = G;
  w.ht = ht;
  w.Gp = Gp;
  w.D = (int)D;
  w.V = (int)V;
  w.R = (int)R;
  w.rcount = (int)rcount;
  w.vc0 = (int)vc0;
  w.tiles_m = (int)(gcols / kTile);
  w.tiles_n = tiles_h;
  w.dW = grad_weight;
  w.accumulate = acc_dw ? 1 : 0;
  w.map = map;
  if (grouped)
    dst_dw_kernel<<<(unsigned)(w.tiles_m * w.tiles_n), kThreads, 0, s>>>(w);
  else
    bwd_dw_kernel<<<(unsigned)(w.tiles_m * w.tiles_n), kThreads, 0, s>>>(w);
  return launched(grouped ? FLCE_KERNEL_DST_DW : FLCE_KERNEL_BWD_DW, s);
}

// dH rows of a row block: sum of the split-K partials, rounded to bf16.
flce_status launch_dh_out(const float *dhacc, void *grad_hidden, int64_t D, int64_t R,
                          int64_t dh_splits, int64_t rb0, int64_t rcount, hipStream_t s,
                          const RowMap &map = RowMap{}, int64_t T = 0) {
  BwdDhOutParams o{};
  o.acc = dhacc;
  o.dH = (uint16_t *)grad_hidden;
  o.T = (int)T;
  o.map = map;
  o.D = (int)D;
  o.R = (int)R;
  o.splits = (int)dh_splits;
  o.rb0 = (int)rb0;
  o.rcount = (int)rcount;
  // a list never holds more tiles for a block than it has as laid out
  const int64_t work = (map.list ? cdiv(rcount, kTile) * kTile : rcount) * (D / 8);
  bwd_dh_out_kernel<<<(unsigned)std::min<int64_t>(cdiv(work, 256), 8192), 256, 0, s>>>(o);
  return launched(FLCE_KERNEL_BWD_DH_OUT, s);
}

flce_status fill(float *dst, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return FLCE_OK;
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
  fill_f32_kernel<<<(unsigned)blocks, 256, 0, s>>>(dst, n, v);
  return launched(FLCE_KERNEL_FILL, s);
}

// Forward KL (jsd = false) or the generalized Jensen-Shannon divergence with
// weight beta (jsd = true); the entry points below differ only in that.
flce_status distill_run(bool jsd, float beta, const void *student_hidden,
                        const void *student_weight, int64_t Ds, const void *teacher_hidden,
                        const void *teacher_weight, int64_t Dt, const int64_t *labels,
                        int64_t ignore_index, int64_t T, int64_t V, int64_t chunk_rows,
                        const flce_logit_transform *transform, float *kl_out, float *mean_out,
                        const float *grad_out, const float *grad_mean, void *grad_student_hidden,
                        float *grad_student_weight, int accumulate_grad_weight, void *workspace,
                        size_t workspace_bytes, void *stream) {
  g_last_error[0] = 0;
  DistillPlan p;
  FLCE_TRY(make_distill_plan(T, Ds, Dt, V, chunk_rows, p));
  Xform xf;
  bool cap;
  FLCE_TRY(make_xform(transform, xf, cap));
  if (jsd && !(beta > 0.f && beta < 1.f))
    return fail(FLCE_ERR_ARG, "JSD weight beta = %g must lie in (0, 1)", (double)beta);
  if (grad_out && grad_mean)
    return fail(FLCE_ERR_ARG, "give at most one of grad_out and grad_mean");
  const bool grads = grad_out || grad_mean;
  if (grads && !grad_student_weight && !grad_student_hidden)
    return fail(FLCE_ERR_ARG,
                "a gradient was requested but grad_student_hidden and grad_student_weight are "
                "both NULL");
  if (grad_student_weight && !aligned(grad_student_weight, 16))
    return fail(FLCE_ERR_ARG, "grad_student_weight not 16-byte aligned");
  if (T > 0) {
    if (!student_hidden || !student_weight || !teacher_hidden || !teacher_weight || !workspace)
      return fail(FLCE_ERR_ARG, "a required pointer is NULL");
    if (!aligned(student_hidden, 16) || !aligned(student_weight, 16) ||
        !aligned(teacher_hidden, 16) || !aligned(teacher_weight, 16) ||
        !aligned(workspace, 16) || (labels && !aligned(labels, 8)) ||
        (kl_out && !aligned(kl_out, 4)) || (mean_out && !aligned(mean_out, 4)) ||
        (grad_out && !aligned(grad_out, 4)) || (grad_mean && !aligned(grad_mean, 4)) ||
        (grad_student_hidden && !aligned(grad_student_hidden, 16)))
      return fail(FLCE_ERR_ARG, "misaligned pointer");
    if (workspace_bytes < p.total)
      return fail(FLCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                  p.total);
  }
  FLCE_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  timing_start(s);
  if (T == 0) {
    if (mean_out) FLCE_TRY(fill(mean_out, 1, 0.f, s));
    if (grads && grad_student_weight && !accumulate_grad_weight)
      FLCE_TRY(fill(grad_student_weight, V * Ds, 0.f, s));
    return FLCE_OK;
  }
  const bool want_dh = grads && grad_student_hidden, want_dw = grads && grad_student_weight;

  char *ws = (char *)workspace;
  float *lse_s = (float *)(ws + p.off_lse_s), *lse_t = (float *)(ws + p.off_lse_t);
  float *l2s = (float *)(ws + p.off_l2s), *l2t = (float *)(ws + p.off_l2t);
  float *cbuf = (float *)(ws + p.off_c);
  float *Abuf = (float *)(ws + p.off_A), *Bbuf = (float *)(ws + p.off_B);
  float *Pbuf = (float *)(ws + p.off_P);
  uint16_t *G = (uint16_t *)Pbuf;  // the student's gradient replaces p_t in place
  float *part_a = (float *)(ws + p.off_pa), *part_b = (float *)(ws + p.off_pb);
  float *dhacc = (float *)(ws + p.off_dh);
  uint16_t *ht = (uint16_t *)(ws + p.off_ht);

  // Log-sum-exp of each head: the fused forward kernel without labels.
  for (int head = 0; head < 2; ++head) {
    FwdLseParams a{};
    a.hidden = (const uint16_t *)(head ? student_hidden : teacher_hidden);
    a.weight = (const uint16_t *)(head ? student_weight : teacher_weight);
    a.labels = nullptr;
    a.ignore_index = ignore_index;
    a.T = (int)T;
    a.D = (int)(head ? Ds : Dt);
    a.V = (int)V;
    a.n_tt = (int)p.n_tt;
    a.n_vt = (int)p.n_vt;
    a.splits = (int)p.splits;
    a.T_pad = (int)p.T_pad;
    a.xf = xf;
    a.part_m = (float *)(ws + p.off_pm);
    a.part_s = (float *)(ws + p.off_ps);
    a.zlab = (float *)(ws + p.off_zl);
    if (cap)
      fwd_lse_kernel<true><<<(unsigned)(p.n_tt * p.splits), kThreads, 0, s>>>(a);
    else
      fwd_lse_kernel<false><<<(unsigned)(p.n_tt * p.splits), kThreads, 0, s>>>(a);
    FLCE_TRY(launched(FLCE_KERNEL_FWD_LSE, s));
    DstLseParams l{};
    l.part_m = a.part_m;
    l.part_s = a.part_s;
    l.T = (int)T;
    l.splits = (int)p.splits;
    l.T_pad = (int)p.T_pad;
    l.n = (int)p.Tb;
    l.lanes = (int)combine_lanes(p.splits);
    l.lse = head ? lse_s : lse_t;
    l.lse2 = head ? l2s : l2t;
    dst_lse_kernel<<<(unsigned)cdiv(p.Tb, 256 / l.lanes), 256, 0, s>>>(l);
    FLCE_TRY(launched(FLCE_KERNEL_DST_LSE, s));
  }

  DstPrepParams pr{};
  pr.labels = labels;
  pr.grad_out = grad_out;
  pr.grad_mean = grad_mean;
  pr.ignore_index = ignore_index;
  pr.T = grads ? (int)T : 0;  // no gradient: c = 0 everywhere
  pr.n = (int)p.Tb;
  pr.c = cbuf;
  dst_prep_kernel<<<1, 1024, 0, s>>>(pr);
  FLCE_TRY(launched(FLCE_KERNEL_DST_PREP, s));

  // One block pass of dst_tile_kernel in the given role over the chunk at vc0.
  auto tile_pass = [&](int role, int64_t rb0, int64_t tiles_n, int64_t vc, float *part,
                       float *part2) -> flce_status {
    const int64_t vc0 = vc * p.Vc;
    const int64_t vcount = std::min<int64_t>(p.Vc, V - vc0);
    const bool teacher = role == kRoleTeacher;
    DstTileParams d{};
    d.hidden = (const uint16_t *)(teacher ? teacher_hidden : student_hidden);
    d.weight = (const uint16_t *)(teacher ? teacher_weight : student_weight);
    d.lse2 = teacher ? l2t : l2s;
    d.c = cbuf;
    d.gbar2 = Bbuf;
    d.beta = beta;
    d.T = (int)T;
    d.D = (int)(teacher ? Dt : Ds);
    d.V = (int)V;
    d.rb0 = (int)rb0;
    d.vc0 = (int)vc0;
    d.n_vt = (int)cdiv(vcount, kTile);
    d.tiles_n = (int)tiles_n;
    d.vsplits = (int)p.vsplits;
    d.R = (int)p.R;
    d.xf = xf;
    d.P = Pbuf;
    d.Pp = (int)p.Vc;
    d.G = G;  // over P, grouped
    d.Gp = (int)(2 * p.Vc);
    d.part = part;
    d.part2 = part2;
    const unsigned grid = (unsigned)(tiles_n * p.vsplits);
#define FLCE_TILE(R)                                                              \
  (cap ? dst_tile_kernel<R, true><<<grid, kThreads, 0, s>>>(d)                   \
       : dst_tile_kernel<R, false><<<grid, kThreads, 0, s>>>(d))
    switch (role) {
      case kRoleTeacher: FLCE_TILE(kRoleTeacher); break;
      case kRoleStudentKL: FLCE_TILE(kRoleStudentKL); break;
      case kRoleJsdStats: FLCE_TILE(kRoleJsdStats); break;
      default: FLCE_TILE(kRoleJsdGrad); break;
    }
#undef FLCE_TILE
    return launched(teacher ? FLCE_KERNEL_DST_TEACHER : FLCE_KERNEL_DST_STUDENT, s);
  };
  auto dh_dw = [&](int64_t rb, int64_t rcount, int64_t vc) -> flce_status {
    const int64_t vc0 = vc * p.Vc;
    const int64_t vcount = std::min<int64_t>(p.Vc, V - vc0);
    return launch_dh_dw(G, (int)(2 * p.Vc), p.Vc, true, student_weight, ht, Ds, V, p.R, rcount,
                        vc0, vcount, p.dh_splits, want_dh ? dhacc : nullptr,
                        want_dw ? grad_student_weight : nullptr, vc > 0,
                        accumulate_grad_weight || rb > 0, RowMap{}, s);
  };
  const int nparts = (int)(p.n_vc * p.vsplits);
  auto reduce = [&](int64_t rb0, int64_t rcount) -> flce_status {
    for (int k = 0; k < 2; ++k) {
      dst_reduce_kernel<<<(unsigned)cdiv(rcount, 64), 256, 0, s>>>(
          k ? part_b : part_a, nparts, (int)p.R, (int)rb0, (int)rcount, k ? Bbuf : Abuf);
      FLCE_TRY(launched(FLCE_KERNEL_DST_REDUCE, s));
    }
    return FLCE_OK;
  };

  for (int64_t rb = 0; rb < p.n_rb; ++rb) {
    const int64_t rb0 = rb * p.R;
    const int64_t rcount = std::min<int64_t>(p.R, T - rb0);
    if (rcount <= 0) break;
    const int64_t tiles_n = cdiv(rcount, kTile);
    if (want_dw) FLCE_TRY(launch_ht(student_hidden, ht, Ds, p.R, rb0, rcount, s));
    for (int64_t vc = 0; vc < p.n_vc; ++vc) {
      float *pa = part_a + (size_t)vc * p.vsplits * p.R;
      float *pb = part_b + (size_t)vc * p.vsplits * p.R;
      // teacher: p_t block (and, for KL, partial sums of A)
      FLCE_TRY(tile_pass(kRoleTeacher, rb0, tiles_n, vc, pa, nullptr));
      if (!jsd) {
        // student: partial sums of B and the gradient block
        FLCE_TRY(tile_pass(kRoleStudentKL, rb0, tiles_n, vc, pb, nullptr));
        if (grads) FLCE_TRY(dh_dw(rb, rcount, vc));
      } else {
        // student: partial sums of the divergence (A) and of gbar (B)
        FLCE_TRY(tile_pass(kRoleJsdStats, rb0, tiles_n, vc, pa, pb));
      }
    }
    FLCE_TRY(reduce(rb0, rcount));
    if (jsd && grads) {
      // the gradient needs each token's complete gbar: a second pass over the chunks
      for (int64_t vc = 0; vc < p.n_vc; ++vc) {
        FLCE_TRY(tile_pass(kRoleTeacher, rb0, tiles_n, vc, part_a, nullptr));
        FLCE_TRY(tile_pass(kRoleJsdGrad, rb0, tiles_n, vc, nullptr, nullptr));
        FLCE_TRY(dh_dw(rb, rcount, vc));
      }
    }
    if (want_dh)
      FLCE_TRY(launch_dh_out(dhacc, grad_student_hidden, Ds, p.R, p.dh_splits, rb0, rcount, s));
  }

  DstCombineParams c{};
  c.jsd = jsd ? 1 : 0;
  c.A = Abuf;
  c.B = Bbuf;
  c.lse_s = lse_s;
  c.lse_t = lse_t;
  c.labels = labels;
  c.ignore_index = ignore_index;
  c.T = (int)T;
  c.kl = kl_out;
  c.blk_sum = (double *)(ws + p.off_bs);
  c.blk_cnt = (int *)(ws + p.off_bc);
  dst_combine_kernel<<<(unsigned)p.n_cblk, 256, 0, s>>>(c);
  FLCE_TRY(launched(FLCE_KERNEL_DST_COMBINE, s));
  if (mean_out) {
    fwd_mean_kernel<<<1, 256, 0, s>>>(c.blk_sum, c.blk_cnt, (int)p.n_cblk, mean_out);
    FLCE_TRY(launched(FLCE_KERNEL_FWD_MEAN, s));
  }
  return FLCE_OK;
}

// Argument checks shared by the two forward entry points (everything but the
// workspace), and the plan and transform they run with.
flce_status forward_checks(const void *hidden, const void *weight, const int64_t *labels,
                           int64_t T, int64_t D, int64_t V, int64_t chunk_rows, int mode,
                           const flce_logit_transform *transform, const float *out,
                           const float *lse, const float *mean_out, Plan &p, Xform &xf,
                           bool &cap) {
  FLCE_TRY(make_plan(T, D, V, chunk_rows, p));
  if (mode != FLCE_MODE_NLL && mode != FLCE_MODE_LOGPROB)
    return fail(FLCE_ERR_ARG, "mode %d is neither NLL (0) nor LOGPROB (1)", mode);
  FLCE_TRY(make_xform(transform, xf, cap));
  if (T > 0) {
    if (!hidden || !weight || !labels || !out || !lse)
      return fail(FLCE_ERR_ARG, "a required pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(labels, 8) ||
        !aligned(out, 4) || !aligned(lse, 4) || (mean_out && !aligned(mean_out, 4)))
      return fail(FLCE_ERR_ARG, "misaligned pointer (hidden/weight/workspace need 16 bytes)");
  }
  return FLCE_OK;
}

// The forward's launches with its partial results at ws (p.fwd_bytes bytes).
flce_status forward_launch(const Plan &p, const Xform &xf, bool cap, const void *hidden,
                           const void *weight, const int64_t *labels, int64_t ignore_index,
                           int mode, float *out, float *lse, float *mean_out, char *ws,
                           hipStream_t s, char *skip_buf = nullptr) {
  const int64_t T = p.T, D = p.D, V = p.V;
  timing_start(s);
  if (T == 0) return mean_out ? fill(mean_out, 1, 0.f, s) : FLCE_OK;

  // skip_buf (8 + 5 n_tt bytes, 4-aligned): the count of the token tiles with a label,
  // the forward's split count for them, their list, then a flag per tile; tiles whose
  // labels are all ignore_index are left out.
  int *n_act = nullptr, *act_list = nullptr, *splits_eff = nullptr;
  uint8_t *tile_act = nullptr;
  if (skip_buf && labels) {
    n_act = (int *)skip_buf;
    splits_eff = n_act + 1;
    act_list = n_act + 2;
    tile_act = (uint8_t *)(act_list + p.n_tt);
    FwdSkipPrepParams q{};
    q.labels = labels;
    q.ignore_index = ignore_index;
    q.T = (int)T;
    q.n_tt = (int)p.n_tt;
    q.n_vt = (int)p.n_vt;
    q.max_splits = (int)p.splits;
    q.tile_act = tile_act;
    q.act_list = act_list;
    q.n_act = n_act;
    q.splits_eff = splits_eff;
    fwd_skip_prep_kernel<<<1, 1024, 0, s>>>(q);
    FLCE_TRY(launched(FLCE_KERNEL_FWD_SKIP_PREP, s));
  }

  FwdLseParams a{};
  a.hidden = (const uint16_t *)hidden;
  a.weight = (const uint16_t *)weight;
  a.labels = labels;
  a.ignore_index = ignore_index;
  a.T = (int)T;
  a.D = (int)D;
  a.V = (int)V;
  a.n_tt = (int)p.n_tt;
  a.n_vt = (int)p.n_vt;
  a.splits = (int)p.splits;
  a.T_pad = (int)p.T_pad;
  a.xf = xf;
  a.part_m = (float *)(ws + p.off_pm);
  a.part_s = (float *)(ws + p.off_ps);
  a.zlab = (float *)(ws + p.off_zl);
  a.act_list = act_list;
  a.n_act = n_act;
  a.splits_eff = splits_eff;
  if (cap)
    fwd_lse_kernel<true><<<(unsigned)(p.n_tt * p.splits), kThreads, 0, s>>>(a);
  else
    fwd_lse_kernel<false><<<(unsigned)(p.n_tt * p.splits), kThreads, 0, s>>>(a);
  FLCE_TRY(launched(FLCE_KERNEL_FWD_LSE, s));

  FwdCombineParams c{};
  c.part_m = a.part_m;
  c.part_s = a.part_s;
  c.zlab = a.zlab;
  c.tile_act = tile_act;
  c.splits_eff = splits_eff;
  c.labels = labels;
  c.ignore_index = ignore_index;
  c.T = (int)T;
  c.V = (int)V;
  c.splits = (int)p.splits;
  c.T_pad = (int)p.T_pad;
  c.mode = mode;
  c.lanes = (int)p.comb_lanes;
  c.out = out;
  c.lse = lse;
  c.blk_sum = (double *)(ws + p.off_bs);
  c.blk_cnt = (int *)(ws + p.off_bc);
  fwd_combine_kernel<<<(unsigned)p.n_cblk, 256, 0, s>>>(c);
  FLCE_TRY(launched(FLCE_KERNEL_FWD_COMBINE, s));
  if (mean_out) {
    fwd_mean_kernel<<<1, 256, 0, s>>>(c.blk_sum, c.blk_cnt, (int)p.n_cblk, mean_out);
    FLCE_TRY(launched(FLCE_KERNEL_FWD_MEAN, s));
  }
  return FLCE_OK;
}

}  // namespace

// Scratch of flce_forward_noalloc: the forward's partial results, for callers
// that cannot allocate.  One copy per GPU, reserved when the library's code is
// loaded on that GPU and kept until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device.  Host code must never use
// the array's name as an address (it is a host-side stand-in); the address is
// asked of the runtime once per device, with that device current, and kept.
flce_status scratch_address(char **out) {
  static std::atomic<void *> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FLCE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(FLCE_ERR_UNSUPPORTED, "device index %d", dev);
  void *ptr = cache[dev].load(std::memory_order_acquire);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FLCE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    cache[dev].store(ptr, std::memory_order_release);
  }
  *out = (char *)ptr;
  return FLCE_OK;
}

}  // namespace

extern "C" {

size_t flce_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk_rows) {
  Plan p;
  if (make_plan(T, D, V, chunk_rows, p) != FLCE_OK) return 0;
  return p.total;
}

flce_status flce_describe_plan(int64_t T, int64_t D, int64_t V, int64_t chunk_rows,
                               int64_t *info) {
  if (!info) return fail(FLCE_ERR_ARG, "info is NULL");
  Plan p;
  FLCE_TRY(make_plan(T, D, V, chunk_rows, p));
  const int64_t v[12] = {p.n_tt, p.n_vt, p.splits, p.R, p.n_rb, p.Vc, p.n_vc, p.dh_splits,
                         (int64_t)p.fwd_bytes, (int64_t)p.bwd_bytes, (int64_t)p.gtile_bytes,
                         (int64_t)p.chunk_bound};
  memcpy(info, v, sizeof(v));
  return FLCE_OK;
}

const char *flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_ARG: return "invalid argument (pointer, alignment or mode)";
    case FLCE_ERR_SHAPE: return "invalid or too large shape";
    case FLCE_ERR_WORKSPACE: return "workspace too small";
    case FLCE_ERR_UNSUPPORTED: return "unsupported shape or device";
    case FLCE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *flce_last_error(void) { return g_last_error; }

const char *flce_kernel_name(int32_t id) { return kernel_name(id); }

flce_status flce_timing_begin(int32_t capacity) {
  g_last_error[0] = 0;
  if (capacity < 1 || capacity > (1 << 20))
    return fail(FLCE_ERR_ARG, "timing capacity %d outside 1 .. 1048576", (int)capacity);
  Timing &t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.on.load(std::memory_order_relaxed)) return fail(FLCE_ERR_ARG, "timing is already on");
  t.ev.assign((size_t)capacity, nullptr);
  for (int32_t i = 0; i < capacity; ++i) {
    const hipError_t e = hipEventCreate(&t.ev[i]);
    if (e != hipSuccess) {
      for (int32_t j = 0; j < i; ++j) (void)hipEventDestroy(t.ev[j]);
      t.ev.clear();
      return fail(FLCE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  t.st.assign((size_t)capacity, nullptr);
  t.id.assign((size_t)capacity, 0);
  t.used = 0;
  t.dropped = 0;
  t.on.store(true, std::memory_order_release);
  return FLCE_OK;
}

flce_status flce_timing_end(int32_t *ids, float *ms, int32_t capacity, int32_t *count,
                            int32_t *dropped) {
  g_last_error[0] = 0;
  if (!ids || !ms || !count || capacity < 0)
    return fail(FLCE_ERR_ARG, "ids, ms and count must not be NULL, capacity >= 0");
  Timing &t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on.load(std::memory_order_relaxed)) return fail(FLCE_ERR_ARG, "timing is not on");
  t.on.store(false, std::memory_order_release);
  flce_status st = FLCE_OK;
  for (int32_t i = 0; i < t.used && st == FLCE_OK; ++i) {
    const hipError_t e = hipEventSynchronize(t.ev[i]);
    if (e != hipSuccess) st = fail(FLCE_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
  }
  int32_t n = 0;
  for (int32_t i = 0; i < t.used && st == FLCE_OK; ++i) {
    if (t.id[i] == 0) continue;  // an entry point's start mark
    float v = -1.f;
    if (i > 0 && t.st[i - 1] == t.st[i]) {
      const hipError_t e = hipEventElapsedTime(&v, t.ev[i - 1], t.ev[i]);
      if (e != hipSuccess)
        st = fail(FLCE_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    }
    if (n < capacity) {
      ids[n] = t.id[i];
      ms[n] = v;
    }
    ++n;
  }
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  *count = n;
  if (dropped) *dropped = t.dropped;
  t.used = t.dropped = 0;
  return st;
}

// flce_forward, or (skip_buf non-null: 8 + 5 ceil(T / 256) bytes of scratch) the same
// with the token tiles whose labels are all ignore_index left out: their out is 0 as
// always, their lse -inf.
static flce_status forward_entry(const void *hidden, const void *weight, const int64_t *labels,
                                 int64_t T, int64_t D, int64_t V, int64_t ignore_index,
                                 int64_t chunk_rows, int mode,
                                 const flce_logit_transform *transform, float *out, float *lse,
                                 float *mean_out, void *workspace, size_t workspace_bytes,
                                 void *stream, char *skip_buf) {
  Plan p;
  Xform xf;
  bool cap;
  FLCE_TRY(forward_checks(hidden, weight, labels, T, D, V, chunk_rows, mode, transform, out,
                          lse, mean_out, p, xf, cap));
  if (T > 0) {
    if (!workspace) return fail(FLCE_ERR_ARG, "a required pointer is NULL");
    if (!aligned(workspace, 16))
      return fail(FLCE_ERR_ARG, "misaligned pointer (hidden/weight/workspace need 16 bytes)");
    if (workspace_bytes < p.total)
      return fail(FLCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                  p.total);
  }
  FLCE_TRY(check_device());
  return forward_launch(p, xf, cap, hidden, weight, labels, ignore_index, mode, out, lse,
                        mean_out, (char *)workspace, (hipStream_t)stream, skip_buf);
}

flce_status flce_forward(const void *hidden, const void *weight, const int64_t *labels,
                         int64_t T, int64_t D, int64_t V, int64_t ignore_index,
                         int64_t chunk_rows, int mode, const flce_logit_transform *transform,
                         float *out, float *lse, float *mean_out,
                         void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error[0] = 0;
  return forward_entry(hidden, weight, labels, T, D, V, ignore_index, chunk_rows, mode,
                       transform, out, lse, mean_out, workspace, workspace_bytes, stream,
                       nullptr);
}

flce_status flce_forward_noalloc(const void *hidden, const void *weight, const int64_t *labels,
                                 int64_t T, int64_t D, int64_t V, int64_t ignore_index,
                                 int64_t chunk_rows, int mode,
                                 const flce_logit_transform *transform, float *out, float *lse,
                                 float *mean_out, void *stream) {
  g_last_error[0] = 0;
  Plan p;
  Xform xf;
  bool cap;
  FLCE_TRY(forward_checks(hidden, weight, labels, T, D, V, chunk_rows, mode, transform, out,
                          lse, mean_out, p, xf, cap));
  if (T > 0 && p.fwd_bytes > kScratchBytes)
    return fail(FLCE_ERR_WORKSPACE,
                "the forward needs %zu bytes of scratch for T = %lld, more than the %zu bytes "
                "of the library's fixed array (use flce_forward with a workspace)",
                p.fwd_bytes, (long long)T, kScratchBytes);
  FLCE_TRY(check_device());
  char *ws = nullptr;
  if (T > 0) FLCE_TRY(scratch_address(&ws));
  return forward_launch(p, xf, cap, hidden, weight, labels, ignore_index, mode, out, lse,
                        mean_out, ws, (hipStream_t)stream);
}

flce_status flce_backward(const void *hidden, const void *weight, const int64_t *labels,
                          const float *lse, int64_t T, int64_t D, int64_t V,
                          int64_t ignore_index, int64_t chunk_rows, int mode,
                          const flce_logit_transform *transform, const float *grad_out,
                          const float *grad_mean, void *grad_hidden, float *grad_weight,
                          int accumulate_grad_weight, void *workspace, size_t workspace_bytes,
                          void *stream) {
  g_last_error[0] = 0;
  Plan p;
  FLCE_TRY(make_plan(T, D, V, chunk_rows, p));
  if (mode != FLCE_MODE_NLL && mode != FLCE_MODE_LOGPROB)
    return fail(FLCE_ERR_ARG, "mode %d is neither NLL (0) nor LOGPROB (1)", mode);
  Xform xf;
  bool cap;
  FLCE_TRY(make_xform(transform, xf, cap));
  if ((grad_out == nullptr) == (grad_mean == nullptr))
    return fail(FLCE_ERR_ARG, "exactly one of grad_out and grad_mean must be given");
  if (!grad_weight && !grad_hidden)
    return fail(FLCE_ERR_ARG, "grad_hidden and grad_weight are both NULL: nothing to compute");
  if (grad_weight && !aligned(grad_weight, 16))
    return fail(FLCE_ERR_ARG, "grad_weight not 16-byte aligned");
  if (T > 0) {
    if (!hidden || !weight || !labels || !lse || !workspace)
      return fail(FLCE_ERR_ARG, "a required pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(labels, 8) ||
        !aligned(lse, 4) || (grad_hidden && !aligned(grad_hidden, 16)) ||
        !aligned(workspace, 16) ||
        (grad_out && !aligned(grad_out, 4)) || (grad_mean && !aligned(grad_mean, 4)))
      return fail(FLCE_ERR_ARG, "misaligned pointer");
    if (workspace_bytes < p.total)
      return fail(FLCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                  p.total);
  }
  FLCE_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  timing_start(s);
  if (T == 0)
    return (accumulate_grad_weight || !grad_weight) ? FLCE_OK : fill(grad_weight, V * D, 0.f, s);

  char *ws = (char *)workspace;
  float *cbuf = (float *)(ws + p.off_c);
  float *l2buf = (float *)(ws + p.off_l2);
  // the token tiles with a gradient: their count, their list, a flag per tile
  int *n_act = (int *)(ws + p.off_list);
  int *act_list = n_act + 1;
  uint8_t *tile_act = (uint8_t *)(act_list + p.Tb / kTile);
  const int64_t n_real = cdiv(T, kTile);
  uint16_t *G = (uint16_t *)(ws + p.off_G);
  float *dhacc = (float *)(ws + p.off_dh);
  uint16_t *ht = (uint16_t *)(ws + p.off_ht);

  BwdPrepParams pr{};
  pr.labels = labels;
  pr.lse = lse;
  pr.grad_out = grad_out;
  pr.grad_mean = grad_mean;
  pr.ignore_index = ignore_index;
  pr.T = (int)T;
  pr.V = (int)V;
  pr.T_pad = (int)p.Tb;
  pr.mode = mode;
  pr.c = cbuf;
  pr.lse2 = l2buf;
  pr.n_real = (int)n_real;
  pr.tile_act = tile_act;
  pr.act_list = act_list;
  pr.n_act = n_act;
  bwd_prep_kernel<<<1, 1024, 0, s>>>(pr);
  FLCE_TRY(launched(FLCE_KERNEL_BWD_PREP, s));
  if (grad_hidden) {  // the rows of tiles left out
    bwd_zero_rows_kernel<<<(unsigned)n_real, 256, 0, s>>>(tile_act, (int)T, (int)D,
                                                          (uint16_t *)grad_hidden);
    FLCE_TRY(launched(FLCE_KERNEL_BWD_ZERO_ROWS, s));
  }

  // Row block rb takes tiles [rb * TR, rb * TR + TR) of the list: tiles without gradient
  // are left out and the rest packed into the leading row blocks (with every tile
  // listed, the blocks are the tiles as laid out).
  const int64_t TR = p.R / kTile;
  for (int64_t rb = 0; rb < p.n_rb; ++rb) {
    const int64_t rb0 = rb * p.R;
    const int64_t rcount = std::min<int64_t>(p.R, T - rb0);
    if (rcount <= 0) break;
    RowMap map{};
    map.list = act_list;
    map.count = n_act;
    map.n_real = (int)n_real;
    map.tile0 = (int)(rb * TR);
    map.tiles_rb = (int)TR;
    if (grad_weight) FLCE_TRY(launch_ht(hidden, ht, D, p.R, rb0, rcount, s, map, T));
    for (int64_t vc = 0; vc < p.n_vc; ++vc) {
      const int64_t vc0 = vc * p.Vc;
      const int64_t vcount = std::min<int64_t>(p.Vc, V - vc0);
      if (vcount <= 0) break;

      BwdGradParams g{};
      g.hidden = (const uint16_t *)hidden;
      g.weight = (const uint16_t *)weight;
      g.labels = labels;
      g.c = cbuf;
      g.lse2 = l2buf;
      g.ignore_index = ignore_index;
      g.T = (int)T;
      g.D = (int)D;
      g.V = (int)V;
      g.vc0 = (int)vc0;
      g.n_vt = (int)cdiv(vcount, kTile);
      g.tiles_n = (int)cdiv(rcount, kTile);
      g.map = map;
      g.xf = xf;
      g.G = G;
      g.Gp = (int)p.Vc;
      // At most one workgroup per CU, each walking n_vt / vsplits vocabulary tiles, for
      // the n tiles the block turns out to hold (at most tiles_n): the grid covers the
      // largest n * vsplits(n), and the kernel's workgroups past its own count exit.
      int64_t grid = 0;
      for (int64_t n = 1; n <= g.tiles_n; ++n)
        grid = std::max(grid, n * std::min<int64_t>(g.n_vt, std::max<int64_t>(1, kCUs / n)));
      if (cap)
        bwd_grad_kernel<true><<<(unsigned)grid, kThreads, 0, s>>>(g);
      else
        bwd_grad_kernel<false><<<(unsigned)grid, kThreads, 0, s>>>(g);
      FLCE_TRY(launched(FLCE_KERNEL_BWD_GRAD, s));

      FLCE_TRY(launch_dh_dw(G, (int)p.Vc, p.Vc, false, weight, ht, D, V, p.R, rcount, vc0, vcount,
                            p.dh_splits, grad_hidden ? dhacc : nullptr, grad_weight, vc > 0,
                            accumulate_grad_weight || rb > 0, map, s));
    }
    if (grad_hidden)
      FLCE_TRY(launch_dh_out(dhacc, grad_hidden, D, p.R, p.dh_splits, rb0, rcount, s, map, T));
  }
  return FLCE_OK;
}

int64_t flce_chunk_rows_for(int64_t context_length, int64_t multiplier) {
  if (context_length < 1) return 0;
  if (multiplier <= 0) multiplier = std::max<int64_t>(4, context_length / 4096);
  return cdiv(context_length, multiplier);
}

flce_status flce_tune(int64_t batch, int64_t context_length, int64_t D, int64_t V,
                      size_t budget_bytes, int64_t *mini_batches, int64_t *chunk_rows,
                      size_t *bytes_needed) {
  g_last_error[0] = 0;
  if (!mini_batches || !chunk_rows) return fail(FLCE_ERR_ARG, "output pointer is NULL");
  if (batch < 1 || context_length < 1)
    return fail(FLCE_ERR_SHAPE, "batch = %lld and context_length = %lld must be >= 1",
                (long long)batch, (long long)context_length);
  if (batch > kMaxTV / context_length)
    return fail(FLCE_ERR_SHAPE, "batch * context_length is too large");
  const int64_t k0 = std::max<int64_t>(4, context_length / 4096);
  // each distinct group size ceil(batch / m) once, smallest m first
  for (int64_t m = 1; m <= batch;) {
    const int64_t g = cdiv(batch, m);
    const int64_t Tmb = g * context_length;
    // chunk_rows = ceil(context / k) takes each value once: walk the distinct ones
    for (int64_t k = std::min(k0, context_length); k <= context_length;) {
      const int64_t cr = cdiv(context_length, k);
      Plan p;
      FLCE_TRY(make_plan(Tmb, D, V, cr, p));
      const size_t need = p.total + (size_t)Tmb * (size_t)D * 4 + (size_t)Tmb * 16;
      if (need <= budget_bytes) {
        *mini_batches = m;
        *chunk_rows = cr;
        if (bytes_needed) *bytes_needed = need;
        return FLCE_OK;
      }
      if (cr == 1) break;
      k = cdiv(context_length, cr - 1);  // smallest multiplier giving fewer rows per chunk
    }
    if (g == 1) break;
    m = cdiv(batch, g - 1);  // smallest m giving smaller groups
  }
  return fail(FLCE_ERR_WORKSPACE, "no mini-batching and chunk size fit in %zu bytes",
              budget_bytes);
}

size_t flce_distill_workspace_bytes(int64_t T, int64_t Ds, int64_t Dt, int64_t V,
                                    int64_t chunk_rows) {
  DistillPlan p;
  if (make_distill_plan(T, Ds, Dt, V, chunk_rows, p) != FLCE_OK) return 0;
  return p.total;
}

flce_status flce_distill(const void *student_hidden, const void *student_weight, int64_t Ds,
                         const void *teacher_hidden, const void *teacher_weight, int64_t Dt,
                         const int64_t *labels, int64_t ignore_index, int64_t T, int64_t V,
                         int64_t chunk_rows, const flce_logit_transform *transform,
                         float *kl_out, float *mean_out, const float *grad_out,
                         const float *grad_mean, void *grad_student_hidden,
                         float *grad_student_weight, int accumulate_grad_weight,
                         void *workspace, size_t workspace_bytes, void *stream) {
  return distill_run(false, 0.f, student_hidden, student_weight, Ds, teacher_hidden,
                     teacher_weight, Dt, labels, ignore_index, T, V, chunk_rows, transform,
                     kl_out, mean_out, grad_out, grad_mean, grad_student_hidden,
                     grad_student_weight, accumulate_grad_weight, workspace, workspace_bytes,
                     stream);
}

flce_status flce_distill_jsd(const void *student_hidden, const void *student_weight, int64_t Ds,
                             const void *teacher_hidden, const void *teacher_weight, int64_t Dt,
                             const int64_t *labels, int64_t ignore_index, int64_t T, int64_t V,
                             int64_t chunk_rows, const flce_logit_transform *transform,
                             float beta, float *jsd_out, float *mean_out, const float *grad_out,
                             const float *grad_mean, void *grad_student_hidden,
                             float *grad_student_weight, int accumulate_grad_weight,
                             void *workspace, size_t workspace_bytes, void *stream) {
  return distill_run(true, beta, student_hidden, student_weight, Ds, teacher_hidden,
                     teacher_weight, Dt, labels, ignore_index, T, V, chunk_rows, transform,
                     jsd_out, mean_out, grad_out, grad_mean, grad_student_hidden,
                     grad_student_weight, accumulate_grad_weight, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"


namespace {

// Workspace of a policy-loss call: the cross-entropy workspace (the log-prob
// forward and backward run in it), then per-token log-probs (when the caller
// keeps none), lse and upstream gradients, and per-sequence values.
struct PolicyLayout {
  size_t flce, off_logp, off_lse, off_c, off_val, off_n, off_g, total;
};

flce_status policy_layout(int64_t T, int64_t D, int64_t V, int64_t chunk_rows, int64_t n_seq,
                          PolicyLayout &l) {
  Plan p;
  FLCE_TRY(make_plan(T, D, V, chunk_rows, p));
  if (n_seq < 1 || n_seq > std::max<int64_t>(T, 1) || T % n_seq)
    return fail(FLCE_ERR_SHAPE, "n_seq = %lld must be >= 1 and divide T = %lld",
                (long long)n_seq, (long long)T);
  size_t off = align256(p.total);
  l.flce = p.total;
  l.off_logp = off; off = align256(off + (size_t)T * 4);
  l.off_lse = off;  off = align256(off + (size_t)T * 4);
  l.off_c = off;    off = align256(off + (size_t)T * 4);
  l.off_val = off;  off = align256(off + (size_t)n_seq * 8);
  l.off_n = off;    off = align256(off + (size_t)n_seq * 4);
  l.off_g = off;    off = align256(off + (size_t)n_seq * 4);
  l.total = off;
  return FLCE_OK;
}

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

struct PolicyInputs {
  const float *advantages, *old_logp, *ref_logp, *ref_seq, *kl_ref;
  const uint8_t *desirable;
};

template <int kKind>
void launch_policy_kernels(const PolicyParams &pp, bool grads, hipStream_t s) {
  pol_seq_kernel<kKind><<<(unsigned)pp.n_seq, 256, 0, s>>>(pp);
  pol_loss_kernel<kKind><<<1, 1024, 0, s>>>(pp);
  if (grads) pol_grad_kernel<kKind><<<(unsigned)cdiv(pp.T, 256), 256, 0, s>>>(pp);
}

flce_status policy_loss(int kind, const PolicyInputs &in, const flce_policy_params *params,
                        const void *hidden, const void *weight, const int64_t *labels,
                        int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                        int64_t chunk_rows, const flce_logit_transform *transform,
                        int64_t n_seq, float *loss_out, float *logp_out,
                        const float *grad_loss, void *grad_hidden, float *grad_weight,
                        int accumulate_grad_weight, void *workspace, size_t workspace_bytes,
                        void *stream) {
  g_last_error[0] = 0;
  PolicyLayout l;
  FLCE_TRY(policy_layout(T, D, V, chunk_rows, n_seq, l));
  Xform xf;
  bool cap;
  FLCE_TRY(make_xform(transform, xf, cap));
  if (!params) return fail(FLCE_ERR_ARG, "params is NULL");
  const flce_policy_params &pr = *params;
  if (kind == kPolicyGrpo) {
    if (!finite_nonneg(pr.beta) || !finite_nonneg(pr.eps_low) || pr.eps_low >= 1.f ||
        !finite_nonneg(pr.eps_high))
      return fail(FLCE_ERR_ARG, "GRPO needs beta >= 0, 0 <= eps_low < 1, eps_high >= 0");
  } else {
    if (!std::isfinite(pr.beta) || pr.beta <= 0.f)
      return fail(FLCE_ERR_ARG, "beta = %g must be positive", (double)pr.beta);
    if (kind == kPolicyDpo && n_seq % 2)
      return fail(FLCE_ERR_SHAPE, "DPO needs an even n_seq (chosen, then rejected); got %lld",
                  (long long)n_seq);
    if (kind == kPolicyKto &&
        (!finite_nonneg(pr.desirable_weight) || !finite_nonneg(pr.undesirable_weight)))
      return fail(FLCE_ERR_ARG, "KTO weights must be finite and >= 0");
  }
  const bool grads = grad_loss != nullptr;
  if (!loss_out) return fail(FLCE_ERR_ARG, "loss_out is NULL");
  if (grads && !grad_weight && !grad_hidden)
    return fail(FLCE_ERR_ARG,
                "a gradient was requested but grad_hidden and grad_weight are both NULL");
  if (grad_weight && !aligned(grad_weight, 16))
    return fail(FLCE_ERR_ARG, "grad_weight not 16-byte aligned");
  if (!aligned(loss_out, 4) || (grad_loss && !aligned(grad_loss, 4)))
    return fail(FLCE_ERR_ARG, "misaligned pointer");
  if (T > 0) {
    const bool need_seq = kind != kPolicyGrpo;
    if (!hidden || !weight || !labels || !workspace ||
        (kind == kPolicyGrpo && !in.advantages) || (need_seq && !in.ref_seq) ||
        (kind == kPolicyKto && !in.desirable))
      return fail(FLCE_ERR_ARG, "a required pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(labels, 8) ||
        !aligned(workspace, 16) || (grad_hidden && !aligned(grad_hidden, 16)) ||
        (logp_out && !aligned(logp_out, 4)) || (in.advantages && !aligned(in.advantages, 4)) ||
        (in.old_logp && !aligned(in.old_logp, 4)) || (in.ref_logp && !aligned(in.ref_logp, 4)) ||
        (in.ref_seq && !aligned(in.ref_seq, 4)) || (in.kl_ref && !aligned(in.kl_ref, 4)))
      return fail(FLCE_ERR_ARG, "misaligned pointer");
    if (workspace_bytes < l.total)
      return fail(FLCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                  l.total);
  }
  FLCE_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  timing_start(s);
  if (T == 0) {
    FLCE_TRY(fill(loss_out, 1, 0.f, s));
    if (grads && grad_weight && !accumulate_grad_weight) FLCE_TRY(fill(grad_weight, V * D, 0.f, s));
    return FLCE_OK;
  }

  char *ws = (char *)workspace;
  float *logp = logp_out ? logp_out : (float *)(ws + l.off_logp);
  float *lse = (float *)(ws + l.off_lse);
  // Non-completion tokens need neither a log-prob nor an lse: tiles holding only those
  // are left out here as in the backward.  Their list borrows the per-token gradient
  // buffer (align256(4 T) >= 8 + 5 ceil(T / 256) bytes), which the loss kernels write
  // only after the forward has read the list.
  FLCE_TRY(forward_entry(hidden, weight, labels, T, D, V, ignore_index, chunk_rows,
                         FLCE_MODE_LOGPROB, transform, logp, lse, nullptr, workspace, l.flce,
                         stream, ws + l.off_c));
  PolicyParams pp{};
  pp.labels = labels;
  pp.ignore_index = ignore_index;
  pp.T = (int)T;
  pp.n_seq = (int)n_seq;
  pp.S = (int)(T / n_seq);
  pp.logp = logp;
  pp.advantages = in.advantages;
  pp.old_logp = in.old_logp;
  pp.ref_logp = in.ref_logp;
  pp.ref_seq = in.ref_seq;
  pp.desirable = in.desirable;
  pp.kl_ref = in.kl_ref;
  pp.grad_loss = grad_loss;
  pp.beta = pr.beta;
  pp.eps_low = pr.eps_low;
  pp.eps_high = pr.eps_high;
  pp.w_des = pr.desirable_weight;
  pp.w_und = pr.undesirable_weight;
  pp.seq_val = (double *)(ws + l.off_val);
  pp.seq_n = (int *)(ws + l.off_n);
  pp.seq_g = (float *)(ws + l.off_g);
  pp.loss = loss_out;
  pp.c = (float *)(ws + l.off_c);
  if (kind == kPolicyGrpo)
    launch_policy_kernels<kPolicyGrpo>(pp, grads, s);
  else if (kind == kPolicyDpo)
    launch_policy_kernels<kPolicyDpo>(pp, grads, s);
  else
    launch_policy_kernels<kPolicyKto>(pp, grads, s);
  FLCE_TRY(launched(FLCE_KERNEL_POLICY, s));
  if (!grads) return FLCE_OK;
  return flce_backward(hidden, weight, labels, lse, T, D, V, ignore_index, chunk_rows,
                       FLCE_MODE_LOGPROB, transform, pp.c, nullptr, grad_hidden, grad_weight,
                       accumulate_grad_weight, workspace, l.flce, stream);
}

}  // namespace

extern "C" {

size_t flce_policy_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk_rows,
                                   int64_t n_seq) {
  PolicyLayout l;
  if (policy_layout(T, D, V, chunk_rows, n_seq, l) != FLCE_OK) return 0;
  return l.total;
}

flce_status flce_grpo_loss(const void *hidden, const void *weight, const int64_t *labels,
                           int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                           int64_t chunk_rows, const flce_logit_transform *transform,
                           int64_t n_seq, const float *advantages, const float *old_logp,
                           const float *ref_logp, const flce_policy_params *params,
                           float *loss_out, float *logp_out, const float *grad_loss,
                           void *grad_hidden, float *grad_weight, int accumulate_grad_weight,
                           void *workspace, size_t workspace_bytes, void *stream) {
  PolicyInputs in = {advantages, old_logp, ref_logp, nullptr, nullptr, nullptr};
  return policy_loss(kPolicyGrpo, in, params, hidden, weight, labels, ignore_index, T, D, V,
                     chunk_rows, transform, n_seq, loss_out, logp_out, grad_loss, grad_hidden,
                     grad_weight, accumulate_grad_weight, workspace, workspace_bytes, stream);
}

flce_status flce_dpo_loss(const void *hidden, const void *weight, const int64_t *labels,
                          int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                          int64_t chunk_rows, const flce_logit_transform *transform,
                          int64_t n_seq, const float *ref_seq_logp,
                          const flce_policy_params *params, float *loss_out, float *logp_out,
                          const float *grad_loss, void *grad_hidden, float *grad_weight,
                          int accumulate_grad_weight, void *workspace, size_t workspace_bytes,
                          void *stream) {
  PolicyInputs in = {nullptr, nullptr, nullptr, ref_seq_logp, nullptr, nullptr};
  return policy_loss(kPolicyDpo, in, params, hidden, weight, labels, ignore_index, T, D, V,
                     chunk_rows, transform, n_seq, loss_out, logp_out, grad_loss, grad_hidden,
                     grad_weight, accumulate_grad_weight, workspace, workspace_bytes, stream);
}

flce_status flce_kto_loss(const void *hidden, const void *weight, const int64_t *labels,
                          int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                          int64_t chunk_rows, const flce_logit_transform *transform,
                          int64_t n_seq, const float *ref_seq_logp, const uint8_t *desirable,
                          const float *kl_ref, const flce_policy_params *params,
                          float *loss_out, float *logp_out, const float *grad_loss,
                          void *grad_hidden, float *grad_weight, int accumulate_grad_weight,
                          void *workspace, size_t workspace_bytes, void *stream) {
  PolicyInputs in = {nullptr, nullptr, nullptr, ref_seq_logp, kl_ref, desirable};
  return policy_loss(kPolicyKto, in, params, hidden, weight, labels, ignore_index, T, D, V,
                     chunk_rows, transform, n_seq, loss_out, logp_out, grad_loss, grad_hidden,
                     grad_weight, accumulate_grad_weight, workspace, workspace_bytes, stream);
}

}  // extern "C"
