// mfma_ceiling.hip - sustained bf16 MFMA rate of an MI355X with no memory
// traffic: the practical ceiling the GEMM kernels of this library are held
// to, beside the 2.5 PFLOP/s dense bf16 figure of the data sheet.
//
// Each wave keeps 8 A and 8 B fragments of pseudo-random bf16 in registers
// and accumulates into 256 fp32 AGPRs, with every MFMA taking a different
// (A, B) pair, so that the multipliers toggle as they do on real data (on
// constant operands the chip holds a higher clock).  One workgroup of 4 waves
// per CU, 8 rounds of workgroups, about 25 ms per launch so that the clock
// settles where power management holds it.  Both instruction shapes used in
// this library's history are timed:
//   v_mfma_f32_32x32x16_bf16 (32 cycles, 16 accumulators per lane per block)
//   v_mfma_f32_16x16x32_bf16 (16 cycles,  4 accumulators per lane per block)
// Prints one JSON line: best of 4 launches per shape, in FLOP/s.  An optional
// argument sets the launches per shape (for example 200, about 5 s per shape,
// long enough to sample board power meanwhile).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

__device__ inline unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ inline bf16x8 random_frag(unsigned seed) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned h = mix(seed * 8 + i);
    v[i] = (__bf16)(((float)(h & 0xffff) / 65536.f - 0.5f) * 0.1f);
  }
  return v;
}

constexpr int kIters = 6000;  // per wave: 6000 x 32 MFMA-slots of 32x32x16 work

// The iteration count is a kernel argument and the loop is kept rolled: an
// unrolled body needs more registers than a wave has and spills accumulators.
__global__ void __launch_bounds__(256) shape32(float *out, int iters) {
  const unsigned t = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = random_frag(t * 16 + i);
    b[i] = random_frag(t * 16 + 8 + i);
  }
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x16{};
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h * 4 + (j >> 2)], b[h * 4 + (j & 3)],
                                                         acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[t] = s;
}

__global__ void __launch_bounds__(256) shape16(float *out, int iters) {
  const unsigned t = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = random_frag(t * 16 + i);
    b[i] = random_frag(t * 16 + 8 + i);
  }
  f32x4 acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = f32x4{};
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 64; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j >> 3], b[j & 7], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[j][r];
  out[t] = s;
}

int check(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  int reps = argc > 1 ? atoi(argv[1]) : 4;
  if (reps < 1 || reps > 100000) reps = 4;
  int dev = 0, cus = 0;
  if (check(hipGetDevice(&dev), "hipGetDevice") ||
      check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "attr"))
    return 1;
  const int blocks = cus * 8;
  float *d = nullptr;
  if (check(hipMalloc(&d, (size_t)blocks * 256 * sizeof(float)), "hipMalloc")) return 1;
  hipEvent_t e0, e1;
  if (check(hipEventCreate(&e0), "event") || check(hipEventCreate(&e1), "event")) return 1;
  // both kernels do 32 x 32768 FLOP per wave and iteration
  const double flops = (double)blocks * 4 * kIters * 32 * 32768.0;
  double best[2] = {0, 0};
  for (int shape = 0; shape < 2; ++shape) {
    for (int rep = 0; rep < reps; ++rep) {
      if (check(hipEventRecord(e0), "record")) return 1;
      if (shape == 0)
        shape32<<<blocks, 256>>>(d, kIters);
      else
        shape16<<<blocks, 256>>>(d, kIters);
      if (check(hipGetLastError(), "launch") || check(hipEventRecord(e1), "record") ||
          check(hipEventSynchronize(e1), "sync"))
        return 1;
      float ms = 0.f;
      if (check(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
      const double rate = flops / (ms * 1e-3);
      if (rate > best[shape]) best[shape] = rate;
    }
  }
  printf("{\"mfma_ceiling\": {\"v_mfma_f32_32x32x16_bf16\": %.4e, \"v_mfma_f32_16x16x32_bf16\": %.4e, "
         "\"unit\": \"FLOP/s\", \"cus\": %d}}\n",
         best[0], best[1], cus);
  return check(hipFree(d), "hipFree");
}
