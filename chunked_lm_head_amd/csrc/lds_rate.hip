// lds_rate.hip - LDS read rate of an MI355X CU as a function of the waves
// reading: each wave issues back-to-back ds_read_b128 (8 in flight, then a
// dependent use) over a bank-conflict-free, in-bounds pattern of a 64 KiB LDS
// array.  One workgroup per CU; prints one JSON line with bytes per ns per CU
// (best of 2 launches) for 4, 8 and 16 waves per CU.  The GEMM engine of this
// library runs one wave per SIMD (4 per CU), so its fragment reads are bounded
// by the first figure, not by the LDS's peak.
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

namespace {

constexpr int kIters = 20000;

template <int kWaves>
__global__ void __launch_bounds__(kWaves * 64) reader(unsigned *out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned lds[16384];  // 64 KiB
  for (int i = threadIdx.x; i < 16384; i += kWaves * 64) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // 16-byte aligned offsets below 65536: always inside the array
      const unsigned off = ((unsigned)((it * 8 + u + w * 3) * 64 + lane) * 16u) & 65535u;
      acc ^= *(const lds_u32x4 *)((const lds_char *)lds + off);
    }
  }
  out[blockIdx.x * kWaves * 64 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

int check(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

template <int kWaves>
int run(int cus, unsigned *d, hipEvent_t e0, hipEvent_t e1, double &best) {
  best = 0;
  for (int rep = 0; rep < 2; ++rep) {
    if (check(hipEventRecord(e0), "record")) return 1;
    reader<kWaves><<<cus, kWaves * 64>>>(d, kIters);
    if (check(hipGetLastError(), "launch") || check(hipEventRecord(e1), "record") ||
        check(hipEventSynchronize(e1), "sync"))
      return 1;
    float ms = 0.f;
    if (check(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
    const double bytes = (double)kWaves * 64 * 16 * 8 * kIters;  // per CU
    const double rate = bytes / (ms * 1e6);
    if (rate > best) best = rate;
  }
  return 0;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  if (check(hipGetDevice(&dev), "hipGetDevice") ||
      check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "attr"))
    return 1;
  unsigned *d = nullptr;
  if (check(hipMalloc(&d, (size_t)cus * 1024 * sizeof(unsigned)), "hipMalloc")) return 1;
  hipEvent_t e0, e1;
  if (check(hipEventCreate(&e0), "event") || check(hipEventCreate(&e1), "event")) return 1;
  double r4, r8, r16;
  if (run<4>(cus, d, e0, e1, r4) || run<8>(cus, d, e0, e1, r8) || run<16>(cus, d, e0, e1, r16))
    return 1;
  printf("{\"lds_read_rate\": {\"waves_4\": %.1f, \"waves_8\": %.1f, \"waves_16\": %.1f, "
         "\"unit\": \"bytes/ns per CU\", \"cus\": %d}}\n",
         r4, r8, r16, cus);
  return check(hipFree(d), "hipFree");
}
