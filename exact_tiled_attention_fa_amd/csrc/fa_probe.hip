// Matrix-core ceiling on given operand data (a measurement helper, not part of
// attention).
//
// The MI355X's MFMA throughput depends on the values it multiplies: operands
// whose mantissas toggle draw more power and the clock drops, so the rate on
// random bf16 data sits well below the rate on constant data.  This kernel
// runs only v_mfma_f32_32x32x16_bf16, in the pattern of the forward step (one
// 8-deep chain like S = Q K^T over D = 128 and four 2-deep chains like P V),
// with its operands taken once from the caller's buffer, so that timing it on
// the benchmark's own Q gives the matrix-core ceiling for that data.
//
// Launch: two 256-thread workgroups per compute unit (two waves per SIMD),
// thread t reads 16-byte operands t*18 .. t*18+17 (modulo the buffer) and
// writes one float: the sum of its accumulators.  With every operand equal to
// bf16 1.0 that sum is exactly 4096 * iters (each MFMA adds 16 to each of its
// outputs; the chain takes 8 per iteration, each of the four 2-deep chains 2).

#include <hip/hip_runtime.h>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeOperands = 18;  // 16-byte operands per thread

__global__ __launch_bounds__(kProbeThreads, 2) void mfma_probe_kernel(const u32x4* __restrict__ ops,
                                                                       long n16, float* __restrict__ out,
                                                                       int iters) {
  const long t = (long)blockIdx.x * kProbeThreads + threadIdx.x;
  const long base = t * kProbeOperands;
  u32x4 a[8], b[8], p[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ops[(base + i) % n16];
    b[i] = ops[(base + 8 + i) % n16];
  }
  p[0] = ops[(base + 16) % n16];
  p[1] = ops[(base + 17) % n16];

  f32x16 s = {}, acc[4] = {};
  for (int it = 0; it < iters; ++it) {
    f32x16 c = s;  // loop-carried: the chain is redone every iteration
#pragma unroll
    for (int k = 0; k < 8; ++k) c = Ops<bf16_t>::mfma32(a[k], b[k], c);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = Ops<bf16_t>::mfma32(a[2 * j + h], p[h], acc[j]);
    s = c;
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += s[i] + acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
  out[t] = r;
}

}  // namespace

double mfma_probe_flops(int nblocks, int iters) {
  // waves x iterations x 16 MFMAs x (2 * 32 * 32 * 16) flops
  return (double)nblocks * (kProbeThreads / 64) * iters * 16 * 32768.0;
}

int mfma_probe_threads(int nblocks) { return nblocks * kProbeThreads; }

hipError_t launch_mfma_probe(const void* ops, long n16, float* out, int nblocks, int iters,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)nblocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(ops), n16, out, iters);
  return hipGetLastError();
}

}  // namespace fa
