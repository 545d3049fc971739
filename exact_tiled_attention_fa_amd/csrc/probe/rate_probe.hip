// Issue-rate probes of the instruction mixes the forward kernel's step is
// made of (a measurement helper of the benchmark, in libfa_probe.so): how
// many cycles a 32x32x16 bf16 MFMA, an fp32 FMA and a v_exp_f32 take per
// wave, and how far MFMA and VALU work overlap -- inside one wave when the
// two are interleaved, and across two waves on one SIMD when one wave issues
// only MFMAs and the other only VALU work.
//
// Launch: one workgroup of 256 * n threads per compute unit (each reserves
// 96 KiB of LDS, so no second one fits): its 4n waves sit n to a SIMD (wave w
// on SIMD w % 4, which each wave reads back from its hardware id).  Every
// wave runs `iters` iterations of one mix and records its loop's s_memtime
// start and end (s_memtime, the shader clock; s_memrealtime, a constant
// 100 MHz clock, to convert) and its hardware id.  What a SIMD sustains is
// its span, from the first of its waves' starts to the last end: a wave's own
// loop time says little when the SIMD serves its waves one after another.  In the split mixes waves 0..3 run the MFMA half and
// waves 4..7 the VALU half, so each SIMD holds one of each.  The instruction
// order inside an iteration is pinned with scheduling barriers, so the
// measured mix is the one named.
//
// The compiler keeps the MFMA accumulators of these loops in AccVGPRs; the
// build also compiles this file a second time with MFMA operands and results
// forced into ArchVGPRs (as the attention kernels hold them), under the entry
// name fa_probe_rates_vgpr.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.hpp"

namespace {

using fa::f32x16;
using fa::u32x4;

enum Mix : int {
  kMfma = 0,        // 8 MFMAs: one dependent chain of 8 (the S = K Q^T step)
  kMfma4 = 1,       // 8 MFMAs: four independent chains of 2 (the P V step)
  kFma = 2,         // 32 independent v_fma_f32
  kExp = 3,         // 32 independent v_exp_f32
  kMfmaFma = 4,     // 8 MFMAs (four chains), 4 FMAs after each MFMA, one wave
  kMfmaExp = 5,     // 8 MFMAs (four chains), 2 exps after each MFMA, one wave
  kSplit = 6,       // waves 0..3: kMfma4; waves 4..7: kFma (two waves per SIMD)
  kSplitExp = 7,    // waves 0..3: kMfma4; waves 4..7: kExp
  kMfmaSoftmax = 8,  // 8 MFMAs (four chains) with the softmax of 16 scores per
                     // lane interleaved: per MFMA 2 FMA, 2 exp, 2 add, 1 cvt (+1 xor
                     // that keeps the packed value live)
  kStep = 9          // a forward step's register work: 8 dependent MFMAs (S) and
                     // 8 in four chains (P V), the softmax of 16 scores per lane
                     // (16 FMA, 16 exp, 16 add, 8 cvt, 8 xor) interleaved, 4 VALU
                     // instructions after each MFMA
};

// Scheduling groups (their order is kept): n MFMAs, then n other VALU instructions.
#define PIN_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, n, 0)
#define PIN_VALU(n) __builtin_amdgcn_sched_group_barrier(0x002, n, 0)

// Every VALU result feeds the same slot in the next iteration, so nothing is
// loop-invariant; exp2(-x) and exp2(y x + z) with y = 0.5 stay finite.
template <int MIX>
__device__ __forceinline__ void run_mix(const u32x4 (&a)[8], const u32x4& b, f32x16 (&acc)[4],
                                        float (&x)[32], float y, float z, int iters) {
  float sum = 0.f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MIX == kMfma) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[0] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[0]);
    } else if constexpr (MIX == kMfma4) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k & 3] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[k & 3]);
    } else if constexpr (MIX == kFma) {
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = __builtin_fmaf(x[j], y, z);
    } else if constexpr (MIX == kExp) {
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    } else if constexpr (MIX == kMfmaFma) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k & 3] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[k & 3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[4 * k + j] = __builtin_fmaf(x[4 * k + j], y, z);
        PIN_MFMA(1);
        PIN_VALU(4);
      }
    } else if constexpr (MIX == kMfmaExp) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k & 3] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[k & 3]);
#pragma unroll
        for (int j = 0; j < 2; ++j) x[2 * k + j] = __builtin_amdgcn_exp2f(-x[2 * k + j]);
        PIN_MFMA(1);
        PIN_VALU(2);
      }
    } else if constexpr (MIX == kMfmaSoftmax) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k & 3] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[k & 3]);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * k], y, z));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * k + 1], y, z));
        sum += p0;
        sum += p1;
        x[16 + k] = __uint_as_float(fa::Ops<fa::bf16_t>::pack2(p0, p1) ^ __float_as_uint(x[16 + k]));
        x[2 * k] = p0;
        x[2 * k + 1] = p1;
        PIN_MFMA(1);
        PIN_VALU(8);
      }
    } else if constexpr (MIX == kStep) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        // MFMAs 0..7: one dependent chain; 8..15: two more chains of four
        if (k < 8)
          acc[0] = fa::Ops<fa::bf16_t>::mfma32(a[k], b, acc[0]);
        else
          acc[1 + (k & 1)] = fa::Ops<fa::bf16_t>::mfma32(a[k & 7], b, acc[1 + (k & 1)]);
        const int j = k >> 1;
        if ((k & 1) == 0) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j], y, z));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j + 1], y, z));
          x[2 * j] = p0;
          x[2 * j + 1] = p1;
        } else {
          sum += x[2 * j];
          sum += x[2 * j + 1];
          x[16 + j] = __uint_as_float(fa::Ops<fa::bf16_t>::pack2(x[2 * j], x[2 * j + 1]) ^
                                      __float_as_uint(x[16 + j]));
        }
        PIN_MFMA(1);
        PIN_VALU(4);
      }
    }
  }
  x[31] += sum;
}

template <int MIX>
__global__ __launch_bounds__(512) void rate_kernel(const u32x4* __restrict__ ops, long n16,
                                                   float* __restrict__ out,
                                                   long long* __restrict__ rec, int iters) {
  extern __shared__ unsigned char lds_reserve[];  // only caps workgroups per CU
  const int w = threadIdx.x >> 6;
  const long wave = (long)blockIdx.x * (blockDim.x >> 6) + w;
  const long base = (wave * 64 + (threadIdx.x & 63)) * 9;
  u32x4 a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = ops[(base + k) % n16];
  const u32x4 b = ops[(base + 8) % n16];
  f32x16 acc[4] = {};
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = 0.001f * (j + (threadIdx.x & 63));
  const float y = 0.5f, z = 1e-3f;
  __syncthreads();  // start together
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const long long t0 = __builtin_amdgcn_s_memtime();
  if constexpr (MIX == kSplit || MIX == kSplitExp) {
    if (w < 4)
      run_mix<kMfma4>(a, b, acc, x, y, z, iters);
    else if constexpr (MIX == kSplit)
      run_mix<kFma>(a, b, acc, x, y, z, iters);
    else
      run_mix<kExp>(a, b, acc, x, y, z, iters);
  } else {
    run_mix<MIX>(a, b, acc, x, y, z, iters);
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
#pragma unroll
  for (int j = 0; j < 32; ++j) r += x[j];
  out[wave * 64 + (threadIdx.x & 63)] = r;
  if ((threadIdx.x & 63) == 0) {
    rec[5 * wave] = t0;
    rec[5 * wave + 1] = t1;
    rec[5 * wave + 2] = r0;
    rec[5 * wave + 3] = r1;
    rec[5 * wave + 4] = (long long)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));
  }
  (void)lds_reserve;
}

template <int MIX>
hipError_t launch(const void* ops, long n16, float* out, long long* rec, int nblocks,
                  int waves_per_simd, int iters, hipStream_t s) {
  hipLaunchKernelGGL(rate_kernel<MIX>, dim3((unsigned)nblocks), dim3(256 * waves_per_simd),
                     (size_t)(96 * 1024), s, static_cast<const u32x4*>(ops), n16, out, rec, iters);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// One launch of mix `mix` (0..9, see the enum above): nblocks workgroups
// (one per compute unit) of 256 * waves_per_simd threads (waves_per_simd 1
// or 2), each wave running `iters` iterations.  ops: device buffer of
// operand_bytes (positive multiple of 16, 16-byte aligned) read as bf16
// operands, modulo its length.  out: device, >= 256 * waves_per_simd *
// nblocks floats (a checksum per thread).  rec: device, 5 int64 per wave
// (s_memtime at its loop's start and end, s_memrealtime at both, the HW_ID
// register).
// Returns 0, 1 for an invalid argument (before any device call), 3 if the
// launch fails.
#ifndef FA_PROBE_RATES_NAME
#define FA_PROBE_RATES_NAME fa_probe_rates
#endif
int FA_PROBE_RATES_NAME(int mix, const void* ops, size_t operand_bytes, float* out,
                        long long* rec, int nblocks, int waves_per_simd, int iters,
                        hipStream_t stream) {
  if (!ops || !out || !rec || ((uintptr_t)ops & 15u)) return 1;
  if (operand_bytes < 16 || operand_bytes % 16) return 1;
  if (nblocks < 1 || nblocks > 4096 || iters < 1 || iters > (1 << 24)) return 1;
  if (waves_per_simd != 1 && waves_per_simd != 2) return 1;
  const long n16 = (long)(operand_bytes / 16);
  const int n = waves_per_simd;
  hipError_t e;
  switch (mix) {
    case kMfma: e = launch<kMfma>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kMfma4: e = launch<kMfma4>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kFma: e = launch<kFma>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kExp: e = launch<kExp>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kMfmaFma: e = launch<kMfmaFma>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kMfmaExp: e = launch<kMfmaExp>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kSplit:
      if (n != 2) return 1;
      e = launch<kSplit>(ops, n16, out, rec, nblocks, n, iters, stream);
      break;
    case kSplitExp:
      if (n != 2) return 1;
      e = launch<kSplitExp>(ops, n16, out, rec, nblocks, n, iters, stream);
      break;
    case kMfmaSoftmax: e = launch<kMfmaSoftmax>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    case kStep: e = launch<kStep>(ops, n16, out, rec, nblocks, n, iters, stream); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 3;
}

}  // extern "C"
