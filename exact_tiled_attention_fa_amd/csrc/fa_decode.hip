// Split-KV decode: one query token per sequence against its KV cache.
//
// The decode step is the per-token inference case of "FlashAttention in the
// CANN ops-transformer library" (ai6s.net), section 3, and the split-K
// decoding backend named by "5 years, 10K stars: xformers"
// (cloud.tencent.com).  The pages give no formulas for the split; the
// reading used here: sequence b's keys are cut into `num_splits` contiguous
// chunks of ceil(len_b / num_splits) keys; each chunk runs the same online
// softmax as the prefill kernel and leaves a normalised partial output and
// its logsumexp; a second kernel merges the chunks with weights
// exp(lse_chunk - lse_total) -- the online-softmax identity applied to chunk
// summaries, exact up to rounding.
//
// gfx950 mapping of the split kernel: one wave64 per (chunk, kv head, head
// group of <= 16 query heads, sequence).  32 keys per step:
//   * S^T = K q^T with v_mfma_f32_16x16x32: A = K rows loaded straight from
//     HBM into registers (16 keys x 32 dims per MFMA), B = q^T (the group's
//     query heads as 16 columns, zero-padded);
//   * O^T += V^T P^T with the same MFMA; V is transposed through a small LDS
//     tile with permuted key positions so each lane's eight keys are 16
//     contiguous bytes.
// Workspace: float32 partial outputs [B, Hq, S, D], then float32 partial
// logsumexps in base 2 [B, Hq, S].
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKS = kDecodeKeysPerStep;  // keys per step (two 16-key MFMA blocks)

template <typename T, int D>
__global__ __launch_bounds__(64)
void decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                         const uint16_t* __restrict__ Vc, const int* __restrict__ seqlens,
                         float* __restrict__ Opart, float* __restrict__ Lpart, int Hq, int Hkv,
                         int Lmax, int S, float scale2, float thr, uint32_t qxor) {
  constexpr int VP = kKS + 8;  // V^T tile row pitch (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];

  const int split = blockIdx.x;
  const int b = blockIdx.z;
  const int g = Hq / Hkv;
  const int nhg = (g + 15) / 16;
  const int kvh = blockIdx.y / nhg;
  const int hg = blockIdx.y - kvh * nhg;
  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int len = seqlens[b];
  len = len < 0 ? 0 : (len > Lmax ? Lmax : len);
  const int C = (len + S - 1) / S;
  const int k0 = split * C;
  const int k1 = min(len, k0 + C);

  const int hloc = hg * 16 + l16;
  const bool hvalid = hloc < g;
  const int hq = kvh * g + hloc;
  const long pidx = ((long)b * Hq + hq) * S + split;  // partial index when hvalid

  if (k1 <= k0) {  // empty chunk: weight 0 in the merge
    if (hvalid && q4 == 0) Lpart[pidx] = -INFINITY;
    return;
  }

  // q^T operand: lane holds head `hloc` (column l16), dims 32*ks + 8*q4 .. +8.
  u32x4 qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = hvalid ? (load16(Q + ((long)b * Hq + hq) * D + 32 * ks + 8 * q4) ^ qxor)
                    : (u32x4){0u, 0u, 0u, 0u};
  }

  const long kstride = (long)Hkv * D;
  const uint16_t* Kb = Kc + (long)b * Lmax * kstride + (long)kvh * D;
  const uint16_t* Vb = Vc + (long)b * Lmax * kstride + (long)kvh * D;

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = (f32x4){};
  float m_ref = -INFINITY;
  float l_part = 0.f;

  for (int j0 = k0; j0 < k1; j0 += kKS) {
    // Issue the V loads first (they go through LDS), then K.
    u32x4 vx[(kKS * D / 8) / 64];
#pragma unroll
    for (int i = 0; i < (kKS * D / 8) / 64; ++i) {
      const int p = lane + 64 * i;
      const int kk = p / (D / 8), c = p % (D / 8);
      vx[i] = (j0 + kk < k1) ? load16(Vb + (long)(j0 + kk) * kstride + 8 * c)
                             : (u32x4){0u, 0u, 0u, 0u};
    }
    u32x4 kx[2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = j0 + 16 * kb + l16;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kx[kb][ks] = (key < k1) ? load16(Kb + (long)key * kstride + 32 * ks + 8 * q4)
                                : (u32x4){0u, 0u, 0u, 0u};
    }

    // S^T: keys j0 + 16*kb + 4*q4 + r (rows) x heads (columns l16).
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x4){};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) s[kb] = Ops<T>::mfma16(kx[kb][ks], qf[ks], s[kb]);
    }

    __syncthreads();  // previous step's V^T reads are complete
#pragma unroll
    for (int i = 0; i < (kKS * D / 8) / 64; ++i) {
      const int p = lane + 64 * i;
      const int kk = p / (D / 8), c = p % (D / 8);
      // key kk = 16a + 4q + r  ->  position 8q + 4a + r
      const int pos = 8 * ((kk >> 2) & 3) + 4 * (kk >> 4) + (kk & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = vx[i][e >> 1];
        sV[(8 * c + e) * VP + pos] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    }
    __syncthreads();

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + 16 * kb + 4 * q4 + r;
        if (key >= k1) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));

    const bool upd = mx > m_ref + thr;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float m_new = upd ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast((m_ref - m_new) * scale2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
      m_ref = m_new;
    }
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * scale2;

    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = j >> 1, r = 2 * (j & 1);
      float p0 = exp2_fast(__builtin_fmaf(s[kb][r], scale2, -mb));
      float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], scale2, -mb));
      p0 = (s[kb][r] == -INFINITY) ? 0.f : p0;
      p1 = (s[kb][r + 1] == -INFINITY) ? 0.f : p1;
      pk[j] = Ops<T>::pack2(p0, p1);
      l_part += p0 + p1;  // unrounded: lse carries no 16-bit rounding
    }
    const u32x4 bop = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(sV + (16 * db + l16) * VP + 8 * q4);
      acc[db] = Ops<T>::mfma16(a, bop, acc[db]);
    }
  }

  float l = l_part + xor16(l_part);
  l = l + xor32(l);
  if (hvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = Opart + pidx * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      f32x4 val = acc[db] * inv;
      *reinterpret_cast<f32x4*>(op + 16 * db + 4 * q4) = val;
    }
    if (q4 == 0) Lpart[pidx] = l > 0.f ? m_ref * scale2 + __builtin_log2f(l) : -INFINITY;
  }
}

// Merge of the chunk summaries: one workgroup of D threads per (b, query head).
template <typename T, int D>
__global__ __launch_bounds__(D)
void decode_combine_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                           uint16_t* __restrict__ O, float* __restrict__ LSE, int S) {
  const long bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* lp = Lpart + bh * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
  float out = 0.f, tot = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = lp[s];
      if (ls == -INFINITY) continue;
      const float wgt = exp2_fast(ls - M);
      tot += wgt;
      out += wgt * Opart[(bh * S + s) * D + d];
    }
    out /= tot;
  }
  const uint32_t w2 = Ops<T>::pack2(out, 0.f);
  O[bh * D + d] = (uint16_t)(w2 & 0xffffu);
  if (d == 0) LSE[bh] = (M != -INFINITY) ? (M + __builtin_log2f(tot)) * kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int nhg = (g + 15) / 16;
  const float scale2 = fabsf(a.scale) * kLog2e;
  const float thr = scale2 > 0.f ? 8.f / scale2 : 1e30f;
  const uint32_t qxor = (a.scale < 0.f) ? 0x80008000u : 0u;
  float* Opart = (float*)a.workspace;
  float* Lpart = Opart + (size_t)a.B * a.Hq * a.num_splits * D;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.num_splits, a.Hkv * nhg, a.B), dim3(64), 0,
                     stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.seqlens, Opart, Lpart, a.Hq, a.Hkv, a.Lk_max, a.num_splits, scale2, thr,
                     qxor);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.B * a.Hq)), dim3(D), 0, stream,
                     (const float*)Opart, (const float*)Lpart, (uint16_t*)a.o, a.lse, a.num_splits);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_dtype(const DecodeArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_decode_t<T, 64>(a, stream);
    case 128: return launch_decode_t<T, 128>(a, stream);
    case 256: return launch_decode_t<T, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  const size_t n = (size_t)B * Hq * num_splits;
  return n * D * sizeof(float) + n * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_decode_dtype<bf16_t>(a, stream) : launch_decode_dtype<f16_t>(a, stream);
}

}  // namespace fa
