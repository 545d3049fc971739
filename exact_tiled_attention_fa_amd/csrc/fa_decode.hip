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
// gfx950 mapping of the split kernel: one workgroup of 4 wave64 per (chunk,
// kv head, group of <= 16 query heads, sequence).  The chunk is walked in
// 16-key steps; wave w takes steps w, w+4, ..., so a long chunk is four short
// serial chains.  Per step:
//   * S^T = K q^T with v_mfma_f32_16x16x32: A = the 16 key rows straight from
//     registers, B = q^T (the group's heads as 16 columns, zero-padded).  The
//     accumulator gives each lane one head and four consecutive keys.
//   * O^T += V^T P^T with v_mfma_f32_16x16x16: its B operand is exactly that
//     accumulator layout (rounded to 16 bits), and its A operand, four keys of
//     one head-dim column per lane, is one ds_read_b64_tr_b16 of the V tile.
//   * K and V rows of step i+1 are loaded into registers while step i
//     computes; V is written row-major into the wave's own small LDS tile (no
//     barrier: only that wave reads it).  All loads go through VGPRs, so the
//     compiler's wait counts stay exact and the prefetch is never drained.
// At the end the four waves' (O, lse) are merged through LDS.  Workspace:
// float32 partial outputs [B, Hq, S, D], then float32 partial logsumexps in
// base 2 [B, Hq, S].
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKS = kDecodeKeysPerStep;  // keys per step (one 16-key MFMA block)
constexpr int kDW = 4;                   // waves per split workgroup
static_assert(kKS == 16, "the decode MFMA layout assumes 16-key steps");

// XOR on the 16-byte chunk index of row r of a V tile: a transpose read of
// one 32-lane half touches 8 consecutive rows x 32 bytes, spread over banks.
template <int D> __device__ __forceinline__ int swz_dv(int r) {
  return D == 64 ? 2 * ((r >> 1) & 3) : 2 * (r & 7);
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kDW)
void decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                         const uint16_t* __restrict__ Vc, const int* __restrict__ seqlens,
                         float* __restrict__ Opart, float* __restrict__ Lpart, int Hq, int Hkv,
                         int Lmax, int S, float scale2, float thr, uint32_t qxor) {
  constexpr int CPR = D / 8;
  constexpr int VT = kKS * D;          // elements per V tile
  constexpr int NVL = kKS * CPR / 64;  // 16-byte V (and K) loads per lane per step
  constexpr int MERGE = 16 * D * 2;    // per-wave merge room in elements (16 heads x D floats)
  constexpr int WS = VT > MERGE ? VT : MERGE;
  __shared__ __attribute__((aligned(16))) uint16_t sV[kDW][WS];
  __shared__ float sL[kDW][16];

  const int split = blockIdx.x;
  const int b = blockIdx.z;
  const int g = Hq / Hkv;
  const int nhg = (g + 15) / 16;
  const int kvh = blockIdx.y / nhg;
  const int hg = blockIdx.y - kvh * nhg;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int len = seqlens[b];
  len = len < 0 ? 0 : (len > Lmax ? Lmax : len);
  const int C = (len + S - 1) / S;
  const int k0 = split * C;
  const int k1 = min(len, k0 + C);
  const long pbase = ((long)b * Hq + kvh * g + hg * 16) * S + split;  // partial of head slot 0

  if (k1 <= k0) {  // empty chunk: weight 0 in the merge
    if (tid < 16 && hg * 16 + tid < g) Lpart[pbase + (long)tid * S] = -INFINITY;
    return;
  }

  const int hloc = hg * 16 + l16;
  const bool hvalid = hloc < g;
  // q^T operand: lane holds head `hloc` (column l16), dims 32*ks + 8*q4 .. +8.
  // Loaded unconditionally (head slots past the group read the group's last
  // head and are zeroed), keeping the count of loads in flight path-independent.
  u32x4 qf[D / 32];
  const int hq_ld = kvh * g + min(hloc, g - 1);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const u32x4 x = load16(Q + ((long)b * Hq + hq_ld) * D + 32 * ks + 8 * q4) ^ qxor;
    qf[ks] = hvalid ? x : (u32x4){0u, 0u, 0u, 0u};
  }

  const long kstride = (long)Hkv * D;
  const uint16_t* Kb = Kc + (long)b * Lmax * kstride + (long)kvh * D;
  const uint16_t* Vb = Vc + (long)b * Lmax * kstride + (long)kvh * D;

  const int nsteps = (k1 - k0 + kKS - 1) / kKS;
  const int my_steps = nsteps > w ? (nsteps - w + kDW - 1) / kDW : 0;

  // Keys past the chunk end are redirected to its last key (finite data;
  // their scores are masked), so padding rows are never read.
  auto kload = [&](int j, u32x4 (&kx)[D / 32]) {
    const int key = min(k0 + kKS * j + l16, k1 - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kx[ks] = load16(Kb + (long)key * kstride + 32 * ks + 8 * q4);
  };
  auto vload = [&](int j, u32x4 (&vx)[NVL]) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int P = 64 * i + lane;
      const int key = min(k0 + kKS * j + P / CPR, k1 - 1);
      vx[i] = load16(Vb + (long)key * kstride + 8 * (P % CPR));
    }
  };
  uint16_t* const sv = sV[w];
  // Row-major V tile [16][D] with 16-byte chunks XOR-swizzled by row.
  auto vstore = [&](const u32x4 (&vx)[NVL]) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int P = 64 * i + lane;
      const int r = P / CPR, c = P % CPR;
      store16(sv + r * D + 8 * (c ^ swz_dv<D>(r)), vx[i]);
    }
  };
  // V^T read for head-dim block db: row 4*q4 + l16/4, columns 16db + 4*(l16%4)
  // .. +3, so lane l16 gets column 16db + l16 of keys 4*q4 .. 4*q4+3.
  const int vr = 4 * q4 + (l16 >> 2);
  int voff[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int col = 16 * db + 4 * (l16 & 3);
    voff[db] = vr * D + 8 * ((col >> 3) ^ swz_dv<D>(vr)) + (col & 7);
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = (f32x4){};
  float m_ref = -INFINITY;
  float l_part = 0.f;

  auto compute = [&](int j, const u32x4 (&kx)[D / 32], const u32x4 (&vx)[NVL]) {
    vstore(vx);  // the previous step's transpose reads of the tile are done (in-order LDS)
    // S^T: keys 4*q4 + r (rows) x heads (columns l16).
    f32x4 s = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) s = Ops<T>::mfma16(kx[ks], qf[ks], s);
    const int lim = k1 - 1 - (k0 + kKS * j) - 4 * q4;  // key offset r visible iff <= lim
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r > lim) s[r] = -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, xor16(mx));
    mx = max_halves(mx);
    const bool upd = mx > m_ref + thr;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(upd) != 0, 0)) {
      asm volatile("" ::: "memory");  // keep the rare rescale a branch
      const float m_new = upd ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast((m_ref - m_new) * scale2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
      m_ref = m_new;
    }
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * scale2;
    const float p0 = exp2_fast(__builtin_fmaf(s[0], scale2, -mb));
    const float p1 = exp2_fast(__builtin_fmaf(s[1], scale2, -mb));
    const float p2 = exp2_fast(__builtin_fmaf(s[2], scale2, -mb));
    const float p3 = exp2_fast(__builtin_fmaf(s[3], scale2, -mb));
    l_part += (p0 + p1) + (p2 + p3);  // unrounded: lse carries no 16-bit rounding
    const u32x2 bop = {Ops<T>::pack2(p0, p1), Ops<T>::pack2(p2, p3)};
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = Ops<T>::mfma16k16(lds_read_tr16(sv + voff[db]), bop, acc[db]);
  };

  // Two-deep pipeline: the next step's K and V rows are requested before this
  // step computes.  The request is unconditional (past the last step it
  // re-reads the chunk's final row, a cache hit) so that the number of loads
  // in flight, and thus each wait, is the same on every path.
  u32x4 kA[D / 32], kB[D / 32], vA[NVL], vB[NVL];
  kload(w, kA);  // (a wave with no step reads the chunk's last row, unused)
  vload(w, vA);
  // The scheduling barriers keep each request ahead of the wait for the step
  // being computed, so two steps are in flight while that wait lasts.
  for (int i = 0; i < my_steps; i += 2) {
    kload(w + kDW * (i + 1), kB);
    vload(w + kDW * (i + 1), vB);
    __builtin_amdgcn_sched_barrier(0);
    compute(w + kDW * i, kA, vA);
    if (i + 1 >= my_steps) break;
    kload(w + kDW * (i + 2), kA);
    vload(w + kDW * (i + 2), vA);
    __builtin_amdgcn_sched_barrier(0);
    compute(w + kDW * (i + 1), kB, vB);
  }

  // Merge the waves: full row sums, per-wave normalised output and lse2 to LDS.
  float l = l_part + xor16(l_part);
  l = sum_halves(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse2 = l > 0.f ? m_ref * scale2 + __builtin_log2f(l) : -INFINITY;
  __syncthreads();  // all waves are done with their V tiles
  float* sO = reinterpret_cast<float*>(&sV[0][0]);
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<f32x4*>(sO + w * (WS / 2) + l16 * D + 16 * db + 4 * q4) = acc[db] * inv;
  if (q4 == 0) sL[w][l16] = lse2;
  __syncthreads();
  for (int e = tid; e < 16 * D; e += 64 * kDW) {
    const int hs = e / D, d = e - hs * D;
    if (hg * 16 + hs >= g) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDW; ++v) M = fmaxf(M, sL[v][hs]);
    float tot = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kDW; ++v) {
        const float lv = sL[v][hs];
        if (lv == -INFINITY) continue;
        const float wt = exp2_fast(lv - M);
        tot += wt;
        o += wt * sO[v * (WS / 2) + hs * D + d];
      }
      o /= tot;
    }
    const long pi = pbase + (long)hs * S;
    Opart[pi * D + d] = o;
    if (d == 0) Lpart[pi] = M != -INFINITY ? M + __builtin_log2f(tot) : -INFINITY;
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
  // |scale| * log2(e), kept >= 1e-30 so masked (-inf) scores give probability 0.
  const float scale2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const float thr = 8.f / scale2;
  const uint32_t qxor = (a.scale < 0.f) ? 0x80008000u : 0u;
  float* Opart = (float*)a.workspace;
  float* Lpart = Opart + (size_t)a.B * a.Hq * a.num_splits * D;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.num_splits, a.Hkv * nhg, a.B), dim3(64 * kDW), 0,
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
