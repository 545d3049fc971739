// Prefill kernel: exact attention computed tile by tile with an online softmax.
//
// The method is the one described in "FlashAttention in the CANN
// ops-transformer library" (ai6s.net), section 2: K/V are cut into blocks
// (step 1), a running row max and row sum are updated after every block so
// that the end result equals standard attention (step 2), and O plus the
// per-row normaliser are accumulated block by block and written once
// (step 3).  From "FlashAttention-2 (TH)" (systems-analysis.info), technical
// architecture items 1-3: little non-matmul work (the division by the row sum
// is deferred to the end, the scale is folded into one FMA in the exponent),
// a grid over query tiles x heads x batch, and query rows split across
// wavefronts so each row's statistics stay in one wavefront's registers.
//
// gfx950 mapping (one workgroup = 4 wave64 = 128 query rows):
//   * S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}: A = K rows from LDS,
//     B = Q^T held in registers for the whole kernel.  The accumulator puts
//     one query per lane column (lane % 32) and 16 of the 32 keys of a block
//     in that lane, so a row's max/sum need only one cross-half exchange.
//   * O^T += V^T P^T with the same MFMA: B = P^T straight from the score
//     registers (rounded to the input type), A = V^T read from an LDS tile
//     that was transposed on the way in.  The output accumulator keeps the
//     query in the lane, so rescaling it is lane-local.
//   * Keys of the transposed V tile are stored at permuted positions (4-key
//     groups with their two low group bits swapped) so that the eight keys a
//     lane needs for one MFMA k-step are 16 contiguous bytes.
//   * Causal: KV tiles entirely above the diagonal are never loaded; only
//     tiles that straddle the diagonal or the ragged key tail take the masked
//     path.  Workgroups are issued heaviest query tile first.
//   * Lazy rescaling: the reference max of a row is only moved when a new
//     score exceeds it by more than 2^8 in the exponent, so the accumulator
//     rescale (D/2 multiplies per lane) runs rarely; probabilities stay
//     <= 256, well inside bf16/fp16 range, and the final O = acc / l and
//     lse = m_ref + log(l) are unchanged up to rounding.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kNT = kFwdWaves * 64;

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(kNT, (D <= 128 ? 2 : 1))
void fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int B, int Hq, int Hkv, int Lq, int Lk,
                float scale2, float thr, uint32_t qxor) {
  constexpr int BM = kFwdBM;
  constexpr int KP = D + 8;   // K tile row pitch (elements): +16 bytes against bank conflicts
  constexpr int VP = BN + 8;  // V^T tile row pitch (elements)
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int nqt = (Lq + BM - 1) / BM;
  const int BH = B * Hq;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = nqt - 1 - qt;  // heaviest query tiles are dispatched first
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);
  const int shift = Lk - Lq;
  const int q0 = qt * BM;
  const int qw0 = q0 + kFwdRowsPerWave * w;
  const int qrow = qw0 + l32;

  const long qstride = (long)Hq * D;
  const long kstride = (long)Hkv * D;
  const uint16_t* Qb = Q + (long)b * Lq * qstride + (long)h * D;
  const uint16_t* Kb = K + (long)b * Lk * kstride + (long)kvh * D;
  const uint16_t* Vb = V + (long)b * Lk * kstride + (long)kvh * D;

  // Q^T operand: lane holds query `qrow`, 8 dims per 16-dim k-step.
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (qrow < Lq) {
      u32x4 x = load16(Qb + (long)qrow * qstride + 16 * s + 8 * hf);
      qf[s] = x ^ qxor;  // negative scales: flip the sign of q, use |scale|
    } else {
      qf[s] = (u32x4){0u, 0u, 0u, 0u};
    }
  }

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, min(q0 + BM, Lq) + shift);
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  const bool wave_live = qw0 < Lq;
  const int qw_last = min(qw0 + kFwdRowsPerWave - 1, Lq - 1);
  const int wave_kmax = CAUSAL ? min(Lk - 1, qw_last + shift) : Lk - 1;
  const int row_kmax = CAUSAL ? min(Lk - 1, qrow + shift) : Lk - 1;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float m_ref = -INFINITY;  // reference max (raw score units) of this lane's row
  float l_part = 0.f;       // this lane's share of the row sum (relative to m_ref)

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BN;
    __syncthreads();  // every wave is done reading the previous tile
    // K tile, row-major [BN][D]; rows past Lk are zero.
    for (int p = tid; p < BN * (D / 8); p += kNT) {
      const int r = p / (D / 8), c = p - r * (D / 8);
      u32x4 x = (u32x4){0u, 0u, 0u, 0u};
      if (j0 + r < Lk) x = load16(Kb + (long)(j0 + r) * kstride + 8 * c);
      store16(sK + r * KP + 8 * c, x);
    }
    // V tile, transposed to [D][BN] with permuted key positions.
    for (int p = tid; p < (BN / 4) * (D / 8); p += kNT) {
      const int g = p % (BN / 4), c = p / (BN / 4);
      u32x4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * g + i;
        x[i] = (j < Lk) ? load16(Vb + (long)j * kstride + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
      }
      const int pg = (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int word = e >> 1;
        const int sh = (e & 1) * 16;
        const uint32_t k0 = (x[0][word] >> sh) & 0xffffu, k1 = (x[1][word] >> sh) & 0xffffu;
        const uint32_t k2 = (x[2][word] >> sh) & 0xffffu, k3 = (x[3][word] >> sh) & 0xffffu;
        u32x2 val = {k0 | (k1 << 16), k2 | (k3 << 16)};
        *reinterpret_cast<u32x2*>(sV + (8 * c + e) * VP + 4 * pg) = val;
      }
    }
    __syncthreads();
    if (!wave_live || j0 > wave_kmax) continue;  // whole tile masked for this wave

    // S^T = K Q^T for BN keys x 32 queries.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sK + (32 * kb + l32) * KP + 16 * ks + 8 * hf);
        s[kb] = Ops<T>::mfma32(a, qf[ks], s[kb]);
      }
    }

    const bool need_mask = (j0 + BN > Lk) || (CAUSAL && j0 + BN - 1 > qw0 + shift);
    float mx = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key > row_kmax) s[kb][r] = -INFINITY;
          mx = fmaxf(mx, s[kb][r]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    }
    mx = fmaxf(mx, xor32(mx));

    const bool upd = mx > m_ref + thr;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float m_new = upd ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast((m_ref - m_new) * scale2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      m_ref = m_new;
    }
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * scale2;

    // P = exp2(s*scale2 - m*scale2).  The MFMA takes P rounded to T; the row
    // sum adds the unrounded fp32 values, so lse carries no 16-bit rounding
    // (summing the rounded values would shift ln(l) by up to 2^-9 for rows
    // with few keys).
    uint32_t pk[BN / 32][8];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float p0 = exp2_fast(__builtin_fmaf(s[kb][2 * j], scale2, -mb));
        float p1 = exp2_fast(__builtin_fmaf(s[kb][2 * j + 1], scale2, -mb));
        if (need_mask) {
          p0 = (s[kb][2 * j] == -INFINITY) ? 0.f : p0;
          p1 = (s[kb][2 * j + 1] == -INFINITY) ? 0.f : p1;
        }
        pk[kb][j] = Ops<T>::pack2(p0, p1);
        l_part += p0 + p1;
      }

    // O^T += V^T P^T, 16 keys per MFMA k-step.
#pragma unroll
    for (int ts = 0; ts < BN / 16; ++ts) {
      const int kb = ts >> 1, c = ts & 1;
      const u32x4 bop = {pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sV + (32 * db + l32) * VP + 16 * ts + 8 * hf);
        acc[db] = Ops<T>::mfma32(a, bop, acc[db]);
      }
    }
  }

  // Epilogue: full row sum, O = acc / l, lse = ln(2) * (m*scale2 + log2 l).
  const float l = l_part + xor32(l_part);
  if (qrow < Lq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* Orow = O + ((long)b * Lq + qrow) * qstride + (long)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * hf;
        u32x2 val = {Ops<T>::pack2(acc[db][4 * a4] * inv, acc[db][4 * a4 + 1] * inv),
                     Ops<T>::pack2(acc[db][4 * a4 + 2] * inv, acc[db][4 * a4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(Orow + d) = val;
      }
    if (hf == 0) {
      LSE[(long)bh * Lq + qrow] =
          l > 0.f ? (m_ref * scale2 + __builtin_log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BN = 64;
  const int nqt = (a.Lq + kFwdBM - 1) / kFwdBM;
  const long nblocks = (long)nqt * a.B * a.Hq;
  const float s = a.scale;
  const float scale2 = fabsf(s) * kLog2e;
  // Rescale threshold of 8 (log2 units) expressed in raw score units.
  const float thr = scale2 > 0.f ? 8.f / scale2 : 1e30f;
  const uint32_t qxor = (s < 0.f) ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<T, D, BN, CAUSAL>), dim3((unsigned)nblocks), dim3(kNT), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Lq, a.Lk, scale2, thr, qxor);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_fwd_t<T, D, true>(a, stream) : launch_fwd_t<T, D, false>(a, stream);
}

template <typename T>
hipError_t launch_fwd_dtype(const FwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_fwd_d<T, 64>(a, stream);
    case 128: return launch_fwd_d<T, 128>(a, stream);
    case 256: return launch_fwd_d<T, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_fwd_dtype<bf16_t>(a, stream) : launch_fwd_dtype<f16_t>(a, stream);
}

}  // namespace fa
