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
//   * K and V tiles of BN keys stream HBM -> LDS with buffer_load_dwordx4
//     ... lds (no VGPR round trip) through four stages (two for the split
//     waves at D = 256), K one tile ahead of V: while tile t's probabilities
//     are formed, S of tile t+1 is computed; one barrier per tile.  The LDS
//     operand reads of each MFMA are issued two MFMAs ahead of it.  Rows are
//     stored row-major
//     with their 16-byte chunks XOR-swizzled by row so that the MFMA operand
//     reads below hit distinct LDS banks.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}: A = K rows from LDS
//     (ds_read_b128), B = Q^T held in registers for the whole kernel.  The
//     accumulator holds one query per lane column (lane % 32) and 16 of a
//     32-key block's scores per lane, so a row's max and sum need one
//     cross-half exchange (v_permlane32_swap).
//   * O^T += V^T P^T with the same MFMA: B = P^T straight from the score
//     registers (rounded to the input type), A = V^T read from the row-major
//     V tile with ds_read_b64_tr_b16, which hands each lane one head-dim
//     column of four consecutive keys.  The output accumulator keeps the
//     query in the lane, so its rescale is lane-local.
//   * Masks: each row sees keys [kmin, kmax] -- causal (bottom-right), a
//     sliding window (left, right), the key count; xformers' structured masks
//     ("5 years, 10K stars: xformers", cloud.tencent.com) are read this way.
//     KV tiles no row of the workgroup sees are never loaded; tiles every row
//     sees whole run a mask-free main loop, the few others a masked one.
//     Workgroups are issued heaviest query tile first within XCD-sized
//     windows of heads (xcd_work_item).
//   * Block-diagonal packing: with cumulative offsets cu_q / cu_k, sequence b
//     is rows cu_q[b] .. cu_q[b+1]-1 of Q/O (cu_k for K/V) and attends only to
//     itself; without them the batch is dense [B, L, H, D].
//   * Lazy rescaling: probabilities are formed against a row's reference max
//     m_ref and the tile is accepted while each lane's share of the tile's
//     probabilities sums to at most 2^8 (so none exceeds 2^8, inside bf16/fp16
//     range).  Only otherwise -- the row's first visible tile, or scores a few
//     units above m_ref -- is the tile's row max taken, the accumulator
//     rescaled and the probabilities formed again.  The common step thus
//     computes no row max at all; O = acc / l and lse = m_ref + log(l) are
//     unchanged up to rounding.
//   * In the main phase the tile copies advance a running pointer with no
//     bounds clamping (every tile there is whole).
//   * The output tile is staged through LDS so each row is written to HBM as
//     full contiguous 16-byte-per-lane stores, non-temporal (O is not read
//     back here).
//   * At D = 256 one wave holding Q^T, the accumulator and two score tiles
//     for all 256 dims needs more than 256 registers (one wave per SIMD).
//     There a workgroup has 8 waves and two share each 32-row slice: wave w
//     and w + 4 each hold half of the head dims (their Q^T, K and V^T columns
//     and accumulator), form a partial S over that half and exchange it
//     through LDS; both then hold the same full S (own half + other half is
//     the same floating-point sum on both sides, addition commuting exactly),
//     so the same softmax, and each forms P V for its own half.  S(t+1) is exchanged during step t and summed after the
//     barrier that opens step t+1, so the exchange needs no barrier of its
//     own.  No MFMA work is done twice.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

// Waves per workgroup and head dims per wave (two waves share a row slice at
// D = 256, each holding half of the dims).
template <int D> constexpr bool fwd_split() { return D == 256; }
template <int D> constexpr int fwd_waves() { return fwd_split<D>() ? 2 * kFwdWaves : kFwdWaves; }

// Keys per KV tile.  The pipelined loop keeps two score tiles, the packed
// probabilities, the output accumulator and Q in registers; at D >= 128 a
// 32-key tile keeps that within 256 VGPRs (two waves per SIMD); at D = 64 it
// leaves room for three waves per SIMD (measured 17% faster than 64 keys).
#ifndef FA_FWD_BN_D64
#define FA_FWD_BN_D64 32
#endif
#ifndef FA_FWD_BN_D128
#define FA_FWD_BN_D128 32
#endif
#ifndef FA_FWD_STAGES
#define FA_FWD_STAGES 4
#endif
// K/V tiles in flight: tile t+NS-1 (and K one further) is requested while
// tile t is computed, which covers the HBM/L2 latency of the copies.
// The split waves at D = 256 keep two stages: their score exchange fills
// the rest of the LDS.
template <int D> constexpr int fwd_stages() { return D == 256 ? 2 : FA_FWD_STAGES; }
#ifndef FA_FWD_PF
#define FA_FWD_PF 2
#endif
// LDS operand reads issued this many MFMAs ahead of their use.
constexpr int kPF = FA_FWD_PF;
static_assert(FA_FWD_STAGES == 2 || FA_FWD_STAGES == 4, "stage count");

template <int D> struct FwdTile { static constexpr int BN = FA_FWD_BN_D64; };
template <> struct FwdTile<128> { static constexpr int BN = FA_FWD_BN_D128; };
template <> struct FwdTile<256> { static constexpr int BN = 32; };

// XOR applied to a row's 16-byte chunk index in the K tile (conflict-free
// ds_read_b128 of 16 consecutive rows at one logical chunk) ...
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}
// ... and in the V tile (conflict-free transpose reads of 4 consecutive rows).
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

struct FwdParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* LSE;
  const int* cu_q;  // nullptr: dense batch
  const int* cu_k;
  int B, Hq, Hkv;
  int Lq, Lk;       // dense: sequence lengths; packed: the longest ones
  int total_q, total_k;
  int win_left, win_right;  // < 0: unbounded
  float scale2;
  uint32_t qxor;
  int xcd_w;  // work-list window, see xcd_work_item
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(fwd_waves<D>() * 64, (D <= 128 ? 2 : 1))
void fwd_kernel(const FwdParams prm) {
  const int B = prm.B, Hq = prm.Hq, Hkv = prm.Hkv;
  const float scale2 = prm.scale2;
  const uint32_t qxor = prm.qxor;
  constexpr bool SPLIT = fwd_split<D>();
  constexpr int NW = fwd_waves<D>();         // waves per workgroup
  constexpr int NT = NW * 64;
  constexpr int DH = SPLIT ? D / 2 : D;      // head dims per wave
  constexpr int BM = kFwdBM;
  constexpr int BN = FwdTile<D>::BN;
  constexpr int kStages = fwd_stages<D>();
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BN * D;               // elements per K or V tile
  constexpr int NLOAD = BN * CPR / NT;       // LDS-direct loads per thread per tile (each of K, V)
  static_assert(BN % 32 == 0 && D % 32 == 0 && (BN * CPR) % NT == 0, "tile shape");
  // The output is staged through LDS: each wave's 32 x DH block in a quarter
  // (an eighth when split) of the four K/V tile arrays.
  static_assert(kFwdWaves == 4 && NW * 32 * DH <= 4 * TILE, "O stage");
  // kStages stages of K and V tiles.  Distinct arrays (not slices of one)
  // let the compiler see that reading one stage does not alias the
  // LDS-direct copy into another, so it inserts no wait between them.
  constexpr int T2 = kStages > 2 ? TILE : 16;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK2[T2];
  __shared__ __attribute__((aligned(16))) uint16_t sV2[T2];
  __shared__ __attribute__((aligned(16))) uint16_t sK3[T2];
  __shared__ __attribute__((aligned(16))) uint16_t sV3[T2];
  // Split waves: partial score tiles, two buffers x NW waves x BN/32 blocks
  // of 1024 floats (lane-major float4s, conflict-free).
  __shared__ __attribute__((aligned(16))) float sX[SPLIT ? 2 * NW * (BN / 32) * 1024 : 4];
  auto kst = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return sK0; else if constexpr (i == 1) return sK1;
    else if constexpr (i == 2) return sK2; else return sK3;
  };
  auto vst = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return sV0; else if constexpr (i == 1) return sV1;
    else if constexpr (i == 2) return sV2; else return sV3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int wr = SPLIT ? (w & (kFwdWaves - 1)) : w;  // 32-row slice
  const int dh0 = SPLIT ? (w / kFwdWaves) * DH : 0;  // first head dim of this wave

  const int nqt = (prm.Lq + BM - 1) / BM;
  int b, h, qt;
  xcd_work_item((int)blockIdx.x, B, Hq, nqt, prm.xcd_w, b, h, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // heaviest query tiles first
  const int bh = b * Hq + h;
  const int kvh = h / (Hq / Hkv);

  // This sequence's rows.  Packed offsets are clamped into the tensors so
  // that inconsistent offsets cannot move an access out of bounds.
  int qs, Lq, ks, Lk;
  if (prm.cu_q) {
    qs = min(max(prm.cu_q[b], 0), prm.total_q);
    Lq = min(max(prm.cu_q[b + 1], qs), prm.total_q) - qs;
    ks = min(max(prm.cu_k[b], 0), prm.total_k);
    Lk = min(max(prm.cu_k[b + 1], ks), prm.total_k) - ks;
  } else {
    qs = b * prm.Lq, Lq = prm.Lq, ks = b * prm.Lk, Lk = prm.Lk;
  }
  const int q0 = qt * BM;
  if (q0 >= Lq) return;  // past this sequence's rows (whole workgroup)
  const int qw0 = q0 + kFwdRowsPerWave * wr;
  const int qrow = qw0 + l32;

  // Keys row i may see: [kmin(i), kmax(i)], both non-decreasing in i.
  const KeyRange kr(Lq, Lk, CAUSAL, prm.win_left, prm.win_right);
  auto kmin = [&](int i) { return kr.kmin(i); };
  auto kmax = [&](int i) { return kr.kmax(i); };

  const long qstride = (long)Hq * D;
  const long kstride = (long)Hkv * D;
  const uint16_t* Qb = prm.Q + (long)qs * qstride + (long)h * D;
  const uint16_t* Kb = prm.K + (long)ks * kstride + (long)kvh * D;
  const uint16_t* Vb = prm.V + (long)ks * kstride + (long)kvh * D;

  // Tiles t_first .. t_first+ntiles-1 hold every key some row of the
  // workgroup sees; below, u = t - t_first indexes them.
  const int q_last = min(q0 + BM, Lq) - 1;
  const FwdWalk walk(kr, q0, q_last, BN);
  const int t_first = walk.t_first;
  const int ntiles = walk.ntiles;

  // Loader: load i of this thread fills 16-byte chunk position P of the tile
  // (row P / CPR, stored chunk P % CPR holding logical chunk (P % CPR) ^ swz).
  // ldk/ldv are that chunk's byte offsets from the tile's first row.
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform copy for LDS bases
  uint32_t ldk[NLOAD], ldv[NLOAD];
#pragma unroll
  for (int i = 0; i < NLOAD; ++i) {
    const int P = (i * NW + wu) * 64 + lane;
    const int r = P / CPR, pc = P % CPR;
    ldk[i] = 2u * (uint32_t)(r * (int)kstride + 8 * (pc ^ swz_k<D>(r)));
    ldv[i] = 2u * (uint32_t)(r * (int)kstride + 8 * (pc ^ swz_v<D>(r)));
  }
  // Rows past Lk (only in the last tile) are redirected to row Lk-1: any
  // finite row will do, their scores are masked.
  auto clamp_off = [&](int i, int j0, uint32_t off) {
    const int r = ((i * NW + wu) * 64 + lane) / CPR;
    return off - 2u * (uint32_t)(((j0 + r) - min(j0 + r, Lk - 1)) * (int)kstride);
  };
  auto issue = [&](const uint16_t* src, const uint32_t (&ld)[NLOAD], int t, uint16_t* dst) {
    const int j0 = t * BN;
    const uint16_t* base = src + (long)j0 * kstride;  // wave-uniform
    if (j0 + BN <= Lk) {
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) load_lds16_buf(base, ld[i], dst + (i * NW + wu) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < NLOAD; ++i)
        load_lds16_buf(base, clamp_off(i, j0, ld[i]), dst + (i * NW + wu) * 512);
    }
  };
  // Main-phase copies: the tile is whole and inside the sequence, no clamping;
  // `base` is a running wave-uniform pointer to the tile's first row.
  auto issue_whole = [&](const uint16_t* base, const uint32_t (&ld)[NLOAD], uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) load_lds16_buf(base, ld[i], dst + (i * NW + wu) * 512);
  };
  const long tstride = (long)BN * kstride;
  const uint16_t* kp = Kb;
  const uint16_t* vp = Vb;
  auto issue_k = [&](int u, uint16_t* dK) { issue(Kb, ldk, t_first + u, dK); };
  auto issue_v = [&](int u, uint16_t* dV) { issue(Vb, ldv, t_first + u, dV); };
  // Q^T operand: lane holds query `qrow`, 8 dims per 16-dim k-step (of this
  // wave's DH dims).
  u32x4 qf[DH / 16];
#pragma unroll
  for (int s = 0; s < DH / 16; ++s) {
    if (qrow < Lq) {
      u32x4 x = load16(Qb + (long)qrow * qstride + dh0 + 16 * s + 8 * hf);
      qf[s] = x ^ qxor;  // negative scales: flip the sign of q, use |scale|
    } else {
      qf[s] = (u32x4){0u, 0u, 0u, 0u};
    }
  }

  // Per-lane LDS element offsets of the MFMA operand reads.
  int koff[DH / 16];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk)
    koff[kk] = l32 * D + 8 * ((dh0 / 8 + 2 * kk + hf) ^ swz_k<D>(l32));
  // V^T read for k-step t, half r, head-dim block db: row 16t + 8r + 4hf + (lane%16)/4,
  // columns 32db + 16*((lane/16)%2) + 4*(lane%4) .. +3.  swz_v depends only on the lane here.
  const int vrow = 4 * hf + ((lane & 15) >> 2);
  int voff[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) {
    const int col = dh0 + 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    voff[db] = vrow * D + 8 * ((col >> 3) ^ swz_v<D>(vrow)) + (col & 7);
  }

  const int qw_last = min(qw0 + kFwdRowsPerWave - 1, Lq - 1);
  const int row_kmin = kmin(qrow), row_kmax = kmax(qrow);
  // Relative tiles first_live .. last_live hold keys some row of this wave sees.
  const bool wave_live = qw0 < Lq && kmax(qw_last) >= kmin(qw0);
  const int first_live = wave_live ? kmin(qw0) / BN - t_first : ntiles;
  const int last_live = wave_live ? kmax(qw_last) / BN - t_first : -1;

  f32x16 acc[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i) acc[i] = (f32x16){};
  float m_ref = -INFINITY;  // reference max (raw score units) of this lane's row
  float l_part = 0.f;       // this lane's half of the row sum (relative to m_ref)


  // S^T = K Q^T for BN keys x 32 queries (raw scores).
  auto scores = [&](f32x16 (&s)[BN / 32], const uint16_t* sK) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sK + 32 * kb * D + koff[kk]);
        s[kb] = Ops<T>::mfma32(a, qf[kk], s[kb]);
      }
    }
  };

  // Sets the scores of keys the row may not see to -inf (only tiles crossing
  // the diagonal, a window edge or the key tail).
  auto mask = [&](f32x16 (&s)[BN / 32], int u) {
    const int j0 = (t_first + u) * BN;
    if (j0 < kmin(qw_last) || j0 + BN - 1 > kmax(qw0)) {
      // key j0 + 32kb + 8(r/4) + 4hf + r%4 is visible iff it is in [row_kmin, row_kmax]
      const int hi = row_kmax - j0 - 4 * hf, lo = row_kmin - j0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          if (off > hi || off < lo) s[kb][r] = -INFINITY;
        }
    }
  };

  // P = exp2(s*scale2 - m_ref*scale2) for a masked tile, rounded to T and packed
  // as the B operand of the PV MFMA.  Masked scores are -inf and give exactly
  // 0 (scale2 > 0, mb finite).  The row sum adds the unrounded fp32 values,
  // so lse carries no 16-bit rounding (summing the rounded values would shift
  // ln(l) by up to 2^-9 for rows with few keys).
  auto exp_pack = [&](const f32x16 (&s)[BN / 32], uint32_t (&pk)[BN / 32][8]) {
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * scale2;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = exp2_fast(__builtin_fmaf(s[kb][2 * j], scale2, -mb));
        const float p1 = exp2_fast(__builtin_fmaf(s[kb][2 * j + 1], scale2, -mb));
        pk[kb][j] = Ops<T>::pack2(p0, p1);
        ls += p0 + p1;
      }
    return ls;
  };
  // The reference max moves lazily: a tile is accepted as long as this lane's
  // probabilities sum to at most 2^8 (so each is <= 2^8).  Otherwise (a score
  // more than a few units above the reference, the first visible tile, or a
  // NaN) the tile's row max is folded in, the accumulator rescaled and the
  // probabilities recomputed.
  auto accept = [&](float ls, const f32x16 (&s)[BN / 32], uint32_t (&pk)[BN / 32][8]) {
    const bool bad = !(ls <= 256.f) || m_ref == -INFINITY;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) {
      asm volatile("" ::: "memory");
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_halves(mx);
      if (mx > m_ref) {
        const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast((m_ref - mx) * scale2);
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < DH / 32; ++i) acc[i] *= alpha;
        m_ref = mx;
      }
      ls = exp_pack(s, pk);
    }
    l_part += ls;
  };
  auto make_p = [&](const f32x16 (&s)[BN / 32], uint32_t (&pk)[BN / 32][8]) {
    accept(exp_pack(s, pk), s, pk);
  };
  // S^T(t+1) = K Q^T fused with the first formation of P(t) from the scores
  // sc: each MFMA is followed by its share of the exponentials, and the K
  // operand of the MFMA kPF places later is read from LDS before it, so the
  // reads' latency is covered by the MFMAs in between.  The scheduling fences
  // keep the compiler from moving each read down to its use.  Returns this
  // lane's sum of the probabilities (as exp_pack).
  auto scores_exp = [&](f32x16 (&s)[BN / 32], const uint16_t* sK, const f32x16 (&sc)[BN / 32],
                        uint32_t (&pk)[BN / 32][8]) {
    constexpr int NK = DH / 16;            // MFMAs per 32-key block
    constexpr int NM = (BN / 32) * NK;     // MFMAs of the tile
    constexpr int NPAIR = (BN / 32) * 8;   // score pairs per lane
    static_assert(NPAIR % NM == 0, "exponentials per MFMA");
    const float mb = (m_ref == -INFINITY) ? 0.f : m_ref * scale2;
    auto kread = [&](int i) {
      return *reinterpret_cast<const u32x4*>(sK + 32 * (i / NK) * D + koff[i % NK]);
    };
    float ls = 0.f;
    u32x4 a[NM];
#pragma unroll
    for (int i = 0; i < kPF; ++i) a[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + kPF < NM) a[i + kPF] = kread(i + kPF);
      const int kb = i / NK, kk = i % NK;
      s[kb] = Ops<T>::mfma32(a[i], qf[kk], kk == 0 ? (f32x16){} : s[kb]);
#pragma unroll
      for (int jp = i * (NPAIR / NM); jp < (i + 1) * (NPAIR / NM); ++jp) {
        const int kc = jp / 8, j = jp % 8;
        const float p0 = exp2_fast(__builtin_fmaf(sc[kc][2 * j], scale2, -mb));
        const float p1 = exp2_fast(__builtin_fmaf(sc[kc][2 * j + 1], scale2, -mb));
        pk[kc][j] = Ops<T>::pack2(p0, p1);
        ls += p0 + p1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return ls;
  };
  // O^T += V^T P^T, 16 keys per MFMA k-step (slots 4r+k <-> key 16t+8r+4hf+k).
  // The V^T operand of the MFMA kPF places later is read before each MFMA
  // (fenced as in scores_exp).
  auto pv = [&](const uint32_t (&pk)[BN / 32][8], const uint16_t* sV) {
    constexpr int NDB = DH / 32;
    constexpr int NM = (BN / 16) * NDB;
    auto vread = [&](int i) {
      const int ts = i / NDB, db = i % NDB;
      const u32x2 lo = lds_read_tr16(sV + 16 * ts * D + voff[db]);
      const u32x2 hi = lds_read_tr16(sV + (16 * ts + 8) * D + voff[db]);
      return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 a[NM];
#pragma unroll
    for (int i = 0; i < kPF; ++i) a[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + kPF < NM) a[i + kPF] = vread(i + kPF);
      const int ts = i / NDB, db = i % NDB;
      const int kb = ts >> 1, c = ts & 1;
      const u32x4 bop = {pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]};
      acc[db] = Ops<T>::mfma32(a[i], bop, acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The same product with the reads left to the compiler's order (the split
  // waves at D = 256, whose registers leave no room for reads ahead).
  auto pv_plain = [&](const uint32_t (&pk)[BN / 32][8], const uint16_t* sV) {
#pragma unroll
    for (int ts = 0; ts < BN / 16; ++ts) {
      const int kb = ts >> 1, c = ts & 1;
      const u32x4 bop = {pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]};
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const u32x2 lo = lds_read_tr16(sV + 16 * ts * D + voff[db]);
        const u32x2 hi = lds_read_tr16(sV + (16 * ts + 8) * D + voff[db]);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        acc[db] = Ops<T>::mfma32(a, bop, acc[db]);
      }
    }
  };

  // Split waves: this wave's partial scores of a tile go to buffer X of the
  // exchange; the partner's (the other half of the head dims) are added in
  // after the next barrier.  The two sums are the same floating-point sum
  // (addition commutes exactly), so both waves hold the same full scores.
  // (A pair whose rows all lie past the sequence runs main-phase steps on
  // whatever the buffer holds; its rows are never stored.)
  auto xput = [&](const f32x16 (&s)[BN / 32], auto X) {
    constexpr int x = decltype(X)::value;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(sX + ((x * NW + w) * (BN / 32) + kb) * 1024 + 4 * (64 * g + lane)) =
            (f32x4){s[kb][4 * g], s[kb][4 * g + 1], s[kb][4 * g + 2], s[kb][4 * g + 3]};
  };
  auto xadd = [&](f32x16 (&s)[BN / 32], auto X) {
    constexpr int x = decltype(X)::value;
    const int other = w ^ kFwdWaves;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(
            sX + ((x * NW + other) * (BN / 32) + kb) * 1024 + 4 * (64 * g + lane));
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][4 * g + i] += o[i];
      }
  };

  // Tile t's K and V live in stage t % kStages.  Requests run kStages-1
  // tiles ahead (K one tile further, since S(t+1) is computed during step t).
  // With more than two stages they are always issued -- past the last tile
  // they re-read it -- so that the number of copies in flight, and the wait
  // below, is the same every step; with two the wait takes every copy.
  constexpr int kPerTile = 2 * NLOAD;  // copies per thread per step (K and V)
  auto tile_wait_barrier = [&](auto young_tag) {
    // This wave's copies older than the `young` most recent have landed and
    // its LDS reads are done; then the workgroup barrier.  (No __syncthreads:
    // its fence would also drain the copies still in flight.)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(young_tag)::value) & ~0x0F00);
    asm volatile("s_barrier" ::: "memory");
  };
  auto clampt = [&](int t) { return min(t, ntiles - 1); };

  // One pipeline step for tile t: its scores sc are masked already, K(t+1)
  // and V(t) have been requested kStages-1 steps ago.  Refills the stages of
  // K(t) and V(t-1) with K(t+kStages) and V(t+kStages-1), then computes
  // S(t+1), P(t) and P(t) V(t) (S first, so its MFMAs overlap the exponentials;
  // the acceptance test of P(t) comes before the PV MFMAs that read it).  In
  // the main phase (TAIL false) tiles t and t+1 are fully visible to every row
  // of the workgroup and the copies lie whole inside the keys (FwdWalk), so
  // nothing is masked, skipped or clamped.
  auto step_sc = [&](int t, auto I, f32x16 (&sc)[BN / 32], f32x16 (&sn)[BN / 32], auto tail_tag) {
    constexpr int i = decltype(I)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    using Inext = std::integral_constant<int, (i + 1) % kStages>;
    using Iprev = std::integral_constant<int, (i + kStages - 1) % kStages>;
    tile_wait_barrier(std::integral_constant<int, (kStages - 2) * kPerTile>{});
    if (TAIL) {
      // With two stages every step waits for all copies, so the copies past
      // the last tile (re-reads, which the epilogue would wait for) can be
      // left out; with more stages the wait counts need them.
      if (kStages > 2 || t + kStages < ntiles) issue_k(clampt(t + kStages), kst(I));
      if (kStages > 2 || t + kStages - 1 < ntiles) issue_v(clampt(t + kStages - 1), vst(Iprev{}));
    } else {
      issue_whole(kp, ldk, kst(I));
      issue_whole(vp, ldv, vst(Iprev{}));
      kp += tstride;
      vp += tstride;
    }
    if constexpr (SPLIT) {
      // S(t+1) is this wave's half; S(t) becomes whole here (the partner's
      // half was stored during step t-1) and is masked only now.
      using Xc = std::integral_constant<int, i & 1>;
      using Xn = std::integral_constant<int, (i + 1) & 1>;
      if (TAIL && (t > last_live || t + 1 < first_live)) return;
      if (TAIL && t + 1 == first_live) {
        scores(sn, kst(Inext{}));
        xput(sn, Xn{});
        return;
      }
      uint32_t pk[BN / 32][8];
      const bool next = !TAIL || t + 1 <= last_live;
      if (next) scores(sn, kst(Inext{}));
      xadd(sc, Xc{});
      if (TAIL) mask(sc, t);
      make_p(sc, pk);
      if (next) xput(sn, Xn{});
      pv_plain(pk, vst(I));
      return;
    }
    if (TAIL && (t > last_live || t + 1 < first_live)) return;  // tile t and t+1 hidden from this wave
    if (TAIL && t + 1 == first_live) {  // tile t hidden, t+1 the wave's first
      scores(sn, kst(Inext{}));
      mask(sn, t + 1);
      return;
    }
    uint32_t pk[BN / 32][8];
    if (!TAIL || t + 1 <= last_live) {
      accept(scores_exp(sn, kst(Inext{}), sc, pk), sc, pk);
      pv(pk, vst(I));
      if (TAIL) mask(sn, t + 1);
    } else {
      make_p(sc, pk);
      pv(pk, vst(I));
    }
  };
  // Score tiles alternate: even steps hold S(t) in sA, odd ones in sB.
  f32x16 sA[BN / 32], sB[BN / 32];
  auto step = [&](int t, auto I, auto tail_tag) {
    if constexpr (decltype(I)::value % 2 == 0)
      step_sc(t, I, sA, sB, tail_tag);
    else
      step_sc(t, I, sB, sA, tail_tag);
  };
  using S2 = std::integral_constant<int, 2 % kStages>;
  using S3 = std::integral_constant<int, 3 % kStages>;

  if (ntiles > 0) {
    // Prologue: K(0), then (K(j), V(j-1)) for j = 1 .. kStages-1.
    issue_k(0, sK0);
    issue_k(clampt(1), sK1);
    issue_v(0, sV0);
    if constexpr (kStages > 2) {
      issue_k(clampt(2), kst(S2{}));
      issue_v(clampt(1), sV1);
      issue_k(clampt(3), kst(S3{}));
      issue_v(clampt(2), vst(S2{}));
    }
    tile_wait_barrier(std::integral_constant<int, (kStages - 1) * kPerTile>{});  // K(0) landed
    if (first_live == 0 && last_live >= 0) {
      scores(sA, sK0);
      if constexpr (SPLIT)
        xput(sA, std::integral_constant<int, 0>{});  // summed and masked in step 0
      else
        mask(sA, 0);
    }
    // Head phase (masked tiles left of some row's window), main phase
    // (unmasked, running tile pointers), tail phase (masked or partly skipped).
    fwd_walk<kStages>(walk, step, [&](int t) {
      kp = Kb + (long)(t_first + t + kStages) * tstride;
      vp = Vb + (long)(t_first + t + kStages - 1) * tstride;
    });
  }
  wait_vmem();  // copies of re-read tiles past the end are still landing

  // Epilogue: full row sum, O = acc / l staged through LDS (wave w uses one
  // stage array, rows [32][D] with 16-byte chunks XOR-swizzled by row), then
  // written as whole rows; lse = ln2 * (m*scale2 + log2 l).
  const float l = sum_halves(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  constexpr int CPH = DH / 8;  // 16-byte chunks of this wave's part of a row
  constexpr int OSW = CPH < 16 ? CPH - 1 : 15;
  {
    __syncthreads();  // all waves are done with the K/V tiles
    uint16_t* so;
    if constexpr (SPLIT)
      so = ((w >> 1) == 0 ? sK0 : (w >> 1) == 1 ? sV0 : (w >> 1) == 2 ? sK1 : sV1) + (w & 1) * 32 * DH;
    else
      so = (w == 0) ? sK0 : (w == 1) ? sV0 : (w == 2) ? sK1 : sV1;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * db + 8 * a4 + 4 * hf;
        u32x2 val = {Ops<T>::pack2(acc[db][4 * a4] * inv, acc[db][4 * a4 + 1] * inv),
                     Ops<T>::pack2(acc[db][4 * a4 + 2] * inv, acc[db][4 * a4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(so + l32 * DH + 8 * ((d >> 3) ^ (l32 & OSW)) + (d & 7)) = val;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32 * CPH / 64; ++i) {
      const int p = lane + 64 * i;
      const int row = p / CPH, c = p % CPH;
      const int q = qw0 + row;
      if (q < Lq)
        // non-temporal: O is written once and not read back here (whole
        // rows per instruction, so no line is written in pieces)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(so + row * DH + 8 * (c ^ (row & OSW))),
            reinterpret_cast<u32x4*>(prm.O + ((long)qs + q) * qstride + (long)h * D + dh0 + 8 * c));
    }
  }
  if (hf == 0 && qrow < Lq && dh0 == 0) {
    // lse: dense [B, Hq, Lq]; packed [Hq, total_q]
    const long li = prm.cu_q ? (long)h * prm.total_q + qs + qrow : ((long)bh * Lq + qrow);
    __builtin_nontemporal_store(
        l > 0.f ? (m_ref * scale2 + __builtin_log2f(l)) * kLn2 : -INFINITY, prm.LSE + li);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.Lq + kFwdBM - 1) / kFwdBM;
  const long nblocks = (long)nqt * a.B * a.Hq;
  const float s = a.scale;
  FwdParams p;
  p.Q = (const uint16_t*)a.q;
  p.K = (const uint16_t*)a.k;
  p.V = (const uint16_t*)a.v;
  p.O = (uint16_t*)a.o;
  p.LSE = a.lse;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.B = a.B, p.Hq = a.Hq, p.Hkv = a.Hkv, p.Lq = a.Lq, p.Lk = a.Lk;
  p.total_q = a.total_q, p.total_k = a.total_k;
  p.win_left = a.win_left, p.win_right = a.win_right;
  // |scale| * log2(e), kept >= 1e-30 so that masked (-inf) scores always give
  // probability 0; for scale 0 this changes no result beyond 1e-30 relative.
  p.scale2 = fmaxf(fabsf(s) * kLog2e, 1e-30f);
  p.qxor = (s < 0.f) ? 0x80008000u : 0u;
  // blocks resident per CU at this kernel's register use: 3 (D=64), 2, 1 (D=256)
  p.xcd_w = xcd_window(a.B, a.Hq, a.Hkv, nqt, D == 64 ? 3 : D == 128 ? 2 : 1);
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3((unsigned)nblocks), dim3(fwd_waves<D>() * 64),
                     0, stream, p);
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
