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
//   * S^T = K q^T with v_mfma_f32_16x16x32: A = the 16 key rows read from the
//     wave's LDS K tile, B = q^T (the group's heads as 16 columns,
//     zero-padded).  The accumulator gives each lane one head and four
//     consecutive keys.
//   * O^T += V^T P^T with v_mfma_f32_16x16x16: its B operand is exactly that
//     accumulator layout (rounded to 16 bits), and its A operand, four keys of
//     one head-dim column per lane, is one ds_read_b64_tr_b16 of the V tile.
//   * K and V rows of step i+1 are loaded into registers while step i
//     computes, whole rows per load instruction, non-temporal; both are
//     written row-major into the wave's own small LDS tiles (no barrier: only
//     that wave reads them).  All loads go through VGPRs, so the compiler's
//     wait counts stay exact and the prefetch is never drained.
// At the end the four waves' (O, lse) are merged through LDS.  Workspace:
// float32 partial outputs [B, Hq, S, D], then float32 partial logsumexps in
// base 2 [B, Hq, S].
//
// Paged and int8 caches (the PagedAttention reference of "FlashAttention-2
// (TH)" (systems-analysis.info), references; the KV-INT8 modes of "MNN LLM
// attention_mode" (lpnh.cn), encoding section).  A paged cache keeps rows in
// pages of P slots; key j of sequence b is slot j % P of page table[b, j / P].
// Chunks are then rounded up to whole 16-key steps and P is a power of two
// >= 16, so each step lies in one page and needs one table entry (a scalar
// load).  An int8 side holds codes with one float scale per cached row: key
// codes are widened exactly to the 16-bit type for the MFMA and the row's
// scale multiplies its scores; value codes are widened exactly when the V
// tile is written to LDS and the row's scale multiplies its probability
// before the 16-bit rounding (the row sum uses the unscaled probabilities).
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKS = kDecodeKeysPerStep;  // keys per step (one 16-key MFMA block)
static_assert(kKS == 16, "the decode MFMA layout assumes 16-key steps");

constexpr int kDW = 4;  // waves per split workgroup

struct SplitParams {
  const uint16_t* Q;
  const void* K;  // dense [B, Lmax, Hkv, D]; paged [num_pages, P, Hkv, D]; 16-bit or int8
  const void* V;
  const float* ksc;  // int8 keys: scales [num_pages, Hkv, P]
  const float* vsc;  // int8 values: scales [num_pages, Hkv, P]
  const int* table;  // paged: [B, max_pages]
  const int* seqlens;
  float* Opart;
  float* Lpart;
  int Hq, Hkv;
  int Lmax;  // longest sequence the cache holds (paged: max_pages * P)
  int page_shift, max_pages, num_pages;
  int S;
  float scale2, thr;
  uint32_t qxor;
};

// K and V rows are read exactly once per call, each load instruction covering
// whole rows, with non-temporal loads that stream them past the caches (on the
// 128-sequence decode workload they took the kernel from 5.45 to 6.13 TB/s).
// A non-temporal load that fetches a line in pieces is slower instead, which
// is why K is not loaded in the MFMA operand layout.
template <typename V> __device__ __forceinline__ V stream_load(const V* p) {
  return __builtin_nontemporal_load(p);
}

// Eight int8 codes (two dwords) widened exactly to eight 16-bit values.
template <typename T> __device__ __forceinline__ u32x4 widen8(u32x2 x) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = x[i >> 1] >> (16 * (i & 1));
    r[i] = Ops<T>::pack2((float)(int8_t)(w & 0xffu), (float)(int8_t)((w >> 8) & 0xffu));
  }
  return r;
}

// The int8 keys-and-values instance at D <= 128 is held to 168 registers,
// three waves per SIMD: it fits there, and each step of it moves half the bytes
// of a 16-bit step, so it needs the extra wave's loads in flight.
template <typename T, int D, bool PAGED, bool KI8, bool VI8>
__global__ __launch_bounds__(64 * kDW, (KI8 && VI8 && D <= 128) ? 3 : 1)
void decode_split_kernel(const SplitParams prm) {
  const int Hq = prm.Hq, Hkv = prm.Hkv, Lmax = prm.Lmax, S = prm.S;
  const float scale2 = prm.scale2, thr = prm.thr;
  const uint32_t qxor = prm.qxor;
  const uint16_t* __restrict__ Q = prm.Q;
  float* __restrict__ Opart = prm.Opart;
  float* __restrict__ Lpart = prm.Lpart;
  constexpr int CPR = D / 8;
  constexpr int VT = kKS * D;          // elements per V tile
  // 16-byte V loads per lane per step (8 16-bit or 16 int8 elements each)
  constexpr int NVL = VI8 ? kKS * D / 16 / 64 : kKS * CPR / 64;
  // The waves' outputs (16 heads x D floats each) are merged through the V
  // tiles' room (16 x D 16-bit values each) in two passes over the head dims.
  constexpr int MP = 2;
  constexpr int DP = D / MP;
  constexpr int WS = VT;
  static_assert(16 * DP * 2 <= WS && DP % 16 == 0, "merge room");
  __shared__ __attribute__((aligned(16))) uint16_t sV[kDW][WS];
  __shared__ float sL[kDW][16];
  // Per-wave K tile [16][D] (16-bit or int8 codes), 16-byte chunks XOR-swizzled by row.
  constexpr int KEB = KI8 ? 1 : 2;         // bytes per cached K element
  constexpr int KLPR = D * KEB / 16;       // 16-byte K loads per row
  constexpr int NKL = kKS * KLPR / 64;     // 16-byte K loads per lane per step
  static_assert(NKL >= 1 && NVL >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t sKt[kDW][kKS * D * KEB];
  __shared__ __attribute__((aligned(16))) float sSc[kDW][64];  // int8 row scales of a step

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

  int len = prm.seqlens[b];
  len = len < 0 ? 0 : (len > Lmax ? Lmax : len);
  int C = (len + S - 1) / S;
  if (PAGED) C = (C + kKS - 1) / kKS * kKS;  // whole steps: a step never straddles a page
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

  const long kstride = (long)Hkv * D;  // elements from one cached row to the next
  using KE = std::conditional_t<KI8, int8_t, uint16_t>;
  using VE = std::conditional_t<VI8, int8_t, uint16_t>;
  const KE* Kb = static_cast<const KE*>(prm.K) + (long)kvh * D;
  const VE* Vb = static_cast<const VE*>(prm.V) + (long)kvh * D;
  if (!PAGED) {
    Kb += (long)b * Lmax * kstride;
    Vb += (long)b * Lmax * kstride;
  }

  const int nsteps = (k1 - k0 + kKS - 1) / kKS;
  const int my_steps = nsteps > w ? (nsteps - w + kDW - 1) / kDW : 0;

  // Step j covers keys k0 + 16j .. +15.  `first` is its first key (a step
  // past the chunk's end maps onto the chunk's last step, whose rows are
  // re-read), row0 the cache row of that key (key first + i lives in row
  // row0 + i) and srow the index of its scale (paged int8).  Keys past the
  // chunk end are redirected to its last key (finite data; their scores are
  // masked), so padding is never read.
  struct StepRows { int first; long row0; long srow; };
  // Paged: a window of 64 table entries in a VGPR (lane i holds the entry of
  // page wstart + i), refilled when a step leaves it, so the page of a step
  // is a readlane rather than a dependent memory load.
  int wstart = -(1 << 30), vtab = 0;
  auto step_rows = [&](int j) -> StepRows {
    if constexpr (PAGED) {
      const int first = min(k0 + kKS * j, (k1 - 1) & ~(kKS - 1));
      const int pg = first >> prm.page_shift;
      if (pg < wstart || pg >= wstart + 64) {
        wstart = pg;
        const int e = min(pg + lane, prm.max_pages - 1);
        vtab = min(max(prm.table[(long)b * prm.max_pages + e], 0), prm.num_pages - 1);
      }
      const long phys = __builtin_amdgcn_readlane(vtab, pg - wstart);
      const int slot = first & ((1 << prm.page_shift) - 1);
      return {first, (phys << prm.page_shift) + slot,
              ((phys * Hkv + kvh) << prm.page_shift) + slot};
    } else {
      const int first = min(k0 + kKS * j, k1 - 1);
      return {first, (long)first, 0};
    }
  };
  // Offset (elements) of key first + i's row from row0's, clamped to the
  // chunk (first <= k1 - 1 always, so the offset is never negative).
  auto row_off = [&](const StepRows& st, int i) {
    return (uint32_t)(min(i, k1 - 1 - st.first) * (int)kstride);
  };
  // K rows are read like V rows, whole rows per instruction (16 lanes per row
  // of 16-bit elements), with non-temporal loads, and staged through the
  // wave's LDS tile: the MFMA operand layout would fetch half a cache line
  // per instruction.
  auto kload = [&](const StepRows& st, u32x4 (&kx)[NKL]) {
    const KE* kr = Kb + st.row0 * kstride;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int P = 64 * i + lane;
      kx[i] = stream_load(
          reinterpret_cast<const u32x4*>(kr + row_off(st, P / KLPR) + (16 / KEB) * (P % KLPR)));
    }
  };
  constexpr int VEPL = VI8 ? 16 : 8;  // elements per 16-byte V load
  constexpr int VLPR = D / VEPL;      // 16-byte V loads per row
  auto vload = [&](const StepRows& st, u32x4 (&vx)[NVL]) {
    const VE* vr = Vb + st.row0 * kstride;
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int P = 64 * i + lane;
      vx[i] = stream_load(
          reinterpret_cast<const u32x4*>(vr + row_off(st, P / VLPR) + VEPL * (P % VLPR)));
    }
  };
  // Int8 sides: a step's row scales, one per lane (lane l holds the scale of
  // key l % 16 of side (l / 16) % NSD, the K side first).  They pass through
  // the wave's LDS like the tiles, which costs one register per step instead
  // of four per side.  Scales of keys past the chunk end hold anything and
  // are masked.
  constexpr int NSD = (KI8 ? 1 : 0) + (VI8 ? 1 : 0);
  const bool s_kside = KI8 && (lane / kKS) % (NSD ? NSD : 1) == 0;
  const float* const s_base = s_kside ? prm.ksc : prm.vsc;
  struct StepRegs {  // one step's rows in registers
    u32x4 k[NKL];
    u32x4 v[NVL];
    float sc;
  };
  auto load_step = [&](int j, StepRegs& r) {
    const StepRows st = step_rows(j);
    kload(st, r.k);
    vload(st, r.v);
    if constexpr (NSD > 0) r.sc = s_base[st.srow + l16];
  };
  float* const ss = sSc[w];
  uint16_t* const sv = sV[w];
  uint8_t* const sk = sKt[w];
  auto kstore = [&](const u32x4 (&kx)[NKL]) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int P = 64 * i + lane;
      const int r = P / KLPR, c = P % KLPR;
      *reinterpret_cast<u32x4*>(sk + 16 * (r * KLPR + (c ^ row_xor<KLPR>(r)))) = kx[i];
    }
  };
  // Row-major V tile [16][D] of 16-bit values with 16-byte chunks
  // XOR-swizzled by row (int8 codes are widened on the way in).
  auto vstore = [&](const u32x4 (&vx)[NVL]) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int P = 64 * i + lane;
      const int r = P / VLPR, c = P % VLPR;
      if constexpr (VI8) {
        store16(sv + r * D + 8 * ((2 * c) ^ swz_dv<D>(r)), widen8<T>((u32x2){vx[i][0], vx[i][1]}));
        store16(sv + r * D + 8 * ((2 * c + 1) ^ swz_dv<D>(r)),
                widen8<T>((u32x2){vx[i][2], vx[i][3]}));
      } else {
        store16(sv + r * D + 8 * (c ^ swz_dv<D>(r)), vx[i]);
      }
    }
  };
  // V^T read for head-dim block db: row 4*q4 + l16/4, columns 16db +
  // 4*(l16%4) .. +3, so lane l16 gets column 16db + l16 of keys 4*q4 .. 4*q4+3.
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

  auto compute = [&](int j, const StepRegs& r) {
    // the previous step's reads of the tiles and scales are done (in-order LDS)
    kstore(r.k);
    vstore(r.v);
    if constexpr (NSD > 0) ss[lane] = r.sc;
    // S^T: keys 4*q4 + i (rows) x heads (columns l16); lane (l16, q4) takes
    // dims 32*ks + 8*q4 .. +7 of key row l16.
    f32x4 s = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      if constexpr (KI8) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(
            sk + 16 * (l16 * KLPR + ((2 * ks + (q4 >> 1)) ^ row_xor<KLPR>(l16))) + 8 * (q4 & 1));
        s = Ops<T>::mfma16(widen8<T>(a), qf[ks], s);
      } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            sk + 16 * (l16 * KLPR + ((4 * ks + q4) ^ row_xor<KLPR>(l16))));
        s = Ops<T>::mfma16(a, qf[ks], s);
      }
    }
    if constexpr (KI8)  // each key row's scale (keys 4*q4 .. +3)
      s *= *reinterpret_cast<const f32x4*>(ss + 4 * q4);
    const int lim = k1 - 1 - (k0 + kKS * j) - 4 * q4;  // key offset i visible iff <= lim
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i > lim) s[i] = -INFINITY;
      mx = fmaxf(mx, s[i]);
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
    u32x2 bop;
    if constexpr (VI8) {  // each value row's scale, folded into its probability
      f32x4 vs = *reinterpret_cast<const f32x4*>(ss + kKS * (NSD - 1) + 4 * q4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i > lim) vs[i] = 0.f;  // masked keys: their slot's scale may be anything
      bop = (u32x2){Ops<T>::pack2(p0 * vs[0], p1 * vs[1]), Ops<T>::pack2(p2 * vs[2], p3 * vs[3])};
    } else
      bop = (u32x2){Ops<T>::pack2(p0, p1), Ops<T>::pack2(p2, p3)};
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = Ops<T>::mfma16k16(lds_read_tr16(sv + voff[db]), bop, acc[db]);
  };

  // Two-deep pipeline: the next step's K and V rows are requested before this
  // step computes.  In the loop the request is unconditional, so that the
  // number of loads in flight, and thus each wait, is the same on every path;
  // the last one or two steps are peeled off, so that no request reaches past
  // the wave's last step (the merge below would wait for it).
  StepRegs rA, rB;
  load_step(w, rA);  // (a wave with no step reads the chunk's last step, unused)
  // The scheduling barriers keep each request ahead of the wait for the step
  // being computed, so two steps are in flight while that wait lasts.  (A
  // third step in flight, or 32-key steps for int8 caches, cost a wave per
  // SIMD in registers or serialise each wave further, and measured slower.)
  int i = 0;
  for (; i + 2 < my_steps; i += 2) {
    load_step(w + kDW * (i + 1), rB);
    __builtin_amdgcn_sched_barrier(0);
    compute(w + kDW * i, rA);
    load_step(w + kDW * (i + 2), rA);
    __builtin_amdgcn_sched_barrier(0);
    compute(w + kDW * (i + 1), rB);
  }
  if (i + 1 < my_steps) {  // two steps left
    load_step(w + kDW * (i + 1), rB);
    __builtin_amdgcn_sched_barrier(0);
    compute(w + kDW * i, rA);
    compute(w + kDW * (i + 1), rB);
  } else if (i < my_steps) {  // one step left
    compute(w + kDW * i, rA);
  }

  // Merge the waves: full row sums, per-wave normalised output and lse2 to LDS.
  float l = l_part + xor16(l_part);
  l = sum_halves(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse2 = l > 0.f ? m_ref * scale2 + __builtin_log2f(l) : -INFINITY;
  __syncthreads();  // all waves are done with their V tiles
  float* sO = reinterpret_cast<float*>(&sV[0][0]);
  if (q4 == 0) sL[w][l16] = lse2;
#pragma unroll
  for (int mp = 0; mp < MP; ++mp) {
    if (mp) __syncthreads();  // the previous pass's reads are done
#pragma unroll
    for (int db = 0; db < DP / 16; ++db)
      *reinterpret_cast<f32x4*>(sO + w * (WS / 2) + l16 * DP +
                                4 * ((4 * db + q4) ^ row_xor<DP / 4>(l16))) =
          acc[mp * (DP / 16) + db] * inv;
    __syncthreads();
    for (int e = tid; e < 16 * DP; e += 64 * kDW) {
      const int hs = e / DP, d = e - hs * DP;
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
          o += wt * sO[v * (WS / 2) + hs * DP + 4 * ((d >> 2) ^ row_xor<DP / 4>(hs)) + (d & 3)];
        }
        o /= tot;
      }
      const long pi = pbase + (long)hs * S;
      __builtin_nontemporal_store(o, Opart + pi * D + mp * DP + d);  // read once, by the merge
      if (mp == 0 && d == 0) Lpart[pi] = M != -INFINITY ? M + __builtin_log2f(tot) : -INFINITY;
    }
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
  for (int s0 = 0; s0 < S; s0 += 8) {
    float l8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) l8[i] = s0 + i < S ? lp[s0 + i] : -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, l8[i]);
  }
  float out = 0.f, tot = 0.f;
  if (M != -INFINITY) {
    // four partials requested at a time (their loads overlap); an empty
    // chunk's partial was never written and is selected away, not weighted
    const float* op = Opart + bh * S * D + d;
    for (int s0 = 0; s0 < S; s0 += 4) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = s0 + i < S ? __builtin_nontemporal_load(op + (s0 + i) * D) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ls = s0 + i < S ? lp[s0 + i] : -INFINITY;
        const float wgt = ls == -INFINITY ? 0.f : exp2_fast(ls - M);
        tot += wgt;
        out += ls == -INFINITY ? 0.f : wgt * o[i];
      }
    }
    out /= tot;
  }
  const uint32_t w2 = Ops<T>::pack2(out, 0.f);
  O[bh * D + d] = (uint16_t)(w2 & 0xffffu);
  if (d == 0) LSE[bh] = (M != -INFINITY) ? (M + __builtin_log2f(tot)) * kLn2 : -INFINITY;
}

template <typename T, int D, bool PAGED, bool KI8, bool VI8>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int nhg = (g + 15) / 16;
  SplitParams p;
  p.Q = (const uint16_t*)a.q;
  p.K = a.k;
  p.V = a.v;
  p.ksc = a.k_scales;
  p.vsc = a.v_scales;
  p.table = a.block_table;
  p.seqlens = a.seqlens;
  p.Opart = (float*)a.workspace;
  p.Lpart = p.Opart + (size_t)a.B * a.Hq * a.num_splits * D;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Lmax = PAGED ? a.max_pages * a.page_size : a.Lk_max;
  p.page_shift = PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.S = a.num_splits;
  // |scale| * log2(e), kept >= 1e-30 so masked (-inf) scores give probability 0.
  p.scale2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  // The running max moves only when a score exceeds it by more than thr, so
  // probabilities reach at most 2^8.  With fp16 and int8 values each
  // probability is multiplied by its value row's scale before the 16-bit
  // rounding; there the max moves at once (p <= 1), so p * scale stays within
  // fp16 wherever the dequantised values themselves fit it (|code| * scale
  // <= 127 * scale, the same bound the output needs).
  p.thr = (VI8 && std::is_same<T, f16_t>::value) ? 0.f : 8.f / p.scale2;
  p.qxor = (a.scale < 0.f) ? 0x80008000u : 0u;
  hipLaunchKernelGGL((decode_split_kernel<T, D, PAGED, KI8, VI8>),
                     dim3(a.num_splits, a.Hkv * nhg, a.B),
                     dim3(64 * kDW), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.B * a.Hq)), dim3(D), 0, stream,
                     (const float*)p.Opart, (const float*)p.Lpart, (uint16_t*)a.o, a.lse, a.num_splits);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_fmt(const DecodeArgs& a, hipStream_t stream) {
  if (!a.paged) return launch_decode_t<T, D, false, false, false>(a, stream);
  if (!a.k_int8 && !a.v_int8) return launch_decode_t<T, D, true, false, false>(a, stream);
  if (a.k_int8 && !a.v_int8) return launch_decode_t<T, D, true, true, false>(a, stream);
  if (a.k_int8 && a.v_int8) return launch_decode_t<T, D, true, true, true>(a, stream);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_decode_dtype(const DecodeArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_decode_fmt<T, 64>(a, stream);
    case 128: return launch_decode_fmt<T, 128>(a, stream);
    case 256: return launch_decode_fmt<T, 256>(a, stream);
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
