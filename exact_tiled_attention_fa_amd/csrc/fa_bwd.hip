// Backward pass: dQ, dK, dV of exact attention from Q, K, V, O, dO and the
// forward's per-row logsumexp.
//
// The gradients are those of the forward's definition (row softmax of the
// scaled scores, weighted sum of values).  Training with the method is
// reported in "FlashAttention-2 (TH)" (systems-analysis.info), performance,
// and "5 years, 10K stars: xformers" (cloud.tencent.com) pairs each attention
// forward with a backward; neither page spells the backward out.  Written
// per (query i, key j) of one head, with P_ij = exp(s_ij - lse_i) rebuilt
// from the saved lse (no N x N buffer, as in the forward):
//   dV_j += P_ij dO_i          dP_ij = dO_i . V_j         D_i = dO_i . O_i
//   dS_ij = P_ij (dP_ij - D_i)  dQ_i += scale dS_ij K_j   dK_j += scale dS_ij Q_i
//
// Three kernels, none of them with atomics (results are bitwise
// reproducible):
//   * prep: D_i and lse_i * log2(e) per row into a workspace (+inf for rows
//     that see no key and for the padding rows past a sequence's end in its
//     last 32-row tile, whose D is 0, so their probabilities and dS come out
//     exactly 0).
//   * dq (query-major, like the forward): a workgroup owns 128 query rows (32
//     per wave, one per lane column) and streams K/V tiles of 32 keys through
//     LDS (LDS-direct copies, two stages).  Per tile and wave:
//     S^T = K Q^T and dP^T = V dO^T with v_mfma_f32_32x32x16 (A = K or V rows
//     from LDS, B = Q^T or dO^T held in registers), then dS^T in registers,
//     then dQ^T += K^T dS^T (A = K^T by transpose reads of the same K tile,
//     B = dS^T straight from the accumulator, rounded to 16 bits).
//   * dkdv (key-major): a workgroup of 8 waves owns 128 keys of one K/V head
//     (32 per pair of waves, one per lane column) and streams tiles of 32
//     query rows of every query head of its group (Q, dO, lse, D) through
//     LDS.  Per tile, one wave of a pair computes S = Q K^T (A = Q rows from
//     LDS, B = K^T in registers), P and dV^T += dO^T P (A by transpose reads
//     of the dO tile) and hands P to its partner through LDS; the partner
//     computes dP = dO V^T, then dS and dK^T += Q^T dS.  Each wave so holds
//     one accumulator and one operand.  The group's query heads add into the
//     same accumulators, so GQA needs no reduction pass.  (At D = 256: 4 waves,
//     64 keys, one wave per SIMD.)
// The gradients are staged through LDS and written as whole rows with
// non-temporal stores.  Masks (causal, sliding window, the key count) and
// packed sequences (cumulative offsets) are those of the forward; tiles a
// wave's rows cannot see are skipped, partly visible ones are masked by
// setting the hidden scores to -inf in a wave-uniform branch, so P and dS are
// then formed with no per-element select.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBW = 4;         // waves per workgroup
constexpr int kBT = kBW * 64;  // threads per workgroup
constexpr int kBR = 32;        // rows per wave (queries in dq, keys in dkdv)
constexpr int kBM = kBW * kBR; // rows per workgroup
constexpr int kTile = 32;      // rows per streamed tile (keys in dq, queries in dkdv)

struct BwdParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;
  const uint16_t* dO;
  const float* LSE;
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
  float* lse2;  // workspace [B, Hq, Lqp]: lse * log2(e), +inf for rows with no key and padding rows
  float* Dd;    // workspace [B, Hq, Lqp]: rowsum(dO * O), 0 for padding rows (those of a
                // sequence's last 32-row tile; the tiles past it are not written)
  const int* cu_q;  // packed sequences: offsets [B + 1] into the rows, or nullptr
  const int* cu_k;
  int total_q, total_k;  // packed row counts
  int B, Hq, Hkv, Lq, Lk, Lqp;  // packed: Lq, Lk are the longest lengths
  int win_left, win_right;
  float scale2;  // |scale| * log2(e), >= 1e-30
  float scale;   // signed scale (factor of dQ and dK)
  uint32_t qxor; // sign flip of q for negative scales
  int xcd_wq, xcd_wk;  // work-list windows of the dq and dkdv grids (xcd_work_item)
};

// Rows of sequence b: queries qs .. qs+Lq-1 and keys ks .. ks+Lk-1.  Packed
// offsets are clamped into the tensors and the lengths to the longest ones
// the grid and the workspace are sized for, so that inconsistent offsets give
// wrong results but no out-of-bounds access.
struct SeqRows {
  int qs, Lq, ks, Lk;
};
__device__ __forceinline__ SeqRows seq_rows(const BwdParams& p, int b) {
  if (!p.cu_q) return {b * p.Lq, p.Lq, b * p.Lk, p.Lk};
  SeqRows r;
  r.qs = min(max(p.cu_q[b], 0), p.total_q);
  r.Lq = min(min(max(p.cu_q[b + 1], r.qs), p.total_q) - r.qs, p.Lq);
  r.ks = min(max(p.cu_k[b], 0), p.total_k);
  r.Lk = min(min(max(p.cu_k[b + 1], r.ks), p.total_k) - r.ks, p.Lk);
  return r;
}

// Per-row statistics: D_i = dO_i . O_i and lse_i * log2(e).  A workgroup
// takes 32 consecutive query rows of one (sequence, head), the workspace's own
// order, so that each of its two stores is one whole 128-byte line; 8 lanes
// share a row (D / 64 16-byte chunks each, whole rows per group of lanes).
// The workspace rows past a sequence's end, up to the end of its last 32-row
// query tile, get lse2 = +inf and D = 0, so that they give P = 0 and dS = 0
// exactly.  Tiles past that (packed sequences shorter than the longest) are
// read by neither later kernel and are left unwritten.
constexpr int kPrepLanes = 8;                         // lanes per row
constexpr int kPrepRows = 256 / kPrepLanes;           // rows per workgroup
static_assert(kPrepRows == kTile, "one workgroup per 32-row query tile");

template <typename T, int D>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(const BwdParams p) {
  constexpr int CPL = D / 8 / kPrepLanes;  // 16-byte chunks per lane
  const int ntile = p.Lqp / kPrepRows;
  const int tile = (int)(blockIdx.x % (unsigned)ntile);
  const int bh = (int)(blockIdx.x / (unsigned)ntile);  // b * Hq + h
  const int h = bh % p.Hq, b = bh / p.Hq;
  const SeqRows sr = seq_rows(p, b);
  const int i0 = tile * kPrepRows;
  if (i0 >= (sr.Lq + kTile - 1) / kTile * kTile) return;  // whole workgroup
  const int r = threadIdx.x / kPrepLanes, c = threadIdx.x % kPrepLanes;
  const int i = i0 + r;
  const bool valid = i < sr.Lq;
  float acc = 0.f;
  if (valid) {
    const long mrow = (long)(sr.qs + i) * p.Hq + h;  // row of O / dO in memory
    // read once here: non-temporal
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int off = 8 * (c + kPrepLanes * k);
      const u32x4 o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.O + mrow * D + off));
      const u32x4 g = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.dO + mrow * D + off));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc += Ops<T>::lo(o[e]) * Ops<T>::lo(g[e]) + Ops<T>::hi(o[e]) * Ops<T>::hi(g[e]);
    }
  }
#pragma unroll
  for (int m = kPrepLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (c == 0) {
    const long oi = (long)bh * p.Lqp + i;
    if (valid) {
      // lse: dense [B, Hq, Lq]; packed [Hq, total_q]
      const long li = p.cu_q ? (long)h * p.total_q + sr.qs + i : (long)bh * p.Lq + i;
      const float l = p.LSE[li];
      p.Dd[oi] = acc;
      p.lse2[oi] = l == -INFINITY ? INFINITY : l * kLog2e;
    } else {
      p.Dd[oi] = 0.f;
      p.lse2[oi] = INFINITY;
    }
  }
}

// LDS-direct copy of `rows` x D 16-bit elements (rows r0 .. r0+rows-1 of a
// matrix with row stride `stride` elements; rows past `last` re-read `last`)
// into an LDS tile, 16-byte chunks XOR-swizzled by row.  Every thread of the
// workgroup takes part.
template <int D, int ROWS>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int NLOAD = ROWS * CPR / kBT;
  static_assert((ROWS * CPR) % kBT == 0, "tile shape");
  uint32_t off[NLOAD];
  int rr[NLOAD];
  __device__ __forceinline__ void init(int wu, int lane, int stride) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int P = (i * kBW + wu) * 64 + lane;
      const int r = P / CPR, pc = P % CPR;
      rr[i] = r;
      off[i] = 2u * (uint32_t)(r * stride + 8 * (pc ^ swz_b<D>(r)));
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* src, int r0, int last, int stride, int wu,
                                        uint16_t* dst) const {
    const uint16_t* base = src + (long)r0 * stride;
    const bool whole = r0 + ROWS - 1 <= last;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      uint32_t o = off[i];
      if (!whole) o -= 2u * (uint32_t)(((r0 + rr[i]) - min(r0 + rr[i], last)) * stride);
      load_lds16_buf(base, o, dst + (i * kBW + wu) * 512);
    }
  }
};

// Wait for this wave's copies, then the workgroup barrier (no __syncthreads:
// its fence would also order the LDS-direct copies issued after it).
__device__ __forceinline__ void copies_done_barrier() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~0x0F00);
  asm volatile("s_barrier" ::: "memory");
}

template <int D>
__device__ __forceinline__ u32x4 ld_row_chunk(const uint16_t* tile, int r, int chunk) {
  return *reinterpret_cast<const u32x4*>(tile + r * D + 8 * (chunk ^ swz_b<D>(r)));
}

// Transpose-read offsets: lane (16-lane group position i) of half hf reads
// row 4*hf + (i/4) (+8 for the second half of a 16-row step), columns
// 32*db + 16*((lane/16)%2) + 4*(lane%4) .. +3; after ds_read_b64_tr_b16 the
// lane holds one column of four consecutive rows: the A operand of an MFMA
// whose B operand is the 32x32 accumulator layout.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&toff)[D / 32][2]) {
  const int hf = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 8 * half + 4 * hf + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      toff[db][half] = row * D + 8 * ((col >> 3) ^ swz_b<D>(row)) + (col & 7);
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ f32x16 mfma_tr(const uint16_t* tile, const int (&toff)[D / 32][2],
                                           int db, int ts, u32x4 bop, f32x16 acc) {
  const u32x2 lo = lds_read_tr16(tile + 16 * ts * D + toff[db][0]);
  const u32x2 hi = lds_read_tr16(tile + 16 * ts * D + toff[db][1]);
  return Ops<T>::mfma32((u32x4){lo[0], lo[1], hi[0], hi[1]}, bop, acc);
}

// Writes a wave's 32 x D accumulator (lane column l32 = row r0 + l32, element
// 4g + i of block db = column 32db + 8g + 4(lane/32) + i) times `sc` as 16-bit
// rows r0 .. r0+31 (those below `rows`) of a matrix with row stride `stride`:
// staged in the wave's LDS area `so` (32 x D, 16-byte chunks XOR-swizzled by
// row) and stored as whole rows with non-temporal stores.  The workgroup
// barriers keep the areas clear of the tiles' last reads.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(const f32x16 (&acc)[D / 32], float sc, uint16_t* so,
                                           int lane, uint16_t* base, long stride, int r0,
                                           int rows) {
  constexpr int CPR = D / 8;
  constexpr int OSW = CPR < 16 ? CPR - 1 : 15;
  const int l32 = lane & 31, hf = lane >> 5;
  __syncthreads();  // every copy has landed and all waves are done with the tiles
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hf;
      const u32x2 val = {Ops<T>::pack2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                         Ops<T>::pack2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc)};
      *reinterpret_cast<u32x2*>(so + l32 * D + 8 * ((d >> 3) ^ (l32 & OSW)) + (d & 7)) = val;
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int pp = lane + 64 * i;
    const int row = pp / CPR, c = pp % CPR;
    if (r0 + row < rows)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(so + row * D + 8 * (c ^ (row & OSW))),
          reinterpret_cast<u32x4*>(base + (long)(r0 + row) * stride + 8 * c));
  }
}

// -------------------------------------------------------------------------
// dQ: query-major.
// -------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kBT, (D <= 128 ? 2 : 1))
void bwd_dq_kernel(const BwdParams p) {
  constexpr int BN = kTile;
  constexpr int TILE = BN * D;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];

  const int Hq = p.Hq;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index, wave-uniform (in an SGPR): so are the bounds derived from it
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wu = w;
  const int l32 = lane & 31, hf = lane >> 5;
  const int nqt = (p.Lq + kBM - 1) / kBM;
  int b, h, tt;
  xcd_work_item((int)blockIdx.x, p.B, Hq, nqt, p.xcd_wq, b, h, tt);
  const int qt = CAUSAL ? nqt - 1 - tt : tt;  // heaviest (last, under a causal mask) first
  const SeqRows sr = seq_rows(p, b);
  const int Lq = sr.Lq, Lk = sr.Lk;
  const int q0 = qt * kBM;
  if (q0 >= Lq) return;  // past this sequence's rows (whole workgroup)
  const int kvh = h / (Hq / p.Hkv);
  const int shift = Lk - Lq;
  const int qw0 = q0 + kBR * w, qrow = qw0 + l32;
  const int wl = p.win_left, wr = p.win_right;
  auto kmin = [&](int i) { return wl < 0 ? 0 : max(0, i + shift - wl); };
  auto kmax = [&](int i) {
    int hi = Lk - 1;
    if (CAUSAL) hi = min(hi, i + shift);
    if (wr >= 0) hi = min(hi, i + shift + wr);
    return hi;
  };
  const long qstride = (long)Hq * D;
  const int kstride = p.Hkv * D;
  const uint16_t* Kb = p.K + (long)sr.ks * kstride + (long)kvh * D;
  const uint16_t* Vb = p.V + (long)sr.ks * kstride + (long)kvh * D;

  // Q^T and dO^T operands: lane holds query qrow, 8 dims per 16-dim k-step.
  u32x4 qf[D / 16], df[D / 16];
  const long rowbase = ((long)sr.qs + min(qrow, Lq - 1)) * qstride + (long)h * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = load16(p.Q + rowbase + 16 * s + 8 * hf) ^ p.qxor;
    df[s] = load16(p.dO + rowbase + 16 * s + 8 * hf);
  }
  const long si = ((long)b * Hq + h) * p.Lqp + qrow;
  const float lse2 = qrow < Lq ? p.lse2[si] : INFINITY;
  const float Dq = qrow < Lq ? p.Dd[si] : 0.f;
  const float scale2 = p.scale2;

  const int q_last = min(q0 + kBM, Lq) - 1;
  const int wg_lo = kmin(q0), wg_hi = kmax(q_last);
  const int t_first = wg_lo / BN;
  const int ntiles = wg_hi >= wg_lo ? wg_hi / BN - t_first + 1 : 0;
  const int qw_last = min(qw0 + kBR - 1, Lq - 1);
  const bool wave_live = qw0 < Lq && kmax(qw_last) >= kmin(qw0);
  const int first_live = wave_live ? kmin(qw0) / BN - t_first : ntiles;
  const int last_live = wave_live ? kmax(qw_last) / BN - t_first : -1;
  const int row_kmin = kmin(qrow), row_kmax = kmax(qrow);

  TileLoader<D, BN> ldr;
  ldr.init(wu, lane, kstride);
  int toff[D / 32][2];
  tr_offsets<D>(lane, toff);

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  auto compute = [&](int u, const uint16_t* sK, const uint16_t* sV) {
    const int j0 = (t_first + u) * BN;
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      s = Ops<T>::mfma32(ld_row_chunk<D>(sK, l32, 2 * kk + hf), qf[kk], s);
      dp = Ops<T>::mfma32(ld_row_chunk<D>(sV, l32, 2 * kk + hf), df[kk], dp);
    }
    // key j0 + 8(r/4) + 4hf + r%4 of query qrow: visible iff in [row_kmin,
    // row_kmax]; hidden scores become -inf, so P and dS are exactly 0 there
    // (rows past the end have lse2 = +inf and D = 0: also P = dS = 0).
    if (!(j0 >= kmin(qw_last) && j0 + BN - 1 <= kmax(qw0))) {
      const int lo = row_kmin - j0 - 4 * hf, hi = row_kmax - j0 - 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off < lo || off > hi) s[r] = -INFINITY;
      }
    }
    uint32_t dsk[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float d2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * jj + e;
        const float pr = exp2_fast(__builtin_fmaf(s[r], scale2, -lse2));
        d2[e] = pr * (dp[r] - Dq);
      }
      dsk[jj] = Ops<T>::pack2(d2[0], d2[1]);
    }
    // dQ^T += K^T dS^T, 16 keys per k-step
#pragma unroll
    for (int ts = 0; ts < BN / 16; ++ts) {
      const u32x4 bop = {dsk[4 * ts], dsk[4 * ts + 1], dsk[4 * ts + 2], dsk[4 * ts + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma_tr<T, D>(sK, toff, db, ts, bop, acc[db]);
    }
  };

  if (ntiles > 0) {
    ldr.issue(Kb, t_first * BN, Lk - 1, kstride, wu, sK0);
    ldr.issue(Vb, t_first * BN, Lk - 1, kstride, wu, sV0);
    for (int u = 0; u < ntiles; u += 2) {
      copies_done_barrier();
      if (u + 1 < ntiles) {
        ldr.issue(Kb, (t_first + u + 1) * BN, Lk - 1, kstride, wu, sK1);
        ldr.issue(Vb, (t_first + u + 1) * BN, Lk - 1, kstride, wu, sV1);
      }
      if (u >= first_live && u <= last_live) compute(u, sK0, sV0);
      if (u + 1 >= ntiles) break;
      copies_done_barrier();
      if (u + 2 < ntiles) {
        ldr.issue(Kb, (t_first + u + 2) * BN, Lk - 1, kstride, wu, sK0);
        ldr.issue(Vb, (t_first + u + 2) * BN, Lk - 1, kstride, wu, sV0);
      }
      if (u + 1 >= first_live && u + 1 <= last_live) compute(u + 1, sK1, sV1);
    }
  }

  // dQ staged through LDS (wave w takes one of the four tile arrays, rows
  // [32][D] with 16-byte chunks XOR-swizzled by row) and written as whole
  // rows with non-temporal stores.
  stage_rows<T, D>(acc, p.scale, (w == 0) ? sK0 : (w == 1) ? sV0 : (w == 2) ? sK1 : sV1, lane,
                   p.dQ + (long)sr.qs * qstride + (long)h * D, qstride, qw0, Lq);
}

// -------------------------------------------------------------------------
// dK, dV: key-major, waves in pairs.
// -------------------------------------------------------------------------
// Waves per dK/dV workgroup (pairs x 32 keys): 8, two per SIMD, where a
// wave's accumulator and operand fit 256 registers (D <= 128); 4, one per SIMD
// with 512 registers, at D = 256.
template <int D> struct KvWaves { static constexpr int value = D <= 128 ? 8 : 4; };

// LDS-direct copy of one query tile of Q and of dO (ROWS x D each; rows past
// `last` re-read `last`) by all the NW waves of a dK/dV workgroup: load i of
// thread t moves chunk (i * NW + wave) * 64 + lane of the list [Q chunks, dO
// chunks], 16-byte chunks XOR-swizzled by row as in TileLoader.
template <int D, int ROWS>
struct PairTileLoader {
  static constexpr int NW = KvWaves<D>::value;
  static constexpr int CPR = D / 8;
  static constexpr int QCH = ROWS * CPR;  // chunks per tile
  static constexpr int NLOAD = 2 * QCH / (NW * 64);
  static_assert((2 * QCH) % (NW * 64) == 0 && QCH % 64 == 0, "tile shape");
  uint32_t off[NLOAD];
  int rr[NLOAD];
  __device__ __forceinline__ void init(int wu, int lane, int stride) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int P = (i * NW + wu) * 64 + lane;
      const int c = P < QCH ? P : P - QCH;
      const int r = c / CPR, pc = c % CPR;
      rr[i] = r;
      off[i] = 2u * (uint32_t)(r * stride + 8 * (pc ^ swz_b<D>(r)));
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* q, const uint16_t* g, int r0, int last,
                                        int stride, int wu, uint16_t* dq, uint16_t* dg) const {
    const long rb = (long)r0 * stride;
    const bool whole = r0 + ROWS - 1 <= last;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int c0 = (i * NW + wu) * 64;  // wave-uniform first chunk
      const bool isg = c0 >= QCH;
      uint32_t o = off[i];
      if (!whole) o -= 2u * (uint32_t)(((r0 + rr[i]) - min(r0 + rr[i], last)) * stride);
      load_lds16_buf((isg ? g : q) + rb, o, (isg ? dg : dq) + (isg ? c0 - QCH : c0) * 8);
    }
  }
};

// A workgroup owns 16 * NW keys of one K/V head: NW / 2 pairs of waves, 32
// keys per pair (one per lane column).  It streams tiles of 32 query rows of every
// query head of the group (Q, dO, lse, D) through LDS.  Within a pair the
// work of a tile is split so that each wave holds one 32 x D accumulator and
// one operand, which keeps two waves per SIMD resident:
//   * wave "P" holds K^T: S = Q K^T, P = exp2(S log2e - lse) on the visible
//     entries, then dV^T += dO^T P; it also stores P (fp32, in its
//     accumulator layout) in LDS for its partner;
//   * wave "S" holds V^T: dP = dO V^T for the tile; one step later (after
//     the barrier that also guards the copies) it reads P back at the same
//     layout, forms dS = P (dP - D) and adds dK^T += Q^T dS.
// The partner's lag keeps the previous tile's Q in LDS: three stages of Q /
// dO tiles (current, previous, next) and two of the P exchange.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(KvWaves<D>::value * 64, 1)
void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NW = KvWaves<D>::value;
  constexpr int KBM = NW / 2 * kBR;  // keys per workgroup
  constexpr int BQ = kTile;
  constexpr int TILE = BQ * D;
  // Distinct arrays per stage: the compiler then sees that reading one stage
  // does not alias the LDS-direct copy into another and adds no wait.
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sG0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sG1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sG2[TILE];
  __shared__ __attribute__((aligned(16))) float sL0[2 * BQ];  // lse2 then D of the tile's rows
  __shared__ __attribute__((aligned(16))) float sL1[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sL2[2 * BQ];
  // P exchange: [step parity][pair][4 x 64 lanes x 4 floats]
  __shared__ __attribute__((aligned(16))) float sX[2][NW / 2][16 * 64];
  auto qst = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return sQ0; else if constexpr (i == 1) return sQ1; else return sQ2;
  };
  auto gst = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return sG0; else if constexpr (i == 1) return sG1; else return sG2;
  };
  auto lst = [&](auto I) -> float* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return sL0; else if constexpr (i == 1) return sL1; else return sL2;
  };

  const int Hq = p.Hq, Hkv = p.Hkv;
  const int g = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int pair = wu >> 1;
  // Role per wave, alternated so that with 8 waves each SIMD (wave w runs on
  // SIMD w % 4) gets one wave of each kind: 1 = the dS / dK wave.
  const bool sw = ((wu & 1) ^ ((wu >> 2) & 1)) != 0;
  // Key tiles ascending: under a causal mask the first see the most queries.
  int b, kvh, kt;
  xcd_work_item((int)blockIdx.x, p.B, Hkv, (p.Lk + KBM - 1) / KBM, p.xcd_wk, b, kvh, kt);
  const SeqRows sr = seq_rows(p, b);
  const int Lq = sr.Lq, Lk = sr.Lk;
  const int k0 = kt * KBM;
  if (k0 >= Lk) return;  // past this sequence's keys (whole workgroup)
  const int shift = Lk - Lq;
  const int kw0 = k0 + kBR * pair, key = kw0 + l32;
  const int k_last = min(k0 + KBM, Lk) - 1;
  const int kw_last = min(kw0 + kBR - 1, Lk - 1);
  const int wl = p.win_left, wr = p.win_right;
  auto kmin = [&](int i) { return wl < 0 ? 0 : max(0, i + shift - wl); };
  auto kmax = [&](int i) {
    int hi = Lk - 1;
    if (CAUSAL) hi = min(hi, i + shift);
    if (wr >= 0) hi = min(hi, i + shift + wr);
    return hi;
  };
  // Query rows that can see some key in [ka, kb]: [qlo(ka), qhi(kb)].
  auto qlo = [&](int ka) {
    int lo = 0;
    if (CAUSAL) lo = max(lo, ka - shift);
    if (wr >= 0) lo = max(lo, ka - shift - wr);
    return lo;
  };
  auto qhi = [&](int kb) { return wl < 0 ? Lq - 1 : min(Lq - 1, kb - shift + wl); };

  const int kstride = Hkv * D;
  const int qstride = Hq * D;
  // This wave's operand: K^T (P wave) or V^T (dS wave); lane holds key `key`
  // (clamped), 8 dims per k-step.  For a negative scale the P wave flips the
  // sign of K (S = Q (-K)^T, the same as flipping Q).
  u32x4 kv[D / 16];
  {
    const long krow = ((long)sr.ks + min(key, Lk - 1)) * kstride + (long)kvh * D;
    const uint16_t* src = sw ? p.V : p.K;
    const uint32_t kx = sw ? 0u : p.qxor;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kv[s] = load16(src + krow + 16 * s + 8 * hf) ^ kx;
  }

  const int i_lo = qlo(k0), i_hi = qhi(k_last);
  const int s_first = i_lo / BQ;
  const int nsteps = (k0 < Lk && i_hi >= i_lo) ? i_hi / BQ - s_first + 1 : 0;
  const int wi_lo = qlo(kw0), wi_hi = qhi(kw_last);
  const bool pair_live = kw0 < Lk && wi_hi >= wi_lo;
  const int first_live = pair_live ? wi_lo / BQ - s_first : nsteps;
  const int last_live = pair_live ? wi_hi / BQ - s_first : -1;
  const int ntiles = g * nsteps;  // (query head of the group, query step) pairs
  // Tile u is query step u % nsteps of query head u / nsteps of the group;
  // the loop keeps these for tiles u - 1, u and u + 1 as running counters.
  auto live_st = [&](int st) { return st >= first_live && st <= last_live; };

  PairTileLoader<D, BQ> ldr;
  ldr.init(wu, lane, qstride);
  int toff[D / 32][2];
  tr_offsets<D>(lane, toff);

  // lse2 / D copy: lanes 0..7 of waves 0 and 1 (8 chunks of 4 rows each).
  auto issue_tile = [&](int hg, int st, uint16_t* dq_tile, uint16_t* dg_tile, float* dl) __attribute__((always_inline)) {
    const int hh = kvh * g + hg;
    const int q0 = (s_first + st) * BQ;
    const long hbase = (long)sr.qs * qstride + (long)hh * D;
    ldr.issue(p.Q + hbase, p.dO + hbase, q0, Lq - 1, qstride, wu, dq_tile, dg_tile);
    if (wu < 2 && lane < 8) {
      // wave 0 copies the 32 rows' lse2 to dl[0..31], wave 1 their D to
      // dl[32..63] (one wave-uniform base each)
      const long sb = ((long)b * Hq + hh) * p.Lqp + q0;  // rows q0..q0+31 < Lqp
      load_lds16_buf(uniform_ptr((wu == 0 ? p.lse2 : p.Dd) + sb), 16u * lane, dl + 32 * wu);
    }
  };

  f32x16 acc[D / 32];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  f32x16 dp = (f32x16){};  // dS wave: dP of the previous step's tile
  const float scale2 = p.scale2;

  // P wave, tile u: S, P (stored for the partner), dV^T += dO^T P.
  auto p_tile = [&](int u, int st, const uint16_t* sQ, const uint16_t* sG, const float* sL) __attribute__((always_inline)) {
    const int q0 = (s_first + st) * BQ;
    f32x16 s = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s = Ops<T>::mfma32(ld_row_chunk<D>(sQ, l32, 2 * kk + hf), kv[kk], s);
    // element r: query q0 + 8(r/4) + 4hf + r%4, key `key`.  Scores the rows
    // may not see become -inf, so P is exactly 0 there (rows past the end
    // have lse2 = +inf: P = 0 as well).
    const int qlast = min(q0 + BQ, Lq) - 1;
    if (!(kw0 >= kmin(qlast) && kw0 + kBR - 1 <= kmax(q0) && kw0 + kBR <= Lk)) {
      // query q0 + 4hf + off sees `key` iff lo <= off <= hi (kmin(i) <= key <=
      // kmax(i) solved for i), so each element is one compare pair against a
      // constant offset, with no branch
      const int base = key - shift - q0 - 4 * hf;
      int lo = -(1 << 30);
      const int hi = wl < 0 ? (1 << 30) : base + wl;
      if (CAUSAL) lo = max(lo, base);
      if (wr >= 0) lo = max(lo, base - wr);
      if (key >= Lk) lo = 1 << 30;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off < lo || off > hi) s[r] = -INFINITY;
      }
    }
    float* xs = &sX[u & 1][pair][0];
    uint32_t pk[8];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 L4 = *reinterpret_cast<const f32x4*>(sL + 8 * gq + 4 * hf);
      f32x4 pr;
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(__builtin_fmaf(s[4 * gq + i], scale2, -L4[i]));
      *reinterpret_cast<f32x4*>(xs + 4 * (gq * 64 + lane)) = pr;
      pk[2 * gq] = Ops<T>::pack2(pr[0], pr[1]);
      pk[2 * gq + 1] = Ops<T>::pack2(pr[2], pr[3]);
    }
    // dV^T += dO^T P, 16 query rows per k-step
#pragma unroll
    for (int ts = 0; ts < BQ / 16; ++ts) {
      const u32x4 pb = {pk[4 * ts], pk[4 * ts + 1], pk[4 * ts + 2], pk[4 * ts + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma_tr<T, D>(sG, toff, db, ts, pb, acc[db]);
    }
  };
  // dS wave, tile u: dP = dO V^T.
  auto dp_tile = [&](const uint16_t* sG) __attribute__((always_inline)) {
    dp = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      dp = Ops<T>::mfma32(ld_row_chunk<D>(sG, l32, 2 * kk + hf), kv[kk], dp);
  };
  // dS wave, tile u (one step later): dS = P (dP - D), dK^T += Q^T dS.
  // Entries the rows may not see have P = 0 and give dS = 0 (padding rows
  // have D = 0).
  auto ds_tile = [&](int u, const uint16_t* sQ, const float* sL) __attribute__((always_inline)) {
    const float* xs = &sX[u & 1][pair][0];
    uint32_t dsk[8];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 D4 = *reinterpret_cast<const f32x4*>(sL + BQ + 8 * gq + 4 * hf);
      const f32x4 pr = *reinterpret_cast<const f32x4*>(xs + 4 * (gq * 64 + lane));
      float ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[i] = pr[i] * (dp[4 * gq + i] - D4[i]);
      dsk[2 * gq] = Ops<T>::pack2(ds[0], ds[1]);
      dsk[2 * gq + 1] = Ops<T>::pack2(ds[2], ds[3]);
    }
#pragma unroll
    for (int ts = 0; ts < BQ / 16; ++ts) {
      const u32x4 db_ = {dsk[4 * ts], dsk[4 * ts + 1], dsk[4 * ts + 2], dsk[4 * ts + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma_tr<T, D>(sQ, toff, db, ts, db_, acc[db]);
    }
  };

  // Step u (0 .. ntiles): tile u sits in stage u % 3, tile u - 1 in the stage
  // before.  The barrier makes tile u's copies visible and ends every wave's
  // step u - 1 (its reads of the stage refilled next, its P stores); then the
  // copies of tile u + 1 are issued and the pair works on tiles u and u - 1.
  // The two kinds of wave run separate loops (so their registers are not
  // allocated side by side) with the same barriers.
  // Query step of tiles u - 1, u, u + 1 and query head (within the group) of
  // tile u + 1.
  int st_prev = 0, st_cur = 0, st_next = nsteps > 1 ? 1 : 0, hg_next = nsteps > 1 ? 0 : 1;
  auto step = [&](int u, auto I, auto role) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    using Inext = std::integral_constant<int, (i + 1) % 3>;
    using Iprev = std::integral_constant<int, (i + 2) % 3>;
    copies_done_barrier();
    if (u + 1 < ntiles) issue_tile(hg_next, st_next, qst(Inext{}), gst(Inext{}), lst(Inext{}));
    if constexpr (!decltype(role)::value) {
      if (u < ntiles && live_st(st_cur)) p_tile(u, st_cur, qst(I), gst(I), lst(I));
    } else {
      if (u >= 1 && live_st(st_prev)) ds_tile(u - 1, qst(Iprev{}), lst(Iprev{}));
      if (u < ntiles && live_st(st_cur)) dp_tile(gst(I));
    }
    st_prev = st_cur;
    st_cur = st_next;
    if (++st_next == nsteps) {
      st_next = 0;
      ++hg_next;
    }
  };
  auto run = [&](auto role) __attribute__((always_inline)) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    for (int u = 0;; u += 3) {
      step(u, S0{}, role);
      if (u + 1 > ntiles) break;
      step(u + 1, S1{}, role);
      if (u + 2 > ntiles) break;
      step(u + 2, S2{}, role);
      if (u + 3 > ntiles) break;
    }
  };

  if (ntiles > 0) {
    issue_tile(0, 0, sQ0, sG0, sL0);
    if (sw)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  // dK (dS waves) or dV (P waves) staged through LDS, one tile-sized area
  // per wave, and written as whole rows with non-temporal stores.
  static_assert(NW <= 6 || sizeof(sX) >= 2 * TILE * sizeof(uint16_t), "dK/dV stage");
  uint16_t* const sxo = reinterpret_cast<uint16_t*>(&sX[0][0][0]);
  uint16_t* const so = wu == 0 ? sQ0 : wu == 1 ? sG0 : wu == 2 ? sQ1 : wu == 3 ? sG1
                     : wu == 4 ? sQ2 : wu == 5 ? sG2 : wu == 6 ? sxo : sxo + TILE;
  stage_rows<T, D>(acc, sw ? p.scale : 1.f, so, lane,
                   (sw ? p.dK : p.dV) + (long)sr.ks * kstride + (long)kvh * D, kstride, kw0, Lk);
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.Q = (const uint16_t*)a.q;
  p.K = (const uint16_t*)a.k;
  p.V = (const uint16_t*)a.v;
  p.O = (const uint16_t*)a.o;
  p.dO = (const uint16_t*)a.dout;
  p.LSE = a.lse;
  p.dQ = (uint16_t*)a.dq;
  p.dK = (uint16_t*)a.dk;
  p.dV = (uint16_t*)a.dv;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Lq = a.Lq;
  p.Lk = a.Lk;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.Lqp = bwd_padded_rows(a.Lq);
  p.lse2 = (float*)a.workspace;
  p.Dd = p.lse2 + (size_t)a.B * a.Hq * p.Lqp;
  p.win_left = a.win_left;
  p.win_right = a.win_right;
  p.scale2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  p.scale = a.scale;
  p.qxor = a.scale < 0.f ? 0x80008000u : 0u;

  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)((long)a.B * a.Hq * (p.Lqp / kPrepRows))),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqt = (a.Lq + kBM - 1) / kBM;
  const dim3 gq((unsigned)((long)nqt * a.Hq * a.B));
  constexpr int NW = KvWaves<D>::value, KBM = NW / 2 * kBR;
  const int nkt = (a.Lk + KBM - 1) / KBM;
  const dim3 gk((unsigned)((long)nkt * a.Hkv * a.B));
  // Block order: each XCD walks windows of a few (sequence, head) rows with
  // the heaviest tiles first (xcd_work_item), so the K/V (dq) or Q/dO (dkdv)
  // streams that run at once on an XCD belong to few heads and stay in its
  // L2.  Workgroups resident per CU: dq 2 (1 at D = 256), dkdv 1.
  p.xcd_wq = xcd_window(a.B, a.Hq, a.Hkv, nqt, D <= 128 ? 2 : 1);
  p.xcd_wk = xcd_window(a.B, a.Hkv, a.Hkv, nkt, 1);
  if (a.causal) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), gq, dim3(kBT), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), gk, dim3(NW * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), gq, dim3(kBT), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), gk, dim3(NW * 64), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dtype(const BwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_bwd_t<T, 64>(a, stream);
    case 128: return launch_bwd_t<T, 128>(a, stream);
    case 256: return launch_bwd_t<T, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int bwd_padded_rows(int Lq) { return (Lq + kTile - 1) / kTile * kTile; }

size_t bwd_workspace_bytes(int B, int Hq, int Lq) {
  return 2 * (size_t)B * Hq * bwd_padded_rows(Lq) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_bwd_dtype<bf16_t>(a, stream) : launch_bwd_dtype<f16_t>(a, stream);
}

}  // namespace fa
