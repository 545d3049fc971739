// FP8 (e4m3) forward: the tiled online-softmax forward with Q, K and V stored
// as 8-bit e4m3 codes plus one float descale each, on gfx950's double-rate
// v_mfma_f32_32x32x64_f8f6f4.
//
// The FP8 variant of the method is the FlashAttention-3 item of
// "FlashAttention-2 (TH)" (systems-analysis.info); the page gives neither the
// format nor the scaling.  Read here as OCP e4m3 codes with per-tensor
// descales (the real value is code * descale), V supplied transposed
// ([B, Hkv, D, stride], keys contiguous per dimension, as written by the
// quantisation step), and P rounded to e4m3 for the PV product.
//
// gfx950 mapping (one workgroup = 4 wave64 = 128 query rows, 64-key tiles):
//   * S^T = K Q^T: two 32x32 blocks per tile, each D/64 MFMAs of k = 64 dims.
//     A = 32 K rows from LDS, B = Q^T in registers (32 bytes per lane per
//     MFMA).  The A rows are taken in the order 16h + 4g + i -> accumulator
//     row 8g + 4h + i, so each lane's 16 scores of a block are 16 consecutive
//     keys (16h .. 16h+15 of the block).
//   * O^T += V^T P^T: one MFMA (k = 64 keys) per 32 head dimensions.  B =
//     P^T straight from the score registers, scaled by 2^kPExp (so that the
//     e4m3 rounding stays clear of subnormals; the factor is added to the
//     exponent and removed through the row sum) and packed with
//     v_cvt_pk_fp8_f32;
//     A = 32 bytes of one V^T row (two ds_read_b128 of keys 16h.. and
//     32+16h..), matching the keys each lane's P bytes carry.  The two
//     operands of the f8f6f4 MFMA share their k layout, so matching byte
//     positions is all that is needed.
//   * Online softmax as in the 16-bit forward, with the lazy rescale limited
//     to a factor of 2^kSlack so that 2^kPExp * P stays below e4m3's 448.  The
//     row sum adds the unrounded fp32 probabilities.
//   * K and V^T tiles stream HBM -> LDS with LDS-direct copies, two stages.
//   * O is staged through the tile arrays and written as whole rows with
//     non-temporal stores.
//   * Packed sequences (cumulative offsets cu_q / cu_k, the block-diagonal
//     structured mask of "5 years, 10K stars: xformers", cloud.tencent.com):
//     V^T is [Hkv, D, stride] with key row r of the packed K at column r, and
//     a sequence's key tiles start at its first key rounded down to 16, so
//     that the 16-byte copies stay aligned; the few keys before its first
//     (the previous sequence's) count as invisible.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kPW = 4;            // waves per workgroup
constexpr int kPT = kPW * 64;     // threads
constexpr int kPR = 32;           // query rows per wave
constexpr int kPBM = kPW * kPR;   // query rows per workgroup
constexpr int kPBN = 64;          // keys per tile
// P enters the PV product as 2^kPExp * P in e4m3, and a row's maximum may grow
// by kSlack (base-2 exponent units) past the reference the accumulators are
// scaled to before they are rescaled: 2^(kPExp + kSlack) ~ 362 stays below
// e4m3's largest finite value, 448, and every P down to 2^-(6 + kPExp) of the
// reference is a normal e4m3 number.  Random scores of unit spread outgrow a
// slack of 0.5 in about half the tiles of a 32-row wave, 2.5 in about one in
// eight; each rescale is a multiply per accumulator.
constexpr float kPExp = 6.f, kSlack = 2.5f;

struct Fp8Params {
  const uint8_t* Q;
  const uint8_t* K;
  const uint8_t* VT;
  uint16_t* O;
  float* LSE;
  const int* cu_q;  // nullptr: dense batch
  const int* cu_k;
  int total_q, total_k;
  int B, Hq, Hkv, Lq, Lk, vt_stride;  // packed: Lq, Lk are the longest lengths
  int win_left, win_right;
  float scale2;  // |scale * q_descale * k_descale| * log2(e)
  float thr;     // lazy-rescale slack in raw score units
  float oscale;  // v_descale
  uint32_t qxor; // sign flip of q for a negative scale
  int xcd_w;     // work-list window, see xcd_work_item
};

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format code 0 for both operands), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat(u32x4 a, u32x4 b) {
  return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2],
                 (int)b[3]};
}

// Output head dimensions one workgroup owns: all of them up to D = 128; at
// D = 256 two workgroups share a query tile, each forming the full scores and
// probabilities and the P V product for 128 of the output dimensions (so its
// accumulator is the D = 128 one: the 256-wide one does not fit beside the
// operands in a wave's registers).
template <int D> struct Fp8Dv { static constexpr int value = D <= 128 ? D : 128; };

template <int D, typename OT, bool CAUSAL>
__global__ __launch_bounds__(kPT, 2)
void fwd_fp8_kernel(const Fp8Params prm) {
  constexpr int DV = Fp8Dv<D>::value;  // output dimensions of this workgroup
  constexpr int NSPLIT = D / DV;       // workgroups per query tile
  constexpr int KT = kPBN * D;   // bytes per K tile
  constexpr int VTB = DV * kPBN; // bytes per V^T tile
  constexpr int CK = D / 16;     // 16-byte chunks per K row
  constexpr int NK = kPBN * CK / kPT;
  constexpr int NV = DV * 4 / kPT;
  static_assert(NK >= 1 && NV >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t sK0[KT];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[VTB];
  __shared__ __attribute__((aligned(16))) uint8_t sK1[KT];
  __shared__ __attribute__((aligned(16))) uint8_t sV1[VTB];

  const int B = prm.B, Hq = prm.Hq, Hkv = prm.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index, wave-uniform (in an SGPR): so are the bounds derived from
  // it, and the mask test of a tile is a scalar branch
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wu = w;
  const int l32 = lane & 31, hf = lane >> 5;

  const int nqt = (prm.Lq + kPBM - 1) / kPBM;
  // the grid holds NSPLIT copies of the nqt * B * Hq work items, one per
  // range of output dimensions
  const int nitems = nqt * B * Hq;
  const int split = (int)blockIdx.x / nitems;
  const int dv0 = split * DV;
  int b, h, qt;
  xcd_work_item((int)blockIdx.x - split * nitems, B, Hq, nqt, prm.xcd_w, b, h, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
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
    qs = b * prm.Lq, Lq = prm.Lq, ks = 0, Lk = prm.Lk;
  }
  const int q0 = qt * kPBM, qw0 = q0 + kPR * w, qrow = qw0 + l32;
  if (q0 >= Lq) return;  // past this sequence's rows (whole workgroup)
  const int shift = Lk - Lq;
  // Key tiles start at a 16-key aligned column of V^T: a packed sequence
  // whose first key is column ks walks tiles from c0 = ks rounded down to 16,
  // and its keys are counted dlt = ks - c0 further on in tile coordinates
  // (its own keys are dlt .. dlt+Lk-1; the dlt keys before them belong to the
  // previous sequence and are never visible).  Dense batches have dlt = 0.
  const int c0 = prm.cu_q ? (ks & ~15) : 0;
  const int dlt = ks - c0;
  const int LkA = Lk + dlt;  // end of this sequence's keys in tile coordinates
  const int wl = prm.win_left, wr = prm.win_right;
  auto kmin = [&](int i) { return dlt + (wl < 0 ? 0 : max(0, i + shift - wl)); };
  auto kmax = [&](int i) {
    int hi = Lk - 1;
    if (CAUSAL) hi = min(hi, i + shift);
    if (wr >= 0) hi = min(hi, i + shift + wr);
    return dlt + hi;
  };

  const long qstride = (long)Hq * D;
  const int kstride = Hkv * D;
  // dense: K [B, Lk, Hkv, D], V^T [B, Hkv, D, vt_stride]; packed: K [total_k,
  // Hkv, D], V^T [Hkv, D, vt_stride] with key row r of K at column r
  const uint8_t* Kb = prm.cu_q ? prm.K + (long)c0 * kstride + (long)kvh * D
                               : prm.K + (long)b * Lk * kstride + (long)kvh * D;
  const uint8_t* Vb = (prm.cu_q ? prm.VT + (long)kvh * D * (long)prm.vt_stride + c0
                                : prm.VT + ((long)b * Hkv + kvh) * D * (long)prm.vt_stride) +
                     (long)dv0 * prm.vt_stride;  // this workgroup's output dimensions

  // Q^T operand: lane holds query qrow, dims 64m + 32hf .. +31 for MFMA m.
  i32x8 qf[D / 64];
  {
    const uint8_t* qr = prm.Q + ((long)qs + min(qrow, Lq - 1)) * qstride + (long)h * D;
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qr + 64 * m + 32 * hf) ^ prm.qxor;
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qr + 64 * m + 32 * hf + 16) ^ prm.qxor;
      qf[m] = cat(x0, x1);
    }
  }

  const int q_last = min(q0 + kPBM, Lq) - 1;
  const int wg_lo = kmin(q0), wg_hi = kmax(q_last);
  const int t_first = wg_lo / kPBN;
  const int ntiles = wg_hi >= wg_lo ? wg_hi / kPBN - t_first + 1 : 0;
  const int qw_last = min(qw0 + kPR - 1, Lq - 1);
  const bool wave_live = qw0 < Lq && kmax(qw_last) >= kmin(qw0);
  const int first_live = wave_live ? kmin(qw0) / kPBN - t_first : ntiles;
  const int last_live = wave_live ? kmax(qw_last) / kPBN - t_first : -1;
  const int row_kmin = kmin(qrow), row_kmax = kmax(qrow);

  // Loaders: LDS byte position 16 * P holds chunk P of the tile.
  uint32_t koff[NK], voff[NV];
  int krow[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int P = (i * kPW + wu) * 64 + lane;
    const int r = P / CK, pc = P % CK;
    krow[i] = r;
    koff[i] = (uint32_t)(r * kstride + 16 * (pc ^ swz_k8<D>(r)));
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int P = (i * kPW + wu) * 64 + lane;
    const int d = P >> 2, pc = P & 3;
    voff[i] = (uint32_t)(d * prm.vt_stride + 16 * (pc ^ swz_v8(d)));
  }
  // Tiles are requested in order, so the K tile pointer advances by one
  // tile's rows per request.
  const long ktile = (long)kPBN * kstride;
  const uint8_t* kbase = Kb + (long)t_first * ktile;
  auto issue = [&](int t, uint8_t* dK, uint8_t* dV) {
    const int j0 = t * kPBN;
    const bool whole = j0 + kPBN <= LkA;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      uint32_t o = koff[i];
      if (!whole) o -= (uint32_t)(((j0 + krow[i]) - min(j0 + krow[i], LkA - 1)) * kstride);
      load_lds16_buf(kbase, o, dK + (i * kPW + wu) * 1024);
    }
    // V^T columns j0 .. j0+63 lie inside the row: dense, the stride is a
    // multiple of 64 >= Lk; packed, it is >= total_k + 64 and j0 <= dlt + Lk - 1
#pragma unroll
    for (int i = 0; i < NV; ++i) load_lds16_buf(Vb + j0, voff[i], dV + (i * kPW + wu) * 1024);
    kbase += ktile;
  };

  // A-operand rows of the S^T MFMA: lane i reads K row 16((i/4)%2) + 4(i/8) + i%4.
  const int arow = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);

  f32x16 acc[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) acc[i] = (f32x16){};
  float m_ref = -INFINITY, l_part = 0.f;
  const float scale2 = prm.scale2, thr = prm.thr;

  auto compute = [&](int u, const uint8_t* sK, const uint8_t* sV) {
    const int j0 = (t_first + u) * kPBN;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
      const int r = 32 * kb + arow;
#pragma unroll
      for (int m = 0; m < D / 64; ++m) {
        const int c0 = 4 * m + 2 * hf;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sK + r * D + 16 * (c0 ^ swz_k8<D>(r)));
        const u32x4 a1 =
            *reinterpret_cast<const u32x4*>(sK + r * D + 16 * ((c0 + 1) ^ swz_k8<D>(r)));
        s[kb] = mfma_fp8(cat(a0, a1), qf[m], s[kb]);
      }
    }
    // score element r of block kb is key j0 + 32kb + 16hf + r; a tile that
    // some row of the wave does not see whole is masked (a scalar branch,
    // then a select per element)
    if (j0 < kmin(qw_last) || j0 + kPBN - 1 > kmax(qw0)) {
      const int lo = row_kmin - j0 - 16 * hf, hi = row_kmax - j0 - 16 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + r;
          if (off < lo || off > hi) s[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx);
    const bool upd = mx > m_ref + thr;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(upd) != 0, 0)) {
      asm volatile("" ::: "memory");
      const float m_new = upd ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast((m_ref - m_new) * scale2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) acc[i] *= alpha;
      m_ref = m_new;
    }
    // 2^kPExp P (the factor keeps the e4m3 rounding clear of subnormals; it
    // enters the exponent and leaves through the row sum), packed four keys
    // per dword: dword j of the B operand carries keys 16(j/4)... i.e. block
    // j/4, elements 4(j%4)..+3.
    const float mb = ((m_ref == -INFINITY) ? 0.f : m_ref * scale2) - kPExp;
    i32x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = j >> 2, r0 = 4 * (j & 3);
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        p[t] = exp2_fast(__builtin_fmaf(s[kb][r0 + t], scale2, -mb));
        l_part += p[t];
      }
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
      pb[j] = wd;
    }
    // O^T += V^T P^T: A = V^T row d, keys 16hf .. +15 and 32+16hf .. +15
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
      const int d = 32 * db + l32;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(sV + d * kPBN + 16 * (hf ^ swz_v8(d)));
      const u32x4 a1 =
          *reinterpret_cast<const u32x4*>(sV + d * kPBN + 16 * ((2 + hf) ^ swz_v8(d)));
      acc[db] = mfma_fp8(cat(a0, a1), pb, acc[db]);
    }
  };

  if (ntiles > 0) {
    issue(t_first, sK0, sV0);
    for (int u = 0; u < ntiles; u += 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~0x0F00);
      asm volatile("s_barrier" ::: "memory");
      if (u + 1 < ntiles) issue(t_first + u + 1, sK1, sV1);
      if (u >= first_live && u <= last_live) compute(u, sK0, sV0);
      if (u + 1 >= ntiles) break;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~0x0F00);
      asm volatile("s_barrier" ::: "memory");
      if (u + 2 < ntiles) issue(t_first + u + 2, sK0, sV0);
      if (u + 1 >= first_live && u + 1 <= last_live) compute(u + 1, sK1, sV1);
    }
  }

  const float l = sum_halves(l_part);
  const float inv = l > 0.f ? prm.oscale / l : 0.f;
  // O = acc / l staged through LDS (wave w takes one of the four tile arrays,
  // rows [32][D] of 16-bit values with 16-byte chunks XOR-swizzled by row) and
  // written as whole rows with non-temporal stores; lse = ln2 * (m*scale2 +
  // log2 l).
  constexpr int CPR = DV / 8;
  constexpr int OSW = CPR < 16 ? CPR - 1 : 15;
  static_assert(32 * DV * 2 <= KT, "O stage");
  __syncthreads();  // every copy has landed and all waves are done with the tiles
  uint16_t* so = reinterpret_cast<uint16_t*>((w == 0) ? sK0 : (w == 1) ? sV0 : (w == 2) ? sK1 : sV1);
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hf;
      const u32x2 val = {Ops<OT>::pack2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                         Ops<OT>::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(so + l32 * DV + 8 * ((d >> 3) ^ (l32 & OSW)) + (d & 7)) = val;
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int p = lane + 64 * i;
    const int row = p / CPR, c = p % CPR;
    const int q = qw0 + row;
    if (q < Lq)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(so + row * DV + 8 * (c ^ (row & OSW))),
          reinterpret_cast<u32x4*>(prm.O + ((long)qs + q) * qstride + (long)h * D + dv0 + 8 * c));
  }
  if (split == 0 && hf == 0 && qrow < Lq)  // lse: dense [B, Hq, Lq]; packed [Hq, total_q]
    __builtin_nontemporal_store(
        l > 0.f ? (m_ref * scale2 + __builtin_log2f(l) - kPExp) * kLn2 : -INFINITY,
        prm.LSE + (prm.cu_q ? (long)h * prm.total_q + qs + qrow : ((long)b * Hq + h) * Lq + qrow));
}

template <int D, typename OT>
hipError_t launch_fp8_t(const Fp8Args& a, hipStream_t stream) {
  Fp8Params p;
  p.Q = (const uint8_t*)a.q;
  p.K = (const uint8_t*)a.k;
  p.VT = (const uint8_t*)a.vt;
  p.O = (uint16_t*)a.o;
  p.LSE = a.lse;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Lq = a.Lq;
  p.Lk = a.Lk;
  p.vt_stride = a.vt_stride;
  p.win_left = a.win_left;
  p.win_right = a.win_right;
  const float sc = a.scale * a.q_descale * a.k_descale;
  p.scale2 = fmaxf(fabsf(sc) * kLog2e, 1e-30f);
  p.thr = kSlack / p.scale2;
  p.oscale = a.v_descale;
  p.qxor = sc < 0.f ? 0x80808080u : 0u;
  const int nqt = (a.Lq + kPBM - 1) / kPBM;
  // blocks resident per CU at this kernel's register use: 4 (D=64), 3 (D=128)
  p.xcd_w = xcd_window(a.B, a.Hq, a.Hkv, nqt, D == 64 ? 4 : 3);
  const dim3 grid((unsigned)((long)nqt * a.B * a.Hq * (D / Fp8Dv<D>::value)));
  if (a.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, OT, true>), grid, dim3(kPT), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, OT, false>), grid, dim3(kPT), 0, stream, p);
  return hipGetLastError();
}

template <typename OT>
hipError_t launch_fp8_out(const Fp8Args& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_fp8_t<64, OT>(a, stream);
    case 128: return launch_fp8_t<128, OT>(a, stream);
    case 256: return launch_fp8_t<256, OT>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  return a.out_bf16 ? launch_fp8_out<bf16_t>(a, stream) : launch_fp8_out<f16_t>(a, stream);
}

}  // namespace fa
