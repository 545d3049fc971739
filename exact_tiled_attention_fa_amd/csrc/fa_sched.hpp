// Integer work scheduling of the attention kernels: which workgroup takes
// which (sequence, head, tile), and the order in which the prefill kernel
// walks its key tiles.  Plain integer code with no HIP dependency, so the
// same functions run in the kernels and in host-side checks of their
// properties (every work item taken exactly once, every unclamped tile copy
// inside the keys).
#pragma once

#include <type_traits>

#if defined(__HIP__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

FA_HD inline int imin(int a, int b) { return a < b ? a : b; }
FA_HD inline int imax(int a, int b) { return a > b ? a : b; }

constexpr int kXcds = 8;  // gfx950: workgroup i runs on XCD i % 8, each with its own L2

// Window W of xcd_work_item: the smallest multiple of gx = gcd(Hq/Hkv, Hq/8)
// that divides the B*Hq/8 rows of an XCD and spans at least twice the blocks
// the XCD holds at once (32 CUs x blocks_per_cu), so that each window's heavy
// ranks start early; the whole row list if none does.  1 when Hq is not a
// multiple of 8 (unused there).
inline int xcd_window(int B, int Hq, int Hkv, int nqt, int blocks_per_cu) {
  if (Hq % kXcds != 0) return 1;
  const int hx = Hq / kXcds, rows = B * hx;
  int gx = Hq / Hkv, m = hx;  // gcd
  while (m != 0) {
    const int t = gx % m;
    gx = m;
    m = t;
  }
  const int want = (2 * 32 * blocks_per_cu + nqt - 1) / nqt;
  for (int w = gx; w < rows; w += gx)
    if (w >= want && rows % w == 0) return w;
  return rows;
}

// Block -> (sequence b, head h, tile rank) over a grid of nqt * B * Hq
// blocks: the forward kernels' (query head, query tile), the backward dq
// kernel's (query head, query tile) and its dkdv kernel's (K/V head, key
// tile).  Blocks are dealt to the 8
// XCDs round-robin and start in index order.  When Hq is a multiple of 8,
// XCD x takes query heads [x*Hq/8, (x+1)*Hq/8) of every sequence, which
// balances the XCDs even when packed sequences differ in length.  Its rows
// (sequence, head) are walked in windows of W adjacent rows, rank-major
// within a window (rank 0 of each row, then rank 1, ...): the heavy ranks of
// every window start together and the grid ends on light blocks, while the
// few rows of a window keep the tiles they stream in L2.  W (from
// xcd_window) is a multiple of gcd(Hq/Hkv, Hq/8), so the heads reading one
// K/V head run side by side.  Otherwise XCD x takes the x-th contiguous slice
// of the (sequence, head, rank) list.  The caller maps rank to a tile.
FA_HD inline void xcd_work_item(int block, int B, int Hq, int nqt, int W, int& b, int& h,
                                int& rank) {
  const int xcd = block % kXcds, slot = block / kXcds;
  if (Hq % kXcds == 0) {
    const int hx = Hq / kXcds, rows = B * hx;
    const int wi = slot / (W * nqt);
    const int w0 = wi * W, wn = imin(W, rows - w0);
    const int r = slot - wi * W * nqt;
    rank = r / wn;
    const int row = w0 + (r - rank * wn);
    b = row / hx;
    h = xcd * hx + (row - b * hx);
  } else {
    const int N = nqt * B * Hq;
    const int item = xcd * (N / kXcds) + imin(xcd, N % kXcds) + slot;
    const int bhi = item / nqt;
    rank = item - bhi * nqt;
    b = bhi / Hq;
    h = bhi - b * Hq;
  }
}

// Keys a query row may see, [kmin(i), kmax(i)], both non-decreasing in i:
// causal (bottom-right aligned: row i of Lq sees keys j <= i + Lk - Lq), a
// sliding window (left, right) measured from the same diagonal (a negative
// side is unbounded), and the key count.
struct KeyRange {
  int Lk, shift, wl, wr;
  bool causal;
  FA_HD KeyRange(int Lq_, int Lk_, bool causal_, int wl_, int wr_)
      : Lk(Lk_), shift(Lk_ - Lq_), wl(wl_), wr(wr_), causal(causal_) {}
  FA_HD int kmin(int i) const { return wl < 0 ? 0 : imax(0, i + shift - wl); }
  FA_HD int kmax(int i) const {
    int hi = Lk - 1;
    if (causal) hi = imin(hi, i + shift);
    if (wr >= 0) hi = imin(hi, i + shift + wr);
    return hi;
  }
};

// The prefill workgroup's key tiles (BN keys each) for query rows
// [q0, q_last]: tiles t_first .. t_first + ntiles - 1 hold every key some row
// sees (u = t - t_first indexes them), and relative tiles [m_lo, m_hi) are
// seen whole by every row.
struct FwdWalk {
  int BN, Lk, t_first, ntiles, m_lo, m_hi;
  FA_HD FwdWalk(const KeyRange& kr, int q0, int q_last, int BN_) : BN(BN_), Lk(kr.Lk) {
    const int lo = kr.kmin(q0), hi = kr.kmax(q_last);
    t_first = lo / BN;
    ntiles = hi >= lo ? hi / BN - t_first + 1 : 0;
    m_lo = imax(0, (kr.kmin(q_last) + BN - 1) / BN - t_first);
    m_hi = imin(ntiles, (kr.kmax(q0) + 1) / BN - t_first);
  }
  // A main-phase group of NS steps starting at relative tile t computes S of
  // tiles t+1 .. t+NS and P of tiles t .. t+NS-1 with no mask, so those must
  // be whole for every row; its copies K(t+NS .. t+2NS-1) and
  // V(t+NS-1 .. t+2NS-2) are not clamped, so they must lie whole inside the
  // keys.  (The V copies stay below K(t+2NS-1).)
  template <int NS> FA_HD bool main_ok(int t) const {
    return t >= m_lo && t + NS < m_hi && (t_first + t + 2 * NS) * BN <= Lk;
  }
};

// The prefill kernel's walk over its tiles in three phases: a masked head
// phase (tiles left of some row's window), the unmasked main phase, and a
// masked tail phase (the diagonal, a window's right edge, the ragged last
// tile).  Every phase walks NS tiles at a time from t = 0, so stages and
// score buffers are in the same roles at every loop head.
// step(t, integral_constant<int, stage>, integral_constant<bool, tail>) runs
// one pipeline step; enter_main(t) runs once before the main phase.
template <int NS, class Step, class EnterMain>
FA_HD inline void fwd_walk(const FwdWalk& w, Step&& step, EnterMain&& enter_main) {
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2 % NS>;
  using S3 = std::integral_constant<int, 3 % NS>;
  using Main = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  const int ntiles = w.ntiles;
  int t = 0;
  // Head phase: running out of tiles here ends the walk (t = ntiles skips
  // the later phases).
  const int m_lo_al = (w.m_lo + NS - 1) / NS * NS;
  while (t < m_lo_al && t < ntiles) {
    step(t, S0{}, Tail{});
    if (t + 1 >= ntiles) { t = ntiles; break; }
    step(t + 1, S1{}, Tail{});
    if constexpr (NS > 2) {
      if (t + 2 >= ntiles) { t = ntiles; break; }
      step(t + 2, S2{}, Tail{});
      if (t + 3 >= ntiles) { t = ntiles; break; }
      step(t + 3, S3{}, Tail{});
    }
    t += NS;
  }
  enter_main(t);
  while (w.template main_ok<NS>(t)) {
    step(t, S0{}, Main{});
    step(t + 1, S1{}, Main{});
    if constexpr (NS > 2) {
      step(t + 2, S2{}, Main{});
      step(t + 3, S3{}, Main{});
    }
    t += NS;
  }
  while (t < ntiles) {
    step(t, S0{}, Tail{});
    if (t + 1 >= ntiles) break;
    step(t + 1, S1{}, Tail{});
    if constexpr (NS > 2) {
      if (t + 2 >= ntiles) break;
      step(t + 2, S2{}, Tail{});
      if (t + 3 >= ntiles) break;
      step(t + 3, S3{}, Tail{});
    }
    t += NS;
  }
}

}  // namespace fa
