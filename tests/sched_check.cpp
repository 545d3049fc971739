// Host-side check of the kernels' integer scheduling (csrc/fa_sched.hpp),
// compiled with g++ against the same header the kernels use:
//   * block -> (sequence, head, tile rank) is a bijection onto
//     [0,B) x [0,H) x [0,ntiles) for every grid shape checked (the forward
//     grids and both backward grids use the same map);
//   * forward tile walk: replaying the prefill kernel's phases, every copy
//     the main phase issues without clamping lies whole inside the keys,
//     every tile the main phase computes unmasked is seen whole by every row
//     of the workgroup, and each wave forms S and P.V exactly once for each
//     tile holding keys its rows see, and for no other;
//   * the score exchange of the split waves (D = 256, two waves per row
//     slice, partial scores through a two-buffer LDS exchange): every tile
//     whose scores a wave completes was stored in the buffer of its parity
//     during the step just before (or the prologue) and not overwritten.
// Prints one line per failure and exits non-zero if there is any.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa_sched.hpp"

namespace {

int failures = 0;

#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      if (failures < 50) {                      \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);               \
        std::printf("\n");                      \
      }                                         \
      ++failures;                               \
    }                                           \
  } while (0)

// Grid of nqt * B * Hq forward blocks at the window the launcher picks.
void check_fwd_map(int B, int Hq, int Hkv, int nqt, int bpc) {
  const int W = fa::xcd_window(B, Hq, Hkv, nqt, bpc);
  const long n = (long)nqt * B * Hq;
  std::vector<unsigned char> seen(n, 0);
  for (long blk = 0; blk < n; ++blk) {
    int b = -1, h = -1, r = -1;
    fa::xcd_work_item((int)blk, B, Hq, nqt, W, b, h, r);
    const bool in = b >= 0 && b < B && h >= 0 && h < Hq && r >= 0 && r < nqt;
    CHECK(in, "fwd map B=%d Hq=%d Hkv=%d nqt=%d W=%d: block %ld -> (%d,%d,%d) out of range", B,
          Hq, Hkv, nqt, W, blk, b, h, r);
    if (!in) continue;
    const long idx = ((long)b * Hq + h) * nqt + r;
    CHECK(!seen[idx], "fwd map B=%d Hq=%d Hkv=%d nqt=%d W=%d: (%d,%d,%d) taken twice", B, Hq, Hkv,
          nqt, W, b, h, r);
    seen[idx] = 1;
  }
  // n blocks, each in range and none repeated: all n items are covered.
}

// Replay of the prefill kernel's walk for one workgroup (rows q0 ..
// q0+BM-1 of a sequence) with kNS K/V stages (4 at D = 64 and 128, 2 for the
// split waves at D = 256), mirroring its pipeline step: K(t+NS) and
// V(t+NS-1) are requested at step t (clamped in the masked phases, unclamped
// in the main phase), then S(t+1), P(t) and P(t).V(t) are formed for the
// waves that see those tiles.
constexpr int kBM = 128, kRows = 32, kWaves = 4;

template <int kNS>
void check_walk(int Lq, int Lk, bool causal, int wl, int wr, int BN) {
  const fa::KeyRange kr(Lq, Lk, causal, wl, wr);
  for (int q0 = 0; q0 < Lq; q0 += kBM) {
    const int q_last = fa::imin(q0 + kBM, Lq) - 1;
    const fa::FwdWalk walk(kr, q0, q_last, BN);
    const int nt = walk.ntiles;
    if (nt <= 0) continue;
    // per wave: the tiles holding keys its rows see, and how often S and PV ran
    int first_live[kWaves], last_live[kWaves];
    std::vector<int> s_cnt[kWaves], p_cnt[kWaves];
    // split waves: the tile and the step (-1: prologue) of each exchange
    // buffer's last store
    int buf_tile[kWaves][2], buf_step[kWaves][2];
    for (int w = 0; w < kWaves; ++w) {
      const int qw0 = q0 + kRows * w, qwl = fa::imin(qw0 + kRows - 1, Lq - 1);
      const bool live = qw0 < Lq && kr.kmax(qwl) >= kr.kmin(qw0);
      first_live[w] = live ? kr.kmin(qw0) / BN - walk.t_first : nt;
      last_live[w] = live ? kr.kmax(qwl) / BN - walk.t_first : -1;
      s_cnt[w].assign(nt + 1, 0);
      p_cnt[w].assign(nt + 1, 0);
      for (int x = 0; x < 2; ++x) buf_tile[w][x] = buf_step[w][x] = -100;
      if (first_live[w] == 0 && last_live[w] >= 0) {  // prologue
        s_cnt[w][0]++;
        buf_tile[w][0] = 0, buf_step[w][0] = -1;
      }
    }
    char tag[160];
    std::snprintf(tag, sizeof tag, "walk NS=%d Lq=%d Lk=%d causal=%d win=(%d,%d) BN=%d q0=%d",
                  kNS, Lq, Lk, (int)causal, wl, wr, BN, q0);
    const int tf = walk.t_first;
    auto visible_whole = [&](int u) {  // every row of the workgroup sees tile u whole
      const int j0 = (tf + u) * BN;
      return kr.kmin(q_last) <= j0 && j0 + BN - 1 <= kr.kmax(q0);
    };
    auto step = [&](int t, auto, auto tail_tag) {
      constexpr bool TAIL = decltype(tail_tag)::value;
      if (!TAIL) {
        // unclamped copies: K tile tf+t+NS and V tile tf+t+NS-1, whole inside [0, Lk)
        for (int tile : {tf + t + kNS, tf + t + kNS - 1}) {
          const int j0 = tile * BN;
          CHECK(j0 >= 0 && j0 + BN <= Lk, "%s: main step %d copies tile %d (keys %d..%d), Lk=%d",
                tag, t, tile, j0, j0 + BN - 1, Lk);
        }
        CHECK(visible_whole(t) && visible_whole(t + 1),
              "%s: main step %d computes tiles %d,%d unmasked but they are not whole for every row",
              tag, t, t, t + 1);
      }
      for (int w = 0; w < kWaves; ++w) {
        auto store = [&](int tile) {  // split: partial of `tile` into its parity's buffer
          buf_tile[w][tile & 1] = tile, buf_step[w][tile & 1] = t;
        };
        if (TAIL && (t > last_live[w] || t + 1 < first_live[w])) continue;
        if (TAIL && t + 1 == first_live[w]) {
          s_cnt[w][t + 1]++;
          store(t + 1);
          continue;
        }
        const bool next = !TAIL || t + 1 <= last_live[w];
        // (waves whose rows all lie past the sequence run the main phase on
        // whatever the buffer holds; their rows are never stored)
        CHECK(q0 + kRows * w >= Lq || (buf_tile[w][t & 1] == t && buf_step[w][t & 1] == t - 1),
              "%s wave %d: split scores of tile %d completed at step %d from a buffer holding "
              "tile %d stored at step %d", tag, w, t, t, buf_tile[w][t & 1], buf_step[w][t & 1]);
        if (next) {
          s_cnt[w][t + 1]++;
          store(t + 1);
        }
        p_cnt[w][t]++;
      }
    };
    fa::fwd_walk<kNS>(walk, step, [](int) {});
    for (int w = 0; w < kWaves; ++w) {
      const int qw0 = q0 + kRows * w;
      if (qw0 >= Lq) continue;  // rows past the sequence are never stored
      for (int u = 0; u < nt; ++u) {
        const bool live = u >= first_live[w] && u <= last_live[w];
        CHECK(s_cnt[w][u] == (live ? 1 : 0), "%s wave %d: S of tile %d formed %d times (live %d)",
              tag, w, u, s_cnt[w][u], (int)live);
        CHECK(p_cnt[w][u] == (live ? 1 : 0), "%s wave %d: P.V of tile %d formed %d times (live %d)",
              tag, w, u, p_cnt[w][u], (int)live);
      }
      CHECK(s_cnt[w][nt] == 0 && p_cnt[w][nt] == 0, "%s wave %d: work past the last tile", tag, w);
    }
  }
}

}  // namespace

int main() {
  // forward grids: the benchmark workloads, then a sweep of head counts
  struct Fwd { int B, Hq, Hkv, L; };
  const Fwd fwd_cfgs[] = {{1, 2, 2, 128},     {4, 32, 32, 4096}, {1, 32, 8, 16384},
                          {2, 16, 16, 4096},  {64, 12, 12, 512}, {2, 32, 8, 16384},
                          {16, 32, 8, 4096},  {1, 128, 16, 147456}, {2, 128, 128, 131072}};
  for (const Fwd& c : fwd_cfgs)
    for (int bpc = 1; bpc <= 4; ++bpc) check_fwd_map(c.B, c.Hq, c.Hkv, (c.L + kBM - 1) / kBM, bpc);
  const int hqs[] = {1, 2, 3, 8, 12, 16, 24, 32, 40, 64, 128};
  for (int Hq : hqs)
    for (int Hkv = 1; Hkv <= Hq; ++Hkv) {
      if (Hq % Hkv) continue;
      for (int B : {1, 2, 3, 4, 7, 16})
        for (int nqt : {1, 2, 3, 5, 32, 128})
          for (int bpc = 1; bpc <= 4; ++bpc) check_fwd_map(B, Hq, Hkv, nqt, bpc);
    }
  // backward grids: dq over (query head, query tile), dkdv over (K/V head,
  // key tile) with one workgroup per CU
  for (int H : {1, 2, 3, 4, 5, 8, 12, 16, 32, 40, 64, 128})
    for (int B : {1, 2, 3, 4, 7, 16, 64})
      for (int nt : {1, 2, 3, 16, 32, 128}) check_fwd_map(B, H, H, nt, 1);
  // forward tile walk
  const int lens[] = {1, 17, 31, 32, 33, 63, 64, 65, 96, 100, 127, 128, 129, 160, 200, 300,
                      331, 1000, 1025};
  const int wins[][2] = {{-1, -1}, {0, 0}, {5, 3}, {64, -1}, {-1, 40}, {127, 0}, {300, 300},
                         {31, 0}, {32, 32}, {4095, 0}};
  for (int Lq : lens)
    for (int Lk : lens)
      for (int causal = 0; causal < 2; ++causal)
        for (const auto& w : wins) {
          check_walk<2>(Lq, Lk, causal != 0, w[0], w[1], 32);
          check_walk<4>(Lq, Lk, causal != 0, w[0], w[1], 32);
        }
  for (int causal = 0; causal < 2; ++causal) {
    check_walk<2>(4096, 4096, causal != 0, -1, -1, 32);
    check_walk<4>(4096, 4096, causal != 0, -1, -1, 32);
    check_walk<2>(16384, 16384, causal != 0, 4095, 0, 32);
    check_walk<4>(16384, 16384, causal != 0, 4095, 0, 32);
    check_walk<2>(1, 4096, causal != 0, -1, -1, 32);
    check_walk<4>(1, 4096, causal != 0, -1, -1, 32);
    check_walk<2>(129, 4097, causal != 0, -1, -1, 32);
    check_walk<4>(129, 4097, causal != 0, -1, -1, 32);
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("scheduling checks passed\n");
  return 0;
}
