// Host-side check of the kernels' LDS layouts (csrc/fa_lds.hpp): every tile
// access the decode, backward and FP8 kernels make is replayed lane by lane
// with the kernels' own XOR functions and scored in the bank model the header
// states (64 banks of 4 bytes; an access served 256 bytes at a time: 16 lanes
// of a 16-byte access, 32 of an 8-byte one, 64 of a 4-byte one).  Every
// access must be free of bank conflicts, except the one the decode kernel
// documents (the widened int8 V stores at D = 256, two-way).  Every XOR must
// be a bijection on its row's chunk indices.
//
// With the argument "old" the pre-fix XORs are checked instead, and the run
// must report conflicts (so the check sees what it claims to).
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <set>
#include <vector>

#include "fa_lds.hpp"

namespace {

int failures = 0;
#define CHECK(cond, ...)          \
  do {                            \
    if (!(cond)) {                \
      std::printf(__VA_ARGS__);   \
      std::printf("\n");          \
      ++failures;                 \
    }                             \
  } while (0)

// Largest number of distinct 4-byte words that one bank serves within one
// 256-byte group of lanes; addrs are byte addresses of the 64 lanes.
int degree(const std::vector<long>& addrs, int width) {
  const int glen = 256 / width;
  int worst = 1;
  for (int g0 = 0; g0 < 64; g0 += glen) {
    std::map<int, std::set<long>> banks;
    for (int l = g0; l < g0 + glen; ++l)
      for (int k = 0; k < width / 4; ++k) {
        const long w = addrs[l] / 4 + k;
        banks[(int)(w % 64)].insert(w);
      }
    for (auto& b : banks) worst = b.second.size() > (size_t)worst ? (int)b.second.size() : worst;
  }
  return worst;
}

void bijection(const char* what, int n, const std::function<int(int)>& f) {
  for (int r = 0; r < 256; ++r) {
    std::vector<int> seen(n, 0);
    for (int c = 0; c < n; ++c) {
      const int p = c ^ f(r);
      CHECK(p >= 0 && p < n && !seen[p], "%s: row %d, chunk %d -> %d not one-to-one", what, r, c, p);
      if (p >= 0 && p < n) seen[p] = 1;
    }
  }
}

struct Xors {
  std::function<int(int, int)> row;      // decode K tile / merge rows: (chunks per row, row)
  std::function<int(int, int)> dv;       // decode V tile: (D, row)
  std::function<int(int, int)> b;        // backward tiles: (D, row)
  std::function<int(int, int)> k8;       // FP8 K tile: (D, row)
  std::function<int(int)> v8;            // FP8 V^T tile: (row)
};

int d_row(int N, int r) {
  switch (N) {
    case 4: return fa::row_xor<4>(r);
    case 8: return fa::row_xor<8>(r);
    case 16: return fa::row_xor<16>(r);
    default: return fa::row_xor<32>(r);
  }
}
int d_dv(int D, int r) { return D == 64 ? fa::swz_dv<64>(r) : D == 128 ? fa::swz_dv<128>(r) : fa::swz_dv<256>(r); }
int d_b(int D, int r) { return D == 64 ? fa::swz_b<64>(r) : D == 128 ? fa::swz_b<128>(r) : fa::swz_b<256>(r); }
int d_k8(int D, int r) { return D == 64 ? fa::swz_k8<64>(r) : D == 128 ? fa::swz_k8<128>(r) : fa::swz_k8<256>(r); }

// The layouts before the bank model was applied.
Xors old_xors() {
  Xors x;
  x.row = [](int N, int r) { return r & ((N < 16 ? N : 16) - 1); };
  x.dv = [](int D, int r) { return D == 64 ? 2 * ((r >> 1) & 3) : 2 * (r & 7); };
  x.b = [](int D, int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); };
  x.k8 = [](int D, int r) { return D >= 128 ? ((r & 3) | (((r >> 4) & 1) << 2)) : (r & 3); };
  x.v8 = [](int d) { return (d >> 1) & 3; };
  return x;
}
Xors cur_xors() { return {d_row, d_dv, d_b, d_k8, fa::swz_v8}; }

// Decode split kernel, one format: 16-key tiles of K (16-bit or int8 codes)
// and V (16-bit, int8 codes widened on the way in), and the wave merge.
void check_decode(const Xors& x, int D, bool ki8, bool vi8) {
  const int KEB = ki8 ? 1 : 2, KLPR = D * KEB / 16, NKL = 16 * KLPR / 64;
  char tag[64];
  std::snprintf(tag, sizeof tag, "decode D=%d K%d V%d", D, ki8 ? 8 : 16, vi8 ? 8 : 16);
  std::vector<long> a(64);
  for (int i = 0; i < NKL; ++i) {  // K tile stores, 16 bytes
    for (int l = 0; l < 64; ++l) {
      const int P = 64 * i + l, r = P / KLPR, c = P % KLPR;
      a[l] = 16L * (r * KLPR + (c ^ x.row(KLPR, r)));
    }
    CHECK(degree(a, 16) == 1, "%s: K store %d conflicts %d-way", tag, i, degree(a, 16));
  }
  for (int ks = 0; ks < D / 32; ++ks) {  // K operand reads
    for (int l = 0; l < 64; ++l) {
      const int l16 = l & 15, q4 = l >> 4;
      a[l] = ki8 ? 16L * (l16 * KLPR + ((2 * ks + (q4 >> 1)) ^ x.row(KLPR, l16))) + 8 * (q4 & 1)
                 : 16L * (l16 * KLPR + ((4 * ks + q4) ^ x.row(KLPR, l16)));
    }
    const int dg = degree(a, ki8 ? 8 : 16);
    CHECK(dg == 1, "%s: K read %d conflicts %d-way", tag, ks, dg);
  }
  const int VLPR = vi8 ? D / 16 : D / 8, NVL = 16 * VLPR / 64;
  for (int i = 0; i < NVL; ++i)
    for (int part = 0; part < (vi8 ? 2 : 1); ++part) {  // V tile stores
      for (int l = 0; l < 64; ++l) {
        const int P = 64 * i + l, r = P / VLPR, c = P % VLPR;
        const int ch = vi8 ? ((2 * c + part) ^ x.dv(D, r)) : (c ^ x.dv(D, r));
        a[l] = 2L * (r * D + 8 * ch);
      }
      const int dg = degree(a, 16), want = (vi8 && D == 256) ? 2 : 1;
      CHECK(dg <= want, "%s: V store %d.%d conflicts %d-way", tag, i, part, dg);
    }
  for (int db = 0; db < D / 16; ++db) {  // V^T transpose reads
    for (int l = 0; l < 64; ++l) {
      const int l16 = l & 15, q4 = l >> 4, vr = 4 * q4 + (l16 >> 2), col = 16 * db + 4 * (l16 & 3);
      a[l] = 2L * (vr * D + 8 * ((col >> 3) ^ x.dv(D, vr)) + (col & 7));
    }
    CHECK(degree(a, 8) == 1, "%s: V read %d conflicts %d-way", tag, db, degree(a, 8));
  }
  const int DP = D / 2, CH = DP / 4;
  for (int db = 0; db < DP / 16; ++db) {  // merge stores (f32x4)
    for (int l = 0; l < 64; ++l) {
      const int l16 = l & 15, q4 = l >> 4;
      a[l] = 4L * (l16 * DP + 4 * ((4 * db + q4) ^ x.row(CH, l16)));
    }
    CHECK(degree(a, 16) == 1, "%s: merge store %d conflicts %d-way", tag, db, degree(a, 16));
  }
  for (int e0 = 0; e0 < 16 * DP; e0 += 64) {  // merge reads (one float per thread)
    for (int l = 0; l < 64; ++l) {
      const int e = e0 + l, hs = e / DP, d = e % DP;
      a[l] = 4L * (hs * DP + 4 * ((d >> 2) ^ x.row(CH, hs)) + (d & 3));
    }
    CHECK(degree(a, 4) == 1, "%s: merge read %d conflicts %d-way", tag, e0, degree(a, 4));
  }
}

// Backward tiles [32][D]: row reads of 16-byte chunks and transpose reads.
void check_bwd(const Xors& x, int D) {
  std::vector<long> a(64);
  for (int kk = 0; kk < D / 16; ++kk) {
    for (int l = 0; l < 64; ++l) {
      const int l32 = l & 31, hf = l >> 5;
      a[l] = 2L * (l32 * D + 8 * ((2 * kk + hf) ^ x.b(D, l32)));
    }
    CHECK(degree(a, 16) == 1, "bwd D=%d: row read %d conflicts %d-way", D, kk, degree(a, 16));
  }
  for (int half = 0; half < 2; ++half)
    for (int db = 0; db < D / 32; ++db) {
      for (int l = 0; l < 64; ++l) {
        const int hf = l >> 5, row = 8 * half + 4 * hf + ((l & 15) >> 2);
        const int col = 32 * db + 16 * ((l >> 4) & 1) + 4 * (l & 3);
        a[l] = 2L * (row * D + 8 * ((col >> 3) ^ x.b(D, row)) + (col & 7));
      }
      CHECK(degree(a, 8) == 1, "bwd D=%d: transpose read %d.%d conflicts %d-way", D, half, db,
            degree(a, 8));
    }
}

// FP8 forward: K A-operand reads (two 16-byte reads per MFMA) and V^T reads.
void check_fp8(const Xors& x, int D) {
  std::vector<long> a(64);
  for (int kb = 0; kb < 2; ++kb)
    for (int m = 0; m < D / 64; ++m)
      for (int h = 0; h < 2; ++h) {
        for (int l = 0; l < 64; ++l) {
          const int l32 = l & 31, hf = l >> 5;
          const int r = 32 * kb + 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
          a[l] = (long)r * D + 16 * ((4 * m + 2 * hf + h) ^ x.k8(D, r));
        }
        CHECK(degree(a, 16) == 1, "fp8 D=%d: K read %d.%d.%d conflicts %d-way", D, kb, m, h,
              degree(a, 16));
      }
  const int DV = D <= 128 ? D : 128;
  for (int db = 0; db < DV / 32; ++db)
    for (int h = 0; h < 2; ++h) {
      for (int l = 0; l < 64; ++l) {
        const int l32 = l & 31, hf = l >> 5, d = 32 * db + l32;
        a[l] = (long)d * 64 + 16 * ((2 * h + hf) ^ x.v8(d));
      }
      CHECK(degree(a, 16) == 1, "fp8 D=%d: V read %d.%d conflicts %d-way", D, db, h, degree(a, 16));
    }
}

}  // namespace

int main(int argc, char** argv) {
  const bool old = argc > 1 && std::strcmp(argv[1], "old") == 0;
  const Xors x = old ? old_xors() : cur_xors();
  for (int D : {64, 128, 256}) {
    check_decode(x, D, false, false);
    check_decode(x, D, true, false);
    check_decode(x, D, true, true);
    check_bwd(x, D);
    check_fp8(x, D);
    char t[64];
    for (int N : {4, 8, 16, 32}) {
      std::snprintf(t, sizeof t, "row_xor<%d>", N);
      bijection(t, N, [&](int r) { return x.row(N, r); });
    }
    std::snprintf(t, sizeof t, "swz_dv<%d>", D);
    bijection(t, D / 8, [&](int r) { return x.dv(D, r); });
    std::snprintf(t, sizeof t, "swz_b<%d>", D);
    bijection(t, D / 8, [&](int r) { return x.b(D, r); });
    std::snprintf(t, sizeof t, "swz_k8<%d>", D);
    bijection(t, D / 16, [&](int r) { return x.k8(D, r); });
  }
  bijection("swz_v8", 4, x.v8);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("LDS layout checks passed\n");
  return 0;
}
