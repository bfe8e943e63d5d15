// Host check of the K/V ring placement: for many (B, H, M, L) and every ring
// start a step can see, each segment token (b, p), head and column d must land
// in K at [b][head][slot][d] and in V^T at [b][slot/32][head][d][slot%32] with
// slot = (start + Mk + p) mod C, through the output maps the projection GEMM
// uses (row map + column map + second column map).  Exit status 0 = pass.
#include <cstdio>
#include <cstdint>
#include "txl_internal.h"

using namespace txl;

static int64_t rm(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int main() {
  const int DP = 64;
  long checked = 0;
  const int shapes[][4] = {{1, 1, 0, 32},   {2, 3, 40, 32},  {2, 2, 70, 64},  {3, 2, 150, 64},
                           {2, 1, 20, 64},  {1, 2, 1600, 128}, {2, 1, 3800, 128}, {1, 1, 31, 96},
                           {4, 2, 96, 32},  {1, 3, 5, 160}};
  for (const auto& sh : shapes) {
    const int B = sh[0], H = sh[1], M = sh[2], L = sh[3];
    const int Mk = (int)rm(M, 32), C = Mk + L;
    // initial projection: tokens b*Mk + r (G zero rows, then the memory) to slots r
    if (Mk > 0) {
      const RingMaps m = ring_maps(H, DP, C, Mk, 0);
      for (int b = 0; b < B; ++b)
        for (int r = 0; r < Mk; ++r)
          for (int head = 0; head < H; ++head) {
            const int tok = b * Mk + r, col = head * DP + 5;
            const int64_t k_got = m.k_base + axis_offset(m.k_row, tok) + axis_offset(m.k_col, col);
            const int64_t v_got = m.v_base + axis_offset(m.v_row, col) +
                                  axis_offset(m.v_col, tok) + axis_offset(m.v_col2, tok);
            const int64_t k_want = (((int64_t)b * H + head) * C + r) * DP + 5;
            const int64_t v_want = ((((int64_t)b * (C / 32) + r / 32) * H + head) * DP + 5) * 32 + r % 32;
            ++checked;
            if (k_got != k_want || v_got != v_want) {
              std::printf("FAIL init B=%d H=%d M=%d L=%d b=%d r=%d\n", B, H, M, L, b, r);
              return 1;
            }
          }
    }
    for (int start = 0; start < C; start += 32) {
      const int base = (start + Mk) % C;
      const int n1 = ring_first_piece(start, Mk, L, C);
      if (n1 < 1 || n1 > L || n1 % 32) { std::printf("FAIL piece %d\n", n1); return 1; }
      for (int piece = 0; piece < 2; ++piece) {
        const int n = piece == 0 ? n1 : L - n1;
        const int slot0 = piece == 0 ? base : 0;
        const int p0 = piece == 0 ? 0 : n1;
        if (n == 0) continue;
        if (slot0 % 32 || slot0 + n > C) { std::printf("FAIL slot0 %d\n", slot0); return 1; }
        const RingMaps m = ring_maps(H, DP, C, n, slot0);
        for (int b = 0; b < B; ++b)
          for (int r = 0; r < n; ++r) {
            const int p = p0 + r;
            const int slot = (start + Mk + p) % C;
            const int tok = b * n + r;
            for (int head = 0; head < H; ++head)
              for (int d = 0; d < DP; d += 7) {
                const int col = head * DP + d;
                const int64_t k_got = m.k_base + axis_offset(m.k_row, tok) + axis_offset(m.k_col, col);
                const int64_t k_want = (((int64_t)b * H + head) * C + slot) * DP + d;
                const int64_t v_got = m.v_base + axis_offset(m.v_row, col) +
                                      axis_offset(m.v_col, tok) + axis_offset(m.v_col2, tok);
                const int64_t v_want =
                    ((((int64_t)b * (C / 32) + slot / 32) * H + head) * DP + d) * 32 + slot % 32;
                ++checked;
                if (k_got != k_want || v_got != v_want) {
                  std::printf("FAIL B=%d H=%d M=%d L=%d start=%d b=%d p=%d head=%d d=%d "
                              "k %lld/%lld v %lld/%lld\n", B, H, M, L, start, b, p, head, d,
                              (long long)k_got, (long long)k_want, (long long)v_got,
                              (long long)v_want);
                  return 1;
                }
              }
          }
      }
    }
  }
  std::printf("ok %ld checks\n", checked);
  return 0;
}
