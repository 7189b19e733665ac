// Host-side exhaustive check of the chunked HGRN2 kernel's LDS address forms: every factored form in
// h2_layout.hpp equals the direct layout function (qk_off / vw_off / gv_off) over all of its lane
// and loop indices, and each layout maps its tile one-to-one into the tile's storage.  Built with hipcc and run on the CPU (no GPU call).
#include <hip/hip_runtime.h>
#include <cstdio>
#include "h2_layout.hpp"
using namespace ssd::h2;
int main() {
  long n = 0, bad = 0;
  for (int l16 = 0; l16 < 16; ++l16)
    for (int lg = 0; lg < 4; ++lg) {
      const int b = l16 >> 2, c = l16 & 3;
      for (int a = 0; a < 4; ++a)
        for (int ks = 0; ks < 4; ++ks) {
          ++n; if (qk_seg_off(l16, qk_seg_lane(l16, lg), a, ks) != qk_off(16 * a + l16, 32 * ks + 8 * lg)) ++bad;
          for (int h = 0; h < 2; ++h) {
            ++n; if (qk_quad_off(l16, lg, qk_quad_lane(l16, lg), a, ks, h) != qk_off(16 * a + l16, 32 * ks + 16 * h + 4 * lg)) ++bad;
          }
        }
      for (int ks = 0; ks < 2; ++ks)
        for (int h = 0; h < 2; ++h)
          for (int jt = 0; jt < 8; ++jt) {
            ++n; if (qk_tr_off(l16, lg, qk_tr_lane(l16, lg), ks, h, jt) != qk_off(32 * ks + 8 * lg + b + 4 * h, 16 * jt + 4 * c)) ++bad;
          }
      for (int rt = 0; rt < 4; ++rt)
        for (int ks = 0; ks < 2; ++ks)
          for (int h = 0; h < 2; ++h) {
            ++n; if (vw_out_off(vw_out_lane(l16, lg, rt), ks, h) != vw_off(32 * ks + 16 * h + 4 * lg + b, 16 * rt + 4 * c)) ++bad;
            ++n; if (vw_state_off(vw_state_lane(l16, lg, rt, h), ks) != vw_off(32 * ks + 8 * lg + b + 4 * h, 16 * rt + 4 * c)) ++bad;
          }
      for (int gp = 0; gp < 8; ++gp)
        for (int h = 0; h < 2; ++h) {
          ++n; if (gv_gate_off(l16, lg, gp, h) != gv_off(8 * gp + b + 4 * h, 16 * lg + 4 * c)) ++bad;
        }
    }
  for (int gi = 0; gi < 64; ++gi)
    for (int gp = 0; gp < 8; ++gp)
      for (int u = 0; u < 8; ++u) {
        ++n; if (vw_gate_wr(gi, vw_gate_lane(gi, gp), gp, u) != vw_off(8 * gp + u, gi)) ++bad;
      }
  // each layout is a bijection of its tile's elements into the tile's storage
  {
    static unsigned char seen[kQkTile];
    for (int r = 0; r < 64; ++r)
      for (int c = 0; c < kQkCols; ++c) {
        const int o = qk_off(r, c);
        ++n; if (o < 0 || o >= kQkTile || seen[o]++) ++bad;
      }
    static unsigned char seen_vw[64 * kVwCols], seen_gv[64 * kVwCols];
    for (int r = 0; r < 64; ++r)
      for (int c = 0; c < kVwCols; ++c) {
        const int o = vw_off(r, c), g = gv_off(r, c);
        ++n; if (o < 0 || o >= 64 * kVwCols || seen_vw[o]++) ++bad;
        ++n; if (g < 0 || g >= 64 * kVwCols || seen_gv[g]++) ++bad;
      }
  }
  printf("%ld cases, %ld mismatches\n", n, bad);
  return bad != 0;
}
