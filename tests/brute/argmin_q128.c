/* Brute-force nearest-grid search in binary128, used to pin the oracle's NVFP4 encoder.
 *
 * For every weight, all 16 E2M1 codes are tried: the candidate value is S * grid[c & 7] with the sign of bit 3, and
 * the distance |w - candidate| is evaluated in __float128 (113-bit significand). The grid comes from the caller
 * (the values the pages print), S per 16-weight block comes from the caller as a double (s_g * s_b, exact).
 *
 * Among codes at the minimal distance: prefer the magnitude index with mantissa bit 0 (round half to even), and
 * between +0 and -0 (both at distance |w|) prefer the sign of w. Non-finite weights get 0xff (not compared).
 */
#include <stdint.h>
#include <string.h>

static __float128 q_abs(__float128 v) { return v < 0 ? -v : v; }

void brute_codes(const uint16_t* w, int64_t n, int64_t k, const double* S_blocks, const double* grid, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      uint16_t b = w[i * k + j];
      if (((b >> 7) & 0xff) == 0xff) { out[i * k + j] = 0xff; continue; }
      uint32_t u = (uint32_t)b << 16;
      float f;
      memcpy(&f, &u, 4);
      int wneg = (b >> 15) & 1;
      __float128 wq = (__float128)f;
      __float128 S = (__float128)S_blocks[i * (k / 16) + j / 16];
      int best = -1;
      __float128 best_d = 0;
      for (int c = 0; c < 16; ++c) {
        __float128 v = S * (__float128)grid[c & 7];
        if (c & 8) v = -v;
        __float128 d = q_abs(wq - v);
        int better;
        if (best < 0 || d < best_d) {
          better = 1;
        } else if (d == best_d) {
          int mag = c & 7, bmag = best & 7;
          if (mag == bmag) {
            better = ((c >> 3) == wneg) && ((best >> 3) != wneg); /* same magnitude (only 0 or S==0): sign of w */
          } else {
            better = ((mag & 1) == 0) && ((bmag & 1) == 1);       /* tie between neighbours: even mantissa */
            if (S == 0) better = (mag < bmag);                     /* all candidates equal: magnitude 0 */
          }
        } else {
          better = 0;
        }
        if (better) { best = c; best_d = d; }
      }
      out[i * k + j] = (uint8_t)best;
    }
}
