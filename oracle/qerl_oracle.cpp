// Reference oracle for the QeRL rollout-decode linear layer: NVFP4 weights, bf16 LoRA, AQN-RMSNorm.
//
// TEST INFRASTRUCTURE ONLY. This file is a plain, slow, single-threaded CPU model of what the HIP library
// computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load it; the product
// path never calls it and shares no code, header, table or constant with it.
//
// Sources (cited by page title and section; the pages are web text about the QeRL paper, arXiv 2510.11696):
//   [review]  "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops"
//             (Zhongzhu Zhou, English technical review, zhongzhuzhou.org)
//   [notes]   "QeRL 阅读笔记" (the same author's Chinese reading notes; near-parallel text)
//
// Arithmetic is fp64 unless a step decides an integer (an E4M3 scale code), where the pages fix no precision
// and the step is defined in IEEE f32 so that the GPU library can take the same decision in the same precision.
// Build: g++ -std=c++17 -O2 -ffp-contract=off (no fast-math), so every f32/f64 operation is a single IEEE op.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>

namespace {

// ---------------------------------------------------------------------------------------------------------------
// Number formats.

// bf16: the upper 16 bits of an IEEE binary32.
double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Round a finite double to a binary format with `p` significand bits and minimum normal exponent `emin`
// (values below 2^emin are rounded on the subnormal grid 2^(emin-p+1)). Round-to-nearest, ties-to-even.
// No upper exponent bound is applied here; callers handle overflow. This is the textbook definition:
// scale by the quantum, round to an integer with rint (current mode = nearest-even), scale back.
double round_to_format(double v, int p, int emin) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  int e;
  std::frexp(std::fabs(v), &e);  // |v| = f * 2^e, f in [0.5, 1)  =>  floor(log2|v|) = e - 1
  int ex = e - 1;
  if (ex < emin) ex = emin;
  double quantum = std::ldexp(1.0, ex - (p - 1));
  double n = std::rint(v / quantum);  // v / quantum is exact (power-of-two scaling, no underflow here)
  return n * quantum;
}

// Double -> bf16 bits, RNE, overflow to infinity, NaN kept.
uint16_t bf16_from_double(double v) {
  float f;
  if (std::isnan(v)) {
    f = std::numeric_limits<float>::quiet_NaN();
  } else {
    double r = round_to_format(v, 8, -126);
    // largest finite bf16 is (2 - 2^-7) * 2^127; rounding beyond it means overflow
    if (std::fabs(r) > 3.3895313892515355e38) r = std::copysign(INFINITY, v);
    f = (float)r;  // exact: r is a bf16 value (or infinity)
  }
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// E2M1 (FP4): 1 sign, 2 exponent, 1 mantissa bit, exponent bias 1, no infinities or NaN.
// Exponent field 0 is subnormal (0 or 0.5); otherwise (1 + m/2) * 2^(e-1).
// Non-negative values {0, 0.5, 1, 1.5, 2, 3, 4, 6} [review §3.1].
double e2m1_value(unsigned code) {
  unsigned e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

// E4M3 (FP8, the OCP "FN" variant): 1 sign, 4 exponent, 3 mantissa bits, bias 7, no infinities,
// S.1111.111 is NaN, max finite 448, min subnormal 2^-9. The pages name only "FP8 E4M3" [review §3.1].
double e4m3_value(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 15u && m == 7u) return std::numeric_limits<double>::quiet_NaN();
  double mag = (e == 0) ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, (int)e - 10);
  return s ? -mag : mag;
}

// Non-negative finite value -> E4M3 code, round-to-nearest-even on the E4M3 grid, saturating at 448.
unsigned e4m3_encode_satfinite(double v) {
  double r = round_to_format(v, 4, -6);
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return 0u;
  if (r < std::ldexp(1.0, -6)) return (unsigned)(r / std::ldexp(1.0, -9));  // subnormal: m * 2^-9
  int e;
  std::frexp(r, &e);
  int ex = e - 1;                                              // r = (8 + m) * 2^(ex - 3)
  unsigned m = (unsigned)(r / std::ldexp(1.0, ex - 3)) - 8u;
  return ((unsigned)(ex + 7) << 3) | m;
}

bool bf16_is_finite(uint16_t b) { return ((b >> 7) & 0xffu) != 0xffu; }

// ---------------------------------------------------------------------------------------------------------------
// NVFP4 scales. The pages leave the choice of s_g and s_b to calibration [review §3.1]; the reading used here is
// the amax rule: the tensor scale maps the tensor's largest magnitude onto (E2M1 max 6) x (E4M3 max 448), and each
// 16-weight block's E4M3 scale maps that block's largest magnitude onto 6. Both divisions are IEEE f32.
float nvfp4_tensor_scale(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int* flags) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      uint16_t b = w[i * ldw + j];
      if (!bf16_is_finite(b)) { if (flags) *flags |= 1; continue; }
      float a = (float)std::fabs(bf16_value(b));
      if (a > amax) amax = a;
    }
  return (amax > 0.0f) ? amax / 2688.0f : 1.0f;  // 2688 = 6 * 448
}

// the block scales of one row (k / 16 blocks) under the tensor scale s_g
void nvfp4_row_block_scales(const uint16_t* row, int64_t k, float s_g, uint8_t* s_b_row) {
  float denom = 6.0f * s_g;
  for (int64_t b = 0; b < k / 16; ++b) {
    float amax_b = 0.0f;
    for (int64_t j = 0; j < 16; ++j) {
      uint16_t v = row[b * 16 + j];
      if (!bf16_is_finite(v)) continue;
      float a = (float)std::fabs(bf16_value(v));
      if (a > amax_b) amax_b = a;
    }
    float t = amax_b / denom;
    s_b_row[b] = (uint8_t)e4m3_encode_satfinite((double)t);
  }
}

void nvfp4_scales(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, float* s_g_out, uint8_t* s_b, int* flags) {
  float s_g = nvfp4_tensor_scale(w, n, k, ldw, flags);
  *s_g_out = s_g;
  for (int64_t i = 0; i < n; ++i) nvfp4_row_block_scales(w + i * ldw, k, s_g, s_b + i * (k / 16));
}

// Exact three-way comparison of the distances |a - x| and |a - y| (a, x, y >= 0 exact doubles, x and y candidate
// grid values S*g). Subtracting in floating point is not exact when a is many binades above S (both distances then
// round to the same value), so the comparison is made by position: two candidates on the same side of a are ordered by
// value; for candidates on both sides, |a - lo| < |hi - a| iff 2a < lo + hi, and lo + hi = S*(g_lo + g_hi) is exact.
// Returns -1 if x is nearer, 0 on a tie, +1 if y is nearer.
int compare_distance(double a, double x, double y) {
  if (x == y) return 0;
  if (x <= a && y <= a) return x > y ? -1 : 1;
  if (x >= a && y >= a) return x < y ? -1 : 1;
  double lo = x < y ? x : y, hi = x < y ? y : x;
  double two_a = 2.0 * a, sum = lo + hi;
  if (two_a == sum) return 0;
  bool lo_nearer = two_a < sum;
  return (lo_nearer == (x == lo)) ? -1 : 1;
}

// Nearest grid point under fixed scales [review §3.1, argmin equation]: q = argmin over E2M1 of |w - s_g s_b q|.
// S = s_g*s_b is exact in fp64 (24 + 4 significant bits) and so is every candidate S*g. Ties (exact midpoints) go to
// the even code (mantissa bit 0), the usual round-half-to-even convention; the pages fix no tie rule. The sign is
// copied from w, so a negative weight that rounds to zero keeps code 8 (-0).
unsigned nvfp4_code(uint16_t wb, double S) {
  if (!bf16_is_finite(wb)) return 0u;
  double w = bf16_value(wb);
  unsigned sign = std::signbit(w) ? 8u : 0u;
  if (S == 0.0) return sign;
  double a = std::fabs(w);
  unsigned best = 0;
  for (unsigned c = 1; c < 8; ++c) {
    int cmp = compare_distance(a, S * e2m1_value(c), S * e2m1_value(best));
    if (cmp < 0 || (cmp == 0 && (c & 1u) == 0u)) best = c;
  }
  return sign | best;
}

// ---------------------------------------------------------------------------------------------------------------
// MXFP4, the OCP Microscaling FP4 format the papers calibrate and compare beside NVFP4 ["QeRL 阅读笔记" §3.1]. The pages
// give it no further detail, so the reading is the OCP MX v1.0 definition: blocks of 32 consecutive weights along k
// share one E8M0 scale X = 2^(E - 127) (E = 255 is NaN; no sign, no mantissa). The shared exponent is the block's
// floor(log2(amax)) minus the largest exponent of the element format (2 for E2M1, whose largest value is
// 6 = 1.5 * 2^2), kept within E8M0's range; each element is the E2M1 value nearest to w / X, ties to the even code,
// values beyond 6 saturating to 6, with the sign of w. A block without a nonzero finite value takes E = 0.
double e8m0_value(unsigned byte) {
  return byte == 255u ? std::numeric_limits<double>::quiet_NaN() : std::ldexp(1.0, (int)byte - 127);
}

unsigned mxfp4_block_exponent(double amax) {
  if (!(amax > 0.0)) return 0u;
  int e;
  std::frexp(amax, &e);  // amax = f 2^e with f in [0.5, 1): floor(log2(amax)) = e - 1
  const int E = (e - 1) - 2 + 127;
  return E < 0 ? 0u : (E > 254 ? 254u : (unsigned)E);
}

// y = W_hat h + lambda B (A h) in fp64, W_hat row o given by row(o, out[k]) (the shared body of the linear oracles).
template <class RowFn>
void lora_linear_rows(const uint16_t* h, int64_t m, int64_t k, int64_t ldh, int64_t n, RowFn row, const uint16_t* A,
                      const uint16_t* B, int r, double lambda, double* y) {
  double* t = new double[(size_t)(m * (r > 0 ? r : 1))];
  bool lora = A && B && r > 0;
  if (lora)
    for (int64_t i = 0; i < m; ++i)
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < k; ++c) acc += bf16_value(A[j * k + c]) * bf16_value(h[i * ldh + c]);
        t[i * r + j] = acc;
      }
  double* wrow = new double[(size_t)k];
  for (int64_t o = 0; o < n; ++o) {
    row(o, wrow);
    for (int64_t i = 0; i < m; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) acc += wrow[c] * bf16_value(h[i * ldh + c]);
      if (lora) {
        double lr = 0.0;
        for (int j = 0; j < r; ++j) lr += bf16_value(B[o * r + j]) * t[i * r + j];
        acc += lambda * lr;
      }
      y[i * n + o] = acc;
    }
  }
  delete[] wrow;
  delete[] t;
}

}  // namespace

// =================================================================================================================
extern "C" {

double orc_bf16_value(uint16_t b) { return bf16_value(b); }
uint16_t orc_bf16_round(double v) { return bf16_from_double(v); }
void orc_bf16_round_array(const double* v, int64_t count, uint16_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = bf16_from_double(v[i]);
}
double orc_e2m1_value(int code) { return e2m1_value((unsigned)code & 15u); }
double orc_e4m3_value(int byte) { return e4m3_value((unsigned)byte & 255u); }
int orc_e4m3_encode(double v) { return (int)e4m3_encode_satfinite(v); }
int orc_nvfp4_code(uint16_t w, double S) { return (int)nvfp4_code(w, S); }

// Bytes of one NVFP4 tensor in the canonical layout: P/2 code bytes + P/16 scale bytes + one f32 tensor scale
// [review §3.1, M_NVFP4 equation: 9P/16 ignoring the tensor-global scale].
int64_t orc_nvfp4_bytes(int64_t n, int64_t k) { return n * k / 2 + n * k / 16; }

// Quantize W [n x k] (bf16, row stride ldw) to NVFP4 in the canonical layout:
//   codes [n][k/2]: byte j holds element 2j in bits 3:0 and element 2j+1 in bits 7:4;
//   s_b   [n][k/16]: E4M3 block scale of 16 consecutive elements along k;
//   s_g   one f32 tensor scale.
// scale_mode 0 computes the scales by the amax rule; scale_mode 1 reads caller-fixed s_b and s_g.
// flags bit 0 is set when a non-finite weight is seen (it is excluded from the amax and encoded as code 0).
void orc_nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int scale_mode, uint8_t* codes,
                        uint8_t* s_b, float* s_g, int* flags) {
  if (scale_mode == 0) nvfp4_scales(w, n, k, ldw, s_g, s_b, flags);
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      uint16_t b = w[i * ldw + j];
      if (!bf16_is_finite(b) && flags) *flags |= 1;
      double S = (double)(*s_g) * e4m3_value(s_b[i * (k / 16) + j / 16]);  // exact product
      unsigned c = nvfp4_code(b, S);
      uint8_t& byte = codes[i * (k / 2) + j / 2];
      if ((j & 1) == 0) byte = (uint8_t)c; else byte = (uint8_t)(byte | (c << 4));
    }
}

// The amax-rule quantization of selected rows of W: s_g from the whole tensor (as orc_nvfp4_quantize computes it),
// block scales and codes for rows[0 .. nrows) only, written as consecutive rows of codes / s_b. Rows are independent
// given s_g, so each output row equals that row of the whole tensor's quantization.
void orc_nvfp4_quantize_rows(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, const int64_t* rows,
                             int64_t nrows, uint8_t* codes, uint8_t* s_b, float* s_g, int* flags) {
  *s_g = nvfp4_tensor_scale(w, n, k, ldw, flags);
  for (int64_t r = 0; r < nrows; ++r) {
    const uint16_t* row = w + rows[r] * ldw;
    uint8_t* sb_row = s_b + r * (k / 16);
    nvfp4_row_block_scales(row, k, *s_g, sb_row);
    for (int64_t j = 0; j < k; ++j) {
      double S = (double)(*s_g) * e4m3_value(sb_row[j / 16]);  // exact product
      unsigned c = nvfp4_code(row[j], S);
      uint8_t& byte = codes[r * (k / 2) + j / 2];
      if ((j & 1) == 0) byte = (uint8_t)c; else byte = (uint8_t)(byte | (c << 4));
    }
  }
}

// Reconstruction w_hat = s_g * s_b * q [review §3.1, reconstruction equation], exact in fp64 (at most 30
// significant bits), and its single RNE rounding to f32.
void orc_nvfp4_dequantize(const uint8_t* codes, const uint8_t* s_b, float s_g, int64_t n, int64_t k,
                          double* w_exact, float* w_f32) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      uint8_t byte = codes[i * (k / 2) + j / 2];
      unsigned c = (j & 1) ? (byte >> 4) : (byte & 15u);
      double v = (double)s_g * (e4m3_value(s_b[i * (k / 16) + j / 16]) * e2m1_value(c));
      if (w_exact) w_exact[i * k + j] = v;
      if (w_f32) w_f32[i * k + j] = (float)v;
    }
}

// Exponential AQN schedule with a zero warm-up stage [review §5.2, schedule equation]:
// sigma_0 = 0, sigma_k = start * (end/start)^((k-1)/8) for k = 1..9.
double orc_aqn_sigma(int stage, double start, double end) {
  if (stage <= 0) return 0.0;
  return start * std::pow(end / start, (double)(stage - 1) / 8.0);
}

// AQN-RMSNorm [review §5.1, RMSNorm identity]: u = x / sqrt(mean_j x_j^2 + eps), h_z = u (.) (w + z), with the
// additive noise z = sigma * eps_noise on the clean scale w (replacement semantics, §9.1: w is never written).
// noise_ld == 0 shares one noise vector [d] across all rows; otherwise row i uses noise[i * noise_ld ...].
// h_exact gets the fp64 value; h_bf16 (if non-null) its RNE bf16 rounding, the activation the linear consumes.
void orc_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, int64_t ldx, const uint16_t* gamma,
                     const float* noise, int64_t noise_ld, float sigma, float eps, double* h_exact,
                     uint16_t* h_bf16) {
  for (int64_t i = 0; i < m; ++i) {
    double ss = 0.0;
    for (int64_t j = 0; j < d; ++j) { double v = bf16_value(x[i * ldx + j]); ss += v * v; }
    double rstd = 1.0 / std::sqrt(ss / (double)d + (double)eps);
    const float* z = noise ? noise + i * noise_ld : nullptr;
    for (int64_t j = 0; j < d; ++j) {
      double g = bf16_value(gamma[j]) + (z ? (double)sigma * (double)z[j] : 0.0);
      double h = bf16_value(x[i * ldx + j]) * rstd * g;
      if (h_exact) h_exact[i * d + j] = h;
      if (h_bf16) h_bf16[i * d + j] = bf16_from_double(h);
    }
  }
}

// ---- AQN noise drawn from a seed -------------------------------------------------------------------------------
// The pages add Gaussian noise z = sigma * eps, eps ~ N(0, 1), to the norm's clean scale at every call and say
// neither how it is drawn nor how wide its scope is [review §5.1 and §9.1]. This draw is one concrete choice, fixed
// here so that a device implementation can be checked against it: a counter-based generator (Philox4x64 with 10
// rounds, Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) keyed by
// (seed, stream), one block per 8 consecutive columns of one draw, and the Box-Muller transform (Box and Muller,
// 1958) on pairs of its 32-bit words.

// One Philox4x64 block: 10 rounds of the 4-word S-box (two 64x64 -> 128-bit multiplications, the high halves
// XOR-ed with the other two words and the round key, words permuted), the key advanced by the Weyl constants
// between rounds. Constants as published for Philox4x64.
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += W0; k1 += W1; }
    const unsigned __int128 p0 = (unsigned __int128)M0 * x0, p1 = (unsigned __int128)M1 * x2;
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0, hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    const uint64_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

// A 32-bit word as a uniform in (0, 1): its top 23 bits b, u = (b + 1/2) / 2^23, exactly representable in f32 and
// f64 alike (so both sides of a comparison start from the same u), never 0 or 1.
double word_uniform(uint32_t w) { return ((double)(w >> 9) + 0.5) / 8388608.0; }

// eps[i][j] (f32, row stride ld) for rows i of a call: row i takes draw index row_offset + i / draw_rows (draw_rows
// > 0: that many consecutive rows share a draw, e.g. the tokens of one response), or draw row_offset for every row
// (draw_rows == 0). Columns 8c .. 8c+7 of draw r come from the block at counter (c, r, 0, 0) under key (seed,
// stream); its words w_0..w_7 (w_2q = low half of output q, w_2q+1 = high half) pair as (w_2p, w_2p+1) -> columns
// 8c+2p, 8c+2p+1: rho = sqrt(-2 ln u(w_2p)), eps = rho cos(2 pi u(w_2p+1)), rho sin(2 pi u(w_2p+1)). fp64, then
// rounded to f32 (the precision the norm reads its noise in).
void orc_aqn_noise(uint64_t seed, uint64_t stream, uint64_t row_offset, int64_t draw_rows, int64_t m, int64_t d,
                   float* eps, int64_t ld) {
  const double two_pi = 6.283185307179586476925286766559;
  const uint64_t key[2] = {seed, stream};
  for (int64_t i = 0; i < m; ++i) {
    const uint64_t r = row_offset + (draw_rows > 0 ? (uint64_t)(i / draw_rows) : 0);
    for (int64_t c = 0; c * 8 < d; ++c) {
      const uint64_t ctr[4] = {(uint64_t)c, r, 0, 0};
      uint64_t o[4];
      orc_philox4x64_10(ctr, key, o);
      for (int p = 0; p < 4; ++p) {
        const uint32_t wa = (uint32_t)o[p], wb = (uint32_t)(o[p] >> 32);
        const double rho = std::sqrt(-2.0 * std::log(word_uniform(wa)));
        const double th = two_pi * word_uniform(wb);
        const int64_t j = c * 8 + 2 * p;
        if (j < d) eps[i * ld + j] = (float)(rho * std::cos(th));
        if (j + 1 < d) eps[i * ld + j + 1] = (float)(rho * std::sin(th));
      }
    }
  }
}

// LoRA-adapted linear with an NVFP4 base [review §2.1, forward map y = W_hat x + lambda B (A x)], row-batched:
//   y[i][o] = sum_c W_hat[o][c] h[i][c] + lambda * sum_j B[o][j] * t[i][j],   t[i][j] = sum_c A[j][c] h[i][c]
// h [m x k] bf16 (row stride ldh), W_hat from the canonical NVFP4 layout [n x k], A [r x k] bf16, B [n x r] bf16.
// Everything in fp64 from the exact input values; t is not rounded. A or B may be null (no LoRA branch).
void orc_lora_linear(const uint16_t* h, int64_t m, int64_t k, int64_t ldh, const uint8_t* codes,
                     const uint8_t* s_b, float s_g, int64_t n, const uint16_t* A, const uint16_t* B, int r,
                     double lambda, double* y) {
  lora_linear_rows(
      h, m, k, ldh, n,
      [&](int64_t o, double* wrow) {
        for (int64_t c = 0; c < k; ++c) {
          uint8_t byte = codes[o * (k / 2) + c / 2];
          unsigned q = (c & 1) ? (byte >> 4) : (byte & 15u);
          wrow[c] = (double)s_g * (e4m3_value(s_b[o * (k / 16) + c / 16]) * e2m1_value(q));
        }
      },
      A, B, r, lambda, y);
}

// MXFP4 quantization of W bf16 [n x k] (k % 32 == 0), canonical layout: codes [n][k/2] packed as for NVFP4 (element
// 2j in bits 3:0 of byte j), E8M0 scales [n][k/32]. Non-finite weights are left out of the block amax, get code 0
// and set bit 0 of *flags.
void orc_mxfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* codes, uint8_t* scales,
                        int* flags) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t b = 0; b < k / 32; ++b) {
      const uint16_t* blk = w + i * ldw + b * 32;
      double amax = 0.0;
      for (int j = 0; j < 32; ++j) {
        if (!bf16_is_finite(blk[j])) {
          if (flags) *flags |= 1;
          continue;
        }
        amax = std::fmax(amax, std::fabs(bf16_value(blk[j])));
      }
      const unsigned E = mxfp4_block_exponent(amax);
      scales[i * (k / 32) + b] = (uint8_t)E;
      const double X = e8m0_value(E);
      for (int j = 0; j < 32; j += 2) {
        const unsigned lo = nvfp4_code(blk[j], X), hi = nvfp4_code(blk[j + 1], X);  // nearest E2M1 under scale X
        codes[i * (k / 2) + (b * 32 + j) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

// W_hat = X * q from the canonical MXFP4 layout: exact (fp64) and rounded once to f32.
void orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, double* w_exact,
                          float* w_f32) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      uint8_t byte = codes[i * (k / 2) + j / 2];
      unsigned c = (j & 1) ? (byte >> 4) : (byte & 15u);
      double v = e8m0_value(scales[i * (k / 32) + j / 32]) * e2m1_value(c);
      if (w_exact) w_exact[i * k + j] = v;
      if (w_f32) w_f32[i * k + j] = (float)v;
    }
}

// The LoRA-adapted linear of orc_lora_linear with an MXFP4 base (canonical layout).
void orc_mxfp4_lora_linear(const uint16_t* h, int64_t m, int64_t k, int64_t ldh, const uint8_t* codes,
                           const uint8_t* scales, int64_t n, const uint16_t* A, const uint16_t* B, int r,
                           double lambda, double* y) {
  lora_linear_rows(
      h, m, k, ldh, n,
      [&](int64_t o, double* wrow) {
        for (int64_t c = 0; c < k; ++c) {
          uint8_t byte = codes[o * (k / 2) + c / 2];
          unsigned q = (c & 1) ? (byte >> 4) : (byte & 15u);
          wrow[c] = e8m0_value(scales[o * (k / 32) + c / 32]) * e2m1_value(q);
        }
      },
      A, B, r, lambda, y);
}

// Backward of the LoRA-adapted linear through the frozen NVFP4 base [review §2.1: the backbone is frozen, gradients
// update A and B, and may need to pass through the frozen projection to reach an earlier adapter; §6, steps 8-10].
// With the upstream gradient g = dL/dy [m x n] (bf16) of y = W_hat h + lambda B (A h):
//   u = B^T g per token   (u[i][j] = sum_o B[o][j] g[i][o]),   t = A h per token (t[i][j] = sum_c A[j][c] h[i][c]),
//   dh[i][c] = sum_o W_hat[o][c] g[i][o] + lambda sum_j A[j][c] u[i][j],
//   dA[j][c] = lambda sum_i u[i][j] h[i][c],     dB[o][j] = lambda sum_i g[i][o] t[i][j].
// Everything in fp64 from the exact inputs (W_hat exact); any output pointer may be null.
void orc_lora_linear_backward(const uint16_t* g, int64_t m, int64_t n, const uint16_t* h, int64_t k,
                              const uint8_t* codes, const uint8_t* s_b, float s_g, const uint16_t* A,
                              const uint16_t* B, int r, double lambda, double* dh, double* dA, double* dB) {
  const bool lora = A && B && r > 0;
  double* u = new double[(size_t)(m * (r > 0 ? r : 1))];
  double* t = new double[(size_t)(m * (r > 0 ? r : 1))];
  if (lora)
    for (int64_t i = 0; i < m; ++i)
      for (int j = 0; j < r; ++j) {
        double su = 0.0, st = 0.0;
        for (int64_t o = 0; o < n; ++o) su += bf16_value(B[o * r + j]) * bf16_value(g[i * n + o]);
        for (int64_t c = 0; c < k; ++c) st += bf16_value(A[(int64_t)j * k + c]) * bf16_value(h[i * k + c]);
        u[i * r + j] = su;
        t[i * r + j] = st;
      }
  if (dh) {
    for (int64_t x = 0; x < m * k; ++x) dh[x] = 0.0;
    double* wrow = new double[(size_t)k];
    for (int64_t o = 0; o < n; ++o) {
      for (int64_t c = 0; c < k; ++c) {
        uint8_t byte = codes[o * (k / 2) + c / 2];
        unsigned q = (c & 1) ? (byte >> 4) : (byte & 15u);
        wrow[c] = (double)s_g * (e4m3_value(s_b[o * (k / 16) + c / 16]) * e2m1_value(q));
      }
      for (int64_t i = 0; i < m; ++i) {
        const double gi = bf16_value(g[i * n + o]);
        if (gi == 0.0) continue;
        for (int64_t c = 0; c < k; ++c) dh[i * k + c] += wrow[c] * gi;
      }
    }
    delete[] wrow;
    if (lora)
      for (int64_t i = 0; i < m; ++i)
        for (int64_t c = 0; c < k; ++c) {
          double acc = 0.0;
          for (int j = 0; j < r; ++j) acc += bf16_value(A[(int64_t)j * k + c]) * u[i * r + j];
          dh[i * k + c] += lambda * acc;
        }
  }
  if (dA)
    for (int j = 0; j < r; ++j)
      for (int64_t c = 0; c < k; ++c) {
        double acc = 0.0;
        if (lora)
          for (int64_t i = 0; i < m; ++i) acc += u[i * r + j] * bf16_value(h[i * k + c]);
        dA[(int64_t)j * k + c] = lambda * acc;
      }
  if (dB)
    for (int64_t o = 0; o < n; ++o)
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        if (lora)
          for (int64_t i = 0; i < m; ++i) acc += bf16_value(g[i * n + o]) * t[i * r + j];
        dB[o * r + j] = lambda * acc;
      }
  delete[] u;
  delete[] t;
}

// Dense bf16 linear y = x W^T (no quantization), used by the tests as the "BF16 LoRA" comparison baseline.
void orc_dense_linear(const uint16_t* h, int64_t m, int64_t k, const uint16_t* w, int64_t n, double* y) {
  for (int64_t o = 0; o < n; ++o)
    for (int64_t i = 0; i < m; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) acc += bf16_value(w[o * k + c]) * bf16_value(h[i * k + c]);
      y[i * n + o] = acc;
    }
}

// Group-relative advantage with the population standard deviation [review §2.2]:
//   A_i = (R_i - mean) / (s_R + eps),  s_R = sqrt(mean (R_i - mean)^2), per group of g consecutive rewards.
void orc_group_advantage(const float* rewards, int groups, int g, double eps, double* adv) {
  for (int q = 0; q < groups; ++q) {
    const float* R = rewards + (int64_t)q * g;
    double mean = 0.0;
    for (int i = 0; i < g; ++i) mean += (double)R[i];
    mean /= (double)g;
    double var = 0.0;
    for (int i = 0; i < g; ++i) { double d = (double)R[i] - mean; var += d * d; }
    double s = std::sqrt(var / (double)g);
    for (int i = 0; i < g; ++i) adv[(int64_t)q * g + i] = ((double)R[i] - mean) / (s + eps);
  }
}

// GRPO token ratio and clipped surrogate [review §2.3]: for token t of response i, sampled by the behavior policy
// pi_b,  rho = exp(log pi_theta - log pi_b)  and the surrogate  s = min(rho A_i, clip(rho, 1 - clip_low, 1 + clip_high) A_i).
// The pages fix neither the clip widths nor how token surrogates are combined; the readings here: both widths are
// arguments, and the loss is -(sum_i,t w_i,t s_i,t) with w = 1 / (all valid tokens) (agg 0, a token mean over the
// batch) or w = 1 / (responses with tokens x tokens of response i) (agg 1, each response's token mean, averaged over
// responses). Response i has lengths[i] valid tokens (clamped to [0, t_max]) at logp[i * ld + t].
// Per token: surrogate s (0 past the length) and grad = d loss / d log pi_theta = -w rho A where the unclipped term
// is the smaller (ties included: inside the clip range both terms are equal), else 0 (the clipped term is constant).
// stats: [0] loss, [1] mean ratio over valid tokens, [2] min ratio, [3] max ratio, [4] valid tokens, [5] tokens whose
// clipped term is strictly smaller. fp64 throughout, from the f32 inputs.
void orc_grpo_surrogate(const float* logp, const float* logp_old, int64_t ld, const int* lengths, const float* adv,
                        int n_seq, int t_max, double clip_low, double clip_high, int agg, double* surrogate,
                        double* grad, double* stats) {
  int64_t n_tok = 0;
  int n_nonempty = 0;
  for (int i = 0; i < n_seq; ++i) {
    int L = lengths[i] < 0 ? 0 : (lengths[i] > t_max ? t_max : lengths[i]);
    n_tok += L;
    if (L > 0) ++n_nonempty;
  }
  double loss = 0.0, rsum = 0.0, rmin = INFINITY, rmax = -INFINITY;
  int64_t clipped = 0;
  for (int i = 0; i < n_seq; ++i) {
    int L = lengths[i] < 0 ? 0 : (lengths[i] > t_max ? t_max : lengths[i]);
    const double A = (double)adv[i];
    const double w = agg == 0 ? (n_tok > 0 ? 1.0 / (double)n_tok : 0.0)
                              : (L > 0 ? 1.0 / ((double)n_nonempty * (double)L) : 0.0);
    for (int t = 0; t < t_max; ++t) {
      const int64_t k = (int64_t)i * ld + t;
      if (t >= L) {
        if (surrogate) surrogate[k] = 0.0;
        if (grad) grad[k] = 0.0;
        continue;
      }
      const double rho = std::exp((double)logp[k] - (double)logp_old[k]);
      const double lo = 1.0 - clip_low, hi = 1.0 + clip_high;
      const double unclipped = rho * A;
      const double clipped_term = (rho < lo ? lo : (rho > hi ? hi : rho)) * A;
      const double sur = unclipped <= clipped_term ? unclipped : clipped_term;
      if (surrogate) surrogate[k] = sur;
      if (grad) grad[k] = unclipped <= clipped_term ? -w * rho * A : 0.0;
      if (clipped_term < unclipped) ++clipped;
      loss -= w * sur;
      rsum += rho;
      rmin = rho < rmin ? rho : rmin;
      rmax = rho > rmax ? rho : rmax;
    }
  }
  stats[0] = loss;
  stats[1] = n_tok > 0 ? rsum / (double)n_tok : 0.0;
  stats[2] = n_tok > 0 ? rmin : 0.0;
  stats[3] = n_tok > 0 ? rmax : 0.0;
  stats[4] = (double)n_tok;
  stats[5] = (double)clipped;
}

// SwiGLU gating of the feed-forward block (the "gating multiplication and nonlinearity" before Down,
// [review §5.1]): a = SiLU(g) * u with SiLU(v) = v / (1 + exp(-v)). fp64, element-wise.
void orc_silu_mul(const double* gate, const double* up, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = gate[i] / (1.0 + std::exp(-gate[i])) * up[i];
}

}  // extern "C"
