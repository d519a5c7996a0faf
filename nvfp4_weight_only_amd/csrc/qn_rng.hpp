// Seeded standard-normal noise for the AQN norm, drawn on the device where the norm consumes it ("QeRL: When
// Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops", technical review §5.1 and §9.1:
// Gaussian noise on the clean norm scale at every call; the pages leave the generator and the scope of a draw open).
// The generator is Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC 2011), keyed by (seed, subseed), one block per 8 consecutive columns of a draw at counter
// (column block, draw index, 0, 0); the Box-Muller transform (Box and Muller, 1958) turns each pair of its 32-bit
// words into two normals. The uniforms keep 23 bits of a word, u = (b + 1/2) 2^-23, so they are exact in f32, never 0
// or 1; the logarithm, square root and sin/cos are the f32 library functions (a few ulp).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace qn {

// The caller's draw parameters, passed by value to the kernels that generate noise.
struct QnDraw {
  int32_t on;
  uint64_t seed, subseed;
  uint64_t row_offset;  // draw index of row 0
  int64_t draw_rows;    // rows per draw; 0: one draw for every row
  int64_t row_base;     // row of the call that row 0 of this launch is (a call run as sub-calls of fewer rows)
};

// Draw index of row `row` of the launch (row row_base + row of the call).
__device__ __forceinline__ uint64_t draw_index(const QnDraw& q, int64_t row) {
  return q.row_offset + (q.draw_rows > 0 ? (uint64_t)((q.row_base + row) / q.draw_rows) : 0ull);
}

// One Philox4x64 block at counter (c0, c1, 0, 0): per round, the two 64 x 64 -> 128-bit products of words 0 and 2
// with the round multipliers; their high halves XOR-ed with words 1 and 3 and the round key become words 0 and 2,
// the low halves words 3 and 1; the key advances by the Weyl increments between rounds (published constants).
__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t k1, uint64_t o[4]) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = c0, x1 = c1, x2 = 0, x3 = 0;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t hi0 = __umul64hi(kM0, x0), lo0 = kM0 * x0;
    const uint64_t hi1 = __umul64hi(kM1, x2), lo1 = kM1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  o[0] = x0;
  o[1] = x1;
  o[2] = x2;
  o[3] = x3;
}

__device__ __forceinline__ float word_uniform(uint32_t w) { return ((float)(w >> 9) + 0.5f) * 0x1p-23f; }

// eps for columns 8c .. 8c+7 of draw r: words (2p, 2p+1) -> columns 8c+2p, 8c+2p+1.
__device__ __forceinline__ void aqn_noise8(const QnDraw& q, uint64_t r, uint64_t c, float z[8]) {
  uint64_t o[4];
  philox4x64_10(c, r, q.seed, q.subseed, o);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float rho = sqrtf(-2.0f * logf(word_uniform((uint32_t)o[p])));
    float sn, cs;
    sincospif(2.0f * word_uniform((uint32_t)(o[p] >> 32)), &sn, &cs);
    z[2 * p] = rho * cs;
    z[2 * p + 1] = rho * sn;
  }
}

}  // namespace qn
