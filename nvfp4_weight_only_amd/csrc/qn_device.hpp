// Device-side helpers shared by the library's HIP sources (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qerl_nvfp4.h"

namespace qn {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kRowGroup = 16;    // rows per MFMA A-fragment
constexpr int kKTile = 128;      // k per tiled-layout tile (four 16x16x32 MFMA slices)
constexpr int kTileCodeBytes = 1024;
constexpr int kTileScaleBytes = 128;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16 bits, round to nearest even (NaN kept quiet).
// (written as a select, not an early return, so that it compiles to straight-line code without exec-mask branches)
__device__ inline uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded);
}

__device__ inline bool bf16_finite(uint16_t b) { return ((b >> 7) & 0xffu) != 0xffu; }

// E4M3 (OCP FN) byte -> f32 value, from the bit fields: bias 7, subnormals m * 2^-9, S.1111.111 = NaN.
__device__ inline float e4m3_to_f32(uint32_t byte) {
  uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0x1p-9f;
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  }
  if (e == 15u && m == 7u) mag = __uint_as_float(0x7fc00000u);
  return (byte & 0x80u) ? -mag : mag;
}

// An MFMA's result registers may be read by a non-MFMA instruction (a VALU operation, an LDS or memory store) only
// once the matrix core has written every pass of them; the program must place enough independent instructions in
// between. Within a basic block the compiler counts them; across a branch or a loop exit it has been seen to count
// too few (an LDS store one instruction after the MFMA on a taken branch, which then stored stale lanes). This waits
// the passes out explicitly: the assembly statement takes the registers as an operand, so it stays between the MFMA
// and every reader on every path, and its no-ops give 16 wait states, more than any 16x16x32 MFMA here needs.
__device__ __forceinline__ void mfma_settle(f32x4& v) { asm volatile("s_nop 7\n\ts_nop 7" : "+v"(v)); }

// Wave-wide reductions (wave64) through ds_swizzle-free shuffles.
__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace qn
