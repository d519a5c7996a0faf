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

// Loads. Every load issued ahead of the weight stream is a buffer load or a global-segment load, never a flat one:
// a pending flat load may be an LDS access, which forces the compiler to drain all loads at every later wait and
// so would serialize the double-buffered stream.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)
constexpr int kNonTemporal = 2;                 // streamed once: do not keep in cache
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every num_records: the load returns 0

// Wave-uniform copies (readfirstlane) of values the compiler cannot prove uniform on its own, so that buffer
// descriptors built from them stay in SGPRs.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Raw buffer descriptor over [base, base + bytes); bytes < 2^31 (checked on the host).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform64((uint64_t)base), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes), kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// A 32-bit word's bits as two f16. Taking the word as a by-value argument matters: applied directly to an element of
// a vector (w[i] of a u32x4), __builtin_bit_cast has been seen to compile to a read of element 0 whatever i is.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// Load through a pointer known to address global memory.
template <class T>
__device__ __forceinline__ T gload(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(reinterpret_cast<uintptr_t>(p));
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
