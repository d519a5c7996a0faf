// NVFP4 quantizer / packer and reconstruction.
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review),
// §3.1: reconstruction w = s_g * s_b * q with q on the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (and negatives), one
// E4M3 block scale per 16 weights and one f32 tensor scale; for fixed scales q is the nearest grid point. §3.2,
// Algorithm 1 steps 4-5: the codes are then packed into the layout the inference kernel reads (QN_LAYOUT_TILED).
//
// The pages leave the choice of scales to calibration; the amax rule used by scale_mode 0 maps the tensor maximum
// onto 6 * 448 and each block maximum onto 6 (E4M3 round-to-nearest-even, saturating).
#include "qn_device.hpp"

namespace qn {
namespace {

constexpr int kQThreads = 256;

// Location of the dword holding elements k0 .. k0+7 (k0 % 8 == 0) of row n, in bytes from the codes base.
__device__ inline int64_t code_dword_offset(int layout, int64_t n, int64_t k0, int64_t k, int64_t KT) {
  if (layout == QN_LAYOUT_ROWMAJOR) return n * (k / 2) + k0 / 2;
  int64_t g = n / kRowGroup, kt = k0 / kKTile;
  int s = (int)((k0 % kKTile) / 32), lhi = (int)((k0 % 32) / 8);
  int lane = lhi * kRowGroup + (int)(n % kRowGroup);
  return ((g * KT + kt) * kWave + lane) * 16 + s * 4;
}

// Location of the scale byte of the 16-block starting at k0 (k0 % 16 == 0) of row n.
__device__ inline int64_t scale_offset(int layout, int64_t n, int64_t k0, int64_t k, int64_t KT) {
  if (layout == QN_LAYOUT_ROWMAJOR) return n * (k / 16) + k0 / 16;
  int64_t g = n / kRowGroup, kt = k0 / kKTile;
  int s = (int)((k0 % kKTile) / 32), h = (int)((k0 % 32) / 16);
  return (g * KT + kt) * kTileScaleBytes + (n % kRowGroup) * 8 + h * 4 + s;
}

// Non-negative finite f32 -> E4M3 code, round to nearest even on the E4M3 grid, saturating at 448 (0x7E).
// Normal range: round the f32 significand to 3 bits on the bit pattern (carry may bump the exponent), then rebias
// 127 -> 7. Below 2^-6 the grid is m * 2^-9: scale by 2^9 (exact) and round to an integer (0..8; 8 is 0x08 = 2^-6).
__device__ inline uint32_t e4m3_encode_satfinite(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  uint32_t u = __float_as_uint(t);
  if (u < 0x3C800000u) return (uint32_t)rintf(t * 512.0f);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

// E2M1 magnitude index of |w| under block scale S, deciding against the midpoints of neighbouring grid values.
// S * midpoint is exact in fp64 (<= 28 + 3 significant bits). An exact midpoint goes to the even index, so the
// comparison is ">" where the lower neighbour is even and ">=" where the upper one is.
__device__ inline uint32_t e2m1_index(double a, double S) {
  if (S == 0.0) return 0u;
  return (uint32_t)(a > 0.25 * S) + (uint32_t)(a >= 0.75 * S) + (uint32_t)(a > 1.25 * S) +
         (uint32_t)(a >= 1.75 * S) + (uint32_t)(a > 2.5 * S) + (uint32_t)(a >= 3.5 * S) + (uint32_t)(a > 5.0 * S);
}

__global__ void k_quant_init(uint32_t* amax_bits) { *amax_bits = 0u; }

// Tensor amax over finite elements (as f32 bit patterns: ordered like the values for non-negative floats). Workgroups
// take whole rows; a thread takes 8 consecutive elements of a row at a time (k is a multiple of 16); VEC: the rows
// start 16-byte aligned at every group, one 16-byte load per group. One atomic per workgroup (the waves' maxima meet
// in LDS): atomics on one word serialize.
template <bool VEC>
__global__ void __launch_bounds__(kQThreads) k_quant_amax(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                           int64_t ldw, uint32_t* amax_bits, int32_t* flags) {
  __shared__ float s_m[kQThreads / kWave];
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  float m = 0.0f;
  bool bad = false;
  const int64_t gpr = k / 8;
  for (int64_t row = blockIdx.x; row < n; row += gridDim.x) {
    for (int64_t c8 = threadIdx.x; c8 < gpr; c8 += kQThreads) {
      const uint16_t* p = w + row * ldw + c8 * 8;
      uint32_t q[4];
      if (VEC) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = (uint32_t)p[2 * e] | ((uint32_t)p[2 * e + 1] << 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t b = (uint16_t)(q[e / 2] >> (16 * (e % 2)));
        if (!bf16_finite(b)) bad = true;
        else m = fmaxf(m, fabsf(bf16_to_f32(b)));
      }
    }
  }
  m = wave_max(m);
  __syncthreads();  // (s_bad initialised)
  if ((threadIdx.x % kWave) == 0) s_m[threadIdx.x / kWave] = m;
  if (bad) s_bad = 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = s_m[0];
    for (int i = 1; i < kQThreads / kWave; ++i) mm = fmaxf(mm, s_m[i]);
    atomicMax(amax_bits, __float_as_uint(mm));
    if (s_bad && flags) atomicOr(flags, 1);
  }
}

// One thread per 16-element block of the padded [np x kp] grid: block scale (scale_mode 0), 16 codes, stores.
__global__ void __launch_bounds__(kQThreads) k_quant_blocks(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                             int64_t ldw, int scale_mode, int layout,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                             const float* tensor_scale, int32_t* flags, int64_t np,
                                                             int64_t kp) {
  const int64_t KT = kp / kKTile;
  const int64_t kb = kp / 16;
  const int64_t idx = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (idx >= np * kb) return;
  const int64_t row = idx / kb, k0 = (idx - row * kb) * 16;
  const bool real = row < n && k0 < k;
  float s_g;
  if (scale_mode == 0) {
    float amax = __uint_as_float(*reinterpret_cast<const uint32_t*>(tensor_scale));
    s_g = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  } else {
    s_g = *tensor_scale;
  }
  uint32_t lo = 0u, hi = 0u, sb = 0u;
  if (real) {
    const uint16_t* src = w + row * ldw + k0;
    uint16_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = src[j];
    if (scale_mode == 0) {
      float amax_b = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (bf16_finite(v[j])) amax_b = fmaxf(amax_b, fabsf(bf16_to_f32(v[j])));
      sb = e4m3_encode_satfinite(__fdiv_rn(amax_b, __fmul_rn(6.0f, s_g)));
    } else {
      sb = scales[scale_offset(layout, row, k0, k, KT)];
    }
    const double S = (double)s_g * (double)e4m3_to_f32(sb);
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t c = 0u;
      if (bf16_finite(v[j])) {
        c = e2m1_index(fabs((double)bf16_to_f32(v[j])), S) | ((uint32_t)(v[j] >> 15) << 3);
      } else {
        bad = true;
      }
      if (j < 8) lo |= c << (4 * j); else hi |= c << (4 * (j - 8));
    }
    if (bad && flags) atomicOr(flags, 1);
  }
  *reinterpret_cast<uint32_t*>(codes + code_dword_offset(layout, row, k0, k, KT)) = lo;
  *reinterpret_cast<uint32_t*>(codes + code_dword_offset(layout, row, k0 + 8, k, KT)) = hi;
  if (scale_mode == 0) scales[scale_offset(layout, row, k0, k, KT)] = (uint8_t)sb;
}

__global__ void k_quant_finalize(float* tensor_scale) {
  float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(tensor_scale));
  *tensor_scale = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
}

// One thread per 16-block: w_hat = s_g * (s_b * q). The E2M1 decode uses the hardware FP4 -> f32 conversion with
// scale 1; s_b * q is exact in f32, so the f32 result is the exact product rounded once.
__global__ void __launch_bounds__(kQThreads) k_dequant(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, const float* tensor_scale,
                                                        int64_t n, int64_t k, int layout, float* __restrict__ out,
                                                        int64_t ldo, int64_t KT) {
  const int64_t kb = k / 16;
  const int64_t idx = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (idx >= n * kb) return;
  const int64_t row = idx / kb, k0 = (idx - row * kb) * 16;
  const float s_g = *tensor_scale;
  const float sbv = e4m3_to_f32(scales[scale_offset(layout, row, k0, k, KT)]);
  float* dst = out + row * ldo + k0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t d = *reinterpret_cast<const uint32_t*>(codes + code_dword_offset(layout, row, k0 + 8 * half, k, KT));
    // the byte selector of the converter is an immediate
    auto q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    auto q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    auto q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    auto q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    const float q[8] = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 * half + i] = __fmul_rn(s_g, __fmul_rn(sbv, q[i]));
  }
}

// ---- MXFP4 ------------------------------------------------------------------------------------------------------
// The OCP Microscaling FP4 format the papers calibrate beside NVFP4 ("QeRL 阅读笔记" §3.1; no detail on the pages, so
// OCP MX v1.0 is the reading): one E8M0 scale X = 2^(E - 127) per 32 weights along k, E = floor(log2(block amax)) - 2
// (2 = the largest E2M1 exponent: 6 = 1.5 * 2^2) within 0..254, elements the nearest E2M1 value to w / X (ties to the
// even code, saturating at 6). A block without a nonzero finite weight takes E = 0.
//
// Tiled form: the kernels read an NVFP4-tiled weight, so an MXFP4 weight is re-expressed exactly in that form. With
// E_ref = (largest E of the tensor) - 8, every 16-half of a block gets the E4M3 block scale 2^(E - E_ref) (a power of
// two from 2^-9 to 2^8, exact in E4M3) and the tensor scale is 2^(E_ref - 127): s_g s_b q = X q, bit for bit. A block
// whose exponent lies more than 17 below the largest cannot be written so (bit 1 of the flag word).
constexpr int kMxRange = 8;  // E - E_ref of the tensor's largest block scale

// floor(log2(a)) for a finite a > 0 (normal or subnormal f32)
__device__ inline int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ef = (int)((u >> 23) & 0xFFu);
  return ef ? ef - 127 : (31 - __clz((int)(u & 0x7FFFFFu))) - 149;
}

__device__ inline uint32_t mx_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0u;
  const int E = floor_log2(amax) - 2 + 127;
  return E < 0 ? 0u : (E > 254 ? 254u : (uint32_t)E);
}

// E4M3 byte of 2^d for d in [-9, 8]: normal (d + 7) << 3 from d = -6 on, else the subnormal m * 2^-9 with m = 2^(d + 9)
__device__ inline uint32_t e4m3_pow2(int d) { return d >= -6 ? (uint32_t)(d + 7) << 3 : 1u << (d + 9); }

__global__ void k_mx_init(int32_t* emax) { *emax = -1; }

// Largest block exponent of the tensor over blocks with a nonzero finite weight.
__global__ void __launch_bounds__(kQThreads) k_mx_emax(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                        int64_t ldw, int32_t* emax) {
  const int64_t kb = k / 32, idx = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  int e = -1;
  if (idx < n * kb) {
    const int64_t row = idx / kb, k0 = (idx - row * kb) * 32;
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      const uint16_t b = w[row * ldw + k0 + j];
      if (bf16_finite(b)) amax = fmaxf(amax, fabsf(bf16_to_f32(b)));
    }
    if (amax > 0.0f) e = (int)mx_block_exponent(amax);
  }
  for (int off = 32; off > 0; off >>= 1) e = max(e, __shfl_xor(e, off, kWave));
  if ((threadIdx.x % kWave) == 0 && e >= 0) atomicMax(emax, e);
}

// One thread per 32-block of the (padded, for the tiled form) grid: exponent, 32 codes, stores.
__global__ void __launch_bounds__(kQThreads) k_mx_blocks(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                          int64_t ldw, int layout, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, const int32_t* emax,
                                                          int32_t* flags, int64_t np, int64_t kp) {
  const int64_t KT = kp / kKTile, kb = kp / 32;
  const int64_t idx = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (idx >= np * kb) return;
  const int64_t row = idx / kb, k0 = (idx - row * kb) * 32;
  const bool real = row < n && k0 < k;
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
  uint32_t E = 0u;
  float amax = 0.0f;
  if (real) {
    const uint16_t* src = w + row * ldw + k0;
    uint16_t v[32];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      v[j] = src[j];
      if (bf16_finite(v[j])) amax = fmaxf(amax, fabsf(bf16_to_f32(v[j])));
      else bad = true;
    }
    E = mx_block_exponent(amax);
    const double X = ldexp(1.0, (int)E - 127);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t c = bf16_finite(v[j]) ? (e2m1_index(fabs((double)bf16_to_f32(v[j])), X) |
                                              ((uint32_t)(v[j] >> 15) << 3))
                                           : 0u;
      cw[j / 8] |= c << (4 * (j % 8));
    }
    if (bad && flags) atomicOr(flags, 1);
  }
  if (layout == QN_LAYOUT_ROWMAJOR) {
    *reinterpret_cast<u32x4*>(codes + row * (k / 2) + k0 / 2) = u32x4{cw[0], cw[1], cw[2], cw[3]};
    scales[row * (k / 32) + k0 / 32] = (uint8_t)E;
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint32_t*>(codes + code_dword_offset(layout, row, k0 + 8 * j, k, KT)) = cw[j];
  uint32_t sb = 0u;  // zero blocks (and padding): scale 0, codes 0
  if (amax > 0.0f) {
    const int e_ref = *emax - kMxRange;
    const int d = (int)E - e_ref;
    if (d < -9) {
      if (flags) atomicOr(flags, 2);
      sb = e4m3_pow2(-9);
    } else {
      sb = e4m3_pow2(d);
    }
  }
  scales[scale_offset(layout, row, k0, k, KT)] = (uint8_t)sb;
  scales[scale_offset(layout, row, k0 + 16, k, KT)] = (uint8_t)sb;
}

// tensor scale of the tiled form: 2^(E_ref - 127), or 1 for a tensor without a nonzero weight
__global__ void k_mx_finalize(float* tensor_scale) {
  const int32_t emax = *reinterpret_cast<const int32_t*>(tensor_scale);
  *tensor_scale = emax < 0 ? 1.0f : (float)ldexp(1.0, emax - kMxRange - 127);
}

// One thread per 32-block of the canonical MXFP4 layout: w_hat = X * q, exact (X a power of two, q two significant
// bits) and rounded once to f32.
__global__ void __launch_bounds__(kQThreads) k_mx_dequant(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales, int64_t n, int64_t k,
                                                           float* __restrict__ out, int64_t ldo) {
  const int64_t kb = k / 32, idx = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (idx >= n * kb) return;
  const int64_t row = idx / kb, k0 = (idx - row * kb) * 32;
  const uint32_t E = scales[row * kb + k0 / 32];
  const double X = E == 255u ? __builtin_nan("") : ldexp(1.0, (int)E - 127);
  const u32x4 cw = *reinterpret_cast<const u32x4*>(codes + row * (k / 2) + k0 / 2);
  float* dst = out + row * ldo + k0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d = cw[j];
    auto q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    auto q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    auto q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    auto q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    const float q[8] = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 * j + i] = (float)(X * (double)q[i]);
  }
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" size_t nvfp4_tiled_codes_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)(ceil_div(n, kRowGroup) * ceil_div(k, kKTile)) * kTileCodeBytes;
}

extern "C" size_t nvfp4_tiled_scales_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)(ceil_div(n, kRowGroup) * ceil_div(k, kKTile)) * kTileScaleBytes;
}

extern "C" qn_status nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int32_t scale_mode,
                                    int32_t layout, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                                    int32_t* d_flags, void* stream) {
  if (n < 0 || k < 0 || k % 16 != 0) return QN_ERR_SHAPE;
  if (scale_mode != 0 && scale_mode != 1) return QN_ERR_VALUE;
  if (layout != QN_LAYOUT_ROWMAJOR && layout != QN_LAYOUT_TILED) return QN_ERR_VALUE;
  if (n == 0 || k == 0) return QN_OK;
  if (ldw < k) return QN_ERR_SHAPE;
  if (!w || !codes || !block_scales || !tensor_scale) return QN_ERR_NULL;
  if (!aligned(w, 2) || !aligned(codes, 16) || !aligned(tensor_scale, 4) || (d_flags && !aligned(d_flags, 4)))
    return QN_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t np = layout == QN_LAYOUT_TILED ? ceil_div(n, kRowGroup) * kRowGroup : n;
  const int64_t kp = layout == QN_LAYOUT_TILED ? ceil_div(k, kKTile) * kKTile : k;
  if (scale_mode == 0) {
    hipLaunchKernelGGL(k_quant_init, dim3(1), dim3(1), 0, s, reinterpret_cast<uint32_t*>(tensor_scale));
    const int64_t blocks = n < 1024 ? n : 1024;  // (whole rows per workgroup)
    if (aligned(w, 16) && ldw % 8 == 0)
      hipLaunchKernelGGL(k_quant_amax<true>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, w, n, k, ldw,
                         reinterpret_cast<uint32_t*>(tensor_scale), d_flags);
    else
      hipLaunchKernelGGL(k_quant_amax<false>, dim3((unsigned)blocks), dim3(kQThreads), 0, s, w, n, k, ldw,
                         reinterpret_cast<uint32_t*>(tensor_scale), d_flags);
  }
  const int64_t nblk = np * (kp / 16);
  hipLaunchKernelGGL(k_quant_blocks, dim3((unsigned)ceil_div(nblk, kQThreads)), dim3(kQThreads), 0, s, w, n, k, ldw,
                     (int)scale_mode, (int)layout, codes, block_scales, (const float*)tensor_scale, d_flags, np, kp);
  if (scale_mode == 0) hipLaunchKernelGGL(k_quant_finalize, dim3(1), dim3(1), 0, s, tensor_scale);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" qn_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale,
                                      int64_t n, int64_t k, int32_t layout, float* w_out, int64_t ldo, void* stream) {
  if (n < 0 || k < 0 || k % 16 != 0) return QN_ERR_SHAPE;
  if (layout != QN_LAYOUT_ROWMAJOR && layout != QN_LAYOUT_TILED) return QN_ERR_VALUE;
  if (n == 0 || k == 0) return QN_OK;
  if (ldo < k) return QN_ERR_SHAPE;
  if (!codes || !block_scales || !tensor_scale || !w_out) return QN_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(tensor_scale, 4) || !aligned(w_out, 4)) return QN_ERR_ALIGN;
  const int64_t KT = ceil_div(k, kKTile);
  const int64_t nblk = n * (k / 16);
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)ceil_div(nblk, kQThreads)), dim3(kQThreads), 0, (hipStream_t)stream,
                     codes, block_scales, tensor_scale, n, k, (int)layout, w_out, ldo, KT);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" size_t mxfp4_scales_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || k % 32 != 0) return 0;
  return (size_t)(n * (k / 32));
}

extern "C" qn_status mxfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int32_t layout,
                                    uint8_t* codes, uint8_t* scales, float* tensor_scale, int32_t* d_flags,
                                    void* stream) {
  if (n < 0 || k < 0 || k % 32 != 0) return QN_ERR_SHAPE;
  if (layout != QN_LAYOUT_ROWMAJOR && layout != QN_LAYOUT_TILED) return QN_ERR_VALUE;
  if (n == 0 || k == 0) return QN_OK;
  if (ldw < k) return QN_ERR_SHAPE;
  const bool tiled = layout == QN_LAYOUT_TILED;
  if (!w || !codes || !scales || (tiled && !tensor_scale)) return QN_ERR_NULL;
  if (!aligned(w, 2) || !aligned(codes, 16) || (tiled && !aligned(tensor_scale, 4)) ||
      (d_flags && !aligned(d_flags, 4)))
    return QN_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t np = tiled ? ceil_div(n, kRowGroup) * kRowGroup : n;
  const int64_t kp = tiled ? ceil_div(k, kKTile) * kKTile : k;
  int32_t* emax = reinterpret_cast<int32_t*>(tensor_scale);
  if (tiled) {
    hipLaunchKernelGGL(k_mx_init, dim3(1), dim3(1), 0, s, emax);
    hipLaunchKernelGGL(k_mx_emax, dim3((unsigned)ceil_div(n * (k / 32), kQThreads)), dim3(kQThreads), 0, s, w, n, k,
                       ldw, emax);
  }
  const int64_t nblk = np * (kp / 32);
  hipLaunchKernelGGL(k_mx_blocks, dim3((unsigned)ceil_div(nblk, kQThreads)), dim3(kQThreads), 0, s, w, n, k, ldw,
                     (int)layout, codes, scales, (const int32_t*)emax, d_flags, np, kp);
  if (tiled) hipLaunchKernelGGL(k_mx_finalize, dim3(1), dim3(1), 0, s, tensor_scale);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" qn_status mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                      float* w_out, int64_t ldo, void* stream) {
  if (n < 0 || k < 0 || k % 32 != 0) return QN_ERR_SHAPE;
  if (n == 0 || k == 0) return QN_OK;
  if (ldo < k) return QN_ERR_SHAPE;
  if (!codes || !scales || !w_out) return QN_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(w_out, 4)) return QN_ERR_ALIGN;
  hipLaunchKernelGGL(k_mx_dequant, dim3((unsigned)ceil_div(n * (k / 32), kQThreads)), dim3(kQThreads), 0,
                     (hipStream_t)stream, codes, scales, n, k, w_out, ldo);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}
