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

// Tensor amax over finite elements (as f32 bit patterns: ordered like the values for non-negative floats).
__global__ void __launch_bounds__(kQThreads) k_quant_amax(const uint16_t* __restrict__ w, int64_t n, int64_t k,
                                                           int64_t ldw, uint32_t* amax_bits, int32_t* flags) {
  float m = 0.0f;
  bool bad = false;
  const int64_t total = n * k;
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kQThreads) {
    int64_t row = i / k, col = i - row * k;
    uint16_t b = w[row * ldw + col];
    if (!bf16_finite(b)) { bad = true; continue; }
    m = fmaxf(m, fabsf(bf16_to_f32(b)));
  }
  m = wave_max(m);
  if ((threadIdx.x % kWave) == 0) atomicMax(amax_bits, __float_as_uint(m));
  if (bad && flags) atomicOr(flags, 1);
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
    int64_t blocks = ceil_div(n * k, kQThreads);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_quant_amax, dim3((unsigned)blocks), dim3(kQThreads), 0, s, w, n, k, ldw,
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
