// AQN-RMSNorm device routines, shared by the standalone norm and the fused prologue of the linear so that both
// produce bit-identical bf16 activations.
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review),
// §5.1: u = x / sqrt(mean_j x_j^2 + delta), h_z = u (.) (w + z); the noise z = sigma * eps is added to the clean
// norm scale w on the fly, so the scale itself is never modified.
//
// A row is held in registers as chunks of 8 bf16: chunk c belongs to thread c % NT, slot c / NT. The sum of squares
// runs in a fixed order (per thread: slots in order, elements in order; then a butterfly over the wave; then the
// waves in order), so every kernel using these routines with the same NT gets the same bits.
#pragma once
#include "qn_device.hpp"
#include "qn_rng.hpp"

namespace qn {

// threads per row: 256 up to 32768 elements, else 1024 (the library rejects rows longer than 131072)
__host__ __device__ inline int norm_threads(int64_t d) { return d <= 32768 ? 256 : 1024; }

template <int CPT>
struct RowRegs {
  uint32_t v[CPT][4];  // chunk i of this thread: 8 bf16, two per dword (low half = even element)
};

// Load the row's chunks (elements beyond d read as 0). vec_ok: the row start is 16-byte aligned.
template <int NT, int CPT>
__device__ inline void load_row(const uint16_t* __restrict__ xr, int64_t d, bool vec_ok, RowRegs<CPT>& r) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
    if (vec_ok && j0 + 8 <= d) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(xr + j0);
      r.v[i][0] = q[0]; r.v[i][1] = q[1]; r.v[i][2] = q[2]; r.v[i][3] = q[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (j0 + 2 * e < d) ? xr[j0 + 2 * e] : 0u;
        const uint32_t hi = (j0 + 2 * e + 1 < d) ? xr[j0 + 2 * e + 1] : 0u;
        r.v[i][e] = lo | (hi << 16);
      }
    }
  }
}

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Block-wide sum of squares of the row in the fixed order above. `red` is __shared__ float[NT / 64].
template <int NT, int CPT>
__device__ inline float row_sumsq(const RowRegs<CPT>& r, float* red) {
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = lo_bf16(r.v[i][e]), b = hi_bf16(r.v[i][e]);
      ss = __fadd_rn(ss, __fmul_rn(a, a));
      ss = __fadd_rn(ss, __fmul_rn(b, b));
    }
  ss = wave_sum(ss);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) tot = __fadd_rn(tot, red[w]);
  __syncthreads();
  return tot;
}

// The same sum of squares computed by one wave alone, in exactly the order row_sumsq<NT, CPT> takes with NT threads:
// lane l stands in for threads l, l + 64, ..., each summing its own chunks (c = t, t + NT, ...); the wave totals of
// those stand-ins are then added in order. The row is read in whole 8-element chunks (d % 8 == 0, 16-byte aligned
// chunks when vec_ok, else element loads). Every lane returns the total.
template <int NT>
__device__ inline float row_sumsq_one_wave(const uint16_t* __restrict__ xr, int64_t d, bool vec_ok) {
  constexpr int V = NT / kWave;           // stand-in threads per lane
  constexpr int VB = V < 8 ? V : 8;       // stand-ins whose chunks are loaded together
  constexpr int IB = 8 / VB;              // chunk rounds loaded together
  const int lane = threadIdx.x % kWave;
  const int64_t nch = d / 8;
  float ss[V];
#pragma unroll
  for (int v = 0; v < V; ++v) ss[v] = 0.0f;
  for (int64_t i0 = 0; i0 * NT < nch; i0 += IB) {
#pragma unroll
    for (int v0 = 0; v0 < V; v0 += VB) {
      uint32_t q[IB][VB][4];
#pragma unroll
      for (int ib = 0; ib < IB; ++ib)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const int64_t c = (i0 + ib) * NT + (v0 + vb) * kWave + lane;
          if (c < nch && vec_ok) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(xr + c * 8);
            q[ib][vb][0] = w[0]; q[ib][vb][1] = w[1]; q[ib][vb][2] = w[2]; q[ib][vb][3] = w[3];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              q[ib][vb][e] = c < nch ? (uint32_t)xr[c * 8 + 2 * e] | ((uint32_t)xr[c * 8 + 2 * e + 1] << 16) : 0u;
          }
        }
      // each stand-in adds its chunks in chunk order (ib ascending), elements in order
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          if ((i0 + ib) * NT + (v0 + vb) * kWave + lane >= nch) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = lo_bf16(q[ib][vb][e]), b = hi_bf16(q[ib][vb][e]);
            ss[v0 + vb] = __fadd_rn(ss[v0 + vb], __fmul_rn(a, a));
            ss[v0 + vb] = __fadd_rn(ss[v0 + vb], __fmul_rn(b, b));
          }
        }
    }
  }
  float tot = 0.0f;
#pragma unroll
  for (int v = 0; v < V; ++v) tot = __fadd_rn(tot, wave_sum(ss[v]));
  return tot;
}

// rstd = 1 / sqrt(ss / d + eps), each operation correctly rounded.
__device__ inline float rms_rstd(float ss, int64_t d, float eps) {
  return __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(ss, (float)d), eps)));
}

// One normalized, noised activation rounded to bf16: h = bf16(x * rstd * (gamma + sigma * noise)).
__device__ inline uint16_t aqn_value(float x, float rstd, uint16_t gb, float noise, float sigma) {
  const float g = __fadd_rn(bf16_to_f32(gb), __fmul_rn(sigma, noise));
  return f32_to_bf16(__fmul_rn(__fmul_rn(x, rstd), g));
}

// The norm scale and noise of this thread's chunks, fetched together with the row so that one memory round trip
// serves all three. vec_g / vec_z: gamma / the noise row are 16-byte aligned at chunk starts. With a draw (q.on) the
// noise of row `row` is generated instead of read.
template <int CPT>
struct ScaleRegs {
  uint32_t g[CPT][4];  // gamma, bf16 pairs
  float z[CPT][8];     // noise
};

template <int NT, int CPT>
__device__ inline void load_scales(const uint16_t* __restrict__ gamma, const float* __restrict__ noise, int64_t d,
                                   bool vec_g, bool vec_z, const QnDraw& q, int64_t row, ScaleRegs<CPT>& sr) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
    if (vec_g && j0 + 8 <= d) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(gamma + j0);
      sr.g[i][0] = q[0]; sr.g[i][1] = q[1]; sr.g[i][2] = q[2]; sr.g[i][3] = q[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (j0 + 2 * e < d) ? gamma[j0 + 2 * e] : 0u;
        const uint32_t hi = (j0 + 2 * e + 1 < d) ? gamma[j0 + 2 * e + 1] : 0u;
        sr.g[i][e] = lo | (hi << 16);
      }
    }
    if (q.on) {
      if (j0 < d) aqn_noise8(q, draw_index(q, row), (uint64_t)(j0 / 8), sr.z[i]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) sr.z[i][e] = 0.0f;
    } else if (noise && vec_z && j0 + 8 <= d) {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(noise + j0);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(noise + j0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { sr.z[i][e] = a[e]; sr.z[i][4 + e] = b[e]; }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) sr.z[i][e] = (noise && j0 + e < d) ? noise[j0 + e] : 0.0f;
    }
  }
}

// Apply the norm to the row in place (elements at or beyond d stay 0).
template <int NT, int CPT>
__device__ inline void apply_aqn(RowRegs<CPT>& r, const ScaleRegs<CPT>& sr, int64_t d, float rstd, float sigma) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t j = j0 + 2 * e;
      uint32_t lo = 0u, hi = 0u;
      if (j < d) lo = aqn_value(lo_bf16(r.v[i][e]), rstd, (uint16_t)sr.g[i][e], sr.z[i][2 * e], sigma);
      if (j + 1 < d) hi = aqn_value(hi_bf16(r.v[i][e]), rstd, (uint16_t)(sr.g[i][e] >> 16), sr.z[i][2 * e + 1], sigma);
      r.v[i][e] = lo | (hi << 16);
    }
  }
}

}  // namespace qn
