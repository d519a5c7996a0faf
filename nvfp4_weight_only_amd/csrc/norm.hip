// Standalone AQN-RMSNorm ("QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops",
// technical review §5.1): h = bf16(x * rstd * (gamma + sigma * noise)), one workgroup per row. It runs the same
// device routines as the fused prologue of nvfp4_lora_linear, so both produce identical bf16 activations.
#include <cmath>

#include "qn_device.hpp"
#include "qn_norm.hpp"

namespace qn {
namespace {

template <int NT, int CPT>
__global__ void __launch_bounds__(NT) k_aqn_rmsnorm(const uint16_t* __restrict__ x, int64_t d, int64_t ldx,
                                                     const uint16_t* __restrict__ gamma, const float* __restrict__ noise,
                                                     int64_t noise_ld, QnDraw q, float sigma, float eps,
                                                     uint16_t* __restrict__ h, int64_t ldh, int vec_in, int vec_out,
                                                     int vec_g, int vec_z) {
  __shared__ float red[NT / kWave];
  const int64_t row = blockIdx.x;
  RowRegs<CPT> r;
  ScaleRegs<CPT> sr;
  const float* nz = noise ? noise + row * noise_ld : nullptr;
  load_row<NT, CPT>(x + row * ldx, d, vec_in != 0, r);
  load_scales<NT, CPT>(gamma, nz, d, vec_g != 0, vec_z != 0, q, row, sr);
  const float rstd = rms_rstd(row_sumsq<NT, CPT>(r, red), d, eps);
  apply_aqn<NT, CPT>(r, sr, d, rstd, sigma);
  uint16_t* hr = h + row * ldh;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
    if (j0 >= d) continue;
    if (vec_out && j0 + 8 <= d) {
      *reinterpret_cast<u32x4*>(hr + j0) = u32x4{r.v[i][0], r.v[i][1], r.v[i][2], r.v[i][3]};
    } else {
      for (int e = 0; e < 8 && j0 + e < d; ++e) hr[j0 + e] = (uint16_t)(r.v[i][e / 2] >> (16 * (e % 2)));
    }
  }
}

template <int NT, int CPT>
void launch_norm(int64_t m, hipStream_t s, const uint16_t* x, int64_t d, int64_t ldx, const qn_aqn* a, uint16_t* h,
                 int64_t ldh, int vec_in, int vec_out) {
  const int vec_g = (uintptr_t)a->gamma % 16 == 0;
  const int vec_z = a->noise && (uintptr_t)a->noise % 16 == 0 && a->noise_ld % 4 == 0;
  const QnDraw q{a->draw ? 1 : 0, a->seed, a->subseed, a->row_offset, a->draw_rows, 0};
  hipLaunchKernelGGL((k_aqn_rmsnorm<NT, CPT>), dim3((unsigned)m), dim3(NT), 0, s, x, d, ldx, a->gamma, a->noise,
                     a->noise_ld, q, a->sigma, a->eps, h, ldh, vec_in, vec_out, vec_g, vec_z);
}

// aqn_noise: one thread per 8-column block of a row.
__global__ void __launch_bounds__(256) k_aqn_noise(QnDraw q, int64_t m, int64_t d, float* __restrict__ eps,
                                                   int64_t ld) {
  const int64_t nb = (d + 7) / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= m * nb) return;
  const int64_t row = id / nb, c = id % nb;
  float z[8];
  aqn_noise8(q, draw_index(q, row), (uint64_t)c, z);
  float* out = eps + row * ld + c * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c * 8 + e < d) out[e] = z[e];
}

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" qn_status aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, int64_t ldx, const qn_aqn* aqn, uint16_t* h,
                                 int64_t ldh, void* stream) {
  if (m < 0 || d < 0) return QN_ERR_SHAPE;
  if (!aqn) return QN_ERR_NULL;
  if (!(aqn->sigma >= 0.0f) || !std::isfinite(aqn->sigma) || !(aqn->eps >= 0.0f) || !std::isfinite(aqn->eps))
    return QN_ERR_VALUE;
  if (m == 0 || d == 0) return QN_OK;
  if (d > 131072) return QN_ERR_UNSUPPORTED;
  if (!x || !h || !aqn->gamma) return QN_ERR_NULL;
  if (ldx < d || ldh < d) return QN_ERR_SHAPE;
  if (aqn->noise && (aqn->noise_ld < 0 || (aqn->noise_ld > 0 && aqn->noise_ld < d))) return QN_ERR_SHAPE;
  if (aqn->draw && aqn->noise) return QN_ERR_VALUE;  // noise is either read or drawn
  if (aqn->draw && aqn->draw_rows < 0) return QN_ERR_SHAPE;
  if (((uintptr_t)x % 2) || ((uintptr_t)h % 2)) return QN_ERR_ALIGN;
  const int vec_in = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0);
  const int vec_out = ((uintptr_t)h % 16 == 0) && (ldh % 8 == 0);
  hipStream_t s = (hipStream_t)stream;
  const int nt = norm_threads(d);
  const int64_t cpt = ceil_div(ceil_div(d, 8), nt);
  if (nt == 256) {
    if (cpt <= 1) launch_norm<256, 1>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
    else if (cpt <= 2) launch_norm<256, 2>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
    else if (cpt <= 4) launch_norm<256, 4>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
    else if (cpt <= 8) launch_norm<256, 8>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
    else launch_norm<256, 16>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
  } else {
    launch_norm<1024, 16>(m, s, x, d, ldx, aqn, h, ldh, vec_in, vec_out);
  }
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" qn_status aqn_noise(uint64_t seed, uint64_t subseed, uint64_t row_offset, int64_t draw_rows, int64_t m,
                               int64_t d, float* eps, int64_t ld, void* stream) {
  if (m < 0 || d < 0 || draw_rows < 0) return QN_ERR_SHAPE;
  if (m == 0 || d == 0) return QN_OK;
  if (!eps) return QN_ERR_NULL;
  if (ld < d) return QN_ERR_SHAPE;
  if ((uintptr_t)eps % 4) return QN_ERR_ALIGN;
  const int64_t blocks = ceil_div(m * ceil_div(d, 8), 256);
  if (blocks > 0x7fffffff) return QN_ERR_UNSUPPORTED;
  const QnDraw q{1, seed, subseed, row_offset, draw_rows, 0};
  hipLaunchKernelGGL(k_aqn_noise, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, q, m, d, eps, ld);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}
