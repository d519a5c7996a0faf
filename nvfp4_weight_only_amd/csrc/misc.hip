// Small pieces of the rollout step around the linear layer.
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review):
//   §5.2 exponential AQN schedule with a zero-noise warm-up stage; §2.2 group-relative advantages with the
//   population standard deviation.
#include <cmath>

#include "qn_device.hpp"

namespace qn {
namespace {

// One thread per group; fp64 on the device, rounded once to f32.
__global__ void k_group_advantage(const float* __restrict__ rewards, int groups, int g, double eps,
                                  float* __restrict__ adv) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= groups) return;
  const float* R = rewards + (int64_t)q * g;
  double mean = 0.0;
  for (int i = 0; i < g; ++i) mean += (double)R[i];
  mean /= (double)g;
  double var = 0.0;
  for (int i = 0; i < g; ++i) {
    const double dv = (double)R[i] - mean;
    var += dv * dv;
  }
  const double denom = sqrt(var / (double)g) + eps;
  for (int i = 0; i < g; ++i) adv[(int64_t)q * g + i] = (float)(((double)R[i] - mean) / denom);
}

// GRPO token ratio and clipped surrogate [review §2.3], one workgroup of 1024 threads over the whole batch: the
// valid-token counts first (they set each token's weight), then per token rho = exp(log pi_theta - log pi_b),
// s = min(rho A, clip(rho) A) and the gradient -w rho A (or 0 where the clipped term is strictly smaller), in fp64 from
// the f32 inputs. Each thread takes tokens q = tid, tid + 1024, ... in order and the block sums in a fixed tree, so the
// statistics do not depend on scheduling.
constexpr int kGrpoThreads = 1024;

__device__ inline double wave_sum_f64(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <class T, class Op>
__device__ inline T block_reduce(T v, T* s_part, Op op) {
  for (int off = 32; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) s_part[w] = v;
  __syncthreads();
  T r = s_part[0];
  for (int i = 1; i < kGrpoThreads / kWave; ++i) r = op(r, s_part[i]);
  return r;
}

__global__ void __launch_bounds__(kGrpoThreads) k_grpo_surrogate(const float* __restrict__ logp,
                                                                 const float* __restrict__ logp_old, int64_t ld,
                                                                 const int32_t* __restrict__ lengths,
                                                                 const float* __restrict__ adv, int n_seq, int t_max,
                                                                 double lo, double hi, int agg,
                                                                 float* __restrict__ sur, float* __restrict__ grad,
                                                                 qn_grpo_stats* __restrict__ stats) {
  __shared__ double s_d[kGrpoThreads / kWave];
  __shared__ int64_t s_i[kGrpoThreads / kWave];
  auto len_of = [&](int i) { const int L = lengths[i]; return L < 0 ? 0 : (L > t_max ? t_max : L); };
  int64_t n_tok = 0, n_ne = 0;
  for (int i = threadIdx.x; i < n_seq; i += kGrpoThreads) {
    const int L = len_of(i);
    n_tok += L;
    n_ne += L > 0 ? 1 : 0;
  }
  const auto add_i = [](int64_t a, int64_t b) { return a + b; };
  n_tok = block_reduce<int64_t>(n_tok, s_i, add_i);
  n_ne = block_reduce<int64_t>(n_ne, s_i, add_i);
  double loss = 0.0, rsum = 0.0, rmin = INFINITY, rmax = -INFINITY;
  int64_t clipped = 0;
  const int64_t total = (int64_t)n_seq * t_max;
  for (int64_t q = threadIdx.x; q < total; q += kGrpoThreads) {
    const int i = (int)(q / t_max), t = (int)(q % t_max);
    const int L = len_of(i);
    const int64_t k = (int64_t)i * ld + t;
    if (t >= L) {
      if (sur) sur[k] = 0.0f;
      if (grad) grad[k] = 0.0f;
      continue;
    }
    const double A = (double)adv[i];
    const double w = agg == 0 ? 1.0 / (double)n_tok : 1.0 / ((double)n_ne * (double)L);
    const double rho = exp((double)logp[k] - (double)logp_old[k]);
    const double unclipped = rho * A;
    const double clipped_term = (rho < lo ? lo : (rho > hi ? hi : rho)) * A;
    const bool take_unclipped = unclipped <= clipped_term;
    const double s = take_unclipped ? unclipped : clipped_term;
    if (sur) sur[k] = (float)s;
    if (grad) grad[k] = take_unclipped ? (float)(-w * unclipped) : 0.0f;
    clipped += take_unclipped ? 0 : 1;
    loss -= w * s;
    rsum += rho;
    rmin = fmin(rmin, rho);
    rmax = fmax(rmax, rho);
  }
  const auto add_d = [](double a, double b) { return a + b; };
  loss = block_reduce<double>(loss, s_d, add_d);
  rsum = block_reduce<double>(rsum, s_d, add_d);
  rmin = block_reduce<double>(rmin, s_d, [](double a, double b) { return fmin(a, b); });
  rmax = block_reduce<double>(rmax, s_d, [](double a, double b) { return fmax(a, b); });
  clipped = block_reduce<int64_t>(clipped, s_i, add_i);
  if (threadIdx.x == 0) {
    stats->loss = loss;
    stats->ratio_mean = n_tok > 0 ? rsum / (double)n_tok : 0.0;
    stats->ratio_min = n_tok > 0 ? (float)rmin : 0.0f;
    stats->ratio_max = n_tok > 0 ? (float)rmax : 0.0f;
    stats->tokens = n_tok;
    stats->clipped = clipped;
  }
}

// Plain streaming read: every 16-byte piece of [src, src + 16 n16) loaded once (non-temporal), four loads in flight per
// thread, folded into an XOR that one lane per wave publishes (so the loads cannot be dropped).
__global__ void __launch_bounds__(256) k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, kWave);
  if (threadIdx.x % kWave == 0) atomicXor(sink, v);
}

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" qn_status grpo_clipped_surrogate(const float* logp, const float* logp_old, int64_t ld, const int32_t* lengths,
                                            const float* adv, int32_t n_seq, int32_t t_max, float clip_low,
                                            float clip_high, int32_t agg, float* surrogate, float* grad,
                                            qn_grpo_stats* stats, void* stream) {
  if (n_seq < 0 || t_max < 0 || (n_seq > 0 && ld < t_max)) return QN_ERR_SHAPE;  // (no row: any stride)
  if (!std::isfinite(clip_low) || !std::isfinite(clip_high) || clip_low < 0.0f || clip_low >= 1.0f ||
      clip_high < 0.0f || (agg != 0 && agg != 1))
    return QN_ERR_VALUE;
  if (!stats) return QN_ERR_NULL;
  if (n_seq > 0 && t_max > 0 && (!logp || !logp_old || !lengths || !adv)) return QN_ERR_NULL;
  if (n_seq > 0 && !lengths) return QN_ERR_NULL;
  if ((int64_t)n_seq * t_max >= ((int64_t)1 << 40)) return QN_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_grpo_surrogate, dim3(1), dim3(kGrpoThreads), 0, (hipStream_t)stream, logp, logp_old, ld,
                     lengths, adv, (int)n_seq, (int)t_max, 1.0 - (double)clip_low, 1.0 + (double)clip_high, (int)agg,
                     surrogate, grad, stats);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" qn_status qn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16 != 0) return QN_ERR_SHAPE;
  if (bytes == 0) return QN_OK;
  if (!src || !sink) return QN_ERR_NULL;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return QN_ERR_ALIGN;
  hipLaunchKernelGGL(k_stream_read, dim3(256 * 8), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" double aqn_sigma(int32_t stage, double sigma_start, double sigma_end) {
  if (stage <= 0) return 0.0;
  return sigma_start * std::pow(sigma_end / sigma_start, (double)(stage - 1) / 8.0);
}

extern "C" qn_status grpo_group_advantage(const float* rewards, int32_t groups, int32_t g, float eps, float* adv,
                                          void* stream) {
  if (groups < 0 || g < 0) return QN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return QN_ERR_VALUE;
  if (groups == 0 || g == 0) return QN_OK;
  if (!rewards || !adv) return QN_ERR_NULL;
  hipLaunchKernelGGL(k_group_advantage, dim3((unsigned)((groups + 63) / 64)), dim3(64), 0, (hipStream_t)stream,
                     rewards, (int)groups, (int)g, (double)eps, adv);
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

extern "C" const char* qn_status_string(qn_status s) {
  switch (s) {
    case QN_OK: return "ok";
    case QN_ERR_NULL: return "a required pointer is NULL";
    case QN_ERR_SHAPE: return "invalid shape or leading dimension";
    case QN_ERR_ALIGN: return "pointer not aligned as required";
    case QN_ERR_VALUE: return "scalar argument out of range";
    case QN_ERR_WORKSPACE: return "workspace missing or too small";
    case QN_ERR_UNSUPPORTED: return "request not supported by this library";
    case QN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}
