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

}  // namespace
}  // namespace qn

using namespace qn;

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
