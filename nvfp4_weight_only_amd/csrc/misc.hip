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
