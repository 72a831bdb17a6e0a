// Two-tap dynamic depthwise convolution (pegainfer issue "DFlash 2 proposer", section
// "What upstream shipped", item 2):  y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}, with
// x_{-1} the last verified token's hidden; channel d uses tap d / group (FreeToken PR
// "Adds DFlash 2", grouped conv).
//
// A thread owns four adjacent channels of one (site, request) and walks the K draft
// positions, keeping x_{t-1} in registers, so x is read exactly once.  HBM-bound:
// 16 B per element (x, two taps, y) at group 1.
#include "device_common.h"
#include "dflash2_internal.h"

namespace df2 {

constexpr int kConvThreads = 64;   // one wave per block -> enough blocks at small batch

__device__ __forceinline__ f32x4 ld4(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)); }

__global__ void __launch_bounds__(kConvThreads) k_conv2tap_vec(const float* __restrict__ x, const float* __restrict__ x_prev,
                                                               const float* __restrict__ taps, long long lanes_per_seq,
                                                               long long nseq, int K, long long hidden,
                                                               float* __restrict__ y) {
  const long long e = (long long)blockIdx.x * kConvThreads + threadIdx.x;
  if (e >= nseq * lanes_per_seq) return;
  const long long seq = e / lanes_per_seq;                 // (site, request)
  const long long d = (e - seq * lanes_per_seq) * 4;
  const float* xs = x + (size_t)seq * K * hidden + d;
  const float* ts = taps + (size_t)seq * K * 2 * hidden + d;
  float* ys = y + (size_t)seq * K * hidden + d;
  f32x4 prev = ld4(x_prev + (size_t)seq * hidden + d);
  int t = 0;
  for (; t + 2 <= K; t += 2) {
    const f32x4 x0 = ld4(xs + (size_t)t * hidden), x1 = ld4(xs + (size_t)(t + 1) * hidden);
    const f32x4 a0 = ld4(ts + (size_t)(2 * t) * hidden), b0 = ld4(ts + (size_t)(2 * t + 1) * hidden);
    const f32x4 a1 = ld4(ts + (size_t)(2 * t + 2) * hidden), b1 = ld4(ts + (size_t)(2 * t + 3) * hidden);
    const f32x4 y0 = a0 * x0 + b0 * prev;
    const f32x4 y1 = a1 * x1 + b1 * x0;
    __builtin_nontemporal_store(y0, reinterpret_cast<f32x4*>(ys + (size_t)t * hidden));
    __builtin_nontemporal_store(y1, reinterpret_cast<f32x4*>(ys + (size_t)(t + 1) * hidden));
    prev = x1;
  }
  if (t < K) {
    const f32x4 x0 = ld4(xs + (size_t)t * hidden);
    const f32x4 a0 = ld4(ts + (size_t)(2 * t) * hidden), b0 = ld4(ts + (size_t)(2 * t + 1) * hidden);
    __builtin_nontemporal_store(a0 * x0 + b0 * prev, reinterpret_cast<f32x4*>(ys + (size_t)t * hidden));
  }
}

// General path: any group size / hidden, one thread per channel.
__global__ void __launch_bounds__(256) k_conv2tap_scalar(const float* __restrict__ x, const float* __restrict__ x_prev,
                                                         const float* __restrict__ taps, long long nseq, int K,
                                                         long long hidden, long long group, float* __restrict__ y) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= nseq * hidden) return;
  const long long seq = e / hidden, d = e - seq * hidden;
  const long long ntap = hidden / group, c = d / group;
  float prev = x_prev[seq * hidden + d];
  for (int t = 0; t < K; ++t) {
    const float xt = x[(seq * K + t) * hidden + d];
    const float* tp = taps + ((seq * K + t) * 2) * ntap + c;
    y[(seq * K + t) * hidden + d] = tp[0] * xt + tp[ntap] * prev;
    prev = xt;
  }
}

hipError_t launch_conv2tap(const float* x, const float* x_prev, const float* taps, int64_t sites, int64_t batch, int K,
                           int64_t hidden, int64_t group, float* y, hipStream_t s) {
  const long long nseq = sites * batch;
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_prev) |
                         reinterpret_cast<uintptr_t>(taps) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  if (group == 1 && hidden % 4 == 0 && aligned) {
    const long long lanes = hidden / 4;
    const long long n = nseq * lanes;
    hipLaunchKernelGGL(k_conv2tap_vec, dim3((unsigned)((n + kConvThreads - 1) / kConvThreads)), dim3(kConvThreads), 0, s,
                       x, x_prev, taps, lanes, nseq, K, hidden, y);
  } else {
    const long long n = nseq * hidden;
    hipLaunchKernelGGL(k_conv2tap_scalar, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, x_prev, taps, nseq, K,
                       hidden, group, y);
  }
  return hipGetLastError();
}

}  // namespace df2
