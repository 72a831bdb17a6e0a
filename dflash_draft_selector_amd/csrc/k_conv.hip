// Two-tap dynamic depthwise convolution (pegainfer issue "DFlash 2 proposer", section
// "What upstream shipped", item 2):  y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}, with
// x_{-1} the last verified token's hidden; channel d uses tap d / group (FreeToken PR
// "Adds DFlash 2", grouped conv).
//
// A thread owns four adjacent channels of one (site, request, position): one round of
// independent 16-byte loads (x_t, x_{t-1} or the previous hidden, both taps) and one
// store.  HBM-bound: 16 B per element (x, two taps, y) at group 1; the second read of
// x_{t-1} is served by the cache the neighbouring position's thread just filled.
#include "device_common.h"
#include "dflash2_internal.h"

namespace df2 {

constexpr int kConvThreads = 256;

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

__global__ void __launch_bounds__(kConvThreads) k_conv2tap_vec(const float* __restrict__ x, const float* __restrict__ x_prev,
                                                               const float* __restrict__ taps, long long lanes_per_row,
                                                               long long nrows, int K, long long hidden,
                                                               float* __restrict__ y) {
  const long long e = (long long)blockIdx.x * kConvThreads + threadIdx.x;
  if (e >= nrows * lanes_per_row) return;
  const long long row = e / lanes_per_row;                 // (site, request, position)
  const long long d = (e - row * lanes_per_row) * 4;
  const long long seq = row / K;
  const int t = (int)(row - seq * K);
  const f32x4 xt = ld4(x + (size_t)row * hidden + d);
  const f32x4 xp = t == 0 ? ld4(x_prev + (size_t)seq * hidden + d) : ld4(x + (size_t)(row - 1) * hidden + d);
  const f32x4 k0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(taps + (size_t)(2 * row) * hidden + d));
  const f32x4 k1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(taps + (size_t)(2 * row + 1) * hidden + d));
  __builtin_nontemporal_store(k0 * xt + k1 * xp, reinterpret_cast<f32x4*>(y + (size_t)row * hidden + d));
}

// General path: any group size / hidden, one thread per (site, request, position,
// channel).
__global__ void __launch_bounds__(256) k_conv2tap_scalar(const float* __restrict__ x, const float* __restrict__ x_prev,
                                                         const float* __restrict__ taps, long long nrows, int K,
                                                         long long hidden, long long group, float* __restrict__ y) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= nrows * hidden) return;
  const long long row = e / hidden, d = e - row * hidden;
  const long long seq = row / K;
  const int t = (int)(row - seq * K);
  const long long ntap = hidden / group, c = d / group;
  const float xt = x[row * hidden + d];
  const float xp = t == 0 ? x_prev[seq * hidden + d] : x[(row - 1) * hidden + d];
  const float* tp = taps + (2 * row) * ntap + c;
  y[row * hidden + d] = tp[0] * xt + tp[ntap] * xp;
}

hipError_t launch_conv2tap(const float* x, const float* x_prev, const float* taps, int64_t sites, int64_t batch, int K,
                           int64_t hidden, int64_t group, float* y, hipStream_t s) {
  const long long nseq = sites * batch;
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_prev) |
                         reinterpret_cast<uintptr_t>(taps) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  if (group == 1 && hidden % 4 == 0 && aligned) {
    const long long lanes = hidden / 4;
    const long long n = nseq * K * lanes;
    hipLaunchKernelGGL(k_conv2tap_vec, dim3((unsigned)((n + kConvThreads - 1) / kConvThreads)), dim3(kConvThreads), 0, s,
                       x, x_prev, taps, lanes, nseq * K, K, hidden, y);
  } else {
    const long long n = nseq * K * hidden;
    hipLaunchKernelGGL(k_conv2tap_scalar, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, x_prev, taps, nseq * K,
                       K, hidden, group, y);
  }
  return hipGetLastError();
}

}  // namespace df2
