// Context gate kernels: the standalone bf16 path (tiles of gate_dev.h, eight waves per
// work-group, then a kernel adding the slices) and the fp32-weight path (plain fp32
// FMA, one thread per output).
#include "dflash2_internal.h"
#include "gate_dev.h"

namespace df2 {

constexpr int kGateThreads = kGateBlockThreads;
constexpr int kGateWaves = kGateThreads / 64;
constexpr int kGateTargetBlocks = 144;
constexpr int kGateRound = 2;             // 32-wide steps per wave with loads in flight together

static int gate_coltile(int64_t dim) { return dim < 64 ? (int)dim : 64; }

int gate_splits(int64_t rows, int64_t hidden, int64_t dim) {
  const int64_t tiles = ((rows + 15) / 16) * (dim / gate_coltile(dim));
  const int64_t steps = (hidden + 31) / 32;
  int64_t s = (kGateTargetBlocks + tiles - 1) / tiles;
  const int64_t ntiles = dim / gate_coltile(dim);
  const int64_t m = 8 / (ntiles % 8 == 0 ? 8 : (ntiles % 4 == 0 ? 4 : (ntiles % 2 == 0 ? 2 : 1)));
  s = (s + m - 1) / m * m;                // blocks of one weight slice land on one XCD
  const int64_t cap = steps / 4 > 1 ? steps / 4 : 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

int64_t gate_grid_blocks(int64_t rows, int64_t hidden, int64_t dim) {
  return ((rows + 15) / 16) * (dim / gate_coltile(dim)) * gate_splits(rows, hidden, dim);
}

GateWs carve_gate(Carver& c, int64_t rows, int64_t hidden, int64_t dim) {
  GateWs w;
  const int ns = gate_splits(rows, hidden, dim);
  w.partial = c.take<float>(ns > 1 ? (size_t)ns * rows * dim : 0);
  w.nsplit = ns;
  return w;
}

// NB = 16-column blocks of the tile (tile width 16 * NB = min(dim, 64)).
template <int NB>
__global__ void __launch_bounds__(kGateThreads) k_gate_bf16(const float* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int ntiles, int nsplit,
                                                            float* __restrict__ H, float* __restrict__ partial) {
  __shared__ float red[kGateWaves * 16 * 16 * NB];
  const int per = ntiles * nsplit;
  const int mt = blockIdx.x / per;
  const int rem = blockIdx.x - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  gate_tile<NB, kGateWaves, kGateRound>(h, w, bias, rows, hidden, dim, act, mt, nt, split, nsplit, red, H, partial);
}

// Sum of the slices in slice order, then bias and activation: one thread per output.
__global__ void __launch_bounds__(256) k_gate_finish(const float* __restrict__ partial, const float* __restrict__ bias,
                                                     long long n_out, int dim, int nsplit, int act,
                                                     float* __restrict__ H) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_out) return;
  const int row = (int)(e / dim), n = (int)(e - (long long)row * dim);
  H[e] = gate_finish(partial, bias, (int)(n_out / dim), dim, nsplit, act, row, n);
}

// fp32 weight: one thread per (row, column); four interleaved partial sums.
__global__ void __launch_bounds__(256) k_gate_f32(const float* __restrict__ h, const float* __restrict__ w,
                                                  const float* __restrict__ bias, int rows, int hidden, int dim, int act,
                                                  float* __restrict__ H) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)rows * dim) return;
  const int row = (int)(e / dim), n = (int)(e - (long long)row * dim);
  const float* hr = h + (size_t)row * hidden;
  const float* wr = w + (size_t)n * hidden;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < hidden; k += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(hr + k);
    const f32x4 y = *reinterpret_cast<const f32x4*>(wr + k);
    s.x = fmaf(x.x, y.x, s.x);
    s.y = fmaf(x.y, y.y, s.y);
    s.z = fmaf(x.z, y.z, s.z);
    s.w = fmaf(x.w, y.w, s.w);
  }
  const float pre = (s.x + s.y) + (s.z + s.w) + (bias ? bias[n] : 0.f);
  H[(size_t)row * dim + n] = gate_act(pre, act);
}

hipError_t launch_gate(const float* h, const void* w_h, bool w_bf16, const float* bias, int rows, int hidden, int dim,
                       int act, float* H, GateWs ws, hipStream_t s) {
  if (!w_bf16) {
    const long long n = (long long)rows * dim;
    hipLaunchKernelGGL(k_gate_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h,
                       static_cast<const float*>(w_h), bias, rows, hidden, dim, act, H);
    return hipGetLastError();
  }
  const int ct = gate_coltile(dim);
  const int ntiles = dim / ct;
  const int mtiles = (rows + 15) / 16;
  const int nsplit = ws.nsplit;
  const dim3 grid((unsigned)((long long)mtiles * ntiles * nsplit));
  const uint16_t* w = static_cast<const uint16_t*>(w_h);
  switch (ct / 16) {
    case 1:
      hipLaunchKernelGGL(k_gate_bf16<1>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, ntiles,
                         nsplit, H, ws.partial);
      break;
    case 2:
      hipLaunchKernelGGL(k_gate_bf16<2>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, ntiles,
                         nsplit, H, ws.partial);
      break;
    case 4:
      hipLaunchKernelGGL(k_gate_bf16<4>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, ntiles,
                         nsplit, H, ws.partial);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (nsplit > 1) {
    const long long n = (long long)rows * dim;
    hipLaunchKernelGGL(k_gate_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws.partial, bias, n, dim,
                       nsplit, act, H);
  }
  return hipGetLastError();
}

}  // namespace df2
