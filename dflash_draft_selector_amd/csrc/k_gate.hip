// Context gate H = act(W_H h + b) (pegainfer issue "DFlash 2 proposer", section
// "What upstream shipped", item 1: 256-dim token embeddings + context gate).
//
// bf16 weight: h is rounded to bf16 (nearest even) as it is loaded and the product
// runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A block owns a 16-row x
// (up to) 64-column output tile over one slice of the hidden dimension; its four
// waves take interleaved 32-wide steps of the slice and are summed in LDS in a fixed
// order.  With several slices, each block stores its tile as a partial sum and a
// second kernel adds the slices in slice order, then the bias and the activation, so
// results never depend on scheduling.  fp32 weight: plain fp32 FMA, one thread per
// output.
#include "device_common.h"
#include "dflash2_internal.h"

namespace df2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGateThreads = 256;
constexpr int kGateTargetBlocks = 288;
constexpr int kGateRound = 4;             // 32-wide steps per wave with loads in flight together

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

__device__ __forceinline__ float gate_act(float x, int act) { return act == 0 ? 1.f / (1.f + expf(-x)) : x; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// NB = 16-column blocks of the tile (tile width 16 * NB = min(dim, 64)).
template <int NB>
__global__ void __launch_bounds__(kGateThreads) k_gate_bf16(const float* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int ntiles, int nsplit,
                                                            float* __restrict__ H, float* __restrict__ partial) {
  constexpr int kCols = 16 * NB;
  __shared__ float red[4][16][kCols];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int per = ntiles * nsplit;
  const int mt = blockIdx.x / per;
  const int rem = blockIdx.x - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  const int nsteps = (hidden + 31) / 32;
  const int s0 = (int)((long long)nsteps * split / nsplit), s1 = (int)((long long)nsteps * (split + 1) / nsplit);

  const int arow = mt * 16 + r16;
  const bool arow_ok = arow < rows;
  const float* hrow = h + (size_t)(arow_ok ? arow : 0) * hidden;
  const uint16_t* wcol[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) wcol[j] = w + (size_t)(nt * kCols + j * 16 + r16) * hidden;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int base = s0 + wv; base < s1; base += 4 * kGateRound) {
    f32x4 x0[kGateRound], x1[kGateRound];
    u32x4 bw[kGateRound][NB];
#pragma unroll
    for (int i = 0; i < kGateRound; ++i) {
      const int st = base + 4 * i;
      const int k = st * 32 + g * 8;
      const bool kok = st < s1 && k < hidden;
      x0[i] = x1[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (kok && arow_ok) {
        x0[i] = *reinterpret_cast<const f32x4*>(hrow + k);
        x1[i] = *reinterpret_cast<const f32x4*>(hrow + k + 4);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        bw[i][j] = (u32x4){0u, 0u, 0u, 0u};
        if (kok) bw[i][j] = *reinterpret_cast<const u32x4*>(wcol[j] + k);
      }
    }
#pragma unroll
    for (int i = 0; i < kGateRound; ++i) {
      u32x4 a;
      a.x = pack_bf16x2(x0[i].x, x0[i].y);
      a.y = pack_bf16x2(x0[i].z, x0[i].w);
      a.z = pack_bf16x2(x1[i].x, x1[i].y);
      a.w = pack_bf16x2(x1[i].z, x1[i].w);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, bw[i][j]), acc[j], 0, 0, 0);
    }
  }

  // D layout: lane l, register r -> row 4 * (l / 16) + r, column l % 16 of each block
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wv][4 * g + r][j * 16 + r16] = acc[j][r];
  __syncthreads();
  for (int e = tid; e < 16 * kCols; e += kGateThreads) {
    const int rr = e / kCols, c = e - rr * kCols;
    const int row = mt * 16 + rr;
    if (row >= rows) continue;
    const int n = nt * kCols + c;
    const float sum = ((red[0][rr][c] + red[1][rr][c]) + red[2][rr][c]) + red[3][rr][c];
    if (nsplit == 1)
      H[(size_t)row * dim + n] = gate_act(sum + (bias ? bias[n] : 0.f), act);
    else
      partial[((size_t)split * rows + row) * dim + n] = sum;
  }
}

// Sum of the slices in slice order, then bias and activation: one thread per output.
__global__ void __launch_bounds__(256) k_gate_finish(const float* __restrict__ partial, const float* __restrict__ bias,
                                                     long long n_out, int dim, int nsplit, int act,
                                                     float* __restrict__ H) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_out) return;
  const int n = (int)(e % dim);
  float sum = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < nsplit; ++sp) sum += partial[(size_t)sp * n_out + e];
  H[e] = gate_act(sum + (bias ? bias[n] : 0.f), act);
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
