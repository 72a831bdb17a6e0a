// Context gate H = act(W_H h + b) (pegainfer issue "DFlash 2 proposer", section
// "What upstream shipped", item 1: 256-dim token embeddings + context gate).
//
// bf16 weight: h is rounded to bf16 (nearest even) as it is loaded and the product
// runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A block owns 16 rows and
// all `dim` columns over one slice of the hidden dimension; the slices of an M-tile
// are reduced in a fixed order by the block that finishes last, so results do not
// depend on scheduling.  fp32 weight: plain fp32 FMA, one thread per output.
#include "device_common.h"
#include "dflash2_internal.h"

namespace df2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGateThreads = 256;
constexpr int kGateTargetBlocks = 512;

int gate_splits(int64_t rows, int64_t hidden) {
  const int64_t mtiles = (rows + 15) / 16;
  const int64_t steps = (hidden + 31) / 32;
  int64_t s = (kGateTargetBlocks + mtiles - 1) / mtiles;
  if (s > 16) s = 16;
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  return (int)s;
}

GateWs carve_gate(Carver& c, int64_t rows, int64_t hidden, int64_t dim) {
  GateWs w;
  const int64_t mtiles = (rows + 15) / 16;
  const int ns = gate_splits(rows, hidden);
  w.partial = c.take<float>(ns > 1 ? (size_t)ns * mtiles * 16 * dim : 0);
  w.ticket = c.take<unsigned int>((size_t)mtiles);
  return w;
}

__device__ __forceinline__ float gate_act(float x, int act) { return act == 0 ? 1.f / (1.f + expf(-x)) : x; }

// NBW = 16-column blocks handled by each of the 4 waves (dim = 64 * NBW, or a smaller
// power of two with NBW = 1 and idle waves).
template <int NBW>
__global__ void __launch_bounds__(kGateThreads) k_gate_bf16(const float* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int nsplit, float* __restrict__ H,
                                                            GateWs ws) {
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int mt = blockIdx.x / nsplit;
  const int split = blockIdx.x - mt * nsplit;
  const int nsteps = (hidden + 31) / 32;
  const int st0 = (int)((long long)nsteps * split / nsplit), st1 = (int)((long long)nsteps * (split + 1) / nsplit);
  const int nblk = dim / 16;

  const int arow = mt * 16 + r16;
  const bool arow_ok = arow < rows;
  const float* hrow = h + (size_t)(arow_ok ? arow : 0) * hidden;

  f32x4 acc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int st = st0; st < st1; ++st) {
    const int k = st * 32 + g * 8;
    const bool kok = k < hidden;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (kok && arow_ok) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(hrow + k);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(hrow + k + 4);
      a.x = f32_to_bf16_rne(x0.x) | (f32_to_bf16_rne(x0.y) << 16);
      a.y = f32_to_bf16_rne(x0.z) | (f32_to_bf16_rne(x0.w) << 16);
      a.z = f32_to_bf16_rne(x1.x) | (f32_to_bf16_rne(x1.y) << 16);
      a.w = f32_to_bf16_rne(x1.z) | (f32_to_bf16_rne(x1.w) << 16);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int blk = wv + 4 * j;
      if (blk < nblk) {
        const int n = blk * 16 + r16;
        u32x4 bfr = {0u, 0u, 0u, 0u};
        if (kok) bfr = *reinterpret_cast<const u32x4*>(w + (size_t)n * hidden + k);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bfr),
                                                         acc[j], 0, 0, 0);
      }
    }
  }

  // D layout: lane l, register r -> row 4 * (l / 16) + r, column l % 16 of the block.
  if (nsplit == 1) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int blk = wv + 4 * j;
      if (blk < nblk) {
        const int n = blk * 16 + r16;
        const float bn = bias ? bias[n] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mt * 16 + 4 * g + r;
          if (row < rows) H[(size_t)row * dim + n] = gate_act(acc[j][r] + bn, act);
        }
      }
    }
    return;
  }
  const int mrows = gridDim.x / nsplit * 16;
  float* part = ws.partial + ((size_t)split * mrows + (size_t)mt * 16) * dim;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int blk = wv + 4 * j;
    if (blk < nblk) {
      const int n = blk * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) st_agent(part + (size_t)(4 * g + r) * dim + n, (float)acc[j][r]);
    }
  }
  if (!arrive_last(ws.ticket + mt, (unsigned)nsplit, &s_flag)) return;
  for (int e = tid; e < 16 * dim; e += kGateThreads) {
    const int rr = e / dim, n = e - rr * dim;
    const int row = mt * 16 + rr;
    float sum = 0.f;
    for (int s = 0; s < nsplit; ++s) sum += ld_agent(ws.partial + ((size_t)s * mrows + (size_t)mt * 16 + rr) * dim + n);
    if (row < rows) H[(size_t)row * dim + n] = gate_act(sum + (bias ? bias[n] : 0.f), act);
  }
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
  const int mtiles = (rows + 15) / 16;
  const int nsplit = gate_splits(rows, hidden);
  const dim3 grid((unsigned)(mtiles * nsplit));
  const uint16_t* w = static_cast<const uint16_t*>(w_h);
  switch (dim <= 64 ? 1 : dim / 64) {
    case 1:
      hipLaunchKernelGGL(k_gate_bf16<1>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, nsplit, H, ws);
      break;
    case 2:
      hipLaunchKernelGGL(k_gate_bf16<2>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, nsplit, H, ws);
      break;
    case 4:
      hipLaunchKernelGGL(k_gate_bf16<4>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, nsplit, H, ws);
      break;
    case 8:
      hipLaunchKernelGGL(k_gate_bf16<8>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, nsplit, H, ws);
      break;
    case 16:
      hipLaunchKernelGGL(k_gate_bf16<16>, grid, dim3(kGateThreads), 0, s, h, w, bias, rows, hidden, dim, act, nsplit, H, ws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace df2
