// Context gate kernels: tiles of gate_dev.h (bf16 weight on bf16 MFMA, fp32 weight on
// fp32 MFMA), eight waves per work-group, then a kernel adding the slices; at hundreds of
// rows with a bf16 weight, wide tiles (k_gate_wide) in place of the first.
#include "dflash2_internal.h"
#include "gate_dev.h"

namespace df2 {

constexpr int kGateThreads = kGateBlockThreads;
constexpr int kGateWaves = kGateThreads / 64;
// Slices of hidden per tile are chosen for about this many work-groups: at 105 rows,
// 28 tiles x 8 slices = 224 fill one round of the 256 compute units (measured 9.1 us
// against 10.0 us for 6 slices; 10 slices, 280 work-groups, took 10.8 us).
constexpr int kGateTargetBlocks = 224;
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

bool gate_wide(int64_t rows, int64_t hidden, int64_t dim) {
  return rows >= kWideMinRows && dim % kWideCols == 0 && hidden % kWideStage == 0;
}

// Parts of the hidden dimension per wide tile: about kGateTargetBlocks work-groups, at
// least two stages each (one-stage parts measured slower at 300 and 512 rows: more
// slice sums to write and add, and no stage to overlap with the next one's loads).
int gate_wide_parts(int64_t rows, int64_t hidden, int64_t dim) {
  const int64_t tiles = ((rows + kWideRows - 1) / kWideRows) * (dim / kWideCols);
  int64_t p = (kGateTargetBlocks + tiles - 1) / tiles;
  const int64_t nst = hidden / kWideStage;
  if (p > nst / 2) p = nst / 2;
  if (p > 64) p = 64;
  return p < 1 ? 1 : (int)p;
}

GateWs carve_gate(Carver& c, int64_t rows, int64_t hidden, int64_t dim) {
  GateWs w;
  const int ns = gate_splits(rows, hidden, dim);
  // the slice sums of either tiling (the weight's type picks one at launch)
  const int nw = gate_wide(rows, hidden, dim) ? gate_wide_parts(rows, hidden, dim) : 1;
  const int most = ns > nw ? ns : nw;
  w.partial = c.take<float>(most > 1 ? (size_t)most * rows * dim : 0);
  w.nsplit = ns;
  return w;
}

// NB = 16-column blocks of the tile (tile width 16 * NB = min(dim, 64)); HB = h in bf16.
template <int NB, bool HB>
__global__ void __launch_bounds__(kGateThreads) k_gate_bf16(const void* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int ntiles, int nsplit,
                                                            float* __restrict__ H, float* __restrict__ partial) {
  __shared__ float red[kGateWaves * 16 * 16 * NB];
  const int per = ntiles * nsplit;
  const int mt = blockIdx.x / per;
  const int rem = blockIdx.x - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  gate_tile<NB, kGateWaves, kGateRound, HB>(h, w, bias, rows, hidden, dim, act, mt, nt, split, nsplit, red, H, partial);
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

template <int NB, bool HB>
__global__ void __launch_bounds__(kGateThreads) k_gate_f32(const void* __restrict__ h, const float* __restrict__ w,
                                                           const float* __restrict__ bias, int rows, int hidden, int dim,
                                                           int act, int ntiles, int nsplit, float* __restrict__ H,
                                                           float* __restrict__ partial) {
  __shared__ float red[kGateWaves * 16 * 16 * NB];
  const int per = ntiles * nsplit;
  const int mt = blockIdx.x / per;
  const int rem = blockIdx.x - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  gate_tile_f32<NB, kGateWaves, kGateRound, HB>(h, w, bias, rows, hidden, dim, act, mt, nt, split, nsplit, red, H,
                                            partial);
}

template <bool HB>
__global__ void __launch_bounds__(kGateThreads) k_gate_wide(const void* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int ctiles, int nparts,
                                                            float* __restrict__ H, float* __restrict__ partial) {
  __shared__ __align__(16) unsigned char lds[2 * kWideLdsBuf];
  const int per = ctiles * nparts;
  const int mg = (int)blockIdx.x / per, rem = (int)blockIdx.x - mg * per;
  const int ct = rem / nparts, part = rem - ct * nparts;
  gate_wide_tile<HB>(h, w, bias, rows, hidden, dim, act, mg, ct, part, nparts, lds, H, partial);
}

hipError_t launch_gate(const void* h, bool h_bf16, const void* w_h, bool w_bf16, const float* bias, int rows,
                       int hidden, int dim, int act, float* H, GateWs ws, hipStream_t s) {
  if (w_bf16 && gate_wide(rows, hidden, dim)) {
    const int ctiles = dim / kWideCols, parts = gate_wide_parts(rows, hidden, dim);
    const dim3 grid((unsigned)((long long)((rows + kWideRows - 1) / kWideRows) * ctiles * parts));
    if (h_bf16)
      hipLaunchKernelGGL((k_gate_wide<true>), grid, dim3(kGateThreads), 0, s, h, static_cast<const uint16_t*>(w_h),
                         bias, rows, hidden, dim, act, ctiles, parts, H, ws.partial);
    else
      hipLaunchKernelGGL((k_gate_wide<false>), grid, dim3(kGateThreads), 0, s, h, static_cast<const uint16_t*>(w_h),
                         bias, rows, hidden, dim, act, ctiles, parts, H, ws.partial);
    if (parts > 1) {
      const long long n = (long long)rows * dim;
      hipLaunchKernelGGL(k_gate_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws.partial, bias, n, dim,
                         parts, act, H);
    }
    return hipGetLastError();
  }
  const int ct = gate_coltile(dim);
  const int ntiles = dim / ct;
  const int mtiles = (rows + 15) / 16;
  const int nsplit = ws.nsplit;
  const dim3 grid((unsigned)((long long)mtiles * ntiles * nsplit));
  const dim3 blk(kGateThreads);
#define DF2_GATE_HB(NB, HB)                                                                                        \
  if (w_bf16)                                                                                                      \
    hipLaunchKernelGGL((k_gate_bf16<NB, HB>), grid, blk, 0, s, h, static_cast<const uint16_t*>(w_h), bias, rows,   \
                       hidden, dim, act, ntiles, nsplit, H, ws.partial);                                           \
  else                                                                                                             \
    hipLaunchKernelGGL((k_gate_f32<NB, HB>), grid, blk, 0, s, h, static_cast<const float*>(w_h), bias, rows,       \
                       hidden, dim, act, ntiles, nsplit, H, ws.partial);
#define DF2_GATE(NB)           \
  case NB:                     \
    if (h_bf16) {              \
      DF2_GATE_HB(NB, true)    \
    } else {                   \
      DF2_GATE_HB(NB, false)   \
    }                          \
    break;
  switch (ct / 16) {
    DF2_GATE(1)
    DF2_GATE(2)
    DF2_GATE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef DF2_GATE
#undef DF2_GATE_HB
  if (nsplit > 1) {
    const long long n = (long long)rows * dim;
    hipLaunchKernelGGL(k_gate_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws.partial, bias, n, dim,
                       nsplit, act, H);
  }
  return hipGetLastError();
}

}  // namespace df2
