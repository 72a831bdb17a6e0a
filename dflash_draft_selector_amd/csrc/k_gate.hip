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

// ---- wide tiles for many rows (bf16 weight) -------------------------------------------
// At hundreds of rows the 16 x 64 tiles re-read W once per 16 rows and h once per 64
// columns, about 1 MB per compute unit at 960 rows, and each compute unit's load path
// (not HBM, not the matrix cores) sets the time.  A wide tile is 64 rows x 256 columns
// over a part of the hidden dimension: the 64 hidden rows of each 128-dim stage go
// through LDS (rounded to bf16 as they are staged), double-buffered with one barrier per
// stage, and each wave streams the W rows of its own 32 columns straight into the MFMA B
// operand, two stages ahead in registers.  The parts' sums go to partial[part][row][col]
// and k_gate_finish adds them in part order, so results never depend on scheduling.
constexpr int kWideRows = 64;
constexpr int kWideCols = 256;
constexpr int kWideStage = 128;                        // hidden dims per stage (4 MFMA steps)
constexpr int kWideSlots = kWideStage / 8;             // 16-byte bf16 slots per staged row
constexpr int kWideMinRows = 256;

static bool gate_wide(int64_t rows, int64_t hidden, int64_t dim) {
  return rows >= kWideMinRows && dim % kWideCols == 0 && hidden % kWideStage == 0;
}

// Parts of the hidden dimension per wide tile: about kGateTargetBlocks work-groups, at
// least two stages each (one-stage parts measured slower at 300 and 512 rows: more
// slice sums to write and add, and no stage to overlap with the next one's loads).
static int gate_wide_parts(int64_t rows, int64_t hidden, int64_t dim) {
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

__device__ __forceinline__ int wide_lds_off(int r, int c) { return r * (kWideSlots * 16) + ((c ^ (r & 15)) << 4); }

template <bool HB>
__global__ void __launch_bounds__(kGateThreads) k_gate_wide(const void* __restrict__ h, const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int rows, int hidden,
                                                            int dim, int act, int ctiles, int nparts,
                                                            float* __restrict__ H, float* __restrict__ partial) {
  static_assert(kGateThreads == 512 && kWideCols == 32 * kGateWaves, "eight waves of 32 columns");
  __shared__ __align__(16) unsigned char lds[2][kWideRows * kWideSlots * 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int per = ctiles * nparts;
  const int mg = (int)blockIdx.x / per, rem = (int)blockIdx.x - mg * per;
  const int ct = rem / nparts, part = rem - ct * nparts;
  const int nst = hidden / kWideStage;
  const int s0 = (int)((long long)nst * part / nparts), s1 = (int)((long long)nst * (part + 1) / nparts);
  const int row0 = mg * kWideRows;

  // this wave's W rows (columns 256 ct + 32 wv + 16 nt + i16), 16 bytes at dims 8 g of
  // each 32-wide step
  const uint16_t* wr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) wr[nt] = w + (size_t)(ct * kWideCols + 32 * wv + 16 * nt + i16) * hidden + 8 * g;
  auto load_b = [&](int st, u32x4 (&b)[4][2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) b[q][nt] = *reinterpret_cast<const u32x4*>(wr[nt] + (size_t)st * kWideStage + 32 * q);
  };

  // staging: thread slot e (0, 1) covers row (tid + 512 e) / 16, 16-byte slot
  // (tid + 512 e) % 16 of the stage.  A row past the input repeats the last row (loaded
  // on every path, so that the compiler's wait counts stay exact); its accumulator rows
  // are never stored, and MFMA rows do not mix.
  f32x4 xa[2][2];
  u32x4 xb[2];
  auto load_a = [&](int st) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + kGateThreads * e;
      const int r = idx / kWideSlots, c = idx % kWideSlots;
      const int grow = row0 + r;
      const size_t off = (size_t)(grow < rows ? grow : rows - 1) * hidden + (size_t)st * kWideStage + 8 * c;
      if constexpr (HB) {
        xb[e] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(h) + off);
      } else {
        xa[e][0] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(h) + off);
        xa[e][1] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(h) + off + 4);
      }
    }
  };
  auto store_a = [&](unsigned char* buf) {
    // row tid / 16 + 32 e has the swizzle of row tid / 16: one offset, plus 32 e rows
    const int base = wide_lds_off(tid / kWideSlots, tid % kWideSlots);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u32x4 a;
      if constexpr (HB) {
        a = xb[e];
      } else {
        a.x = pack_bf16x2(xa[e][0].x, xa[e][0].y);
        a.y = pack_bf16x2(xa[e][0].z, xa[e][0].w);
        a.z = pack_bf16x2(xa[e][1].x, xa[e][1].y);
        a.w = pack_bf16x2(xa[e][1].z, xa[e][1].w);
      }
      *reinterpret_cast<u32x4*>(buf + base + e * (kGateThreads / kWideSlots) * kWideSlots * 16) = a;
    }
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[m][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // stage st on LDS buffer cur and W slot wb; meanwhile the next stage's hidden rows are
  // loaded (and stored to nxt at the end) and this W slot is refilled with the stage
  // after next (the part's last stage again past its end: valid, unused, so that every
  // path issues the same loads; staging the rows two stages ahead measured no faster)
  u32x4 wb0[4][2], wb1[4][2];
  auto stage = [&](int st, unsigned char* cur, unsigned char* nxt, u32x4 (&wb)[4][2]) {
    load_a(st + 1 < s1 ? st + 1 : st);
    __builtin_amdgcn_sched_barrier(0);                // issued before the stage's MFMAs
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(cur + wide_lds_off(16 * m + i16, 4 * q + g));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                               __builtin_bit_cast(bf16x8, wb[q][nt]), acc[m][nt], 0,
                                                               0, 0);
      }
    }
    load_b(st + 2 < s1 ? st + 2 : s1 - 1, wb);
    __builtin_amdgcn_sched_barrier(0);
    store_a(nxt);
    __syncthreads();
  };
  load_b(s0, wb0);
  load_b(s0 + 1 < s1 ? s0 + 1 : s0, wb1);
  load_a(s0);
  store_a(lds[0]);
  __syncthreads();
  int st = s0;
  for (; st + 1 < s1; st += 2) {
    stage(st, lds[0], lds[1], wb0);
    stage(st + 1, lds[1], lds[0], wb1);
  }
  if (st < s1) stage(st, lds[0], lds[1], wb0);

  // D layout: lane (g, i16), register r -> row 16 m + 4 g + r, column 16 nt + i16 of
  // this wave's 32
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * m + 4 * g + r;
        const int col = ct * kWideCols + 32 * wv + 16 * nt + i16;
        if (row < rows) {
          if (nparts == 1)
            H[(size_t)row * dim + col] = gate_act(acc[m][nt][r] + (bias ? bias[col] : 0.f), act);
          else
            partial[((size_t)part * rows + row) * dim + col] = acc[m][nt][r];
        }
      }
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
