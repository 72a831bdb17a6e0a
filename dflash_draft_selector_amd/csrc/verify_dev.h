// Wave-level helpers of the verify kernels (gfx950, wave64): target weights, DPP
// scans and the inverse-CDF lane pick.
#pragma once

#include "device_common.h"
#include "topk_dev.h"

namespace df2 {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---- sub-chunks: a wave's contiguous share of a top-16 chunk ---------------------------
constexpr int kSubPerChunk = kTopkWaves;                  // one contiguous sub-chunk per wave
constexpr int kMaxSub = kMaxChunks * kSubPerChunk;       // sub-chunks of the longest row
constexpr int kSubVec = kTopkVecPerThread * kWave;       // 1216 vectors: the longest sub-chunk
static_assert(kChunkVec == kSubPerChunk * kSubVec, "a chunk is its waves' sub-chunks");
static_assert(kMaxSub <= kWave, "one sub-chunk per lane of the deciding wave");

// First vector of sub-chunk s = 8c + j (wave j's share of chunk c); s = 8 * nchunks gives
// the row's end.  Chunk c starts at vector floor(nvec * c / nchunks), as in the top-16
// split (32-bit arithmetic: nvec <= 2^16, c <= 8); every sub-chunk but a chunk's last has
// ceil(len / 8) vectors.
__host__ __device__ __forceinline__ int sub_begin(int V, int nchunks, int s) {
  const unsigned nvec = ((unsigned)V + 7u) >> 3;
  const unsigned c = (unsigned)s / kSubPerChunk, j = (unsigned)s % kSubPerChunk;
  const unsigned a = nvec * c / (unsigned)nchunks;
  const unsigned b = nvec * (c + 1u) / (unsigned)nchunks;
  const unsigned span = (b - a + kSubPerChunk - 1) / kSubPerChunk;
  return (int)(a + j * span < b ? a + j * span : b);
}
static_assert((int64_t)kMaxChunks * kChunkVec * (kWave / kSubPerChunk + 1) < (1ll << 32), "sub_begin's products fit 32 bits");

constexpr float kLog2e = 1.44269504088896341f;

// exp((l - m) / T) formed as 2^((l - m) * c2) with c2 = log2(e) / T: one v_exp_f32 per
// weight.  Every weight of the target distribution (sub-chunk sums, the accept test and
// the draws) is formed this one way.
__device__ __forceinline__ float tweight(float l, float m, float c2) { return __builtin_amdgcn_exp2f((l - m) * c2); }

// ---- wave-wide sums on DPP ------------------------------------------------------------
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f32(float x) {
  // lanes whose source lies outside the pattern (or in a row outside ROWS) read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}

// Inclusive sum over the wave's lanes: within each 16-lane row by shifts of 1, 2, 4 and
// 8 lanes, then across rows by broadcasting lane 15 into rows 1 and 3 and lane 31 into
// rows 2 and 3.  Every lane must be active.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_f32<0x111>(x);           // row_shr:1
  x += dpp_f32<0x112>(x);           // row_shr:2
  x += dpp_f32<0x114>(x);           // row_shr:4
  x += dpp_f32<0x118>(x);           // row_shr:8
  x += dpp_f32<0x142, 0xa>(x);      // row_bcast:15
  x += dpp_f32<0x143, 0xc>(x);      // row_bcast:31
  return x;
}

// The scan's exclusive form (wave_shr:1; lane 0 reads 0).
__device__ __forceinline__ float wave_excl_from_incl(float incl) { return dpp_f32<0x138>(incl); }

// The wave's total, the same in every lane (lane 63 of the inclusive scan).
__device__ __forceinline__ float wave_total(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_scan(x)), kWave - 1));
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Inverse-CDF step over one non-negative value per lane (incl: their inclusive scan):
// the first lane holding a positive value whose running sum exceeds x (in exact
// arithmetic the first lane whose running sum exceeds x holds one), or the last positive
// lane when rounding leaves x at or past the total (x = +inf asks for that).  -1 when no
// lane is positive.  The whole wave calls it.
__device__ __forceinline__ int wave_pick_lane(float v, float incl, float x) {
  const unsigned long long pos = __ballot(v > 0.f);
  if (pos == 0ull) return -1;
  const unsigned long long hit = __ballot(x < incl) & pos;
  return hit != 0ull ? __builtin_ctzll(hit) : 63 - __builtin_clzll(pos);
}


// Inclusive integer sum over the wave's lanes (the DPP pattern of wave_incl_scan).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_add_src(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += dpp_add_src<0x111>(x);
  x += dpp_add_src<0x112>(x);
  x += dpp_add_src<0x114>(x);
  x += dpp_add_src<0x118>(x);
  x += dpp_add_src<0x142, 0xa>(x);
  x += dpp_add_src<0x143, 0xc>(x);
  return x;
}

}  // namespace df2
