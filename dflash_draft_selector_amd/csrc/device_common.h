// Device helpers shared by the libdflash2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df2 {

constexpr int kNC = 16;       // candidates per draft position
constexpr int kWave = 64;     // CDNA wavefront width

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 -------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Order key of a bf16 pattern: a larger key is a larger value, -0 and +0 share the
// key 0x8000, every NaN maps to 0 (below -inf, whose key is 0x0080).
__device__ __forceinline__ uint32_t bf16_key(uint32_t b16) {
  const uint32_t mag = b16 & 0x7fffu;
  if (mag > 0x7f80u) return 0u;
  return (b16 & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
}

// Round-to-nearest-even fp32 -> bf16 for finite and infinite inputs (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- Philox4x32-10 (Salmon et al., SC'11) -----------------------------------------

struct Philox4 {
  uint32_t x0, x1, x2, x3;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// Uniform in [0, 1): top 24 bits of a word times 2^-24 (exact in fp32).
__device__ __forceinline__ float word_to_uniform(uint32_t x) { return (float)(x >> 8) * 5.9604644775390625e-08f; }

__device__ __forceinline__ float walk_uniform(uint64_t seed, uint32_t b, uint32_t t) {
  const Philox4 r = philox4x32_10(t, b, 0u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
  return word_to_uniform(r.x0);
}

// ---- 16-slot row decisions (lane-parallel) --------------------------------------------
// A row of 16 scores lives in a group of 16 consecutive lanes (lane j of the group
// holds slot j); the group reduces and scans it with DPP row operations.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// max over the 16 lanes of the row (every lane gets it)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4e>(v));     // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));    // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));    // row_mirror
  return v;
}

// inclusive prefix sum over slots 0..j of the row (Hillis-Steele, fixed order)
__device__ __forceinline__ float row16_scan(float v) {
  v += dpp_f<0x111>(v);             // row_shr:1 (lanes without a source read 0)
  v += dpp_f<0x112>(v);             // row_shr:2
  v += dpp_f<0x114>(v);             // row_shr:4
  v += dpp_f<0x118>(v);             // row_shr:8
  return v;
}

// Slot chosen from the row held by this lane's group (same in all 16 lanes):
//   temperature 0: the lowest slot holding the row maximum;
//   temperature T: w_j = exp((s_j - max) / T), the first slot whose prefix weight
//   exceeds u * (total weight), slot order.
// Non-finite scores never win (weight 0); an all-non-finite row picks slot 0.  *q gets
// this lane's slot probability (one-hot when greedy).  All 64 lanes of the wave must
// call it, with whole 16-lane rows active.
__device__ __forceinline__ int row16_pick(float s, float inv_t, float u, float* q) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int shift = lane & 48;
  const bool fin = __builtin_isfinite(s);
  const float sv = fin ? s : -__builtin_inff();
  const float m = row16_max(sv);
  const unsigned int anyfin = (unsigned int)((__ballot(fin) >> shift) & 0xffffull);
  if (!anyfin) {
    *q = j == 0 ? 1.f : 0.f;
    return 0;
  }
  if (inv_t == 0.f) {
    const unsigned int hit = (unsigned int)((__ballot(fin && sv == m) >> shift) & 0xffffull);
    const int pick = __builtin_ctz(hit);
    *q = j == pick ? 1.f : 0.f;
    return pick;
  }
  const float w = fin ? expf((s - m) * inv_t) : 0.f;
  const float pre = row16_scan(w);
  const float total = __shfl(pre, shift + 15);
  const float target = u * total;
  const unsigned int hit = (unsigned int)((__ballot(target < pre) >> shift) & 0xffffull);
  int pick;
  if (hit) {
    pick = __builtin_ctz(hit);
  } else {
    // rounding left u * total at or above the last prefix: the last slot with weight;
    // with no positive weight at all (a scale the host checks rule out), the lowest
    // slot holding the row maximum, so the slot is always in [0, 16)
    const unsigned int pos = (unsigned int)((__ballot(w > 0.f) >> shift) & 0xffffull);
    const unsigned int top = (unsigned int)((__ballot(fin && sv == m) >> shift) & 0xffffull);
    pick = pos ? 31 - __builtin_clz(pos) : __builtin_ctz(top);
  }
  *q = w * (1.f / total);
  return pick;
}

// ---- kernel arguments -------------------------------------------------------------

// Keeps the given kernel arguments in scalar registers from the kernel's first
// instructions on.  Left alone, the compiler loads an argument from the kernel-argument
// segment only where it is first used; in a kernel whose last phase is on the critical
// path, that scalar load then stalls the first LDS wait after it (both count in
// lgkmcnt) for a full memory round trip.
template <typename T>
__device__ __forceinline__ void pin_arg(T a) {
  if constexpr (sizeof(T) == 8)
    asm volatile("" ::"s"(__builtin_bit_cast(uint64_t, a)));
  else if constexpr (sizeof(T) == 4)
    asm volatile("" ::"s"(__builtin_bit_cast(uint32_t, a)));
  else
    asm volatile("" ::"s"((uint32_t)a));
}
template <typename... T>
__device__ __forceinline__ void args_in_sgprs(T... a) {
  (pin_arg(a), ...);
}

// ---- hand-offs between work-groups of one launch ---------------------------------------
// Relaxed stores and loads at agent scope are performed where every compute unit sees
// them (written through to the device's coherence point; no stale L1 or L2 copy is
// read), so a value stored this way by one work-group is read by another once the
// storing wave's memory counter has drained and the reader has learnt so through an
// atomic.  The drain carries a memory clobber so that the compiler moves no access across
// it.  (A release / acquire fence pair would also order plain stores, but its release
// writes back the whole L2 of the work-group's XCD.)

template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- wave / block helpers ----------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t other = __shfl_xor(v, o);
    v = other > v ? other : v;
  }
  return v;
}

}  // namespace df2
