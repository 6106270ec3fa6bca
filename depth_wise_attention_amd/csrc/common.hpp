// Device helpers shared by the AttnRes kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

typedef uint16_t bf16_t;
typedef _Float16 f16_t;

constexpr int kWave = 64;

// Buffer descriptors (gfx9 family): word 3 of a raw, unswizzled descriptor
// with 32-bit data format, and the cache-policy bit of a nontemporal access.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNt = 2;

// ---------------------------------------------------------------- element I/O
__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two fp32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
  bf2v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Low / high bf16 of a packed pair, as fp32.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// q = w * g (G) or q = w for 8 consecutive channels, 16-byte aligned rows,
// with vector loads.  Callers branch on the gain once, outside their fold
// loops, and fold every chunk inside: a per-element branch on the gain makes
// the compiler wait for each load in turn, and even a select lets it sink the
// gain loads into a branch per chunk.
template <bool G>
__device__ __forceinline__ void fold_q8(const float* w, const float* g, float (&q)[8]) {
  const float4 w0 = reinterpret_cast<const float4*>(w)[0], w1 = reinterpret_cast<const float4*>(w)[1];
  q[0] = w0.x; q[1] = w0.y; q[2] = w0.z; q[3] = w0.w;
  q[4] = w1.x; q[5] = w1.y; q[6] = w1.z; q[7] = w1.w;
  if constexpr (G) {
    const float4 g0 = reinterpret_cast<const float4*>(g)[0], g1 = reinterpret_cast<const float4*>(g)[1];
    q[0] *= g0.x; q[1] *= g0.y; q[2] *= g0.z; q[3] *= g0.w;
    q[4] *= g1.x; q[5] *= g1.y; q[6] *= g1.z; q[7] *= g1.w;
  }
}

template <typename E> __device__ __forceinline__ float ld(const E* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <> __device__ __forceinline__ float ld<f16_t>(const f16_t* p) { return (float)*p; }

template <typename E> __device__ __forceinline__ void st(E* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }
template <> __device__ __forceinline__ void st<f16_t>(f16_t* p, float v) { *p = (f16_t)v; }

// Per-token power-of-two scale for an fp16 state whose values are bounded by
// `bound` (>= max |value|): returns 2^e with bound / 32768 = m * 2^e, m in
// [0.5, 1), so the stored values value * 2^-e satisfy |.| < 32768 (below the
// fp16 limit 65504) and the bound itself lands in [16384, 32768): the top of
// fp16's range, where its 11 significant bits apply.  Zero, NaN and infinite
// bounds give 1.
__device__ __forceinline__ float f16_state_scale(float bound) {
  if (!(bound > 0.f) || !(bound <= 3.0e38f)) return 1.0f;
  int e = 0;
  frexpf(bound * (1.0f / 32768.0f), &e);
  e = e < -120 ? -120 : (e > 120 ? 120 : e);
  return ldexpf(1.0f, e);
}

// -------------------------------------------------------------- cross-lane ops
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Butterfly reduction: every lane ends with the total over the 64 lanes.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Value held by lane `src` (wave-uniform index), broadcast as a scalar.
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Workgroup barrier that orders LDS only: the fences are restricted to the
// local address space, so the wait before s_barrier is lgkmcnt(0) alone and
// this wave's global loads and stores stay in flight across it.
// (__syncthreads' workgroup fence also covers global memory and waits for
// every outstanding load and store, which defeats loads issued ahead.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Compiler barrier: keeps the memory operations before it (a prefetch) where
// they are instead of letting the compiler sink them towards their first use.
__device__ __forceinline__ void keep_memory_order() { asm volatile("" ::: "memory"); }

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace attnres
