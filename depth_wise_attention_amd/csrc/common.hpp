// Device helpers shared by the AttnRes kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

typedef uint16_t bf16_t;

constexpr int kWave = 64;

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

template <typename E> __device__ __forceinline__ float ld(const E* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf2f(*p); }

template <typename E> __device__ __forceinline__ void st(E* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

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

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace attnres
