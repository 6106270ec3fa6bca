// One thread's share of a bf16 row for the vector kernels that hold whole
// source rows in registers (gfx950): C = 8 channels (16 bytes, a uint4) or
// C = 4 channels (8 bytes, a uint2) at a per-thread byte offset, through
// buffer descriptors whose record count can be zero (then a load reads
// nothing and returns zeros, and a store writes nothing).
#pragma once

#include "common.hpp"

namespace attnres {

// 16 bytes at byte offset `off` of a row through a buffer descriptor of
// `records` bytes (nontemporal).  With zero records the load reads nothing and
// returns zeros, and the store writes nothing: a row that does not exist
// costs no memory traffic and no branch.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_rec(const void* row, uint32_t off, int records = 0x7fffffff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, records, kBufferWord3);
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kBufferNt);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_rec(void* row, uint32_t off, int records, const uint4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, records, kBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, (int)off, 0, kBufferNt);
}

// Eight bf16 (one 16-byte piece) as fp32.
__device__ __forceinline__ void unpack_bf8(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One thread's C channels of a bf16 row: 16 bytes (C = 8, a uint4) or 8
// bytes (C = 4, a uint2), through a buffer descriptor of `records` bytes
// (zero: nothing is read or written, and a load returns zeros).
template <int C> struct PieceOf { typedef uint4 type; };
template <> struct PieceOf<4> { typedef uint2 type; };

template <int C>
__device__ __forceinline__ typename PieceOf<C>::type piece_ld(const void* row, uint32_t off, int records) {
  if constexpr (C == 8) {
    return ld16_rec(row, off, records);
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, records, kBufferWord3);
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kBufferNt);
    return make_uint2(v.x, v.y);
  }
}

__device__ __forceinline__ void piece_st(void* row, uint32_t off, int records, const float (&x)[8]) {
  st16_rec(row, off, records,
           make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])));
}
__device__ __forceinline__ void piece_st(void* row, uint32_t off, int records, const float (&x)[4]) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, records, kBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])}, r, (int)off, 0, kBufferNt);
}

__device__ __forceinline__ void piece_unpack(const uint4 u, float (&x)[8]) { unpack_bf8(u, x); }
__device__ __forceinline__ void piece_unpack(const uint2 u, float (&x)[4]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
}

// An opaque copy: the compiler cannot reuse an earlier unpacking of it.
__device__ __forceinline__ uint4 piece_opaque(uint4 u) {
  asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
  return u;
}
__device__ __forceinline__ uint2 piece_opaque(uint2 u) {
  asm volatile("" : "+v"(u.x), "+v"(u.y));
  return u;
}

// q = w * g (or w) for C consecutive channels.
template <int C>
__device__ __forceinline__ void fold_q(const float* w, const float* g, float (&q)[C]) {
#pragma unroll
  for (int k = 0; k < C; k += 4) {
    const float4 wv = *reinterpret_cast<const float4*>(w + k);
    q[k] = wv.x; q[k + 1] = wv.y; q[k + 2] = wv.z; q[k + 3] = wv.w;
    if (g != nullptr) {
      const float4 gv = *reinterpret_cast<const float4*>(g + k);
      q[k] *= gv.x; q[k + 1] *= gv.y; q[k + 2] *= gv.z; q[k + 3] *= gv.w;
    }
  }
}

}  // namespace attnres
