// MFMA tile helpers shared by the Full AttnRes kernels (gfx950, wave64,
// v_mfma_f32_32x32x16_bf16).
//
// Operand layouts (checked on the device with a probe):
//   A operand: lane l holds A[l % 32][8 (l / 32) + e], e = 0..7
//   B operand: lane l holds B[8 (l / 32) + e][l % 32]
//   result:    element r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
// A 64-channel chunk of 32 rows is staged in LDS as 32 rows of 128 bytes whose
// 16-byte pieces are XOR-swizzled by row, so that both the coalesced staging
// writes (8 whole rows per wave instruction) and the operand reads (one row
// per lane) are free of bank conflicts.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace attnres {
namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef float f16acc __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;         // MFMA tile: 32 destinations x 32 sources
constexpr int kChunk = 64;        // channels per staged chunk
constexpr int kVRow = 128;        // bytes per staged source row (64 bf16)
constexpr int kORow = 160;        // bytes per staged output row (64 bf16 + pad)
constexpr int kARow = 36;         // floats per alpha row (32 + pad, 16-byte aligned)

__device__ __forceinline__ bf8v as_bf8(uint4 u) { return __builtin_bit_cast(bf8v, u); }

__device__ __forceinline__ f16acc mfma(uint4 a, uint4 b, f16acc c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                       float a7) {
  return make_uint4(pack_bf2(a0, a1), pack_bf2(a2, a3), pack_bf2(a4, a5), pack_bf2(a6, a7));
}

// Coalesced load of one 64-channel chunk of the token's sources: instruction u
// of lane l reads row 8u + l/8, 16-byte piece l%8.  The loads carry no branch
// (rows >= n_src point at row 0 and are zeroed when staged), so the wait
// counters stay exact and a chunk's loads overlap the work on earlier chunks.
__device__ __forceinline__ void load_chunk(const bf16_t* const rowp[4], int ch, uint4 v[4]) {
  const int piece = lane_id() & 7;
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(rowp[u] + ch + 8 * piece);
}

// Swizzled position of (row, 16-byte piece) in a staged source tile.
__device__ __forceinline__ int vpos(int row, int piece) { return row * kVRow + ((piece ^ (row & 7)) << 4); }

// Rows 8u + l/8 share the swizzle of row l/8, so one per-lane base serves all
// four writes (constant offsets u * 1 KiB).
// rowmask[u] is all ones for a real source row and zero past n_src (a mask, not
// a select, so no branch splits the wait for the loads).
__device__ __forceinline__ void stage_chunk(unsigned char* tile, const uint4 v[4], const uint32_t rowmask[4]) {
  const int lane = lane_id();
  unsigned char* base = tile + vpos(lane >> 3, lane & 7);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t m = rowmask[u];
    *reinterpret_cast<uint4*>(base + u * 8 * kVRow) = make_uint4(v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m);
  }
}

// Operand of k-step s (channels 16 s .. 16 s + 15 of the chunk): lane l holds
// row l % 32, channels 16 s + 8 (l / 32) .. + 7.
__device__ __forceinline__ uint4 tile_operand(const unsigned char* tile, int s) {
  const int lane = lane_id();
  return *reinterpret_cast<const uint4*>(tile + vpos(lane & 31, 2 * s + (lane >> 5)));
}

// Identity B operand of k-step a2 for the transposes: I[k][n] = 1 when
// 16 a2 + k == n, with k = 8 h + e held by lane (h, n).
__device__ __forceinline__ uint4 ident_operand(int a2) {
  const int lane = lane_id(), h = lane >> 5, n = lane & 31;
  uint32_t wds[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo16 = (16 * a2 + 8 * h + 2 * q == n) ? 0x3F80u : 0u;
    const uint32_t hi16 = (16 * a2 + 8 * h + 2 * q + 1 == n) ? 0x3F80u : 0u;
    wds[q] = lo16 | (hi16 << 16);
  }
  return make_uint4(wds[0], wds[1], wds[2], wds[3]);
}

// After the identity transpose of a row-operand tile, k-step b of the
// transposed operand holds (in lane half h, element e) row number
// 16 b + 8 (e / 4) + 4 h + e % 4 of the original tile.
__device__ __forceinline__ int transposed_row(int b, int h, int e) { return 16 * b + 8 * (e / 4) + 4 * h + (e % 4); }

}  // namespace
}  // namespace attnres
