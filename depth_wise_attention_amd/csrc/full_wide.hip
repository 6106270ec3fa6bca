// Full AttnRes forward for 33 .. 64 sources on the matrix cores (gfx950, bf16
// I/O, one head).  A model with L sublayers has destinations that read up to
// L + 1 sources (b-lab.team summary §1; dimensionstp "Attention Residuals
// Review" §3 (2) runs 54 sublayers), past the 32-source tile of the kernels in
// full_fast.hip.  The contractions are the same (S = Q V^T with q split into
// bf16 high + low parts, G = V V^T for the sums of squares, H = alpha V with
// alpha split the same way, v_mfma_f32_32x32x16_bf16), over two 32-source
// tiles and TD = 1 or 2 tiles of 32 destinations.
//
// A workgroup of 4 waves owns one token at a time; wave w covers channels
// [w d/4, (w+1) d/4) in 64-channel chunks.  Each chunk of the token's 64
// source rows is loaded with coalesced 16-byte loads (8 whole rows per wave
// instruction, two chunks in flight), staged in a per-wave LDS tile with
// row-swizzled pieces, and read back one row per lane as MFMA operands.  Stage
// 2 transposes the staged tile with an MFMA against the identity (exact) and
// stages the outputs through the same tile for whole-row stores.
//
// LDS: the per-wave S partials share one region with the per-wave tiles and
// with the stage-2 operands of alpha (laid out next to the tiles), separated
// by workgroup barriers, so that two workgroups fit on a compute unit; the
// per-wave sums of squares have their own.
#include <math.h>

#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kWW = 4;             // waves per workgroup
constexpr int kWB = kWW * 64;      // threads per workgroup
constexpr int kWSrc = 2 * kTile;   // source rows staged per chunk (two tiles)

// Bytes of one wave's tile: 64 staged source rows, or TD x 32 output rows.
template <int TD>
constexpr int wide_tile_bytes() {
  return kWSrc * kVRow > TD * kTile * kORow ? kWSrc * kVRow : TD * kTile * kORow;
}
// The alpha operands of stage 2 follow the tiles: for destination tile td,
// source tile ts, k-step b and part p, 64 lanes of 16 bytes at operand
// ((td * 2 + ts) * 2 + b) * 2 + p.
template <int TD>
constexpr int wide_op_offset() {
  return kWW * wide_tile_bytes<TD>();
}
template <int TD>
constexpr int wide_union_bytes() {
  constexpr int ops = wide_op_offset<TD>() + TD * 8 * 64 * 16;
  constexpr int sred = kWW * TD * kTile * kWSrc * 4;
  return ops > sred ? ops : sred;
}
template <int TD>
constexpr size_t wide_lds_bytes() {
  return (size_t)wide_union_bytes<TD>() + kWW * kWSrc * 4;  // + the sums of squares
}

// q = w * g packed for TD destination tiles: for chunk g (64 channels), k-step
// s, destination tile td and part p (0 = bf16 high, 1 = low), lane l holds
// q_p[32 td + l % 32][64 g + 16 s + 8 (l / 32) + e], e = 0..7, at uint4
// ((g * 4 + s) * TD + td) * 2 + p) * 64 + l.  Rows past n_dst are zero.
template <int TD>
__global__ __launch_bounds__(256) void k_full_wide_qsplit(FullArgs a, uint4* qpk) {
  const int64_t units = a.d / kChunk * 4 * TD * 64;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < units;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(x % 64);
    const int td = (int)((x / 64) % TD);
    const int64_t gs = x / (64 * TD);  // g * 4 + s
    const int j = td * kTile + lane % 32;
    const int64_t k0 = gs * 16 + 8 * (lane / 32);
    const int jc = j < a.n_dst ? j : (int)a.n_dst - 1;  // in bounds; stored as zeros
    float q[8], hi[8], lo[8];
    if (a.gain != nullptr)
      fold_q8<true>(a.w + jc * a.d + k0, a.gain + jc * a.gain_ld + k0, q);
    else
      fold_q8<false>(a.w + jc * a.d + k0, nullptr, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qe = j < a.n_dst ? q[e] : 0.f;
      hi[e] = bf2f(f2bf(qe));
      lo[e] = qe - hi[e];
    }
    uint4* dst = qpk + (gs * TD + td) * 2 * 64 + lane;
    dst[0] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
    dst[64] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
  }
}

// One 64-channel chunk of the token's 64 source rows (tok: the token's row in
// source 0 at this wave's first channel; plane: T d): instruction u of lane l
// reads piece l % 8 of row 8 u + l / 8.  Rows past n_src read row 0 (no
// branch, exact wait counts) and are zeroed when staged.  The row offsets are
// recomputed from an opaque lane id at each call rather than held across the
// token loop.
__device__ __forceinline__ void wide_load(const bf16_t* tok, int64_t plane, int n_src, int ch, uint4 (&v)[8]) {
  int l = lane_id();
  asm volatile("" : "+v"(l));
  const bf16_t* base = tok + ch + 8 * (l & 7);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = 8 * u + (l >> 3);
    v[u] = *reinterpret_cast<const uint4*>(base + (int64_t)(r < n_src ? r : 0) * plane);
  }
}

__device__ __forceinline__ void wide_stage(unsigned char* tile, const uint4 (&v)[8], int n_src) {
  int l = lane_id();
  asm volatile("" : "+v"(l));
  unsigned char* base = tile + vpos(l >> 3, l & 7);  // rows 8 u + l / 8 share the swizzle
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t m = 8 * u + (l >> 3) < n_src ? 0xFFFFFFFFu : 0u;
    *reinterpret_cast<uint4*>(base + u * 8 * kVRow) = make_uint4(v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m);
  }
}

// 16-byte load at byte voff + soff of a buffer whose base is uniform over the
// wave (base and soff in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferWord3);
}
__device__ __forceinline__ uint4 wide_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Operand of k-step s from a staged tile, for lane id ol (an opaque copy, so
// that the swizzled addresses are recomputed per chunk, not held).
__device__ __forceinline__ uint4 wide_operand(const unsigned char* tile, int ol, int s) {
  return *reinterpret_cast<const uint4*>(tile + vpos(ol & 31, 2 * s + (ol >> 5)));
}

template <int TD>
__global__ __launch_bounds__(kWB, 2) void k_full_wide(FullArgs a, const uint4* qpk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char wide_smem[];
  constexpr int ND = TD * kTile;                 // destination rows of the tables
  constexpr int TPD = kWB / ND;                  // softmax threads per destination
  constexpr int SPT = kWSrc / TPD;               // sources per softmax thread
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const int kw = d / kWW;                        // channels per wave
  const int nch = kw / kChunk;                   // chunks per wave (even, >= 2)
  const int ch_base = wave * kw;
  const int64_t plane = T * d;
  unsigned char* vt = wide_smem + wave * wide_tile_bytes<TD>();
  float* sred = reinterpret_cast<float*>(wide_smem);  // [kWW][ND][kWSrc], after stage 1
  unsigned char* aop = wide_smem + wide_op_offset<TD>();  // alpha operands, after the softmax reads
  float* gred = reinterpret_cast<float*>(wide_smem + wide_union_bytes<TD>());  // [kWW][kWSrc]
  const int h = lane >> 5, n = lane & 31;
  // This wave's query operands: chunk c at byte c * 8 TD KiB, (k-step s,
  // tile td, part p) at ((s TD + td) 2 + p) KiB, lane at 16 lane.
  const __amdgpu_buffer_rsrc_t qrs = wide_rsrc(qpk + (int64_t)(ch_base / kChunk) * 4 * TD * 2 * 64);
  const uint4 ident0 = ident_operand(0), ident1 = ident_operand(1);

  // Two chunks are always in flight: each chunk's slot is refilled with the
  // chunk two ahead in the order stage 1 (chunks 0 .. nch - 1), stage 2 (0 ..
  // nch - 1), the next token's stage 1, ...  So neither stage starts cold,
  // and the loads stay in flight across the barriers and the softmax.
  int64_t t = blockIdx.x;
  uint4 va[8], vb[8];
  if (t < T) {
    wide_load(src + t * d + ch_base, plane, n_src, 0, va);
    __builtin_amdgcn_sched_barrier(0);  // keep the loop's load order (va, then vb)
    wide_load(src + t * d + ch_base, plane, n_src, kChunk, vb);
  }
  for (; t < T; t += gridDim.x) {
    const bf16_t* tok = src + t * d + ch_base;
    // The next token's rows (this token's again after the last one: loaded,
    // never used, so that every path has the same loads in flight).
    const bf16_t* tokn = src + (t + gridDim.x < T ? t + gridDim.x : t) * d + ch_base;

    // ---------------- stage 1: S = Q V^T and G = V V^T over this wave's channels
    f16acc S[TD][2], G[2];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      G[ts] = f16acc{};
#pragma unroll
      for (int td = 0; td < TD; ++td) S[td][ts] = f16acc{};
    }
    {
      auto chunk1 = [&](int c, uint4 (&v)[8]) {
        int ol = lane;
        asm volatile("" : "+v"(ol));
        const uint32_t qoff = (uint32_t)ol * 16u + (uint32_t)c * (uint32_t)(4 * TD * 2 * 1024);
        wide_stage(vt, v, n_src);
        // Chunk c + 2, or stage 2's chunk c + 2 - nch (the same rows again).
        wide_load(tok, plane, n_src, (c + 2 < nch ? c + 2 : c + 2 - nch) * kChunk, v);
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 q[TD][2];
#pragma unroll
          for (int td = 0; td < TD; ++td) {
            q[td][0] = wide_ld(qrs, qoff, ((s * TD + td) * 2 + 0) * 1024);
            q[td][1] = wide_ld(qrs, qoff, ((s * TD + td) * 2 + 1) * 1024);
          }
#pragma unroll
          for (int ts = 0; ts < 2; ++ts) {
            const uint4 b = wide_operand(vt + ts * kTile * kVRow, ol, s);
#pragma unroll
            for (int td = 0; td < TD; ++td) {
              S[td][ts] = mfma(q[td][0], b, S[td][ts]);
              S[td][ts] = mfma(q[td][1], b, S[td][ts]);
            }
            G[ts] = mfma(b, b, G[ts]);
          }
          // One k-step's operands at a time: with two destination tiles the
          // accumulators leave no room for the whole chunk's.
          __builtin_amdgcn_sched_barrier(0);
        }
        wave_lds_sync();  // operand reads done before the tile is rewritten
      };
      // The first pair is peeled so that the loop head sees the same
      // outstanding loads on entry as on the back edge.
      chunk1(0, va);
      chunk1(1, vb);
      for (int c = 2; c < nch; c += 2) {
        chunk1(c, va);
        chunk1(c + 1, vb);
      }
    }
    lds_barrier();  // every wave is done with its tile: the partials overwrite them
    // D layout: element r of lane l is D[8 (r/4) + 4 (l/32) + r%4][l%32].
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r / 4) + 4 * h + (r % 4);
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
#pragma unroll
        for (int td = 0; td < TD; ++td)
          sred[(wave * ND + td * kTile + m) * kWSrc + ts * kTile + n] = S[td][ts][r];
        if (m == n) gred[wave * kWSrc + ts * kTile + n] = G[ts][r];
      }
    }
    lds_barrier();

    // ---------------- softmax: thread -> destination j = tid / TPD, sources SPT (tid % TPD) .. + SPT - 1
    {
      const int j = tid / TPD, i0 = SPT * (tid % TPD);
      const int lim = n_src - n_dst + j;  // destination j reads sources 0..lim
      float sc[SPT];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const int i = i0 + q;
        float sv = 0.f, gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWW; ++w2) {
          sv += sred[(w2 * ND + j) * kWSrc + i];
          gv += gred[w2 * kWSrc + i];
        }
        const float r = 1.0f / sqrtf(gv / (float)d + a.eps);
        sc[q] = (j < n_dst && i <= lim) ? r * sv : -INFINITY;
        m = fmaxf(m, sc[q]);
      }
      m = group_max<TPD>(m);
      float e[SPT], l = 0.f;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        e[q] = (sc[q] == -INFINITY) ? 0.f : expf(sc[q] - m);
        l += e[q];
      }
      l = group_sum<TPD>(l);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      lds_barrier();  // every thread has read the partials: the operands overwrite them
      // Stage 2's A operand of (destination tile td, source tile ts, k-step b)
      // holds, in lane (h, j % 32) element e, alpha[j][32 ts + 16 b + 8 (e / 4)
      // + 4 h + e % 4] (the source order the transpose leaves in the B
      // operand): four consecutive sources are four consecutive elements.
      const int td = j / kTile, jn = j % kTile;
#pragma unroll
      for (int q = 0; q < SPT; q += 4) {
        const int i = i0 + q, ts = i / kTile, b = (i % kTile) / 16, r16 = i % 16;
        const int lane_h = (r16 >> 2) & 1, e0 = 4 * (r16 >> 3);
        float hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = e[q + k] * inv;
          hi[k] = bf2f(f2bf(x));
          lo[k] = x - hi[k];
        }
        unsigned char* dst = aop + ((((td * 2 + ts) * 2 + b) * 2) * 64 + lane_h * 32 + jn) * 16 + 2 * e0;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3]));
        *reinterpret_cast<uint2*>(dst + 64 * 16) = make_uint2(pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]));
      }
    }
    lds_barrier();

    // ---------------- stage 2: H = alpha V (the operands stay in LDS, next to the tiles)
    const uint4* opl = reinterpret_cast<const uint4*>(aop) + lane;
    {
      // Output tile (the wave's tile, reused once the chunk's operands are in
      // registers): row j = 32 td + 8 (r/4) + 4 h + r%4, channel 32 half + n.
      unsigned char* obase = vt + 4 * h * kORow + 2 * n;
      auto chunk2 = [&](int c, uint4 (&v)[8]) {
        wide_stage(vt, v, n_src);
        // Chunk c + 2, or the next token's stage-1 chunk c + 2 - nch.
        wide_load(c + 2 < nch ? tok : tokn, plane, n_src, (c + 2 < nch ? c + 2 : c + 2 - nch) * kChunk, v);
        wave_lds_sync();
        int ol = lane;
        asm volatile("" : "+v"(ol));
        uint4 op[2][4];
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
          for (int s = 0; s < 4; ++s) op[ts][s] = wide_operand(vt + ts * kTile * kVRow, ol, s);
        wave_lds_sync();  // operands read: the tile takes the outputs
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // bt[ts][b]: lane (h, n') element e holds source 32 ts +
          // transposed_row(b, h, e) of channel 32 half + n'.
          uint4 bt[2][2];
#pragma unroll
          for (int ts = 0; ts < 2; ++ts) {
            f16acc D1 = {};
            D1 = mfma(op[ts][2 * half], ident0, D1);
            D1 = mfma(op[ts][2 * half + 1], ident1, D1);
            bt[ts][0] = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
            bt[ts][1] = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
          }
#pragma unroll
          for (int td = 0; td < TD; ++td) {
            f16acc D2 = {};
#pragma unroll
            for (int ts = 0; ts < 2; ++ts)
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                const int o = ((td * 2 + ts) * 2 + b) * 2 * 64;
                D2 = mfma(opl[o], bt[ts][b], D2);       // alpha, bf16 high part
                D2 = mfma(opl[o + 64], bt[ts][b], D2);  //        low part
              }
#pragma unroll
            for (int r = 0; r < 16; ++r)
              *reinterpret_cast<bf16_t*>(obase + (td * kTile + 8 * (r / 4) + (r % 4)) * kORow + 64 * half) =
                  f2bf(D2[r]);
          }
        }
        wave_lds_sync();
        const int ch = ch_base + c * kChunk + 8 * (ol & 7);
        // Rows past n_dst store row n_dst - 1 again (identical bytes): no branch.
#pragma unroll
        for (int u = 0; u < 4 * TD; ++u) {
          const int j = min(8 * u + (ol >> 3), n_dst - 1);
          const uint4 o = *reinterpret_cast<const uint4*>(vt + j * kORow + ((ol & 7) << 4));
          __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w},
                                      reinterpret_cast<v4u*>(out + ((int64_t)j * T + t) * d + ch));
        }
        wave_lds_sync();  // the tile is rewritten by the next chunk
      };
      chunk2(0, va);
      chunk2(1, vb);
      for (int c = 2; c < nch; c += 2) {
        chunk2(c, va);
        chunk2(c + 1, vb);
      }
    }
    // The next token's stage 1 writes only this wave's tile; the partials
    // (over every tile) follow its first barrier, which every wave reaches
    // only after finishing this token's stage 2.
  }
}

template <int TD>
hipError_t launch_wide(const FullArgs& a, hipStream_t st) {
  uint4* qpk = static_cast<uint4*>(a.ws);
  hipLaunchKernelGGL(k_full_wide_qsplit<TD>, dim3(64), dim3(256), 0, st, a, qpk);
  auto kern = k_full_wide<TD>;
  constexpr size_t lds = wide_lds_bytes<TD>();
  if (lds > 64 * 1024) {
    static std::atomic<bool> allowed{false};  // dynamic LDS above 64 KiB is allowed per kernel, once
    if (!allowed.load(std::memory_order_relaxed)) {
      const hipError_t e =
          hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      allowed.store(true, std::memory_order_relaxed);
    }
  }
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), kWB, &per_cu, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWB), lds, st, a, (const uint4*)qpk);
  return hipGetLastError();
}

}  // namespace

size_t full_wide_workspace_bytes(int64_t n_dst, int64_t d) {
  return (size_t)2 * (n_dst > kTile ? 2 : 1) * kTile * (size_t)d * sizeof(bf16_t);
}

bool full_wide_shape(int64_t n_src, int64_t n_dst, int64_t d, int H, int dtype) {
  return dtype == kBF16 && H == 1 && n_src > kTile && n_src <= kWSrc && n_dst >= 1 && n_dst <= n_src &&
         d % (2 * kWW * kChunk) == 0 && d <= ((int64_t)1 << 16);
}

hipError_t launch_full_wide(const FullArgs& a, hipStream_t st) {
  return a.n_dst > kTile ? launch_wide<2>(a, st) : launch_wide<1>(a, st);
}

}  // namespace attnres
