// Block AttnRes backward for every block depth on gfx950 (bf16 I/O, fp32
// arithmetic): gradients of L = sum_j <dh_j, h_j> for one block of Block
// AttnRes / MHAR (the analytic form in attnres.h).  Destination j of the
// block reads the N reps and, for j >= 1, the partial sum b_{j} (b-lab.team
// summary §2, the value matrix); the pages give no backward, so this is the
// chain rule through that forward.  One kernel per (N, S) with N = 1..12 and
// S = 1..4.  A block of more than 4 sublayers runs as two chunks of
// consecutive destinations: the first chunk writes its rep gradients in fp32
// to the workspace, and the second chunk's kernel (PO = 0), whose first
// destination reads a partial too, adds its own to them before the one
// rounding to bf16 (the gradient is a sum over destinations) and writes its
// Z rows into the same slabs.
//
// A persistent workgroup of B = d / 8 threads owns all channels of one token
// at a time, thread `tid` owning the 8 channels at tid * 8.  Per token the
// workgroup
//   1. loads the N reps, the S-PO partials and the S upstream gradients once,
//   2. accumulates per-thread partial sums per source i -- its sum of squares
//      and, for every destination j reading it, q_j . v_i and dh_j . v_i --
//      and reduces them across the wave one source group at a time (at most
//      64 values a group, so few partial sums are live at once), then across
//      waves through LDS,
//   3. forms, in lanes (one per (destination, source) pair), alpha,
//      c = alpha (a - sum alpha a), c r_i and the normalisation-path
//      coefficient r_i^2 sum_j c s / d,
//   4. writes dv_i = sum_j (alpha dh_j + c r_i q_j) - coef_i v_i, and
//   5. accumulates Z_j += sum_i c r_i v_i in registers across its tokens.
// At the end each workgroup writes its Z slab; the fixed-order reduction
// (k_bwd_reduce) turns the slabs into dw and dgain.
//
// Heads (chatpaper.ai MHAR abstract): wave w owns channels [512 w, 512 w +
// 512), so a head of d/H channels is W/H consecutive waves.  The sums of
// squares reduce over the whole workgroup (the RMS spans all of d), the dot
// products over the head's waves; the one quantity mixing heads, the sum over
// (j, h) of c s in the normalisation path, takes a second LDS exchange.
//
// This header holds the kernel and its launcher; block_nNN.hip instantiate
// them per rep count and bwd_fast.hip plans and dispatches a call.
#pragma once

#include <math.h>

#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {

// How a backward call runs on the specialised kernel (B == 0: not eligible).
struct BwdPlan {
  int B = 0;
  int hh = 1;
  size_t lds = 0;  // the larger chunk's
  int s0 = 0;      // destinations of the first chunk (all of them unless S > 4)
};

template <int N>
hipError_t bwd_launch_n(const BwdArgs& a, const BwdPlan& p, int po, bool dry, int64_t* slots_used, hipStream_t st);
#define ATTNRES_BWD_DECLARE(n)                                                                  \
  template <>                                                                                   \
  hipError_t bwd_launch_n<n>(const BwdArgs& a, const BwdPlan& p, int po, bool dry, int64_t* slots_used, \
                             hipStream_t st);
ATTNRES_BWD_DECLARE(1) ATTNRES_BWD_DECLARE(2) ATTNRES_BWD_DECLARE(3) ATTNRES_BWD_DECLARE(4)
ATTNRES_BWD_DECLARE(5) ATTNRES_BWD_DECLARE(6) ATTNRES_BWD_DECLARE(7) ATTNRES_BWD_DECLARE(8)
ATTNRES_BWD_DECLARE(9) ATTNRES_BWD_DECLARE(10) ATTNRES_BWD_DECLARE(11) ATTNRES_BWD_DECLARE(12)
#undef ATTNRES_BWD_DECLARE

// Layout of one wave's reduction row: source i (i < N a rep, else partial
// i - N, read only by destination i - N + PO) owns bwd_cnt(i) consecutive
// values from bwd_off(i): its sum of squares, then q_j . v_i and dh_j . v_i
// for each destination j reading it, in destination order.
template <int N, int S>
constexpr int bwd_cnt(int i) { return i < N ? 1 + 2 * S : 3; }
template <int N, int S>
constexpr int bwd_off(int i) { return i < N ? i * (1 + 2 * S) : N * (1 + 2 * S) + (i - N) * 3; }
// PO = 1: partial k is read by destination k + 1 (a whole block, or its first
// chunk); PO = 0: by destination k (a later chunk).  N + S - PO sources.
template <int N, int S, int PO>
constexpr int bwd_row_len() { return (bwd_off<N, S>(N + S - PO) + 7) / 8 * 8; }

namespace {

constexpr int bwd_pow2(int n) { return n <= 1 ? 1 : 2 * bwd_pow2((n + 1) / 2); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bwd_row(const void* row) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, 0x7fffffff, kBufferWord3);
}
__device__ __forceinline__ uint4 bwd_ld(const void* row, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(bwd_row(row), (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bwd_st(void* row, uint32_t off, uint4 u) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(v4u{u.x, u.y, u.z, u.w}, bwd_row(row), (int)off, 0, 0);
}
// 8 fp32 values at byte offset off of an fp32 row: stored, or added to x.
__device__ __forceinline__ void bwd_st32(float* row, uint32_t off, const float (&x)[8]) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(v4f{x[0], x[1], x[2], x[3]}, bwd_row(row), (int)off, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(v4f{x[4], x[5], x[6], x[7]}, bwd_row(row), (int)off + 16, 0, 0);
}
__device__ __forceinline__ void bwd_add32(const float* row, uint32_t off, float (&x)[8]) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f lo = __builtin_amdgcn_raw_buffer_load_b128(bwd_row(row), (int)off, 0, 0);
  const v4f hi = __builtin_amdgcn_raw_buffer_load_b128(bwd_row(row), (int)off + 16, 0, 0);
  x[0] += lo.x; x[1] += lo.y; x[2] += lo.z; x[3] += lo.w;
  x[4] += hi.x; x[5] += hi.y; x[6] += hi.z; x[7] += hi.w;
}
__device__ __forceinline__ void bwd_unpack8(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}
__device__ __forceinline__ uint4 bwd_pack8(const float (&x)[8]) {
  return make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7]));
}

// Reduce values v[OFF .. OFF + REM) over the wave into dst[OFF + k] (one lane
// per value), in transposing reductions of 64, 32, 16 or 8 values (the
// largest that fits; a remainder below 8 is padded with zeros).
template <int OFF, int REM, int P>
__device__ __forceinline__ void bwd_reduce_store(const float (&v)[P], float* dst, int rl) {
  if constexpr (REM > 0) {
    constexpr int SZ = REM >= 64 ? 64 : REM >= 32 ? 32 : REM >= 16 ? 16 : 8;
    constexpr int TAKE = SZ < REM ? SZ : REM;
    float seg[SZ];
#pragma unroll
    for (int k = 0; k < SZ; ++k) seg[k] = k < TAKE ? v[OFF + k] : 0.f;
    if constexpr (SZ == 64) {
      dst[OFF + rl] = transpose_reduce64(seg);
    } else if constexpr (SZ == 32) {
      const float r = transpose_reduce_pow2<32>(seg);
      if ((rl & 1) == 0) dst[OFF + (rl >> 1)] = r;
    } else if constexpr (SZ == 16) {
      const float r = transpose_reduce16(seg);
      if ((rl & 3) == 0) dst[OFF + (rl >> 2)] = r;
    } else {
      const float r = transpose_reduce_pow2<8>(seg);
      if ((rl & 7) == 0 && (rl >> 3) < TAKE) dst[OFF + (rl >> 3)] = r;
    }
    bwd_reduce_store<OFF + TAKE, REM - TAKE, P>(v, dst, rl);
  }
}

// The end of the source group starting at I0: sources I0 .. I1-1 with at most
// 64 values between them (at least one source).
template <int N, int S, int PO>
constexpr int bwd_group_end(int i0) {
  int i1 = i0 + 1;
  while (i1 < N + S - PO && bwd_off<N, S>(i1 + 1) - bwd_off<N, S>(i0) <= 64) ++i1;
  return i1;
}

// Partial sums of the sources from I0 on, one group at a time, each group
// reduced into its slots of the wave's row before the next is accumulated.
template <int N, int S, int PO, int I0>
__device__ __forceinline__ void bwd_partials(const uint4 (&v)[N + S - PO], const float (&qc)[S][8],
                                             const float (&dg)[S][8], float* row, int rl) {
  if constexpr (I0 < N + S - PO) {
    constexpr int I1 = bwd_group_end<N, S, PO>(I0);
    constexpr int O0 = bwd_off<N, S>(I0);
    constexpr int GC = bwd_off<N, S>(I1) - O0;
    float part[GC];
#pragma unroll
    for (int p = 0; p < GC; ++p) part[p] = 0.f;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      float x[8];
      bwd_unpack8(v[i], x);
      const int o = bwd_off<N, S>(i) - O0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        part[o] = fmaf(x[e], x[e], part[o]);
        if (i < N) {
#pragma unroll
          for (int j = 0; j < S; ++j) {
            part[o + 1 + 2 * j] = fmaf(qc[j][e], x[e], part[o + 1 + 2 * j]);
            part[o + 2 + 2 * j] = fmaf(dg[j][e], x[e], part[o + 2 + 2 * j]);
          }
        } else {
          const int j = i - N + PO;
          part[o + 1] = fmaf(qc[j][e], x[e], part[o + 1]);
          part[o + 2] = fmaf(dg[j][e], x[e], part[o + 2]);
        }
      }
    }
    bwd_reduce_store<0, GC, GC>(part, row + O0, rl);
    bwd_partials<N, S, PO, I1>(v, qc, dg, row, rl);
  }
}

// q = w * g into this thread's own LDS slots; out of line, like Phase 1's fold.
template <int S>
__device__ __noinline__ void bwd_fold(const float* w, const float* gain, int64_t gain_ld, int d, int B, int tid,
                                      float4* qs) {
#pragma unroll
  for (int j = 0; j < S; ++j) {
    float qq[8];
    const int col = tid * 8;
    if (gain != nullptr)
      fold_q8<true>(w + (int64_t)j * d + col, gain + j * gain_ld + col, qq);
    else
      fold_q8<false>(w + (int64_t)j * d + col, gain, qq);
    qs[(j * B + tid) * 2 + 0] = make_float4(qq[0], qq[1], qq[2], qq[3]);
    qs[(j * B + tid) * 2 + 1] = make_float4(qq[4], qq[5], qq[6], qq[7]);
  }
}

template <int N, int S, int HH, int PO>
__global__ __launch_bounds__(512, 1) void k_bwd(BwdArgs a) {
  constexpr int NS = N + S - PO;              // sources: N reps, then S-PO partials
  constexpr int PR = bwd_row_len<N, S, PO>();  // floats per wave row
  constexpr int NP = bwd_pow2(N + 1);       // lanes per destination group
  static_assert(S * NP <= 64, "pair table must fit one wave");
  extern __shared__ float4 bwd_smem[];
  __shared__ float csx[2][HH > 1 ? HH : 1][64];  // per-head sum of c s, heads > 1 only

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int B = blockDim.x, W = B >> 6, WH = W / HH;  // waves per head
  const int d = (int)a.d;
  const int64_t T = a.T;
  float4* qs = bwd_smem;                                         // [S][B][2], this thread's slots
  float* red = reinterpret_cast<float*>(bwd_smem + S * 2 * B);   // [2][W][PR]

  bwd_fold<S>(a.w, a.gain, a.gain_ld, d, B, tid, qs);

  float zacc[S][8];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[j][e] = 0.f;

  const bf16_t* reps = static_cast<const bf16_t*>(a.reps);
  const bf16_t* parts = static_cast<const bf16_t*>(a.partials);
  const bf16_t* dhp = static_cast<const bf16_t*>(a.dh);
  bf16_t* d_reps = static_cast<bf16_t*>(a.d_reps);
  bf16_t* d_parts = static_cast<bf16_t*>(a.d_partials);
  const int64_t td = T * d;
  const uint32_t coff = (uint32_t)tid * 16u;  // this thread's byte offset in a bf16 row
  auto src_row = [&](int i, int64_t t) { return i < N ? reps + i * td + t * d : parts + (i - N) * td + t * d; };
  auto dsrc_row = [&](int i, int64_t t) { return i < N ? d_reps + i * td + t * d : d_parts + (i - N) * td + t * d; };

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    // Wave priority: a token's loads and partial sums at 0, its source
    // gradients and stores at 2.
    __builtin_amdgcn_s_setprio(0);
    uint4 v[NS], g[S];
#pragma unroll
    for (int i = 0; i < NS; ++i) v[i] = bwd_ld(src_row(i, t), coff);
#pragma unroll
    for (int j = 0; j < S; ++j) g[j] = bwd_ld(dhp + j * td + t * d, coff);

    float qc[S][8], dg[S][8];
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const float4 q0 = qs[(j * B + tid) * 2 + 0];
      const float4 q1 = qs[(j * B + tid) * 2 + 1];
      qc[j][0] = q0.x; qc[j][1] = q0.y; qc[j][2] = q0.z; qc[j][3] = q0.w;
      qc[j][4] = q1.x; qc[j][5] = q1.y; qc[j][6] = q1.z; qc[j][7] = q1.w;
      bwd_unpack8(g[j], dg[j]);
    }
    {
      // Lane-dependent LDS addresses from an opaque copy of the lane id,
      // recomputed per token (held across the loop they cost registers).
      int rl = lane;
      asm volatile("" : "+v"(rl));
      bwd_partials<N, S, PO, 0>(v, qc, dg, red + (buf * W + wave) * PR, rl);
    }
    __syncthreads();

    // Per-pair scalars, one lane per (destination pj, slot pu): slot pu < N
    // is rep pu, slot N the partial destination pj >= PO reads.
    int sl = lane;
    asm volatile("" : "+v"(sl));
    const int pj = sl / NP, pu = sl % NP;
    const bool pvalid = pj < S && (pu < N || (pu == N && pj >= PO));
    // This pair's source values in the row: its sum of squares at soff, q . v
    // at pslot and dh . v right after.
    const int soff = pu < N ? pu * (1 + 2 * S) : N * (1 + 2 * S) + (pj - PO) * 3;
    const int pslot = soff + 1 + (pu < N ? 2 * pj : 0);
    float alpha = 0.f, cr = 0.f, coef = 0.f;
    {
      const float* rb = red + buf * W * PR;
      float ss = 0.f, sd = 0.f, ad = 0.f;
      if (pvalid) {
        const int h0 = (wave / WH) * WH;  // first wave of this head
        for (int w2 = 0; w2 < W; ++w2) ss += rb[w2 * PR + soff];
        for (int w2 = 0; w2 < WH; ++w2) {
          sd += rb[(h0 + w2) * PR + pslot];
          ad += rb[(h0 + w2) * PR + pslot + 1];
        }
      }
      const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
      const float s = pvalid ? r * sd : -INFINITY;
      const float av = pvalid ? ad : 0.f;
      const float m = group_max<NP>(s);
      const float e = pvalid ? expf(s - m) : 0.f;
      const float l = group_sum<NP>(e);
      alpha = e / l;
      const float sa = group_sum<NP>(alpha * av);
      const float c = alpha * (av - sa);
      cr = c * r;
      // sum_j c s over the destinations reading the same rep (same slot, other groups)
      const float cs = pvalid ? c * s : 0.f;
      const float csum = butterfly<NP, 64>(cs, SumOp());
      float csh = pu < N ? csum : cs;
      if constexpr (HH > 1) {
        // Sum over heads, in head order, from the first wave of each head.
        if (wave % WH == 0) csx[buf][wave / WH][sl] = csh;
        __syncthreads();
        csh = 0.f;
#pragma unroll
        for (int h = 0; h < HH; ++h) csh += csx[buf][h][sl];
      }
      coef = pvalid ? r * r * csh / (float)d : 0.f;
    }

    __builtin_amdgcn_s_setprio(2);
    // Source gradients and Z, from registers.
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float x[8], gr[8];
      bwd_unpack8(v[i], x);
      const int u = i < N ? i : N;
      const float cf = read_lane(coef, (i < N ? 0 : i - N + PO) * NP + u);
#pragma unroll
      for (int e = 0; e < 8; ++e) gr[e] = -cf * x[e];
#pragma unroll
      for (int j = 0; j < S; ++j) {
        if (i < N || i == N + j - PO) {
          const float al = read_lane(alpha, j * NP + u);
          const float crl = read_lane(cr, j * NP + u);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            gr[e] = fmaf(al, dg[j][e], gr[e]);
            gr[e] = fmaf(crl, qc[j][e], gr[e]);
            zacc[j][e] = fmaf(crl, x[e], zacc[j][e]);
          }
        }
      }
      bf16_t* out = dsrc_row(i, t);
      if (i < N && a.rep_mode != 0) {
        // Rep gradients of a block split into destination chunks, in fp32.
        float* r32 = a.rep32 + i * td + t * d;
        if (a.rep_mode == 1) {
          bwd_st32(r32, coff * 2u, gr);
          continue;
        }
        bwd_add32(r32, coff * 2u, gr);
      }
      if (a.accumulate) {
        float old[8];
        bwd_unpack8(bwd_ld(out, coff), old);
#pragma unroll
        for (int e = 0; e < 8; ++e) gr[e] += old[e];
      }
      bwd_st(out, coff, bwd_pack8(gr));
    }
    buf ^= 1;
  }

  // This workgroup's slab of Z partial sums: zslots[blockIdx][j][channel],
  // slabs zld floats apart.
  float* z = a.zslots + (int64_t)blockIdx.x * a.zld;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    float4* zp = reinterpret_cast<float4*>(z + (int64_t)j * d + tid * 8);
    zp[0] = make_float4(zacc[j][0], zacc[j][1], zacc[j][2], zacc[j][3]);
    zp[1] = make_float4(zacc[j][4], zacc[j][5], zacc[j][6], zacc[j][7]);
  }
}

// Launches one chunk (or, with dry set, only reports the grid it would use).
template <int N, int S, int HH, int PO>
hipError_t bwd_go(const BwdArgs& a, const BwdPlan& p, bool dry, int64_t* slots_used, hipStream_t st) {
  auto kern = k_bwd<N, S, HH, PO>;
  static std::atomic<size_t> allowed{64 * 1024};
  if (p.lds > allowed.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
    allowed.store(p.lds, std::memory_order_relaxed);
  }
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), p.B, &per_cu, p.lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  if (grid > a.slots) grid = a.slots;
  *slots_used = grid;
  if (dry) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((unsigned)p.B), p.lds, st, a);
  return hipGetLastError();
}

template <int N, int S, int PO>
hipError_t bwd_go_s(const BwdArgs& a, const BwdPlan& p, bool dry, int64_t* slots_used, hipStream_t st) {
  switch (p.hh) {
    case 1: return bwd_go<N, S, 1, PO>(a, p, dry, slots_used, st);
    case 2: return bwd_go<N, S, 2, PO>(a, p, dry, slots_used, st);
    case 4: return bwd_go<N, S, 4, PO>(a, p, dry, slots_used, st);
    case 8: return bwd_go<N, S, 8, PO>(a, p, dry, slots_used, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

// a.S destinations of one chunk: PO = 1 for S = 1..4, PO = 0 for S = 2..4
// (a later chunk of a block of 5..8).
template <int N>
hipError_t bwd_launch_for(const BwdArgs& a, const BwdPlan& p, int po, bool dry, int64_t* slots_used,
                          hipStream_t st) {
  if (po == 0) {
    switch (a.S) {
      case 2: return bwd_go_s<N, 2, 0>(a, p, dry, slots_used, st);
      case 3: return bwd_go_s<N, 3, 0>(a, p, dry, slots_used, st);
      case 4: return bwd_go_s<N, 4, 0>(a, p, dry, slots_used, st);
      default: return hipErrorNotSupported;
    }
  }
  switch (a.S) {
    case 1: return bwd_go_s<N, 1, 1>(a, p, dry, slots_used, st);
    case 2: return bwd_go_s<N, 2, 1>(a, p, dry, slots_used, st);
    case 3: return bwd_go_s<N, 3, 1>(a, p, dry, slots_used, st);
    case 4: return bwd_go_s<N, 4, 1>(a, p, dry, slots_used, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attnres
