// Block AttnRes Phase 1 for every block depth on gfx950 (bf16 sources, fp32
// arithmetic): the S pseudo-queries of a block against its N cached block
// representations in one pass over the reps (b-lab.team summary §3, Inference:
// Phase 1; dimensionstp "Attention Residuals Review" §3-2 (4)).  Block n of a
// model reads N = n reps (b-lab.team summary §2, the value matrix), so one
// kernel is compiled per (N, S) with N = 1..12 and S = 1..8.
//
// A persistent workgroup of B threads owns every channel of one token at a
// time: thread `tid` owns CH chunks of 8 consecutive channels at
// (c * B + tid) * 8, so each wave's 16-byte loads cover a contiguous 1 KiB per
// chunk and d = 8 * CH * B.  Per token the workgroup
//   1. streams the N rep rows once into registers (16-byte buffer loads),
//   2. accumulates per-thread partial sums of squares (N) and dot products
//      q_l . v_i (S * N, per chunk when heads differ between chunks),
//   3. reduces them across the wave with transposing reductions (lane p ends
//      with value p) and across waves through LDS (one barrier),
//   4. forms scores, softmax and lse per (layer, head) in lanes, and
//   5. writes o_l = sum_i alpha_{l,i} v_i from the registers; as each rep row
//      is used for the last time its register is refilled with the rep row
//      of the workgroup's next token.
// q = w * g sits in LDS; each thread reads back only its own channels.
//
// This header holds the kernel and its launcher; block_nNN.hip instantiate them
// for one rep count each (so the instantiations compile in parallel) and
// p1_fast.hip plans and dispatches a call.
#pragma once

#include <math.h>

#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {

// How a Phase 1 call runs on the specialised kernel (p1_plan; ch == 0: not
// eligible).  B threads per workgroup own CH chunks of 8 channels each; mh:
// heads (H > 1); lds: bytes of dynamic LDS per workgroup (q, then the
// reduction rows).
struct P1Plan {
  int ch = 0;
  bool mh = false;
  int B = 0;
  size_t lds = 0;
};

// Launches the kernel instantiated for N reps (defined in block_nNN.hip).
template <int N>
hipError_t p1_launch_n(const Phase1Args& a, const P1Plan& p, hipStream_t st);
#define ATTNRES_P1_DECLARE(n) \
  template <>                 \
  hipError_t p1_launch_n<n>(const Phase1Args& a, const P1Plan& p, hipStream_t st);
ATTNRES_P1_DECLARE(1) ATTNRES_P1_DECLARE(2) ATTNRES_P1_DECLARE(3) ATTNRES_P1_DECLARE(4)
ATTNRES_P1_DECLARE(5) ATTNRES_P1_DECLARE(6) ATTNRES_P1_DECLARE(7) ATTNRES_P1_DECLARE(8)
ATTNRES_P1_DECLARE(9) ATTNRES_P1_DECLARE(10) ATTNRES_P1_DECLARE(11) ATTNRES_P1_DECLARE(12)
#undef ATTNRES_P1_DECLARE

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int p1_pow2(int n) { return n <= 1 ? 1 : 2 * p1_pow2((n + 1) / 2); }

// Buffer descriptor of a row whose address is the same for the whole wave:
// loads and stores then take the row as a scalar base plus a 32-bit vector
// byte offset (no 64-bit address per lane in registers).  The range,
// 2^31 - 1 bytes, covers any row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t p1_row(const void* row) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, 0x7fffffff, kBufferWord3);
}

__device__ __forceinline__ uint4 p1_ld(const void* row, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(p1_row(row), (int)off, 0, kBufferNt);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void p1_st(void* row, uint32_t off, uint4 u) {
  __builtin_amdgcn_raw_buffer_store_b128(v4u{u.x, u.y, u.z, u.w}, p1_row(row), (int)off, 0, kBufferNt);
}

__device__ __forceinline__ void p1_unpack8(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}

// Reduce values v[OFF .. OFF + REM) over the wave and write total k to
// dst[OFF + k], one lane per value.  The values are taken in transposing
// reductions of 64, 32, 16 or 8 (the largest that fits; a remainder below 8
// is padded with zeros).  rl is the lane id.
template <int OFF, int REM, int P>
__device__ __forceinline__ void p1_reduce_store(const float (&v)[P], float* dst, int rl) {
  if constexpr (REM > 0) {
    constexpr int SZ = REM >= 64 ? 64 : REM >= 32 ? 32 : REM >= 16 ? 16 : 8;
    constexpr int TAKE = SZ < REM ? SZ : REM;
    float seg[SZ];
#pragma unroll
    for (int k = 0; k < SZ; ++k) seg[k] = k < TAKE ? v[OFF + k] : 0.f;
    if constexpr (SZ == 64) {
      dst[OFF + rl] = transpose_reduce64(seg);
    } else if constexpr (SZ == 32) {
      const float r = transpose_reduce_pow2<32>(seg);  // lane L: value L >> 1
      if ((rl & 1) == 0) dst[OFF + (rl >> 1)] = r;
    } else if constexpr (SZ == 16) {
      const float r = transpose_reduce16(seg);         // lane L: value L >> 2
      if ((rl & 3) == 0) dst[OFF + (rl >> 2)] = r;
    } else {
      const float r = transpose_reduce_pow2<8>(seg);   // lane L: value L >> 3
      if ((rl & 7) == 0 && (rl >> 3) < TAKE) dst[OFF + (rl >> 3)] = r;
    }
    p1_reduce_store<OFF + TAKE, REM - TAKE, P>(v, dst, rl);
  }
}

// q = w * g into this thread's own LDS slots (two float4 per chunk and
// query).  Out of line, so that the prologue cannot change how the token loop
// is scheduled and allocated.
template <int S, int CH, bool G>
__device__ __noinline__ void p1_fold(const float* w, const float* gain, int64_t gain_ld, int d, int B, int tid,
                                     float4* qs) {
#pragma unroll
  for (int l = 0; l < S; ++l)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float qq[8];
      const int col = (c * B + tid) * 8;
      fold_q8<G>(w + (int64_t)l * d + col, gain + l * gain_ld + col, qq);
      qs[((l * CH + c) * B + tid) * 2 + 0] = make_float4(qq[0], qq[1], qq[2], qq[3]);
      qs[((l * CH + c) * B + tid) * 2 + 1] = make_float4(qq[4], qq[5], qq[6], qq[7]);
    }
}

// Floats of one wave's reduction row (the S N (per chunk with heads) dot
// products and N sums of squares of a token, padded to a multiple of 8).
template <int N, int S, int CH, bool MH>
constexpr int p1_row_len() {
  return (((MH ? CH : 1) * S * N + N) + 7) / 8 * 8;
}

// q = w * g into this thread's own LDS slots, inline (the small-T kernel
// issues its token's rep loads first, so both latencies overlap).
template <int S, int CH, bool G>
__device__ __forceinline__ void p1_fold_inline(const float* w, const float* gain, int64_t gain_ld, int d, int B,
                                               int tid, float4* qs) {
#pragma unroll
  for (int l = 0; l < S; ++l)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float qq[8];
      const int col = (c * B + tid) * 8;
      fold_q8<G>(w + (int64_t)l * d + col, gain + l * gain_ld + col, qq);
      qs[((l * CH + c) * B + tid) * 2 + 0] = make_float4(qq[0], qq[1], qq[2], qq[3]);
      qs[((l * CH + c) * B + tid) * 2 + 1] = make_float4(qq[4], qq[5], qq[6], qq[7]);
    }
}

// The token loop; q = w * g is already in the thread's LDS slots, or, with
// FOLD (one token per workgroup), is folded right after the first token's
// rep loads are issued, so that the two memory latencies overlap.
template <int N, int S, int CH, bool MH, bool FOLD = false>
__device__ __forceinline__ void p1_body(const Phase1Args& a, float4* smem) {
  constexpr int CHH = MH ? CH : 1;           // dot-product groups per thread
  constexpr int NDOT = CHH * S * N;
  constexpr int P = NDOT + N;                // values reduced per token
  constexpr int PP = p1_row_len<N, S, CH, MH>();
  constexpr int NP = p1_pow2(N);             // lanes per softmax group
  constexpr int TAB = CHH * S * NP;          // softmax lanes
  constexpr int R = (TAB + 63) / 64;         // rounds of 64 lanes

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // d = 8 CH B: the block size from a kernel argument (blockDim.x is read
  // from memory, a round trip at the start of every launch).
  const int B = (int)a.d / (8 * CH), W = B >> 6;
  const int d = (int)a.d;
  const int64_t T = a.T;
  const int segs_per_head = (d / a.H) / 512;  // 512-channel segments per head
  float4* qs = smem;
  float* red = reinterpret_cast<float*>(smem + S * CH * B * 2);  // [2][W][PP]
  const bool f16_state = a.orest_dtype == kF16;

  const bf16_t* reps = static_cast<const bf16_t*>(a.reps);
  const int64_t rs = a.rep_stride != 0 ? a.rep_stride : T * d;
  const int64_t os = a.orest_stride != 0 ? a.orest_stride : T * d;  // state rows
  const uint32_t coff = (uint32_t)tid * 16u;  // this thread's byte offset in a bf16 row (chunk 0)
  const int64_t Gs = gridDim.x;
  int buf = 0;

  auto load_all = [&](uint4 (&v)[N][CH], int64_t t) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int c = 0; c < CH; ++c) v[i][c] = p1_ld(reps + (int64_t)i * rs + t * d, coff + (uint32_t)(c * B * 16));
  };

  auto token = [&](uint4 (&v)[N][CH], const int64_t t) {
    const int64_t tn = t + Gs;
    // Wave priority: scores at 1, reductions and softmax at 3, weighted sums
    // and stores at 0.  With two workgroups per CU the one heading for its
    // barrier issues first; the weighted sums issue the next token's loads
    // and fill the gaps.
    __builtin_amdgcn_s_setprio(1);
    float part[P];
#pragma unroll
    for (int p = 0; p < P; ++p) part[p] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = MH ? c : 0;
      float qc[S][8];
#pragma unroll
      for (int l = 0; l < S; ++l) {
        const float4 q0 = qs[((l * CH + c) * B + tid) * 2 + 0];
        const float4 q1 = qs[((l * CH + c) * B + tid) * 2 + 1];
        qc[l][0] = q0.x; qc[l][1] = q0.y; qc[l][2] = q0.z; qc[l][3] = q0.w;
        qc[l][4] = q1.x; qc[l][5] = q1.y; qc[l][6] = q1.z; qc[l][7] = q1.w;
      }
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float x[8];
        p1_unpack8(v[i][c], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          part[NDOT + i] = fmaf(x[e], x[e], part[NDOT + i]);
#pragma unroll
          for (int l = 0; l < S; ++l)
            part[(cc * S + l) * N + i] = fmaf(qc[l][e], x[e], part[(cc * S + l) * N + i]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(3);
    {
      // Lane-dependent LDS addresses come from an opaque copy of the lane id,
      // recomputed per token: held across the loop they would take registers
      // the token needs (and a spill reload waits for every outstanding load).
      int rl = lane;
      asm volatile("" : "+v"(rl));
      p1_reduce_store<0, P, P>(part, red + (buf * W + wave) * PP, rl);
    }
    __syncthreads();

    // Scores, softmax and lse, one lane per (chunk, layer, rep) of this wave
    // in R rounds of 64 lanes.
    int sl = lane;
    asm volatile("" : "+v"(sl));
    const float* rb = red + buf * W * PP;
    // The scaled fp16 state of layers >= 2: every |o| <= sqrt(max_i ss_i), so
    // the token's power-of-two scale follows from the sums of squares alone.
    float inv_scale = 1.0f;
    if (f16_state) {
      float ss0 = 0.f;
      if (sl < N)
        for (int w2 = 0; w2 < W; ++w2) ss0 += rb[w2 * PP + NDOT + sl];
      const float scale = f16_state_scale(sqrtf(group_max<64>(ss0)));
      inv_scale = 1.0f / scale;  // exact: a power of two
      if (wave == 0 && lane == 0) a.oscale[t] = scale;
    }
    float alpha[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = r * 64 + sl;
      const int sm_cc = idx / (S * NP), sm_l = (idx / NP) % S, sm_i = idx % NP;
      const bool valid = idx < TAB && sm_i < N;
      const int seg = sm_cc * W + wave;           // 512-channel segment of chunk sm_cc (MH only)
      const int head = MH ? seg / segs_per_head : 0;
      float ss = 0.f, dot = 0.f;
      if (valid) {
        for (int w2 = 0; w2 < W; ++w2) ss += rb[w2 * PP + NDOT + sm_i];
        if constexpr (!MH) {
          for (int w2 = 0; w2 < W; ++w2) dot += rb[w2 * PP + sm_l * N + sm_i];
        } else {
#pragma unroll
          for (int c2 = 0; c2 < CHH; ++c2)
            for (int w2 = 0; w2 < W; ++w2)
              if ((c2 * W + w2) / segs_per_head == head) dot += rb[w2 * PP + (c2 * S + sm_l) * N + sm_i];
        }
      }
      const float rinv = 1.0f / sqrtf(ss / (float)d + a.eps);
      const float s = valid ? rinv * dot : -INFINITY;
      const float m = group_max<NP>(s);
      const float e = valid ? expf(s - m) : 0.f;
      const float l = group_sum<NP>(e);
      alpha[r] = e / l;
      if (sm_l >= 1) alpha[r] *= inv_scale;
      const bool lse_writer = valid && sm_i == 0 && (MH ? seg % segs_per_head == 0 : wave == 0);
      if (lse_writer) a.lse[((int64_t)sm_l * a.H + head) * T + t] = m + logf(l);
    }

    __builtin_amdgcn_s_setprio(0);
    // o_l = sum_i alpha_{l,i} v_i for each of this thread's chunks, from registers.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = MH ? c : 0;
      float acc[S][8];
#pragma unroll
      for (int l = 0; l < S; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float x[8];
        p1_unpack8(v[i][c], x);
        if constexpr (!MH) {
          // The next token's row goes into the register as soon as its last
          // use here is done: the loads overlap the rest of the weighted sums
          // and the stores.  (With heads there are no registers to spare.)
          if (tn < T) v[i][c] = p1_ld(reps + (int64_t)i * rs + tn * d, coff + (uint32_t)(c * B * 16));
        }
#pragma unroll
        for (int l = 0; l < S; ++l) {
          const int idx = (cc * S + l) * NP + i;
          const float al = read_lane(alpha[idx >> 6], idx & 63);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[l][e] = fmaf(al, x[e], acc[l][e]);
        }
      }
      const uint32_t off = coff + (uint32_t)(c * B * 16);
      p1_st(static_cast<bf16_t*>(a.o0) + t * d, off,
            make_uint4(pack_bf2(acc[0][0], acc[0][1]), pack_bf2(acc[0][2], acc[0][3]),
                       pack_bf2(acc[0][4], acc[0][5]), pack_bf2(acc[0][6], acc[0][7])));
#pragma unroll
      for (int l = 1; l < S; ++l) {
        const int64_t row_off = (int64_t)(l - 1) * os + t * d;
        if (f16_state) {
          typedef _Float16 h8 __attribute__((ext_vector_type(8)));
          const h8 h = {(f16_t)acc[l][0], (f16_t)acc[l][1], (f16_t)acc[l][2], (f16_t)acc[l][3],
                        (f16_t)acc[l][4], (f16_t)acc[l][5], (f16_t)acc[l][6], (f16_t)acc[l][7]};
          p1_st(static_cast<f16_t*>(a.orest) + row_off, off, __builtin_bit_cast(uint4, h));
        } else {
          float* orow = static_cast<float*>(a.orest) + row_off;
          p1_st(orow, 2 * off, make_uint4(__float_as_uint(acc[l][0]), __float_as_uint(acc[l][1]),
                                         __float_as_uint(acc[l][2]), __float_as_uint(acc[l][3])));
          p1_st(orow, 2 * off + 16, make_uint4(__float_as_uint(acc[l][4]), __float_as_uint(acc[l][5]),
                                              __float_as_uint(acc[l][6]), __float_as_uint(acc[l][7])));
        }
      }
    }
    buf ^= 1;
    if constexpr (MH) {
      if (tn < T) load_all(v, tn);
    }
  };

  uint4 v[N][CH];
  int64_t t = blockIdx.x;
  if (t < T) load_all(v, t);
  if constexpr (FOLD) {
    // Each thread reads back only its own slots, so no barrier is needed.
    if (a.gain != nullptr)
      p1_fold_inline<S, CH, true>(a.w, a.gain, a.gain_ld, d, B, tid, qs);
    else
      p1_fold_inline<S, CH, false>(a.w, a.gain, a.gain_ld, d, B, tid, qs);
  }
  for (; t < T; t += Gs) token(v, t);
}

template <int N, int S, int CH, bool MH>
__global__ __launch_bounds__(512, 2) void k_p1(Phase1Args a) {
  extern __shared__ float4 p1_smem[];
  if (a.gain != nullptr)
    p1_fold<S, CH, true>(a.w, a.gain, a.gain_ld, (int)a.d, (int)a.d / (8 * CH), (int)threadIdx.x, p1_smem);
  else
    p1_fold<S, CH, false>(a.w, a.gain, a.gain_ld, (int)a.d, (int)a.d / (8 * CH), (int)threadIdx.x, p1_smem);
  p1_body<N, S, CH, MH>(a, p1_smem);
}

// Small T (every workgroup gets at most one token): the same kernel with the
// fold of q moved after the issue of the token's rep loads (inline), instead
// of a prologue that completes before the rows are requested.  Same channel
// map and reductions as k_p1, so the same bits.
template <int N, int S, int CH, bool MH>
__global__ __launch_bounds__(512, 2) void k_p1s(Phase1Args a) {
  extern __shared__ float4 p1_smem[];
  p1_body<N, S, CH, MH, true>(a, p1_smem);
}

template <int N, int S, int CH, bool MH>
hipError_t p1_go(const Phase1Args& a, const P1Plan& p, hipStream_t st) {
  auto kern = k_p1<N, S, CH, MH>;
  // Dynamic LDS above the default limit has to be allowed per kernel, once.
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
  if (grid >= a.T) {
    // One token per workgroup: the small-T kernel.
    auto ks = k_p1s<N, S, CH, MH>;
    static std::atomic<size_t> allowed_s{64 * 1024};
    if (p.lds > allowed_s.load(std::memory_order_relaxed)) {
      const hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(ks),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
      if (e2 != hipSuccess) return e2;
      allowed_s.store(p.lds, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL(ks, dim3((unsigned)a.T), dim3((unsigned)p.B), p.lds, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((unsigned)p.B), p.lds, st, a);
  return hipGetLastError();
}

// The kernels built for N reps, per the plan's (CH, heads); the two-chunk
// kernels exist only where p1_plan can select them (N <= 8, S <= 4).
template <int N, int S>
hipError_t p1_go_s(const Phase1Args& a, const P1Plan& p, hipStream_t st) {
  if (p.ch == 2) {
    if constexpr (N <= 8 && S <= 4) return p.mh ? p1_go<N, S, 2, true>(a, p, st) : p1_go<N, S, 2, false>(a, p, st);
    return hipErrorNotSupported;
  }
  return p.mh ? p1_go<N, S, 1, true>(a, p, st) : p1_go<N, S, 1, false>(a, p, st);
}

}  // namespace

template <int N>
hipError_t p1_launch_for(const Phase1Args& a, const P1Plan& p, hipStream_t st) {
  switch (a.S) {
    case 1: return p1_go_s<N, 1>(a, p, st);
    case 2: return p1_go_s<N, 2>(a, p, st);
    case 3: return p1_go_s<N, 3>(a, p, st);
    case 4: return p1_go_s<N, 4>(a, p, st);
    case 5: return p1_go_s<N, 5>(a, p, st);
    case 6: return p1_go_s<N, 6>(a, p, st);
    case 7: return p1_go_s<N, 7>(a, p, st);
    case 8: return p1_go_s<N, 8>(a, p, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attnres
