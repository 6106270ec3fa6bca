// Specialised Block AttnRes kernels for gfx950 (bf16 sources, fp32 arithmetic).
//
// Phase 1 (b-lab.team summary §3 Inference: all S queries of a block against
// the N cached reps in one pass).  A persistent workgroup of B = d/(8*CH)
// threads owns every channel of a token: thread `tid` owns CH chunks of 8
// consecutive channels at (c*B + tid)*8, so each wave's 16-byte loads cover a
// contiguous 1 KiB per chunk.  q = w*g for the thread's channels stays in
// registers for the whole kernel.  Per token the workgroup
//   1. streams the N reps once (16-byte loads, bf16),
//   2. accumulates per-thread partial sums of squares (N) and dot products
//      q_l . v_i (S*N, per chunk when heads differ between chunks),
//   3. reduces them across the wave (transpose-reduce: lane p ends with value p)
//      and across waves through a double-buffered LDS array (one barrier),
//   4. forms scores, softmax and lse per (layer, head) in lanes, and
//   5. writes o_l = sum_i alpha_{l,i} v_i from the registers (no second read).
//
// Phase 2 (Review §3-2 (4) online-softmax merge): one wavefront per token,
// lane owns CPL chunks of 8 channels at (c*64 + lane)*8; sum of squares and
// the per-head dots reduce inside the wave, then each element is merged.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

struct RowsOut {
  void* o0;      // layer 0
  void* orest;   // layers 1..S-1
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte global load; NT marks it nontemporal (streamed once: no reuse in cache).
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (NT) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

__device__ __forceinline__ void unpack8(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}

template <bool NT>
__device__ __forceinline__ void st16(void* p, uint4 u) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v4u{u.x, u.y, u.z, u.w}, reinterpret_cast<v4u*>(p));
  } else {
    *reinterpret_cast<uint4*>(p) = u;
  }
}

// 8 values -> one 16-byte store (two for fp32), optionally nontemporal.
template <typename O, bool NT> __device__ __forceinline__ void store8nt(O* p, const float (&x)[8]) {
  if constexpr (__is_same(O, float)) {
    st16<NT>(p, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                           __float_as_uint(x[3])));
    st16<NT>(p + 4, make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                               __float_as_uint(x[7])));
  } else if constexpr (__is_same(O, f16_t)) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = {(f16_t)x[0], (f16_t)x[1], (f16_t)x[2], (f16_t)x[3],
                  (f16_t)x[4], (f16_t)x[5], (f16_t)x[6], (f16_t)x[7]};
    st16<NT>(p, __builtin_bit_cast(uint4, h));
  } else {
    st16<NT>(p, make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]),
                           pack_bf2(x[6], x[7])));
  }
}

template <typename O> __device__ __forceinline__ void store8(O* p, const float (&x)[8]);
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&x)[8]) {
  uint4 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  u.z = pack_bf2(x[4], x[5]);
  u.w = pack_bf2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
template <> __device__ __forceinline__ void store8<f16_t>(f16_t* p, const float (&x)[8]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 h = {(f16_t)x[0], (f16_t)x[1], (f16_t)x[2], (f16_t)x[3],
          (f16_t)x[4], (f16_t)x[5], (f16_t)x[6], (f16_t)x[7]};
  *reinterpret_cast<h8*>(p) = h;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

constexpr int next_pow2(int n) { return n <= 1 ? 1 : 2 * next_pow2((n + 1) / 2); }

// Compile-time tuning knobs.  The defaults are the fastest combination measured on
// MI355X for the d=4096, N=8, S=4 block (bf16 I/O, scaled fp16 state):
//   ATTNRES_P1_PREFETCH  issue the next token's rep loads before computing the
//                        current token (keeps HBM requests in flight)
//   ATTNRES_P1_QLDS      keep q in LDS (read per chunk) instead of registers
//   ATTNRES_P1_CH        preferred chunks of 8 channels per thread (1 or 2)
//   ATTNRES_P2_PREFETCH  same as above for the Phase-2 partial and state
//   ATTNRES_P2_QLDS      Phase-2 q in LDS instead of registers
//   ATTNRES_P1_NT / ATTNRES_P2_NT  nontemporal loads of the streamed-once inputs
//   ATTNRES_P1_MINWAVES / ATTNRES_P2_MINWAVES  minimum waves per SIMD the
//                        register allocation must leave room for
//   ATTNRES_P1_DOT2      Phase-1 sums of squares and scores with v_dot2_f32_bf16 on
//                        packed bf16 pairs, q split into bf16 hi + lo (q to about
//                        16 significant bits; the reps are bf16 already)
//   ATTNRES_P1_NTST      nontemporal Phase-1 output stores
#ifndef ATTNRES_P1_PREFETCH
#define ATTNRES_P1_PREFETCH 0
#endif
#ifndef ATTNRES_P1_QLDS
#define ATTNRES_P1_QLDS 1
#endif
#ifndef ATTNRES_P1_CH
#define ATTNRES_P1_CH 2
#endif
#ifndef ATTNRES_P2_PREFETCH
#define ATTNRES_P2_PREFETCH 0
#endif
#ifndef ATTNRES_P2_QLDS
#define ATTNRES_P2_QLDS 1
#endif
#ifndef ATTNRES_P1_NT
#define ATTNRES_P1_NT 1
#endif
#ifndef ATTNRES_P2_NT
#define ATTNRES_P2_NT 1
#endif
#ifndef ATTNRES_P1_MINWAVES
#define ATTNRES_P1_MINWAVES 2
#endif
#ifndef ATTNRES_P1_DOT2
#define ATTNRES_P1_DOT2 0
#endif
#ifndef ATTNRES_P1_NTST
#define ATTNRES_P1_NTST 1
#endif
constexpr bool kP1Dot2 = ATTNRES_P1_DOT2 != 0;
constexpr bool kP1NtSt = ATTNRES_P1_NTST != 0;
#ifndef ATTNRES_P2_MINWAVES
#define ATTNRES_P2_MINWAVES 2
#endif
constexpr bool kP1Nt = ATTNRES_P1_NT != 0;
constexpr bool kP2Nt = ATTNRES_P2_NT != 0;
constexpr bool kP1Prefetch = ATTNRES_P1_PREFETCH != 0;
constexpr bool kP1QLds = ATTNRES_P1_QLDS != 0;
constexpr bool kP2Prefetch = ATTNRES_P2_PREFETCH != 0;
constexpr bool kP2QLds = ATTNRES_P2_QLDS != 0;

// ------------------------------------------------------------------ Phase 1
// rs: elements between consecutive reps.
template <int N, int CH, int B>
__device__ __forceinline__ void load_reps(uint4 (&v)[N][CH], const bf16_t* reps, int64_t rs, int d,
                                          int64_t t, int tid) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int c = 0; c < CH; ++c)
      v[i][c] = ld16<kP1Nt>(reps + (int64_t)i * rs + t * d + (c * B + tid) * 8);
}

// q = w * g into this thread's own LDS slots (fp32, two float4 per chunk).  Kept
// out of line so that the prologue's code shape cannot change how the token
// loop is scheduled and allocated.
template <int S, int CH, int B, bool G>
__device__ __noinline__ void p1_fold_lds(const float* w, const float* gain, int64_t gain_ld, int d, int tid,
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

template <int N, int S, int CH, int B, bool MH, typename O0, typename OR>
__global__ __launch_bounds__(B, ATTNRES_P1_MINWAVES) void k_phase1_fast(Phase1Args a) {
  constexpr int CHH = MH ? CH : 1;          // dot-product groups per thread
  constexpr int NDOT = CHH * S * N;
  constexpr int P = NDOT + N;               // values reduced per token
  constexpr int NG = (P + 63) / 64;
  constexpr int NP = next_pow2(N);          // lanes per softmax group
  static_assert(CHH * S * NP <= 64, "softmax table must fit one wave");
  constexpr int W = B / 64;
  constexpr bool QL = kP1QLds || kP1Dot2;    // q in LDS (always with packed pairs)
  constexpr int QR = QL ? 1 : S;            // q rows kept in registers
  __shared__ float red[2][W][NG * 64];
  __shared__ float4 qs[QL ? S * CH * B * 2 : 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d = (int)a.d;
  const int64_t T = a.T;
  const int segs_per_head = (d / a.H) / 512;  // 512-channel segments per head

  // q = w * g for this thread's channels: registers, or this thread's own LDS
  // slots (each thread reads back only what it wrote, so no barrier is needed).
  float qreg[QR][CH][8];
  auto fold = [&](auto with_gain) {
#pragma unroll
  for (int l = 0; l < S; ++l)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float qq[8];
      const int col = (c * B + tid) * 8;
      fold_q8<decltype(with_gain)::value>(a.w + (int64_t)l * d + col, a.gain + l * a.gain_ld + col, qq);
      if constexpr (kP1Dot2) {
        // packed bf16 pairs: first 16 bytes q_hi, second 16 bytes q_lo = q - q_hi
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float h0 = bf2f(f2bf(qq[2 * k])), h1 = bf2f(f2bf(qq[2 * k + 1]));
          hi[k] = pack_bf2(h0, h1);
          lo[k] = pack_bf2(qq[2 * k] - h0, qq[2 * k + 1] - h1);
        }
        qs[((l * CH + c) * B + tid) * 2 + 0] =
            make_float4(__uint_as_float(hi[0]), __uint_as_float(hi[1]), __uint_as_float(hi[2]), __uint_as_float(hi[3]));
        qs[((l * CH + c) * B + tid) * 2 + 1] =
            make_float4(__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]), __uint_as_float(lo[3]));
      } else if constexpr (kP1QLds) {
        qs[((l * CH + c) * B + tid) * 2 + 0] = make_float4(qq[0], qq[1], qq[2], qq[3]);
        qs[((l * CH + c) * B + tid) * 2 + 1] = make_float4(qq[4], qq[5], qq[6], qq[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[QL ? 0 : l][c][e] = qq[e];
      }
      // One query row's loads at a time: all rows at once spill registers.
      if (c == CH - 1) __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (kP1QLds && !kP1Dot2) {
    if (a.gain != nullptr)
      p1_fold_lds<S, CH, B, true>(a.w, a.gain, a.gain_ld, d, tid, qs);
    else
      p1_fold_lds<S, CH, B, false>(a.w, a.gain, a.gain_ld, d, tid, qs);
  } else if (a.gain != nullptr) {
    fold(std::true_type());
  } else {
    fold(std::false_type());
  }

  // The softmax lane of this wave: (cc, l, i) = decomposition of the lane.
  const int sm_cc = lane / (S * NP), sm_l = (lane / NP) % S, sm_i = lane % NP;
  const bool sm_valid = sm_cc < CHH && sm_i < N;
  // Head of the softmax group and whether this wave writes its lse.
  const int sm_seg = sm_cc * W + wave;  // segment of chunk sm_cc in this wave (MH only)
  const int sm_head = MH ? sm_seg / segs_per_head : 0;
  const bool lse_writer = MH ? (sm_valid && sm_i == 0 && sm_seg % segs_per_head == 0)
                             : (sm_valid && sm_i == 0 && wave == 0);

  const bf16_t* reps = static_cast<const bf16_t*>(a.reps);
  const int64_t rs = a.rep_stride != 0 ? a.rep_stride : T * d;
  int buf = 0;
  uint4 v[N][CH];
  int64_t t = blockIdx.x;
  if (t < T) load_reps<N, CH, B>(v, reps, rs, d, t, tid);
  for (; t < T; t += gridDim.x) {
    const int64_t tn = t + gridDim.x;
    uint4 vn[N][CH];
    if (kP1Prefetch && tn < T) load_reps<N, CH, B>(vn, reps, rs, d, tn, tid);

    // Wave priority: a token's scores run at 1, its reductions and softmax at 3
    // and its weighted sums and stores at 0.  With two workgroups per CU, the
    // one heading for its barrier then issues first, which shortens the time
    // its waves wait for each other there; the weighted sums issue the next
    // token's loads and fill the gaps.
    __builtin_amdgcn_s_setprio(1);
    float part[P];
#pragma unroll
    for (int p = 0; p < P; ++p) part[p] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = MH ? c : 0;
      if constexpr (kP1Dot2) {
        typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
        auto dot2 = [](uint32_t x, uint32_t y, float acc) {
          return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2v, x), __builtin_bit_cast(bf2v, y),
                                                 acc, false);
        };
        uint4 qh[S], ql[S];
#pragma unroll
        for (int l = 0; l < S; ++l) {
          const float4 h = qs[((l * CH + c) * B + tid) * 2 + 0];
          const float4 o = qs[((l * CH + c) * B + tid) * 2 + 1];
          qh[l] = make_uint4(__float_as_uint(h.x), __float_as_uint(h.y), __float_as_uint(h.z), __float_as_uint(h.w));
          ql[l] = make_uint4(__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z), __float_as_uint(o.w));
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const uint4 u = v[i][c];
          const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            part[NDOT + i] = dot2(uw[k], uw[k], part[NDOT + i]);
#pragma unroll
            for (int l = 0; l < S; ++l) {
              const uint32_t hw[4] = {qh[l].x, qh[l].y, qh[l].z, qh[l].w};
              const uint32_t lw[4] = {ql[l].x, ql[l].y, ql[l].z, ql[l].w};
              float& acc = part[(cc * S + l) * N + i];
              acc = dot2(uw[k], hw[k], acc);
              acc = dot2(uw[k], lw[k], acc);
            }
          }
        }
      } else {
        float qc[S][8];
#pragma unroll
        for (int l = 0; l < S; ++l) {
          if constexpr (QL) {
            const float4 q0 = qs[((l * CH + c) * B + tid) * 2 + 0];
            const float4 q1 = qs[((l * CH + c) * B + tid) * 2 + 1];
            qc[l][0] = q0.x; qc[l][1] = q0.y; qc[l][2] = q0.z; qc[l][3] = q0.w;
            qc[l][4] = q1.x; qc[l][5] = q1.y; qc[l][6] = q1.z; qc[l][7] = q1.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qc[l][e] = qreg[QL ? 0 : l][c][e];
          }
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float x[8];
          unpack8(v[i][c], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            part[NDOT + i] = fmaf(x[e], x[e], part[NDOT + i]);
#pragma unroll
            for (int l = 0; l < S; ++l)
              part[(cc * S + l) * N + i] = fmaf(qc[l][e], x[e], part[(cc * S + l) * N + i]);
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(3);
    if constexpr ((NDOT == 32 || NDOT == 64) && N == 8) {
      // The dot products and the sums of squares reduced separately, each with
      // a transposing reduction of its own size: no padded 64-value group.
      float dv[NDOT], sv[N];
#pragma unroll
      for (int p = 0; p < NDOT; ++p) dv[p] = part[p];
#pragma unroll
      for (int i = 0; i < N; ++i) sv[i] = part[NDOT + i];
      if constexpr (NDOT == 64) {
        red[buf][wave][lane] = transpose_reduce64(dv);
      } else {
        const float td = transpose_reduce_pow2<32>(dv);  // lane L: dot product L >> 1
        if ((lane & 1) == 0) red[buf][wave][lane >> 1] = td;
      }
      const float ts = transpose_reduce_pow2<8>(sv);     // lane L: sum of squares L >> 3
      if ((lane & 7) == 0) red[buf][wave][NDOT + (lane >> 3)] = ts;
    } else {
      float tot[NG];
      wave_reduce_values<P>(part, tot);
#pragma unroll
      for (int g = 0; g < NG; ++g) red[buf][wave][g * 64 + lane] = tot[g];
    }
    __syncthreads();

    // Scores, softmax and lse for this wave's (chunk, layer, rep) lanes.
    float alpha = 0.f;
    {
      float ss = 0.f, dot = 0.f;
      if (sm_valid) {
        for (int w2 = 0; w2 < W; ++w2) ss += red[buf][w2][NDOT + sm_i];
        if (!MH) {
          for (int w2 = 0; w2 < W; ++w2) dot += red[buf][w2][sm_l * N + sm_i];
        } else {
          for (int c2 = 0; c2 < CHH; ++c2)
            for (int w2 = 0; w2 < W; ++w2)
              if ((c2 * W + w2) / segs_per_head == sm_head)
                dot += red[buf][w2][(c2 * S + sm_l) * N + sm_i];
        }
      }
      const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
      const float s = sm_valid ? r * dot : -INFINITY;
      float m = s;
      m = group_max<NP>(m);
      const float e = sm_valid ? expf(s - m) : 0.f;
      float l = e;
      l = group_sum<NP>(l);
      alpha = e / l;
      if (lse_writer) a.lse[((int64_t)sm_l * a.H + sm_head) * T + t] = m + logf(l);
      if constexpr (__is_same(OR, f16_t)) {
        // Scaled fp16 state for layers >= 2: every |o| <= sqrt(max_i ss_i).
        float mss = ss;
        mss = group_max<64>(mss);
        const float scale = f16_state_scale(sqrtf(mss));
        if (sm_l >= 1) alpha *= 1.0f / scale;  // exact: a power of two
        if (wave == 0 && lane == 0) a.oscale[t] = scale;
      }
    }

    __builtin_amdgcn_s_setprio(0);
    // o_l = sum_i alpha_{l,i} v_i for each of this thread's chunks, from registers.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = MH ? c : 0;
      const int col = (c * B + tid) * 8;
      float acc[S][8];
#pragma unroll
      for (int l = 0; l < S; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float x[8];
        unpack8(v[i][c], x);
        if constexpr (!kP1Prefetch && !MH) {
          // The next token's rows go into each register as soon as its last
          // use here is done: the loads overlap the rest of the weighted sums
          // and the stores instead of starting after them.  (With heads the
          // kernel has no registers to spare for it: it would spill.)
          if (tn < T) v[i][c] = ld16<kP1Nt>(reps + (int64_t)i * rs + tn * d + (c * B + tid) * 8);
        }
#pragma unroll
        for (int l = 0; l < S; ++l) {
          const float al = read_lane(alpha, (cc * S + l) * NP + i);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[l][e] = fmaf(al, x[e], acc[l][e]);
        }
      }
      store8nt<O0, kP1NtSt>(static_cast<O0*>(a.o0) + t * d + col, acc[0]);
#pragma unroll
      for (int l = 1; l < S; ++l)
        store8nt<OR, kP1NtSt>(static_cast<OR*>(a.orest) + ((int64_t)(l - 1) * T + t) * d + col, acc[l]);
    }
    buf ^= 1;
    if constexpr (kP1Prefetch) {
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int c = 0; c < CH; ++c) v[i][c] = vn[i][c];
    } else if constexpr (MH) {
      if (tn < T) load_reps<N, CH, B>(v, reps, rs, d, tn, tid);
    }
  }
}

// ------------------------------------------------------------------ Phase 2
// Raw 16-byte words of one 8-channel chunk of the state (fp32 takes two).
template <typename OT> struct StateWords { static constexpr int kWords = sizeof(OT) == 4 ? 2 : 1; };

template <typename OT>
__device__ __forceinline__ void state_unpack(const uint4 (&u)[StateWords<OT>::kWords], float (&x)[8]) {
  if constexpr (__is_same(OT, float)) {
    x[0] = __uint_as_float(u[0].x); x[1] = __uint_as_float(u[0].y);
    x[2] = __uint_as_float(u[0].z); x[3] = __uint_as_float(u[0].w);
    x[4] = __uint_as_float(u[1].x); x[5] = __uint_as_float(u[1].y);
    x[6] = __uint_as_float(u[1].z); x[7] = __uint_as_float(u[1].w);
  } else if constexpr (__is_same(OT, f16_t)) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = __builtin_bit_cast(h8, u[0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
  } else {
    unpack8(u[0], x);
  }
}

template <int CPL, typename OT>
__device__ __forceinline__ void load_p2(uint4 (&p)[CPL], uint4 (&o)[CPL][StateWords<OT>::kWords],
                                        const bf16_t* part, const OT* oin, int64_t t, int d, int lane) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    p[c] = ld16<kP2Nt>(part + t * d + (c * 64 + lane) * 8);
#pragma unroll
    for (int k = 0; k < StateWords<OT>::kWords; ++k)
      o[c][k] = ld16<kP2Nt>(oin + t * d + (c * 64 + lane) * 8 + k * 4);
  }
}

// UPD: 0 = plain merge; 1 = fused update partial + f; 2 = fused update with
// no previous partial (the block's first update: the partial is f).  With a
// fused update the kernel also stores the merged partial and the inverse RMS
// of the stored h (see Phase2Args).
template <int CPL, bool MH, typename OT, int UPD>
__global__ __launch_bounds__(256, ATTNRES_P2_MINWAVES) void k_phase2_fast(Phase2Args a) {
  constexpr int OW = StateWords<OT>::kWords;
  constexpr bool kPref = kP2Prefetch && UPD == 0;
  const int lane = lane_id();
  const int d = (int)a.d;
  const int64_t T = a.T;
  const int segs_per_head = (d / a.H) / 512;
  constexpr int QR = kP2QLds ? 1 : CPL;
  __shared__ float4 qs[kP2QLds ? CPL * 64 * 2 : 1];
  float qreg[QR][8];
  if constexpr (kP2QLds) {
    // Every wave uses the same lane -> channel map, so the block shares one copy.
    // One branch on the gain outside the loop: loads in the loop are unconditional.
    const float4* w4 = reinterpret_cast<const float4*>(a.w);
    const float4* g4 = reinterpret_cast<const float4*>(a.gain);
    if (a.gain != nullptr) {
      for (int k = threadIdx.x; k < d / 4; k += blockDim.x) {
        float4 q = w4[k];
        const float4 g = g4[k];
        q.x *= g.x; q.y *= g.y; q.z *= g.z; q.w *= g.w;
        qs[k] = q;
      }
    } else {
      for (int k = threadIdx.x; k < d / 4; k += blockDim.x) qs[k] = w4[k];
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = (c * 64 + lane) * 8 + e;
        qreg[kP2QLds ? 0 : c][e] = a.gain ? a.w[col] * a.gain[col] : a.w[col];
      }
  }
  // With UPD == 2 the partial loads read f itself.
  const bf16_t* part = static_cast<const bf16_t*>(UPD == 2 ? a.f : a.partial);
  const bf16_t* fin = static_cast<const bf16_t*>(a.f);
  bf16_t* pout = static_cast<bf16_t*>(a.partial_out);
  const OT* oin = static_cast<const OT*>(a.o);
  bf16_t* hout = static_cast<bf16_t*>(a.h);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  uint4 p[CPL];
  uint4 o[CPL][OW];
  uint4 fv[UPD == 1 ? CPL : 1];
  auto load_f = [&](int64_t tt) {
    if constexpr (UPD == 1) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) fv[c] = ld16<kP2Nt>(fin + tt * d + (c * 64 + lane) * 8);
    }
  };
  if (t < T) {
    load_p2<CPL, OT>(p, o, part, oin, t, d, lane);
    load_f(t);
  }
  for (; t < T; t += nw) {
    const int64_t tn = t + nw;
    uint4 pn[CPL];
    uint4 on[CPL][OW];
    if (kPref && tn < T) load_p2<CPL, OT>(pn, on, part, oin, tn, d, lane);

    if constexpr (UPD != 0) {
      // The partial this sublayer reads: partial + f rounded once (or f), stored.
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if constexpr (UPD == 1) {
          float x[8], y[8];
          unpack8(p[c], x);
          unpack8(fv[c], y);
          p[c] = make_uint4(pack_bf2(x[0] + y[0], x[1] + y[1]), pack_bf2(x[2] + y[2], x[3] + y[3]),
                            pack_bf2(x[4] + y[4], x[5] + y[5]), pack_bf2(x[6] + y[6], x[7] + y[7]));
        }
        st16<false>(pout + t * d + (c * 64 + lane) * 8, p[c]);
      }
    }

    float ss = 0.f;
    float dot[MH ? CPL : 1];
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) dot[c] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float x[8], qc[8];
      unpack8(p[c], x);
      if constexpr (kP2QLds) {
        const float4 q0 = qs[(c * 64 + lane) * 2 + 0];
        const float4 q1 = qs[(c * 64 + lane) * 2 + 1];
        qc[0] = q0.x; qc[1] = q0.y; qc[2] = q0.z; qc[3] = q0.w;
        qc[4] = q1.x; qc[5] = q1.y; qc[6] = q1.z; qc[7] = q1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qc[e] = qreg[kP2QLds ? 0 : c][e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(x[e], x[e], ss);
        dot[MH ? c : 0] = fmaf(qc[e], x[e], dot[MH ? c : 0]);
      }
    }
    ss = wave_allsum(ss);
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) dot[c] = wave_allsum(dot[c]);
    const float r = 1.0f / sqrtf(ss / (float)d + a.eps);

    // Merge weights per head: ca = e^{lse-m}/(..), cb = e^{s_p-m}/(..).
    float ca[MH ? CPL : 1], cb[MH ? CPL : 1];
    const float oscale = __is_same(OT, f16_t) ? a.oscale[t] : 1.0f;
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) {
      const int head = MH ? c / segs_per_head : 0;
      float dh = 0.f;
      if (MH) {
#pragma unroll
        for (int c2 = 0; c2 < CPL; ++c2)
          if (c2 / segs_per_head == head) dh += dot[MH ? c2 : 0];
      } else {
        dh = dot[0];
      }
      const float s_p = r * dh;
      const float L = a.lse[head * T + t];
      const float m = fmaxf(L, s_p);
      const float wa = expf(L - m), wb = expf(s_p - m);
      const float inv = 1.0f / (wa + wb);
      ca[c] = wa * inv * oscale;
      cb[c] = wb * inv;
    }
    float sh = 0.f;  // sum of squares of the stored h (fused update only)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float x[8], ov[8], h[8];
      unpack8(p[c], x);
      state_unpack<OT>(o[c], ov);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = fmaf(ca[MH ? c : 0], ov[e], cb[MH ? c : 0] * x[e]);
      if constexpr (UPD == 0) {
        store8(hout + t * d + (c * 64 + lane) * 8, h);
      } else {
        const uint4 hv = make_uint4(pack_bf2(h[0], h[1]), pack_bf2(h[2], h[3]), pack_bf2(h[4], h[5]),
                                    pack_bf2(h[6], h[7]));
        st16<false>(hout + t * d + (c * 64 + lane) * 8, hv);
        float hr[8];
        unpack8(hv, hr);
#pragma unroll
        for (int e = 0; e < 8; ++e) sh = fmaf(hr[e], hr[e], sh);
      }
    }
    if constexpr (UPD != 0) {
      sh = wave_allsum(sh);
      if (a.h_inv_rms != nullptr && lane == 0) a.h_inv_rms[t] = 1.0f / sqrtf(sh / (float)d + a.norm_eps);
    }
    if constexpr (kPref) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        p[c] = pn[c];
#pragma unroll
        for (int k = 0; k < OW; ++k) o[c][k] = on[c][k];
      }
    } else {
      if (tn < T) {
        load_p2<CPL, OT>(p, o, part, oin, tn, d, lane);
        load_f(tn);
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
template <int N, int S, int CH, bool MH>
constexpr bool p1_fits() { return (MH ? CH : 1) * S * next_pow2(N) <= 64; }

template <int N, int S, int CH, int B, bool MH>
hipError_t launch_p1(const Phase1Args& a, hipStream_t st) {
  if constexpr (!p1_fits<N, S, CH, MH>()) {
    return hipErrorNotSupported;
  } else {
  auto pick = [&](auto kern) -> hipError_t {
    int per_cu = 0;
    hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), B, &per_cu);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    if (grid > a.T) grid = a.T;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(B), 0, st, a);
    return hipGetLastError();
  };
  if (a.orest_dtype == kF16) return pick(k_phase1_fast<N, S, CH, B, MH, bf16_t, f16_t>);
  if (a.orest_dtype == kF32) return pick(k_phase1_fast<N, S, CH, B, MH, bf16_t, float>);
  return pick(k_phase1_fast<N, S, CH, B, MH, bf16_t, bf16_t>);
  }
}

// Chunks of 8 channels per thread (CH) and threads per block (B = d / (8*CH)).
// Built pairs: CH in {1, 2} with B in {128, 256, 512}; ATTNRES_P1_CH is the
// preferred CH where both fit.
int phase1_ch(int64_t d) {
  auto fits = [&](int ch) {
    if (d % (8 * ch) != 0) return false;
    const int64_t B = d / (8 * ch);
    return B == 128 || B == 256 || B == 512;
  };
  constexpr int pref = ATTNRES_P1_CH == 1 ? 1 : 2;
  if (fits(pref)) return pref;
  if (fits(3 - pref)) return 3 - pref;
  return 0;
}

template <int N, int S, int CH, bool MH>
hipError_t launch_p1_b(const Phase1Args& a, hipStream_t st) {
  switch (a.d / (8 * CH)) {
    case 128: return launch_p1<N, S, CH, 128, MH>(a, st);
    case 256: return launch_p1<N, S, CH, 256, MH>(a, st);
    default: return launch_p1<N, S, CH, 512, MH>(a, st);
  }
}

template <int N, int S>
hipError_t launch_p1_ns(const Phase1Args& a, hipStream_t st) {
  const int ch = phase1_ch(a.d);
  const bool mh = a.H > 1;
  if (ch == 2) return mh ? launch_p1_b<N, S, 2, true>(a, st) : launch_p1_b<N, S, 2, false>(a, st);
  return mh ? launch_p1_b<N, S, 1, true>(a, st) : launch_p1_b<N, S, 1, false>(a, st);
}

template <int CPL>
hipError_t launch_p2(const Phase2Args& a, hipStream_t st) {
  auto pick = [&](auto kern) -> hipError_t {
    int per_cu = 0;
    hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), 256, &per_cu);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    const int64_t need = (a.T + 3) / 4;
    if (grid > need) grid = need;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
  };
  const bool mh = a.H > 1;
  auto by_state = [&](auto upd) -> hipError_t {
    constexpr int U = decltype(upd)::value;
    if (a.o_dtype == kF32)
      return mh ? pick(k_phase2_fast<CPL, true, float, U>) : pick(k_phase2_fast<CPL, false, float, U>);
    if (a.o_dtype == kF16)
      return mh ? pick(k_phase2_fast<CPL, true, f16_t, U>) : pick(k_phase2_fast<CPL, false, f16_t, U>);
    return mh ? pick(k_phase2_fast<CPL, true, bf16_t, U>) : pick(k_phase2_fast<CPL, false, bf16_t, U>);
  };
  if (a.f == nullptr) return by_state(std::integral_constant<int, 0>());
  if (a.partial != nullptr) return by_state(std::integral_constant<int, 1>());
  return by_state(std::integral_constant<int, 2>());
}

bool heads_fit_segments(int64_t d, int H) { return (d / H) % 512 == 0; }

// The specialised kernels use 16-byte vector loads and stores.
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool phase1_fast_ok(const Phase1Args& a) {
  if (a.dtype != kBF16 || a.T < 1 || !heads_fit_segments(a.d, a.H)) return false;
  if (!aligned16(a.reps) || !aligned16(a.o0) || !aligned16(a.orest) || !aligned16(a.w) ||
      !aligned16(a.gain))
    return false;
  const int ch = phase1_ch(a.d);
  if (ch == 0) return false;
  if (!((a.N == 8 && a.S == 4) || (a.N == 4 && a.S == 4))) return false;
  return (a.H > 1 ? ch : 1) * a.S * next_pow2((int)a.N) <= 64;
}

hipError_t launch_phase1_fast(const Phase1Args& a, hipStream_t st) {
  if (a.N == 8 && a.S == 4) return launch_p1_ns<8, 4>(a, st);
  return launch_p1_ns<4, 4>(a, st);
}

bool phase2_fast_ok(const Phase2Args& a) {
  if (a.dtype != kBF16 || a.T < 1 || !heads_fit_segments(a.d, a.H)) return false;
  if (!aligned16(a.o) || !aligned16(a.partial) || !aligned16(a.h) || !aligned16(a.w) ||
      !aligned16(a.gain) || !aligned16(a.f) || !aligned16(a.partial_out))
    return false;
  const int64_t cpl = a.d / 512;
  return a.d % 512 == 0 && (cpl == 4 || cpl == 8);
}

hipError_t launch_phase2_fast(const Phase2Args& a, hipStream_t st) {
  return a.d / 512 == 4 ? launch_p2<4>(a, st) : launch_p2<8>(a, st);
}

}  // namespace attnres
