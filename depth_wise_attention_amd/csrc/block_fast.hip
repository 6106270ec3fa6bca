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
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

struct RowsOut {
  void* o0;      // layer 0
  void* orest;   // layers 1..S-1
};

__device__ __forceinline__ void unpack8(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
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
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

template <typename O> __device__ __forceinline__ void load8(const O* p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&x)[8]) {
  unpack8(*reinterpret_cast<const uint4*>(p), x);
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

constexpr int next_pow2(int n) { return n <= 1 ? 1 : 2 * next_pow2((n + 1) / 2); }

// ------------------------------------------------------------------ Phase 1
template <int N, int S, int CH, int B, bool MH, typename O0, typename OR>
__global__ __launch_bounds__(B) void k_phase1_fast(Phase1Args a) {
  constexpr int CHH = MH ? CH : 1;          // dot-product groups per thread
  constexpr int NDOT = CHH * S * N;
  constexpr int P = NDOT + N;               // values reduced per token
  constexpr int NG = (P + 63) / 64;
  constexpr int NP = next_pow2(N);          // lanes per softmax group
  static_assert(CHH * S * NP <= 64, "softmax table must fit one wave");
  constexpr int W = B / 64;
  __shared__ float red[2][W][NG * 64];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d = (int)a.d;
  const int64_t T = a.T;
  const int segs_per_head = (d / a.H) / 512;  // 512-channel segments per head

  // q = w * g for this thread's channels, resident for the whole kernel.
  float q[S][CH][8];
#pragma unroll
  for (int l = 0; l < S; ++l)
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = (c * B + tid) * 8 + e;
        const float wv = a.w[(int64_t)l * d + col];
        q[l][c][e] = a.gain ? wv * a.gain[l * a.gain_ld + col] : wv;
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
  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    uint4 v[N][CH];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        v[i][c] = *reinterpret_cast<const uint4*>(reps + ((int64_t)i * T + t) * d + (c * B + tid) * 8);

    float part[P];
#pragma unroll
    for (int p = 0; p < P; ++p) part[p] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float x[8];
        unpack8(v[i][c], x);
        const int cc = MH ? c : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          part[NDOT + i] = fmaf(x[e], x[e], part[NDOT + i]);
#pragma unroll
          for (int l = 0; l < S; ++l)
            part[(cc * S + l) * N + i] = fmaf(q[l][c][e], x[e], part[(cc * S + l) * N + i]);
        }
      }
    float tot[NG];
    wave_reduce_values<P>(part, tot);
#pragma unroll
    for (int g = 0; g < NG; ++g) red[buf][wave][g * 64 + lane] = tot[g];
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
#pragma unroll
      for (int off = 1; off < NP; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
      const float e = sm_valid ? expf(s - m) : 0.f;
      float l = e;
#pragma unroll
      for (int off = 1; off < NP; off <<= 1) l += __shfl_xor(l, off, kWave);
      alpha = e / l;
      if (lse_writer) a.lse[((int64_t)sm_l * a.H + sm_head) * T + t] = m + logf(l);
    }

    // o_l = sum_i alpha_{l,i} v_i for each of this thread's chunks.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cc = MH ? c : 0;
      float x[N][8];
#pragma unroll
      for (int i = 0; i < N; ++i) unpack8(v[i][c], x[i]);
      const int col = (c * B + tid) * 8;
#pragma unroll
      for (int l = 0; l < S; ++l) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float al = read_lane(alpha, (cc * S + l) * NP + i);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(al, x[i][e], acc[e]);
        }
        if (l == 0)
          store8(static_cast<O0*>(a.o0) + t * d + col, acc);
        else
          store8(static_cast<OR*>(a.orest) + ((int64_t)(l - 1) * T + t) * d + col, acc);
      }
    }
    buf ^= 1;
  }
}

// ------------------------------------------------------------------ Phase 2
template <int CPL, bool MH, typename OT>
__global__ __launch_bounds__(256) void k_phase2_fast(Phase2Args a) {
  const int lane = lane_id();
  const int d = (int)a.d;
  const int64_t T = a.T;
  const int segs_per_head = (d / a.H) / 512;
  float q[CPL][8];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = (c * 64 + lane) * 8 + e;
      q[c][e] = a.gain ? a.w[col] * a.gain[col] : a.w[col];
    }
  const bf16_t* part = static_cast<const bf16_t*>(a.partial);
  const OT* oin = static_cast<const OT*>(a.o);
  bf16_t* hout = static_cast<bf16_t*>(a.h);
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = wave0; t < T; t += nw) {
    uint4 p[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      p[c] = *reinterpret_cast<const uint4*>(part + t * d + (c * 64 + lane) * 8);
    float ss = 0.f;
    float dot[MH ? CPL : 1];
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) dot[c] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float x[8];
      unpack8(p[c], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(x[e], x[e], ss);
        dot[MH ? c : 0] = fmaf(q[c][e], x[e], dot[MH ? c : 0]);
      }
    }
    ss = wave_allsum(ss);
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) dot[c] = wave_allsum(dot[c]);
    const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
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
      const float ca = wa * inv, cb = wb * inv;
      float o[8], x[8], h[8];
      load8(oin + t * d + (c * 64 + lane) * 8, o);
      unpack8(p[c], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = fmaf(ca, o[e], cb * x[e]);
      store8(hout + t * d + (c * 64 + lane) * 8, h);
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
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, B, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    if (grid > a.T) grid = a.T;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(B), 0, st, a);
    return hipGetLastError();
  };
  if (a.o0_dtype == kBF16 && a.orest_dtype == kF32) return pick(k_phase1_fast<N, S, CH, B, MH, bf16_t, float>);
  if (a.o0_dtype == kBF16 && a.orest_dtype == kBF16) return pick(k_phase1_fast<N, S, CH, B, MH, bf16_t, bf16_t>);
  return pick(k_phase1_fast<N, S, CH, B, MH, float, float>);
  }
}

// Chunks of 8 channels per thread (CH) and threads per block (B = d / (8*CH)).
// Built pairs: CH in {1, 2} with B in {128, 256, 512}.  CH = 2 halves the
// number of waves that share a token (and so the cross-wave reduction work);
// ATTNRES_PHASE1_CH=1 or 2 forces one choice where both fit.
int phase1_ch(int64_t d) {
  static const int forced = [] {
    const char* e = getenv("ATTNRES_PHASE1_CH");
    return e ? atoi(e) : 0;
  }();
  auto fits = [&](int ch) {
    if (d % (8 * ch) != 0) return false;
    const int64_t B = d / (8 * ch);
    return B == 128 || B == 256 || B == 512;
  };
  if ((forced == 1 || forced == 2) && fits(forced)) return forced;
  if (fits(2)) return 2;
  if (fits(1)) return 1;
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
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    const int64_t need = (a.T + 3) / 4;
    if (grid > need) grid = need;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
  };
  const bool mh = a.H > 1;
  if (a.o_dtype == kF32)
    return mh ? pick(k_phase2_fast<CPL, true, float>) : pick(k_phase2_fast<CPL, false, float>);
  return mh ? pick(k_phase2_fast<CPL, true, bf16_t>) : pick(k_phase2_fast<CPL, false, bf16_t>);
}

bool heads_fit_segments(int64_t d, int H) { return (d / H) % 512 == 0; }

}  // namespace

bool phase1_fast_ok(const Phase1Args& a) {
  if (a.dtype != kBF16 || a.T < 1 || !heads_fit_segments(a.d, a.H)) return false;
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
  const int64_t cpl = a.d / 512;
  return a.d % 512 == 0 && (cpl == 4 || cpl == 8);
}

hipError_t launch_phase2_fast(const Phase2Args& a, hipStream_t st) {
  return a.d / 512 == 4 ? launch_p2<4>(a, st) : launch_p2<8>(a, st);
}

}  // namespace attnres
