// MSAR specialised path: bf16, one destination (a Block MSAR sublayer), at
// most 12 sources, d a multiple of 512.
//
// The streams of a source at token t need the source's rows t-11 .. t, and
// the routing needs sums over all d channels per token.  Workgroups own a
// 512-channel slice (two channels per thread) over a range of consecutive
// tokens, walked in chunks of 8 tokens; within a chunk the sources are taken
// one at a time, so a thread holds the 19 rows (t0-11 .. t0+7) of one source's
// two channels in registers, unpacked once, and the 24 taps of its channels:
//   k_msar_slice<0>  per token and slice: each source's per-stream sum of
//                    squares and query product (8 values per source) -> part
//   k_msar_alpha<N>  per token: sum the slices, scores, four depth softmaxes,
//                    and the power-of-two scale of the stored Z      -> alpha, zscale
//   k_msar_slice<1>  per token and slice: Z^(r) for the slice's channels
//                    (stored once, fp16 scaled per token), the sum of squares
//                    of Flatten(Z) and its four projections by P     -> zbuf, part2
//   k_msar_out       per token: sum the slices, beta = sigmoid(...), and
//                    h = sum_r beta_r Z^(r)                          -> out
// The streams themselves are never stored.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kMfB = 256;        // threads per workgroup
constexpr int kMfSlice = 512;    // channels per slice (2 per thread)
constexpr int kMfRange = 64;     // tokens per workgroup (measured: 64 beats 128 and 256)
constexpr int kMfTC = 8;         // tokens per chunk
constexpr int kMfHalo = 11;      // rows before a token that its longest stream reads
constexpr int kMfWin = kMfTC + kMfHalo;
constexpr int kMfAlphaRow = 16;  // alpha[t][r][16]
constexpr int kMfPart2 = 8;      // part2[t][slice][8] (5 used)

struct MsarFastBufs {
  float* part;    // [T][S][8 n]: per source i, [i*8 + r] sum of squares, [i*8 + 4 + r] query product
  float* alpha;   // [T][4][16]
  float* part2;   // [T][S][8]: [0] sum of squares of Z, [1 + q] projection q
  // Z^(r) in fp16, divided per token by zscale[t], a power of two that maps a
  // bound on every |Z| (the largest stream norm over the sources: Z is a
  // convex combination of the streams) to [16384, 32768).  The Block MSAR
  // Phase 1 keeps its sublayer-1 states in fp32 instead (zbuf32, no scale):
  // the conversion in its weighting pass costs registers it does not have.
  f16_t* zbuf;      // [T][4][d]
  float* zscale;    // [T]
  float* zbuf32;    // [T][4][d]
};

// Sum of v[p] over the workgroup's 256 threads, for p < 64, into the
// returned value of thread p (other threads return garbage).  One barrier;
// red is double-buffered by the caller's buf.
__device__ __forceinline__ float block_reduce64(const float (&v)[64], float (&red)[2][4][64], int buf) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  red[buf][wave][lane] = transpose_reduce64(v);
  lds_barrier();
  const int p = tid & 63;
  return (red[buf][0][p] + red[buf][1][p]) + (red[buf][2][p] + red[buf][3][p]);
}

// PASS 0: per-source statistics; PASS 1: retrieved states (stored to zbuf)
// and the mixer's sums.
template <int PASS>
__global__ __launch_bounds__(kMfB, 2) void k_msar_slice(MsarArgs a, MsarFastBufs b) {
  __shared__ float red[2][4][64];
  __shared__ __attribute__((aligned(16))) float alpha_s[PASS == 1 ? kMfTC * kMsarStreams * kMfAlphaRow : 4];
  __shared__ float zis_s[kMfTC];
  const int tid = threadIdx.x;
  const int64_t d = a.d, T = a.T;
  const int n = (int)a.n_src;
  const int S = (int)(d / kMfSlice);
  const int slice = blockIdx.x;
  const int64_t c0 = (int64_t)slice * kMfSlice + 2 * tid;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);

  // Taps of this thread's two channels.
  float2 tap[kMsarTaps];
#pragma unroll
  for (int k = 0; k < kMsarTaps; ++k) tap[k] = *reinterpret_cast<const float2*>(a.conv + k * d + c0);
  // Pass 0: the pseudo-queries of the two channels; pass 1: their rows of P.
  float2 wq[kMsarStreams];
  float4 pm[kMsarStreams][2];
#pragma unroll
  for (int r = 0; r < kMsarStreams; ++r) {
    if constexpr (PASS == 0) {
      wq[r] = *reinterpret_cast<const float2*>(a.w + r * d + c0);
    } else {
      pm[r][0] = *reinterpret_cast<const float4*>(a.mix + (r * d + c0) * kMsarStreams);
      pm[r][1] = *reinterpret_cast<const float4*>(a.mix + (r * d + c0 + 1) * kMsarStreams);
    }
  }

  const int64_t t_begin = (int64_t)blockIdx.y * kMfRange;
  const int64_t t_end = t_begin + kMfRange < T ? t_begin + kMfRange : T;
  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kMfTC) {
    float2 z[kMfTC][kMsarStreams];
    if constexpr (PASS == 1) {
#pragma unroll
      for (int q = 0; q < kMfTC; ++q)
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) z[q][r] = make_float2(0.f, 0.f);
      // The chunk's softmax weights, into LDS: per-source reads then go through
      // the LDS counter instead of queueing behind the prefetched rows.  The
      // barrier also orders the previous chunk's reads before these writes.
      lds_barrier();
      // Stored [token][source][stream]: one 16-byte LDS read per (token, source).
      for (int e = tid; e < kMfTC * kMsarStreams * kMfAlphaRow; e += kMfB) {
        const int q = e / (kMsarStreams * kMfAlphaRow), rem = e % (kMsarStreams * kMfAlphaRow);
        const int r = rem / kMfAlphaRow, i = rem % kMfAlphaRow;
        const int64_t tq = t0 + q;
        alpha_s[(q * kMfAlphaRow + i) * kMsarStreams + r] =
            b.alpha[(tq < T ? tq : T - 1) * (kMsarStreams * kMfAlphaRow) + rem];
      }
      if (tid < kMfTC) zis_s[tid] = 1.0f / b.zscale[t0 + tid < T ? t0 + tid : T - 1];
      lds_barrier();
    }
    // Rows t0-11 .. t0+7 of source i; rows outside [0, T) read as zero (before
    // the first token: the causal zero; past the end: unused).  Loads are
    // unconditional (clamped row and source), so the next source's rows stay
    // in flight while this one computes.
    auto load_rows = [&](int i, uint32_t (&raw)[kMfWin]) {
      const bf16_t* col = src + (int64_t)(i < n ? i : n - 1) * T * d + c0;
#pragma unroll
      for (int h = 0; h < kMfWin; ++h) {
        const int64_t row = t0 - kMfHalo + h;
        const int64_t rc = row < 0 ? 0 : (row >= T ? T - 1 : row);
        raw[h] = *reinterpret_cast<const uint32_t*>(col + rc * d);
      }
    };
    auto source = [&](int i, const uint32_t (&raw)[kMfWin]) {
      __builtin_amdgcn_s_setprio(0);
      float2 x[kMfWin];
#pragma unroll
      for (int h = 0; h < kMfWin; ++h) {
        const int64_t row = t0 - kMfHalo + h;
        const uint32_t u = (row >= 0 && row < T) ? raw[h] : 0u;
        x[h] = make_float2(bf_lo(u), bf_hi(u));
      }
      float v[64];  // pass 0: [token q][8]
#pragma unroll
      for (int q = 0; q < kMfTC; ++q) {
        // Token t0 + q is window row q + 11; lag k is row q + 11 - k.
        float2 sv[kMsarStreams];
        sv[0] = x[q + kMfHalo];
#pragma unroll
        for (int r = 1; r < kMsarStreams; ++r) {
          const int K = msar_kernel(r), off = msar_offset(r);
          float2 acc = make_float2(0.f, 0.f);
#pragma unroll
          for (int k = 0; k < K; ++k) {
            acc.x = fmaf(tap[off + k].x, x[q + kMfHalo - k].x, acc.x);
            acc.y = fmaf(tap[off + k].y, x[q + kMfHalo - k].y, acc.y);
          }
          sv[r] = acc;
        }
        if constexpr (PASS == 0) {
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            v[q * 8 + r] = fmaf(sv[r].x, sv[r].x, sv[r].y * sv[r].y);
            v[q * 8 + 4 + r] = fmaf(wq[r].x, sv[r].x, wq[r].y * sv[r].y);
          }
        } else {
          const float4 wv = *reinterpret_cast<const float4*>(&alpha_s[(q * kMfAlphaRow + i) * kMsarStreams]);
          const float wr[kMsarStreams] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            z[q][r].x = fmaf(wr[r], sv[r].x, z[q][r].x);
            z[q][r].y = fmaf(wr[r], sv[r].y, z[q][r].y);
          }
        }
      }
      if constexpr (PASS == 0) {
        __builtin_amdgcn_s_setprio(2);
        const float tot = block_reduce64(v, red, buf);
        buf ^= 1;
        const int p = tid;
        if (p < 64 && t0 + p / 8 < t_end) b.part[((t0 + p / 8) * S + slice) * (8 * n) + i * 8 + (p & 7)] = tot;
      }
    };
    // Ping-pong over pairs of sources: each buffer's loads are issued one
    // source ahead of its use.
    uint32_t ra[kMfWin], rb[kMfWin];
    // One source per iteration: the next source's rows load into rb while
    // this one computes, then move to ra.  (A two-buffer ping-pong inlines the
    // source twice, and the weighted sums then change registers between the
    // two copies: more moves than the row copy.)
    load_rows(0, ra);
    for (int i = 0; i < n; ++i) {
      load_rows(i + 1, rb);
      source(i, ra);
#pragma unroll
      for (int h = 0; h < kMfWin; ++h) ra[h] = rb[h];
    }
    if constexpr (PASS == 1) {
      __builtin_amdgcn_s_setprio(2);
      float v[64];
#pragma unroll
      for (int q = 0; q < kMfTC; ++q) {
        float e[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          const float2 zr = z[q][r];
          if (t0 + q < t_end) {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            const float isc = zis_s[q];  // a power of two: exact
            const h2 hv = {(f16_t)(zr.x * isc), (f16_t)(zr.y * isc)};
            *reinterpret_cast<uint32_t*>(b.zbuf + ((t0 + q) * kMsarStreams + r) * d + c0) =
                __builtin_bit_cast(uint32_t, hv);
          }
          e[0] = fmaf(zr.x, zr.x, fmaf(zr.y, zr.y, e[0]));
          e[1] = fmaf(zr.x, pm[r][0].x, fmaf(zr.y, pm[r][1].x, e[1]));
          e[2] = fmaf(zr.x, pm[r][0].y, fmaf(zr.y, pm[r][1].y, e[2]));
          e[3] = fmaf(zr.x, pm[r][0].z, fmaf(zr.y, pm[r][1].z, e[3]));
          e[4] = fmaf(zr.x, pm[r][0].w, fmaf(zr.y, pm[r][1].w, e[4]));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[q * 8 + j] = j < 5 ? e[j] : 0.f;
      }
      const float tot = block_reduce64(v, red, buf);
      buf ^= 1;
      const int p = tid;
      if (p < 64 && (p & 7) < 5 && t0 + p / 8 < t_end)
        b.part2[((t0 + p / 8) * S + slice) * kMfPart2 + (p & 7)] = tot;
    }
  }
}

// One wavefront per token: lane r*16 + i holds source i of stream r.
template <int N>
__global__ __launch_bounds__(256) void k_msar_alpha(MsarArgs a, MsarFastBufs b) {
  constexpr int NV = 8 * N;
  const int lane = lane_id();
  const int64_t T = a.T, d = a.d;
  const int S = (int)(d / kMfSlice);
  const int r = lane >> 4, i = lane & 15;
  const bool valid = i < N;
  const int ii = valid ? i : 0;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += (int64_t)gridDim.x * 4) {
    float ss = 0.f, dot = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = b.part + (t * S + s) * NV;
      ss += p[ii * 8 + r];
      dot += p[ii * 8 + 4 + r];
    }
    const float score = valid ? dot / sqrtf(ss / (float)d + a.eps) : -INFINITY;
    const float m = group_max<16>(score);
    const float e = valid ? expf(score - m) : 0.f;
    const float l = group_sum<16>(e);
    b.alpha[t * (kMsarStreams * kMfAlphaRow) + r * kMfAlphaRow + i] = e / l;
    const float mss = group_max<64>(valid ? ss : 0.f);
    if (lane == 0) b.zscale[t] = f16_state_scale(sqrtf(mss));
  }
}

// Per token: beta from the slices' sums, then h = sum_r beta_r Z^(r) (with
// the fp16 Z, its per-token scale is applied once at the end: exact).
template <bool F16>
__global__ __launch_bounds__(256) void k_msar_out(MsarArgs a, MsarFastBufs b) {
  const int64_t T = a.T, d = a.d;
  const int S = (int)(d / kMfSlice);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int q = 0; q < 5; ++q) v[q] += b.part2[(t * S + s) * kMfPart2 + q];
    }
    const float inv = 1.0f / sqrtf(v[0] / (float)(kMsarStreams * d) + a.eps);
    float beta[kMsarStreams];
#pragma unroll
    for (int q = 0; q < kMsarStreams; ++q) beta[q] = 1.0f / (1.0f + expf(-v[1 + q] * inv));
    const float sc = F16 ? b.zscale[t] : 1.0f;
    for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += (int64_t)blockDim.x * 4) {
      float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) {
        float4 zr;
        if constexpr (F16) {
          const uint2 u = *reinterpret_cast<const uint2*>(b.zbuf + (t * kMsarStreams + r) * d + c);
          zr.x = (float)__builtin_bit_cast(f16_t, (uint16_t)(u.x & 0xffffu));
          zr.y = (float)__builtin_bit_cast(f16_t, (uint16_t)(u.x >> 16));
          zr.z = (float)__builtin_bit_cast(f16_t, (uint16_t)(u.y & 0xffffu));
          zr.w = (float)__builtin_bit_cast(f16_t, (uint16_t)(u.y >> 16));
        } else {
          zr = *reinterpret_cast<const float4*>(b.zbuf32 + (t * kMsarStreams + r) * d + c);
        }
        h.x = fmaf(beta[r], zr.x, h.x);
        h.y = fmaf(beta[r], zr.y, h.y);
        h.z = fmaf(beta[r], zr.z, h.z);
        h.w = fmaf(beta[r], zr.w, h.w);
      }
      if constexpr (F16) {
        h.x *= sc; h.y *= sc; h.z *= sc; h.w *= sc;
      }
      *reinterpret_cast<uint2*>(out + t * d + c) = make_uint2(pack_bf2(h.x, h.y), pack_bf2(h.z, h.w));
    }
  }
}

// ------------------------------------------------------------ Block MSAR
// Phase 1 ([MSAR] "How to use it": AttnRes's two-phase computation carries
// over): the block's SB sublayers' queries against the N reps, each rep's
// streams expanded once per pass for all of them.  Same slicing as
// k_msar_slice, with 4-token chunks (the state pass keeps SB x 4 streams of
// weighted sums per token).
constexpr int kBmTC = 4;   // statistics pass (its reductions are shaped for 4 tokens)
#ifndef ATTNRES_BM_TC1
#define ATTNRES_BM_TC1 4
#endif
constexpr int kBmTC1 = ATTNRES_BM_TC1;  // weighting pass (measured: 2 tokens is 16% slower)

struct BmsarArgs {
  const void* reps;    // [N][T][d] bf16
  int64_t N, T, d;
  const float* w;      // [SB][4][d]
  const float* conv;   // [24][d]
  const float* mix1;   // [4 d][4], sublayer 1's mixer
  float eps;
  f16_t* o_state;      // [SB-1][4][T][d], fp16 scaled per token
  float* o_scale;      // [T]: o_state * o_scale[t] is the state
  float* lse;          // [SB-1][4][T]
  float* part;         // [T][slices][N][4 + 4 SB]
  float* alpha;        // [T][SB][4][16]
  float* part2;        // [T][slices][8]
  float* zbuf;         // [T][4][d], sublayer 1's retrieved states
};

// Workgroup sum of NV <= 256 values per thread: thread p < NV returns value p's total.
template <int NV>
__device__ __forceinline__ float block_reduce_values(const float (&v)[NV], float (&red)[2][4][256], int buf) {
  constexpr int NG = (NV + 63) / 64;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  float tot[NG];
  wave_reduce_values<NV>(v, tot);
#pragma unroll
  for (int g = 0; g < NG; ++g) red[buf][wave][g * 64 + lane] = tot[g];
  lds_barrier();
  return (red[buf][0][tid] + red[buf][1][tid]) + (red[buf][2][tid] + red[buf][3][tid]);
}

// Workgroup sums of 32 values per thread, one barrier: thread p < 32 returns
// value p (other threads return garbage).  A 32-value transposing reduction
// instead of a 64-value one padded with zeros.
__device__ __forceinline__ float block_reduce32(const float (&v)[32], float (&red)[2][4][256], int buf) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const float t = transpose_reduce_pow2<32>(v);  // lane L: value L >> 1
  if ((lane & 1) == 0) red[buf][wave][lane >> 1] = t;
  lds_barrier();
  return (red[buf][0][tid & 31] + red[buf][1][tid & 31]) + (red[buf][2][tid & 31] + red[buf][3][tid & 31]);
}

// Workgroup sums of ND query products and 16 sums of squares per thread, one
// barrier: thread p < ND returns product p, thread R + s (R = ND rounded up to
// 64, s < 16) sum of squares s; other threads return garbage.
template <int ND>
__device__ __forceinline__ float block_reduce_stats(const float (&dv)[ND], const float (&sq)[16],
                                                    float (&red)[2][4][256], int buf) {
  constexpr int NG = (ND + 63) / 64;
  static_assert(NG * 64 + 16 <= 256, "reduction table");
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  float td[NG];
  wave_reduce_values<ND>(dv, td);
  const float ts = transpose_reduce16(sq);  // lane L: sum of squares L >> 2
#pragma unroll
  for (int g = 0; g < NG; ++g) red[buf][wave][g * 64 + lane] = td[g];
  if ((lane & 3) == 0) red[buf][wave][NG * 64 + (lane >> 2)] = ts;
  lds_barrier();
  return (red[buf][0][tid] + red[buf][1][tid]) + (red[buf][2][tid] + red[buf][3][tid]);
}

template <int SB, int PASS>
__global__ __launch_bounds__(kMfB, 2) void k_bmsar_p1(BmsarArgs a) {
  constexpr int V = 4 + 4 * SB;          // per rep and token: 4 sums of squares, 4 SB query products
  constexpr int TC = PASS == 0 ? kBmTC : kBmTC1;  // tokens per chunk
  constexpr int WIN = TC + kMfHalo;
  __shared__ float red[2][4][256];
  __shared__ float alpha_s[PASS == 1 ? TC * SB * kMsarStreams * kMfAlphaRow : 1];
  __shared__ float iscale_s[TC];
  // Pass 1: this thread's rows of sublayer 1's mixer P, in LDS rather than in
  // registers (the weighted sums of SB sublayers fill the register file).
  __shared__ float4 pm_s[PASS == 1 ? kMsarStreams * 2 * kMfB : 1];
  const int tid = threadIdx.x;
  const int64_t d = a.d, T = a.T;
  const int n = (int)a.N;
  const int S = (int)(d / kMfSlice);
  const int slice = blockIdx.x;
  const int64_t c0 = (int64_t)slice * kMfSlice + 2 * tid;
  const bf16_t* src = static_cast<const bf16_t*>(a.reps);

  float2 tap[kMsarTaps];
#pragma unroll
  for (int k = 0; k < kMsarTaps; ++k) tap[k] = *reinterpret_cast<const float2*>(a.conv + k * d + c0);
  float2 wq[PASS == 0 ? SB : 1][kMsarStreams];
#pragma unroll
  for (int r = 0; r < kMsarStreams; ++r) {
    if constexpr (PASS == 0) {
#pragma unroll
      for (int i = 0; i < SB; ++i) wq[i][r] = *reinterpret_cast<const float2*>(a.w + (i * kMsarStreams + r) * d + c0);
    } else {
      // Read back only by this thread: no barrier needed.
      pm_s[(r * 2 + 0) * kMfB + tid] = *reinterpret_cast<const float4*>(a.mix1 + (r * d + c0) * kMsarStreams);
      pm_s[(r * 2 + 1) * kMfB + tid] = *reinterpret_cast<const float4*>(a.mix1 + (r * d + c0 + 1) * kMsarStreams);
    }
  }

  const int64_t t_begin = (int64_t)blockIdx.y * kMfRange;
  const int64_t t_end = t_begin + kMfRange < T ? t_begin + kMfRange : T;
  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TC) {
    float2 z[TC][SB][kMsarStreams];
    if constexpr (PASS == 1) {
#pragma unroll
      for (int q = 0; q < TC; ++q)
#pragma unroll
        for (int i = 0; i < SB; ++i)
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) z[q][i][r] = make_float2(0.f, 0.f);
      lds_barrier();
      constexpr int NA = TC * SB * kMsarStreams * kMfAlphaRow;
      for (int e = tid; e < NA; e += kMfB) {
        const int64_t tq = t0 + e / (SB * kMsarStreams * kMfAlphaRow);
        alpha_s[e] = a.alpha[(tq < T ? tq : T - 1) * (SB * kMsarStreams * kMfAlphaRow) +
                             e % (SB * kMsarStreams * kMfAlphaRow)];
      }
      if (tid < TC) iscale_s[tid] = 1.0f / a.o_scale[t0 + tid < T ? t0 + tid : T - 1];
      lds_barrier();
    }
    auto load_rows = [&](int i, uint32_t (&raw)[WIN]) {
      const bf16_t* col = src + (int64_t)(i < n ? i : n - 1) * T * d + c0;
#pragma unroll
      for (int h = 0; h < WIN; ++h) {
        const int64_t row = t0 - kMfHalo + h;
        const int64_t rc = row < 0 ? 0 : (row >= T ? T - 1 : row);
        raw[h] = *reinterpret_cast<const uint32_t*>(col + rc * d);
      }
    };
    auto source = [&](int i, const uint32_t (&raw)[WIN]) {
      __builtin_amdgcn_s_setprio(0);
      float2 x[WIN];
#pragma unroll
      for (int h = 0; h < WIN; ++h) {
        const int64_t row = t0 - kMfHalo + h;
        const uint32_t u = (row >= 0 && row < T) ? raw[h] : 0u;
        x[h] = make_float2(bf_lo(u), bf_hi(u));
      }
      // Pass 0: the chunk's query products [token][sublayer][stream] and sums
      // of squares [token][stream], reduced separately (no padded group).
      float dv[PASS == 0 ? TC * 4 * SB : 1], sq[PASS == 0 ? TC * kMsarStreams : 1];
#pragma unroll
      for (int q = 0; q < TC; ++q) {
        float2 sv[kMsarStreams];
        sv[0] = x[q + kMfHalo];
#pragma unroll
        for (int r = 1; r < kMsarStreams; ++r) {
          const int K = msar_kernel(r), off = msar_offset(r);
          float2 acc = make_float2(0.f, 0.f);
#pragma unroll
          for (int k = 0; k < K; ++k) {
            acc.x = fmaf(tap[off + k].x, x[q + kMfHalo - k].x, acc.x);
            acc.y = fmaf(tap[off + k].y, x[q + kMfHalo - k].y, acc.y);
          }
          sv[r] = acc;
        }
        if constexpr (PASS == 0) {
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            sq[q * kMsarStreams + r] = fmaf(sv[r].x, sv[r].x, sv[r].y * sv[r].y);
#pragma unroll
            for (int j = 0; j < SB; ++j)
              dv[(q * SB + j) * kMsarStreams + r] = fmaf(wq[j][r].x, sv[r].x, wq[j][r].y * sv[r].y);
          }
        } else {
#pragma unroll
          for (int j = 0; j < SB; ++j)
#pragma unroll
            for (int r = 0; r < kMsarStreams; ++r) {
              const float w_ri = alpha_s[((q * SB + j) * kMsarStreams + r) * kMfAlphaRow + i];
              z[q][j][r].x = fmaf(w_ri, sv[r].x, z[q][j][r].x);
              z[q][j][r].y = fmaf(w_ri, sv[r].y, z[q][j][r].y);
            }
        }
      }
      if constexpr (PASS == 0) {
        __builtin_amdgcn_s_setprio(2);
        constexpr int ND = TC * 4 * SB, DROWS = (ND + 63) / 64 * 64;
        const float tot = block_reduce_stats<ND>(dv, sq, red, buf);
        buf ^= 1;
        const int p = tid;
        int q = -1, k = 0;
        if (p < ND) {
          q = p / (4 * SB);
          k = 4 + p % (4 * SB);
        } else if (p >= DROWS && p < DROWS + TC * kMsarStreams) {
          q = (p - DROWS) / kMsarStreams;
          k = (p - DROWS) % kMsarStreams;
        }
        if (q >= 0 && t0 + q < t_end) a.part[(((t0 + q) * S + slice) * n + i) * V + k] = tot;
      }
    };
    uint32_t ra[WIN], rb[WIN];
    // One source per iteration: the next source's rows load into rb while
    // this one computes, then move to ra.  (A two-buffer ping-pong inlines the
    // source twice, and the weighted sums then change registers between the
    // two copies: more moves than the row copy.)
    load_rows(0, ra);
    for (int i = 0; i < n; ++i) {
      load_rows(i + 1, rb);
      source(i, ra);
#pragma unroll
      for (int h = 0; h < WIN; ++h) ra[h] = rb[h];
    }
    if constexpr (PASS == 1) {
      __builtin_amdgcn_s_setprio(2);
      // Sublayers 2..SB: the per-stream states; sublayer 1: its retrieved
      // states and the mixer's sums.
      float v[TC * 8];
#pragma unroll
      for (int q = 0; q < TC; ++q) {
        const bool ok = t0 + q < t_end;
        const float isc = iscale_s[q];  // a power of two: exact
#pragma unroll
        for (int j = 1; j < SB; ++j)
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            const h2 hv = {(f16_t)(z[q][j][r].x * isc), (f16_t)(z[q][j][r].y * isc)};
            if (ok)
              *reinterpret_cast<uint32_t*>(a.o_state + (((j - 1) * kMsarStreams + r) * T + t0 + q) * d + c0) =
                  __builtin_bit_cast(uint32_t, hv);
          }
        float e[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          const float2 zr = z[q][0][r];
          const float4 pm0 = pm_s[(r * 2 + 0) * kMfB + tid], pm1 = pm_s[(r * 2 + 1) * kMfB + tid];
          if (ok) *reinterpret_cast<float2*>(a.zbuf + ((t0 + q) * kMsarStreams + r) * d + c0) = zr;
          e[0] = fmaf(zr.x, zr.x, fmaf(zr.y, zr.y, e[0]));
          e[1] = fmaf(zr.x, pm0.x, fmaf(zr.y, pm1.x, e[1]));
          e[2] = fmaf(zr.x, pm0.y, fmaf(zr.y, pm1.y, e[2]));
          e[3] = fmaf(zr.x, pm0.z, fmaf(zr.y, pm1.z, e[3]));
          e[4] = fmaf(zr.x, pm0.w, fmaf(zr.y, pm1.w, e[4]));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[q * 8 + j] = j < 5 ? e[j] : 0.f;
      }
      float tot;
      if constexpr (TC * 8 == 32)
        tot = block_reduce32(v, red, buf);
      else
        tot = block_reduce_values<TC * 8>(v, red, buf);
      buf ^= 1;
      const int p = tid;
      if (p < TC * 8 && (p & 7) < 5 && t0 + p / 8 < t_end)
        a.part2[((t0 + p / 8) * S + slice) * kMfPart2 + (p & 7)] = tot;
    }
  }
}

// Per token, wave j handles sublayer j: lane r*16 + n holds rep n of stream r.
// Writes the weights, and for sublayers 2..SB the log-sum-exp Phase 2 merges with.
template <int SB>
__global__ __launch_bounds__(256) void k_bmsar_alpha(BmsarArgs a) {
  constexpr int V = 4 + 4 * SB;
  const int lane = lane_id(), j = threadIdx.x >> 6;
  const int64_t T = a.T, d = a.d;
  const int S = (int)(d / kMfSlice), n = (int)a.N;
  const int r = lane >> 4, i = lane & 15;
  const bool valid = i < n;
  const int ii = valid ? i : 0;
  if (j >= SB) return;  // whole waves: no cross-lane work below in a partial wave
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    float ss = 0.f, dot = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = a.part + ((t * S + s) * n + ii) * V;
      ss += p[r];
      dot += p[4 + j * kMsarStreams + r];
    }
    const float score = valid ? dot / sqrtf(ss / (float)d + a.eps) : -INFINITY;
    const float m = group_max<16>(score);
    const float e = valid ? expf(score - m) : 0.f;
    const float l = group_sum<16>(e);
    a.alpha[((t * SB + j) * kMsarStreams + r) * kMfAlphaRow + i] = e / l;
    if (j >= 1 && i == 0) a.lse[((j - 1) * kMsarStreams + r) * T + t] = m + logf(l);
    // fp16 state scale: every |o^(r)| <= max_n sqrt(ss_n^(r)), a power of two.
    const float mss = group_max<64>(valid ? ss : 0.f);
    if (j == 0 && lane == 0) a.o_scale[t] = f16_state_scale(sqrtf(mss));
  }
}

// ------------------------------------------------------------ Block MSAR Phase 2
// One source, the intra-block partial b, merged by online softmax into the
// Phase-1 state of each stream ([MSAR] "How to use it"; the merge is Block
// AttnRes's, per stream): Z^(r) = a_r o^(r) + b_r x^(r), with a_r, b_r from
// the state's log-sum-exp and the partial's score.  Same slicing as the
// other passes, but with one source each thread keeps a sliding window of the
// partial's rows (t0-11 .. t0+TC-1 of its two channels) in registers across
// its chunks and prefetches the next chunk's rows and state one chunk ahead:
// no halo row is read twice, and each chunk's loads have the previous chunk's
// work to arrive.  Per-token weights are read with uniform (scalar) loads.
//   k_bmsar_p2<0>       the partial's per-stream sum of squares and query
//                       product per token and slice                  -> part
//   k_bmsar_p2_merge    per token: a_r * state scale, b_r            -> mw
//   k_bmsar_p2<1>       Z^(r) per token, the sum of squares of Flatten(Z)
//                       and its four projections by P, per slice     -> part2
//   k_bmsar_p2_beta     per token: beta = sigmoid(RMSNorm(Flatten(Z)) P)
//   k_bmsar_p2<2>       Z^(r) again and h = sum_r beta_r Z^(r)       -> out
constexpr int kP2Range = 256;  // tokens per workgroup (measured: 256 beats 128 and 512)

template <int PASS, int TC>
__global__ __launch_bounds__(kMfB, 2) void k_bmsar_p2(const bf16_t* __restrict__ part,
                                                      const f16_t* __restrict__ base,
                                                      const float* __restrict__ conv,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ mix,
                                                      const float* __restrict__ mw,
                                                      const float* __restrict__ beta,
                                                      float* __restrict__ sums, bf16_t* __restrict__ out,
                                                      int64_t T, int64_t d) {
  constexpr int WIN = TC + kMfHalo;
  constexpr int NV = TC * 8;
  __shared__ float red[2][4][256];
  const int tid = threadIdx.x;
  const int S = (int)(d / kMfSlice);
  const int slice = blockIdx.x;
  const int64_t c0 = (int64_t)slice * kMfSlice + 2 * tid;

  float2 tap[kMsarTaps];
#pragma unroll
  for (int k = 0; k < kMsarTaps; ++k) tap[k] = *reinterpret_cast<const float2*>(conv + k * d + c0);
  float2 wq[kMsarStreams];
  float4 pm[kMsarStreams][2];
#pragma unroll
  for (int r = 0; r < kMsarStreams; ++r) {
    if constexpr (PASS == 0) {
      wq[r] = *reinterpret_cast<const float2*>(w + r * d + c0);
    } else if constexpr (PASS == 1) {
      pm[r][0] = *reinterpret_cast<const float4*>(mix + (r * d + c0) * kMsarStreams);
      pm[r][1] = *reinterpret_cast<const float4*>(mix + (r * d + c0 + 1) * kMsarStreams);
    }
  }

  const int64_t t_begin = (int64_t)blockIdx.y * kP2Range;
  const int64_t t_end = t_begin + kP2Range < T ? t_begin + kP2Range : T;
  const bf16_t* col = part + c0;
  // Unconditional loads of clamped rows; rows outside [0, T) are zeroed when
  // unpacked (before the first token: the causal zero; past the end: unused).
  auto row_ld = [&](int64_t row) {
    const int64_t rc = row < 0 ? 0 : (row >= T ? T - 1 : row);
    return *reinterpret_cast<const uint32_t*>(col + rc * d);
  };
  auto unpack_row = [&](int64_t row, uint32_t u) {
    u = (row >= 0 && row < T) ? u : 0u;
    return make_float2(bf_lo(u), bf_hi(u));
  };
  auto base_ld = [&](int64_t t0, uint32_t (&bb)[TC][kMsarStreams]) {
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int64_t tq = t0 + q < T ? t0 + q : T - 1;
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r)
        bb[q][r] = *reinterpret_cast<const uint32_t*>(base + (r * T + tq) * d + c0);
    }
  };

  float2 win[WIN];
  {
    uint32_t raw[WIN];
#pragma unroll
    for (int h = 0; h < WIN; ++h) raw[h] = row_ld(t_begin - kMfHalo + h);
#pragma unroll
    for (int h = 0; h < WIN; ++h) win[h] = unpack_row(t_begin - kMfHalo + h, raw[h]);
  }
  uint32_t bcur[PASS >= 1 ? TC : 1][kMsarStreams], bnxt[PASS >= 1 ? TC : 1][kMsarStreams];
  if constexpr (PASS >= 1) base_ld(t_begin, bcur);

  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TC) {
    // The next chunk's rows and state, in flight during this chunk.
    uint32_t nxt[TC];
#pragma unroll
    for (int q = 0; q < TC; ++q) nxt[q] = row_ld(t0 + TC + q);
    if constexpr (PASS >= 1) base_ld(t0 + TC, bnxt);
    // Keep the prefetch here: without this the compiler may sink the loads to
    // their first use in the next chunk, where their latency is exposed.
    keep_memory_order();
    if constexpr (PASS <= 1) __builtin_amdgcn_s_setprio(0);

    float v[PASS <= 1 ? NV : 1];
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      // Token t0 + q is window row q + 11; lag k is row q + 11 - k.
      float2 sv[kMsarStreams];
      sv[0] = win[q + kMfHalo];
#pragma unroll
      for (int r = 1; r < kMsarStreams; ++r) {
        const int K = msar_kernel(r), off = msar_offset(r);
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          acc.x = fmaf(tap[off + k].x, win[q + kMfHalo - k].x, acc.x);
          acc.y = fmaf(tap[off + k].y, win[q + kMfHalo - k].y, acc.y);
        }
        sv[r] = acc;
      }
      if constexpr (PASS == 0) {
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          v[q * 8 + r] = fmaf(sv[r].x, sv[r].x, sv[r].y * sv[r].y);
          v[q * 8 + 4 + r] = fmaf(wq[r].x, sv[r].x, wq[r].y * sv[r].y);
        }
      } else {
        const int64_t tq = t0 + q < T ? t0 + q : T - 1;
        const float* mq = mw + tq * 8;
        float2 z[kMsarStreams];
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          const uint32_t u = bcur[q][r];
          const float ox = (float)__builtin_bit_cast(f16_t, (uint16_t)(u & 0xffffu));
          const float oy = (float)__builtin_bit_cast(f16_t, (uint16_t)(u >> 16));
          const float ca = mq[r], cb = mq[4 + r];
          z[r] = make_float2(fmaf(cb, sv[r].x, ca * ox), fmaf(cb, sv[r].y, ca * oy));
        }
        if constexpr (PASS == 1) {
          float e[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            const float2 zr = z[r];
            e[0] = fmaf(zr.x, zr.x, fmaf(zr.y, zr.y, e[0]));
            e[1] = fmaf(zr.x, pm[r][0].x, fmaf(zr.y, pm[r][1].x, e[1]));
            e[2] = fmaf(zr.x, pm[r][0].y, fmaf(zr.y, pm[r][1].y, e[2]));
            e[3] = fmaf(zr.x, pm[r][0].z, fmaf(zr.y, pm[r][1].z, e[3]));
            e[4] = fmaf(zr.x, pm[r][0].w, fmaf(zr.y, pm[r][1].w, e[4]));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[q * 8 + j] = j < 5 ? e[j] : 0.f;
        } else {
          const float* bq = beta + tq * kMsarStreams;
          float2 h = make_float2(0.f, 0.f);
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            h.x = fmaf(bq[r], z[r].x, h.x);
            h.y = fmaf(bq[r], z[r].y, h.y);
          }
          if (t0 + q < t_end) *reinterpret_cast<uint32_t*>(out + (t0 + q) * d + c0) = pack_bf2(h.x, h.y);
        }
      }
    }
    if constexpr (PASS <= 1) {
      __builtin_amdgcn_s_setprio(2);
      float tot;
      if constexpr (NV == 32)
        tot = block_reduce32(v, red, buf);
      else
        tot = block_reduce_values<NV>(v, red, buf);
      buf ^= 1;
      const int p = tid;
      if (p < NV && t0 + p / 8 < t_end) sums[((t0 + p / 8) * S + slice) * 8 + (p & 7)] = tot;
    }
    // The prefetched values are consumed here, at the end of this chunk.
#pragma unroll
    for (int q = 0; q < TC; ++q) asm volatile("" ::"v"(nxt[q]));
    if constexpr (PASS >= 1) {
#pragma unroll
      for (int q = 0; q < TC; ++q)
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) asm volatile("" ::"v"(bnxt[q][r]));
    }
    // Slide the window by one chunk.
#pragma unroll
    for (int h = 0; h < kMfHalo; ++h) win[h] = win[h + TC];
#pragma unroll
    for (int q = 0; q < TC; ++q) win[kMfHalo + q] = unpack_row(t0 + TC + q, nxt[q]);
    if constexpr (PASS >= 1) {
#pragma unroll
      for (int q = 0; q < TC; ++q)
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) bcur[q][r] = bnxt[q][r];
    }
  }
}

// Per (token, stream): the partial's score from the slices' sums and the
// online-softmax merge weights a = e^{lse-m}/(...) (times the state's scale)
// and b = e^{s_p-m}/(...).
__global__ __launch_bounds__(256) void k_bmsar_p2_merge(const float* stats, const float* lse_i, const float* o_scale,
                                                        float* mw, int64_t T, int64_t d, float eps) {
  const int S = (int)(d / kMfSlice);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < T * kMsarStreams;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / kMsarStreams;
    const int r = (int)(e % kMsarStreams);
    float ss = 0.f, dot = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = stats + (t * S + s) * 8;
      ss += p[r];
      dot += p[4 + r];
    }
    const float sp = dot / sqrtf(ss / (float)d + eps);
    const float L = lse_i[r * T + t];
    const float m = fmaxf(L, sp);
    const float wa = expf(L - m), wb = expf(sp - m);
    const float inv = 1.0f / (wa + wb);
    mw[t * 8 + r] = (wa * inv) * o_scale[t];
    mw[t * 8 + 4 + r] = wb * inv;
  }
}

// Per token: beta_q = sigmoid((Flatten(Z) . P_q) / RMS(Flatten(Z))) from the
// slices' sums, summed in slice order.
__global__ __launch_bounds__(256) void k_bmsar_p2_beta(const float* sums, float* beta, int64_t T, int64_t d,
                                                       float eps) {
  const int S = (int)(d / kMfSlice);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += (int64_t)gridDim.x * blockDim.x) {
    float e[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int q = 0; q < 5; ++q) e[q] += sums[(t * S + s) * 8 + q];
    const float inv = 1.0f / sqrtf(e[0] / (float)(kMsarStreams * d) + eps);
#pragma unroll
    for (int q = 0; q < kMsarStreams; ++q) beta[t * kMsarStreams + q] = 1.0f / (1.0f + expf(-e[1 + q] * inv));
  }
}

bool al16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

MsarFastBufs carve(const MsarArgs& a) {
  const int64_t S = a.d / kMfSlice, T = a.T, N = a.n_src;
  char* p = static_cast<char*>(a.ws);
  MsarFastBufs b;
  b.part = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * S * 8 * N) * 4);
  b.alpha = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * kMsarStreams * kMfAlphaRow) * 4);
  b.part2 = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * S * kMfPart2) * 4);
  b.zscale = reinterpret_cast<float*>(p);
  p += align256((size_t)T * 4);
  b.zbuf = reinterpret_cast<f16_t*>(p);
  b.zbuf32 = nullptr;
  return b;
}

template <int N>
hipError_t launch_n(const MsarArgs& a, hipStream_t st) {
  const MsarFastBufs b = carve(a);
  const dim3 grid((unsigned)(a.d / kMfSlice), (unsigned)((a.T + kMfRange - 1) / kMfRange));
  hipLaunchKernelGGL(k_msar_slice<0>, grid, dim3(kMfB), 0, st, a, b);
  int64_t ablocks = (a.T + 3) / 4;
  if (ablocks > 8 * (int64_t)num_cus()) ablocks = 8 * (int64_t)num_cus();
  hipLaunchKernelGGL((k_msar_alpha<N>), dim3((unsigned)ablocks), dim3(256), 0, st, a, b);
  hipLaunchKernelGGL(k_msar_slice<1>, grid, dim3(kMfB), 0, st, a, b);
  int64_t oblocks = a.T < 4 * (int64_t)num_cus() ? a.T : 4 * (int64_t)num_cus();
  hipLaunchKernelGGL(k_msar_out<true>, dim3((unsigned)oblocks), dim3(256), 0, st, a, b);
  return hipGetLastError();
}

}  // namespace

size_t msar_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int dtype) {
  if (dtype != kBF16 || n_dst != 1 || n_src < 1 || n_src > kMsarFastMaxSources || T < 1 || d % kMfSlice != 0)
    return 0;
  const int64_t S = d / kMfSlice;
  return align256((size_t)(T * S * 8 * n_src) * 4) + align256((size_t)(T * kMsarStreams * kMfAlphaRow) * 4) +
         align256((size_t)(T * S * kMfPart2) * 4) + align256((size_t)T * 4) + align256((size_t)(T * kMsarStreams * d) * 2);
}

bool msar_fast_ok(const MsarArgs& a) {
  const size_t need = msar_fast_workspace_bytes(a.n_src, a.n_dst, a.T, a.d, a.dtype);
  if (need == 0 || a.ws == nullptr || a.ws_bytes < need) return false;
  if (a.T > ((int64_t)1 << 30) || a.d > ((int64_t)1 << 20)) return false;
  return al16(a.src) && al16(a.out) && al16(a.w) && al16(a.conv) && al16(a.mix) && al16(a.ws);
}

namespace {

template <int SB>
hipError_t launch_bmsar_p1_sb(const BmsarArgs& a, void* h1, hipStream_t st) {
  const dim3 grid((unsigned)(a.d / kMfSlice), (unsigned)((a.T + kMfRange - 1) / kMfRange));
  hipLaunchKernelGGL((k_bmsar_p1<SB, 0>), grid, dim3(kMfB), 0, st, a);
  int64_t blocks = a.T < 8 * (int64_t)num_cus() ? a.T : 8 * (int64_t)num_cus();
  hipLaunchKernelGGL((k_bmsar_alpha<SB>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_bmsar_p1<SB, 1>), grid, dim3(kMfB), 0, st, a);
  MsarArgs ma{nullptr, a.N, a.T, a.d, a.w, a.conv, a.mix1, 1, a.eps, kBF16, h1, nullptr, 0};
  MsarFastBufs mb{nullptr, nullptr, a.part2, nullptr, nullptr, a.zbuf};
  int64_t oblocks = a.T < 4 * (int64_t)num_cus() ? a.T : 4 * (int64_t)num_cus();
  hipLaunchKernelGGL(k_msar_out<false>, dim3((unsigned)oblocks), dim3(256), 0, st, ma, mb);
  return hipGetLastError();
}

}  // namespace

size_t bmsar_phase1_workspace_bytes(int64_t N, int64_t SB, int64_t T, int64_t d) {
  if (N < 1 || N > kMsarFastMaxSources || SB < 1 || SB > 4 || T < 1 || T > ((int64_t)1 << 30) ||
      d % kMfSlice != 0 || d > ((int64_t)1 << 20))
    return 0;
  const int64_t S = d / kMfSlice, V = 4 + 4 * SB;
  return align256((size_t)(T * S * N * V) * 4) + align256((size_t)(T * SB * kMsarStreams * kMfAlphaRow) * 4) +
         align256((size_t)(T * S * kMfPart2) * 4) + align256((size_t)(T * kMsarStreams * d) * 4);
}

hipError_t launch_bmsar_phase1(const BmsarCall& c, hipStream_t st) {
  const int64_t S = c.d / kMfSlice, V = 4 + 4 * c.SB;
  char* p = static_cast<char*>(c.ws);
  BmsarArgs a;
  a.reps = c.reps;
  a.N = c.N;
  a.T = c.T;
  a.d = c.d;
  a.w = c.w;
  a.conv = c.conv;
  a.mix1 = c.mix1;
  a.eps = c.eps;
  a.o_state = static_cast<f16_t*>(c.o_state);
  a.o_scale = c.o_scale;
  a.lse = c.lse;
  a.part = reinterpret_cast<float*>(p);
  p += align256((size_t)(c.T * S * c.N * V) * 4);
  a.alpha = reinterpret_cast<float*>(p);
  p += align256((size_t)(c.T * c.SB * kMsarStreams * kMfAlphaRow) * 4);
  a.part2 = reinterpret_cast<float*>(p);
  p += align256((size_t)(c.T * S * kMfPart2) * 4);
  a.zbuf = reinterpret_cast<float*>(p);
  switch (c.SB) {
    case 1: return launch_bmsar_p1_sb<1>(a, c.h1, st);
    case 2: return launch_bmsar_p1_sb<2>(a, c.h1, st);
    case 3: return launch_bmsar_p1_sb<3>(a, c.h1, st);
    case 4: return launch_bmsar_p1_sb<4>(a, c.h1, st);
    default: return hipErrorNotSupported;
  }
}

size_t bmsar_phase2_workspace_bytes(int64_t T, int64_t d) {
  if (T < 1 || T > ((int64_t)1 << 30) || d % kMfSlice != 0 || d > ((int64_t)1 << 20)) return 0;
  const int64_t S = d / kMfSlice;
  // stats [T][S][8], merge weights [T][8], mixer sums [T][S][8], beta [T][4]
  return align256((size_t)(T * S * 8) * 4) + align256((size_t)(T * 8) * 4) + align256((size_t)(T * S * 8) * 4) +
         align256((size_t)(T * kMsarStreams) * 4);
}

hipError_t launch_bmsar_phase2(const Bmsar2Call& c, hipStream_t st) {
  const int64_t S = c.d / kMfSlice, T = c.T, d = c.d;
  char* p = static_cast<char*>(c.ws);
  float* stats = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * S * 8) * 4);
  float* mw = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * 8) * 4);
  float* sums = reinterpret_cast<float*>(p);
  p += align256((size_t)(T * S * 8) * 4);
  float* beta = reinterpret_cast<float*>(p);
  const bf16_t* part = static_cast<const bf16_t*>(c.partial);
  const f16_t* base = static_cast<const f16_t*>(c.o_i);
  bf16_t* out = static_cast<bf16_t*>(c.h_i);
  const dim3 grid((unsigned)S, (unsigned)((T + kP2Range - 1) / kP2Range));
  const int64_t cap = 8 * (int64_t)num_cus();
  int64_t mblocks = (T * kMsarStreams + 255) / 256, bblocks = (T + 255) / 256;
  if (mblocks > cap) mblocks = cap;
  if (bblocks > cap) bblocks = cap;
  hipLaunchKernelGGL((k_bmsar_p2<0, 8>), grid, dim3(kMfB), 0, st, part, base, c.conv, c.w_i, c.mix_i,
                     (const float*)nullptr, (const float*)nullptr, stats, (bf16_t*)nullptr, T, d);
  hipLaunchKernelGGL(k_bmsar_p2_merge, dim3((unsigned)mblocks), dim3(256), 0, st, (const float*)stats, c.lse_i,
                     c.o_scale, mw, T, d, c.eps);
  hipLaunchKernelGGL((k_bmsar_p2<1, 4>), grid, dim3(kMfB), 0, st, part, base, c.conv, c.w_i, c.mix_i,
                     (const float*)mw, (const float*)nullptr, sums, (bf16_t*)nullptr, T, d);
  hipLaunchKernelGGL(k_bmsar_p2_beta, dim3((unsigned)bblocks), dim3(256), 0, st, (const float*)sums, beta, T, d,
                     c.eps);
  hipLaunchKernelGGL((k_bmsar_p2<2, 8>), grid, dim3(kMfB), 0, st, part, base, c.conv, c.w_i, c.mix_i,
                     (const float*)mw, (const float*)beta, (float*)nullptr, out, T, d);
  return hipGetLastError();
}

hipError_t launch_msar_fast(const MsarArgs& a, hipStream_t st) {
  switch (a.n_src) {
    case 1: return launch_n<1>(a, st);
    case 2: return launch_n<2>(a, st);
    case 3: return launch_n<3>(a, st);
    case 4: return launch_n<4>(a, st);
    case 5: return launch_n<5>(a, st);
    case 6: return launch_n<6>(a, st);
    case 7: return launch_n<7>(a, st);
    case 8: return launch_n<8>(a, st);
    case 9: return launch_n<9>(a, st);
    case 10: return launch_n<10>(a, st);
    case 11: return launch_n<11>(a, st);
    case 12: return launch_n<12>(a, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attnres
