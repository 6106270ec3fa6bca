// Specialised Block AttnRes backward for gfx950 (bf16 I/O, fp32 arithmetic).
//
// Gradient of L = sum_j <dh_j, h_j> for one block (the analytic form in
// attnres.h).  Like Phase 1, a persistent workgroup of B = d/(8*CH) threads owns
// all channels of one token at a time, thread `tid` owning CH chunks of 8
// channels at (c*B + tid)*8.  Per token the workgroup
//   1. loads the N reps, the S-1 partials and the S upstream gradients once,
//   2. accumulates per-thread partial sums of squares (per source), q_j . v_i
//      and dh_j . v_i for every (destination j, source i) pair,
//   3. reduces them across the wave (transpose-reduce) and the workgroup (LDS),
//   4. forms, in lanes (one per pair), alpha, c = alpha (a - sum alpha a),
//      c * r_i and the normalisation-path coefficient r_i^2 sum_j c s / d,
//   5. writes dv_i = sum_j (alpha dh_j + c r_i q_j) - coef_i v_i, and
//   6. accumulates Z_j += sum_i c r_i v_i in registers across its tokens.
// At the end each workgroup writes its Z slab; the fixed-order reduction
// (k_bwd_reduce) turns the slabs into dw and dgain.
//
// Heads (MHAR, chatpaper.ai abstract): with one chunk of 8 channels per thread,
// wave w owns channels [512 w, 512 w + 512), so a head of d/H channels is
// exactly WH = (B/64)/H consecutive waves.  The sums of
// squares are reduced over the whole workgroup (the RMS spans all of d), the
// dot products only over the head's waves, and every lane table then holds the
// wave's own head.  The one quantity mixing heads, sum over (j, h) of c s in
// the normalisation path, takes a second LDS exchange per token.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

#ifndef ATTNRES_BWD_MINWAVES
#define ATTNRES_BWD_MINWAVES 1
#endif

namespace attnres {
namespace {

constexpr int next_pow2b(int n) { return n <= 1 ? 1 : 2 * next_pow2b((n + 1) / 2); }

__device__ __forceinline__ void unpack8b(const uint4 u, float (&x)[8]) {
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
  x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
  x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}

__device__ __forceinline__ uint4 pack8b(const float (&x)[8]) {
  uint4 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  u.z = pack_bf2(x[4], x[5]);
  u.w = pack_bf2(x[6], x[7]);
  return u;
}

// Pair (destination j, slot u): slot u < N is rep u; slot N is the partial
// read only by destinations j >= 1 (partial j-1).
template <int N>
constexpr int pair_index(int j, int u) { return j == 0 ? u : N + (j - 1) * (N + 1) + u; }

template <int N, int S, int CH, int B, int HH>
__global__ __launch_bounds__(B, ATTNRES_BWD_MINWAVES) void k_bwd_fast(BwdArgs a) {
  constexpr int NS = N + S - 1;                   // sources: N reps, then S-1 partials
  constexpr int NPAIR = N + (S - 1) * (N + 1);    // (destination, source) pairs
  constexpr int P = NS + 2 * NPAIR;               // ss_i, q.v per pair, dh.v per pair
  constexpr int NG = (P + 63) / 64;
  constexpr int NP = next_pow2b(N + 1);           // lanes per destination group
  static_assert(S * NP <= 64, "pair table must fit one wave");
  constexpr int W = B / 64;
  static_assert(HH == 1 || (CH == 1 && W % HH == 0), "a head must be whole waves");
  constexpr int WH = W / HH;                      // waves per head
  __shared__ float red[2][W][NG * 64];
  __shared__ float csx[2][HH > 1 ? HH : 1][64];   // per-head sum of c s, heads > 1 only
  __shared__ float4 qs[S * CH * B * 2];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d = (int)a.d;
  const int64_t T = a.T;

  // q = w * g for this thread's channels, in this thread's own LDS slots.
  auto fold = [&](auto with_gain) {
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float qq[8];
      const int col = (c * B + tid) * 8;
      fold_q8<decltype(with_gain)::value>(a.w + (int64_t)j * d + col, a.gain + j * a.gain_ld + col, qq);
      qs[((j * CH + c) * B + tid) * 2 + 0] = make_float4(qq[0], qq[1], qq[2], qq[3]);
      qs[((j * CH + c) * B + tid) * 2 + 1] = make_float4(qq[4], qq[5], qq[6], qq[7]);
    }
  };
  if (a.gain != nullptr)
    fold(std::true_type());
  else
    fold(std::false_type());

  // This lane's pair in the table: destination pj, slot pu.
  const int pj = lane / NP, pu = lane % NP;
  const bool pvalid = pj < S && (pu < N || (pu == N && pj >= 1));
  const int psrc = pu < N ? pu : N + pj - 1;                 // source index of the pair
  const int pidx = pj == 0 ? pu : N + (pj - 1) * (N + 1) + pu;

  float zacc[S][CH][8];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) zacc[j][c][e] = 0.f;

  const bf16_t* reps = static_cast<const bf16_t*>(a.reps);
  const bf16_t* parts = static_cast<const bf16_t*>(a.partials);
  const bf16_t* dhp = static_cast<const bf16_t*>(a.dh);
  bf16_t* d_reps = static_cast<bf16_t*>(a.d_reps);
  bf16_t* d_parts = static_cast<bf16_t*>(a.d_partials);
  auto src_row = [&](int i, int64_t t) {
    return i < N ? reps + ((int64_t)i * T + t) * d : parts + ((int64_t)(i - N) * T + t) * d;
  };
  auto dsrc_row = [&](int i, int64_t t) {
    return i < N ? d_reps + ((int64_t)i * T + t) * d : d_parts + ((int64_t)(i - N) * T + t) * d;
  };

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    // Wave priority: the loads and partial sums of a token at 0, its source
    // gradients and stores at 2 (measured about 1% faster than either the
    // opposite order or none).
    __builtin_amdgcn_s_setprio(0);
    uint4 v[NS][CH], g[S][CH];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        v[i][c] = *reinterpret_cast<const uint4*>(src_row(i, t) + (c * B + tid) * 8);
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        g[j][c] = *reinterpret_cast<const uint4*>(dhp + ((int64_t)j * T + t) * d + (c * B + tid) * 8);

    // ---- per-thread partial sums
    float part[P];
#pragma unroll
    for (int p = 0; p < P; ++p) part[p] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float qc[S][8], dg[S][8];
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const float4 q0 = qs[((j * CH + c) * B + tid) * 2 + 0];
        const float4 q1 = qs[((j * CH + c) * B + tid) * 2 + 1];
        qc[j][0] = q0.x; qc[j][1] = q0.y; qc[j][2] = q0.z; qc[j][3] = q0.w;
        qc[j][4] = q1.x; qc[j][5] = q1.y; qc[j][6] = q1.z; qc[j][7] = q1.w;
        unpack8b(g[j][c], dg[j]);
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        float x[8];
        unpack8b(v[i][c], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          part[i] = fmaf(x[e], x[e], part[i]);
#pragma unroll
          for (int j = 0; j < S; ++j) {
            if (i < N || i == N + j - 1) {
              const int pp = pair_index<N>(j, i < N ? i : N);
              part[NS + pp] = fmaf(qc[j][e], x[e], part[NS + pp]);
              part[NS + NPAIR + pp] = fmaf(dg[j][e], x[e], part[NS + NPAIR + pp]);
            }
          }
        }
      }
    }
    if constexpr (P == 64 + 16 + 1) {
      // 81 values (N = 8, S = 4): one full 64-value transposing reduction, a
      // 16-value one and a single wave sum, instead of a second 64-value group
      // padded from 17.
      float a64[64], a16[16];
#pragma unroll
      for (int p = 0; p < 64; ++p) a64[p] = part[p];
#pragma unroll
      for (int p = 0; p < 16; ++p) a16[p] = part[64 + p];
      red[buf][wave][lane] = transpose_reduce64(a64);
      const float t16 = transpose_reduce16(a16);  // lane L: value 64 + (L >> 2)
      if ((lane & 3) == 0) red[buf][wave][64 + (lane >> 2)] = t16;
      const float t80 = wave_allsum(part[80]);
      if (lane == 0) red[buf][wave][80] = t80;
    } else {
      float tot[NG];
      wave_reduce_values<P>(part, tot);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) red[buf][wave][gi * 64 + lane] = tot[gi];
    }
    __syncthreads();

    // ---- per-pair scalars, one lane per (destination, source)
    float alpha = 0.f, cr = 0.f, coef = 0.f;
    {
      float ss = 0.f, sd = 0.f, ad = 0.f;
      if (pvalid) {
        const int h0 = (wave / WH) * WH;                    // first wave of this head
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) ss += red[buf][w2][psrc];
#pragma unroll
        for (int w2 = 0; w2 < WH; ++w2) {
          sd += red[buf][h0 + w2][NS + pidx];
          ad += red[buf][h0 + w2][NS + NPAIR + pidx];
        }
      }
      const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
      const float s = pvalid ? r * sd : -INFINITY;
      const float av = pvalid ? ad : 0.f;
      float m = s;
      m = group_max<NP>(m);
      const float e = pvalid ? expf(s - m) : 0.f;
      float l = e;
      l = group_sum<NP>(l);
      alpha = e / l;
      float sa = alpha * av;
      sa = group_sum<NP>(sa);
      const float c = alpha * (av - sa);
      cr = c * r;
      // sum_j c s over the destinations reading the same rep (same slot, other groups)
      const float cs = pvalid ? c * s : 0.f;
      float csum = cs;
      csum = butterfly<NP, 64>(csum, SumOp());
      float csh = pu < N ? csum : cs;
      if constexpr (HH > 1) {
        // Sum over heads, in head order, from the first wave of each head.
        if (wave % WH == 0) csx[buf][wave / WH][lane] = csh;
        __syncthreads();
        csh = 0.f;
#pragma unroll
        for (int h = 0; h < HH; ++h) csh += csx[buf][h][lane];
      }
      coef = pvalid ? r * r * csh / (float)d : 0.f;
    }

    __builtin_amdgcn_s_setprio(2);
    // ---- source gradients and Z, from registers
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = (c * B + tid) * 8;
      float qc[S][8], dg[S][8];
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const float4 q0 = qs[((j * CH + c) * B + tid) * 2 + 0];
        const float4 q1 = qs[((j * CH + c) * B + tid) * 2 + 1];
        qc[j][0] = q0.x; qc[j][1] = q0.y; qc[j][2] = q0.z; qc[j][3] = q0.w;
        qc[j][4] = q1.x; qc[j][5] = q1.y; qc[j][6] = q1.z; qc[j][7] = q1.w;
        unpack8b(g[j][c], dg[j]);
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        float x[8], gr[8];
        unpack8b(v[i][c], x);
        const int u = i < N ? i : N;
        const float cf = read_lane(coef, (i < N ? 0 : i - N + 1) * NP + u);
#pragma unroll
        for (int e = 0; e < 8; ++e) gr[e] = -cf * x[e];
#pragma unroll
        for (int j = 0; j < S; ++j) {
          if (i < N || i == N + j - 1) {
            const float al = read_lane(alpha, j * NP + u);
            const float crl = read_lane(cr, j * NP + u);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              gr[e] = fmaf(al, dg[j][e], gr[e]);
              gr[e] = fmaf(crl, qc[j][e], gr[e]);
              zacc[j][c][e] = fmaf(crl, x[e], zacc[j][c][e]);
            }
          }
        }
        bf16_t* out = dsrc_row(i, t) + col;
        if (a.accumulate) {
          float old[8];
          unpack8b(*reinterpret_cast<const uint4*>(out), old);
#pragma unroll
          for (int e = 0; e < 8; ++e) gr[e] += old[e];
        }
        *reinterpret_cast<uint4*>(out) = pack8b(gr);
      }
    }
    buf ^= 1;
  }

  // This workgroup's slab of Z partial sums: zslots[blockIdx][j][channel].
  float* z = a.zslots + (int64_t)blockIdx.x * S * d;
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float4* zp = reinterpret_cast<float4*>(z + (int64_t)j * d + (c * B + tid) * 8);
      zp[0] = make_float4(zacc[j][c][0], zacc[j][c][1], zacc[j][c][2], zacc[j][c][3]);
      zp[1] = make_float4(zacc[j][c][4], zacc[j][c][5], zacc[j][c][6], zacc[j][c][7]);
    }
}

template <int N, int S, int CH, int B, int HH>
hipError_t launch_bwd_nsb(const BwdArgs& a, int64_t* slots_used, hipStream_t st) {
  auto kern = k_bwd_fast<N, S, CH, B, HH>;
  int per_cu = 0;
  hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), B, &per_cu);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  if (grid > a.slots) grid = a.slots;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(B), 0, st, a);
  *slots_used = grid;
  return hipGetLastError();
}

// One chunk of 8 channels per thread (B = d/8 threads) keeps the kernel within
// 2 waves per SIMD without spills.
bool bwd_width_ok(int64_t d) { return d == 1024 || d == 2048 || d == 4096; }

bool aligned16b(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool bwd_fast_ok(const BwdArgs& a) {
  if (a.dtype != kBF16 || a.N != 8 || a.S != 4 || a.T < 1) return false;
  if (!bwd_width_ok(a.d) || a.slots < 1) return false;
  // Heads of whole waves: H in {1, 2, 4, 8} dividing the d/512 waves.
  const int64_t waves = a.d / 512;
  if (a.H != 1 && a.H != 2 && a.H != 4 && a.H != 8) return false;
  if (waves % a.H != 0) return false;
  return aligned16b(a.reps) && aligned16b(a.partials) && aligned16b(a.dh) && aligned16b(a.d_reps) &&
         aligned16b(a.d_partials) && aligned16b(a.zslots) && aligned16b(a.w) && aligned16b(a.gain);
}

template <int B>
hipError_t launch_bwd_b(const BwdArgs& a, int64_t* slots_used, hipStream_t st) {
  switch (a.H) {
    case 1: return launch_bwd_nsb<8, 4, 1, B, 1>(a, slots_used, st);
    case 2: return launch_bwd_nsb<8, 4, 1, B, 2>(a, slots_used, st);
    case 4:
      if constexpr (B >= 256) return launch_bwd_nsb<8, 4, 1, B, 4>(a, slots_used, st);
      break;
    case 8:
      if constexpr (B >= 512) return launch_bwd_nsb<8, 4, 1, B, 8>(a, slots_used, st);
      break;
  }
  return hipErrorInvalidValue;  // excluded by bwd_fast_ok
}

hipError_t launch_bwd_fast(const BwdArgs& a, int64_t* slots_used, hipStream_t st) {
  if (a.d == 1024) return launch_bwd_b<128>(a, slots_used, st);
  if (a.d == 2048) return launch_bwd_b<256>(a, slots_used, st);
  return launch_bwd_b<512>(a, slots_used, st);
}

}  // namespace attnres
