// MSAR, multi-stream depth attention (onedev.kr summary of the MSAR paper,
// "How it differs" and "How to use it"): every source v_i expands into four
// full-width streams -- the identity and causal depthwise convolutions along
// the tokens with kernel sizes 4, 8 and 12 -- each stream runs its own depth
// softmax with its own pseudo-query, and the H^pre mixer
// beta = sigmoid(RMSNorm(Flatten(Z)) P) weights the retrieved stream states:
// h = sum_r beta_r Z^(r).  The streams are never written: each kernel expands
// them from the sources on demand.
//
// General kernel: one wavefront per (token, destination), any d, n_src <= 64.
// Three passes over the channels, each expanding the streams again from the
// source rows (t-11 .. t, cache-resident): scores, then the retrieved states
// with the mixer's statistics, then the output.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace attnres {
namespace {

constexpr int kMsWaves = 4;

// The 24 taps of channel c.
__device__ __forceinline__ void msar_taps(const float* conv, int64_t d, int64_t c, float (&tap)[kMsarTaps]) {
#pragma unroll
  for (int k = 0; k < kMsarTaps; ++k) tap[k] = conv[k * d + c];
}

// Streams 1..3 of one source at one channel: tap k of a stream multiplies the
// value k tokens back.  win[k] = v[t - k] (zero before the first token).
__device__ __forceinline__ void msar_streams(const float (&win)[kMsarMaxTaps], const float (&tap)[kMsarTaps],
                                             float (&x)[kMsarStreams]) {
  x[0] = win[0];
#pragma unroll
  for (int r = 1; r < kMsarStreams; ++r) {
    const int K = msar_kernel(r), off = msar_offset(r);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kMsarMaxTaps; ++k)
      if (k < K) acc = fmaf(tap[off + k], win[k], acc);
    x[r] = acc;
  }
}

template <typename E>
__device__ __forceinline__ void msar_window(const E* col, int64_t t, int64_t d, float (&win)[kMsarMaxTaps]) {
#pragma unroll
  for (int k = 0; k < kMsarMaxTaps; ++k) win[k] = (k <= t) ? ld(col + (t - k) * d) : 0.f;
}

template <typename E>
__global__ __launch_bounds__(kMsWaves * 64) void k_msar_generic(MsarArgs a) {
  __shared__ float alpha_tab[kMsWaves][kMsarStreams][64];
  const E* src = static_cast<const E*>(a.src);
  E* out = static_cast<E*>(a.out);
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int64_t d = a.d, T = a.T, td = a.T * a.d, units = a.T * a.n_dst;
  const int64_t wave = (int64_t)blockIdx.x * kMsWaves + wv;
  const int64_t nw = (int64_t)gridDim.x * kMsWaves;
  for (int64_t u = wave; u < units; u += nw) {
    const int64_t t = u / a.n_dst, j = u % a.n_dst;
    const int n = (int)(a.n_src - a.n_dst + j + 1);
    const float* wj = a.w + j * kMsarStreams * d;
    const float* Pj = a.mix + j * kMsarStreams * d * kMsarStreams;

    // Pass 1: scores.  Lane i keeps source i's score per stream.
    float score[kMsarStreams];
#pragma unroll
    for (int r = 0; r < kMsarStreams; ++r) score[r] = -INFINITY;
    for (int i = 0; i < n; ++i) {
      float ss[kMsarStreams] = {0.f, 0.f, 0.f, 0.f}, dot[kMsarStreams] = {0.f, 0.f, 0.f, 0.f};
      for (int64_t c0 = 0; c0 < d; c0 += kWave) {  // uniform bounds, predicated channel
        const int64_t c = c0 + lane;
        if (c < d) {
          float win[kMsarMaxTaps], x[kMsarStreams], tap[kMsarTaps];
          msar_window<E>(src + i * td + c, t, d, win);
          msar_taps(a.conv, d, c, tap);
          msar_streams(win, tap, x);
#pragma unroll
          for (int r = 0; r < kMsarStreams; ++r) {
            ss[r] = fmaf(x[r], x[r], ss[r]);
            dot[r] = fmaf(wj[r * d + c], x[r], dot[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) {
        const float s = wave_sum(dot[r]) / sqrtf(wave_sum(ss[r]) / (float)d + a.eps);
        if (lane == i) score[r] = s;
      }
    }
    // Depth softmax per stream, over lanes 0 .. n-1; weights to this wave's table.
#pragma unroll
    for (int r = 0; r < kMsarStreams; ++r) {
      const float m = wave_max(score[r]);
      const float e = lane < n ? expf(score[r] - m) : 0.f;
      alpha_tab[wv][r][lane] = e / wave_sum(e);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // Pass 2: Z^(r) per channel, sum of squares of Flatten(Z) and its projections.
    float ssz = 0.f, proj[kMsarStreams] = {0.f, 0.f, 0.f, 0.f};
    auto z_at = [&](int64_t c, float (&z)[kMsarStreams]) {
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) z[r] = 0.f;
      float tap[kMsarTaps];
      msar_taps(a.conv, d, c, tap);
      for (int i = 0; i < n; ++i) {
        float win[kMsarMaxTaps], x[kMsarStreams];
        msar_window<E>(src + i * td + c, t, d, win);
        msar_streams(win, tap, x);
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) z[r] = fmaf(alpha_tab[wv][r][i], x[r], z[r]);
      }
    };
    for (int64_t c0 = 0; c0 < d; c0 += kWave) {
      const int64_t c = c0 + lane;
      if (c < d) {
        float z[kMsarStreams];
        z_at(c, z);
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          ssz = fmaf(z[r], z[r], ssz);
          const float* prow = Pj + (r * d + c) * kMsarStreams;  // row r*d + c of P
#pragma unroll
          for (int q = 0; q < kMsarStreams; ++q) proj[q] = fmaf(z[r], prow[q], proj[q]);
        }
      }
    }
    const float inv = 1.0f / sqrtf(wave_sum(ssz) / (float)(kMsarStreams * d) + a.eps);
    float beta[kMsarStreams];
#pragma unroll
    for (int q = 0; q < kMsarStreams; ++q) beta[q] = 1.0f / (1.0f + expf(-wave_sum(proj[q]) * inv));

    // Pass 3: h = sum_r beta_r Z^(r).
    for (int64_t c0 = 0; c0 < d; c0 += kWave) {
      const int64_t c = c0 + lane;
      if (c < d) {
        float z[kMsarStreams];
        z_at(c, z);
        float h = 0.f;
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) h = fmaf(beta[r], z[r], h);
        st(out + (j * T + t) * d + c, h);
      }
    }
    // The table is rewritten by this wave's next unit only after every lane
    // has finished reading it.
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_msar_generic(const MsarArgs& a, hipStream_t st) {
  int64_t units = a.T * a.n_dst;
  int64_t blocks = (units + kMsWaves - 1) / kMsWaves;
  const int64_t cap = 8 * (int64_t)num_cus();
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  if (a.dtype == kF32)
    hipLaunchKernelGGL(k_msar_generic<float>, dim3((unsigned)blocks), dim3(kMsWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(k_msar_generic<bf16_t>, dim3((unsigned)blocks), dim3(kMsWaves * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace attnres
