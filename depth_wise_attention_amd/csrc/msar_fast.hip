// MSAR specialised path: bf16, one destination (a Block MSAR sublayer), at
// most 12 sources, d a multiple of 512.
//
// The streams of a source at token t need the source's rows t-11 .. t, and
// the routing needs sums over all d channels per token.  The work is split
// over channel slices of 512 so that a workgroup keeps the 12-token history of
// every source for its slice in LDS and the 24 taps of its channels in
// registers, while walking a range of consecutive tokens:
//   k_msar_slice<N, 0>  per token and slice: each source's per-stream sum of
//                       squares and query product (8 N values)      -> part
//   k_msar_alpha<N>     per token: sum the slices, scores, the four depth
//                       softmaxes                                   -> alpha
//   k_msar_slice<N, 1>  per token and slice: Z^(r) for the slice's channels
//                       (stored once, fp32), the sum of squares of Flatten(Z)
//                       and its four projections by P               -> zbuf, part2
//   k_msar_out          per token: sum the slices, beta = sigmoid(...), and
//                       h = sum_r beta_r Z^(r)                      -> out
// The streams themselves are never stored.  Thread tid of a slice owns the two
// channels 2 tid, 2 tid + 1; its ring words in LDS are private to it, so the
// ring needs no barrier (LDS operations of a wave complete in order).

#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kMfB = 256;        // threads per workgroup
constexpr int kMfSlice = 512;    // channels per slice (2 per thread)
constexpr int kMfRange = 128;    // tokens per workgroup
constexpr int kMfHist = 12;      // history ring slots (the longest kernel)
constexpr int kMfAlphaRow = 16;  // alpha[t][r][16]
constexpr int kMfPart2 = 8;      // part2[t][slice][8] (5 used)

struct MsarFastBufs {
  float* part;    // [T][S][8 N]: per source i, [i*8 + r] sum of squares, [i*8 + 4 + r] query product
  float* alpha;   // [T][4][16]
  float* part2;   // [T][S][8]: [0] sum of squares of Z, [1 + q] projection q
  float* zbuf;    // [T][4][d]
};

__device__ __forceinline__ float2 bf2_to_f2(uint32_t u) { return make_float2(bf_lo(u), bf_hi(u)); }

template <int N, int PASS>
__global__ __launch_bounds__(kMfB, 2) void k_msar_slice(MsarArgs a, MsarFastBufs b) {
  constexpr int NV = 8 * N;                 // values reduced per token in pass 0
  constexpr int NG = (NV + 63) / 64;
  __shared__ uint32_t ring[kMfHist * N * kMfB];
  __shared__ float red[2][4][PASS == 0 ? NG * 64 : kMfPart2];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t d = a.d, T = a.T;
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

  // Zero the history, so positions before the first token read as zero.
#pragma unroll
  for (int s = 0; s < kMfHist * N; ++s) ring[s * kMfB + tid] = 0u;

  const int64_t t_begin = (int64_t)blockIdx.y * kMfRange;
  const int64_t t_end = t_begin + kMfRange < T ? t_begin + kMfRange : T;
  const int64_t t_warm = t_begin >= kMfHist - 1 ? t_begin - (kMfHist - 1) : 0;
  uint32_t nxt[N];
#pragma unroll
  for (int i = 0; i < N; ++i) nxt[i] = *reinterpret_cast<const uint32_t*>(src + ((int64_t)i * T + t_warm) * d + c0);
  int buf = 0;
  for (int64_t t = t_warm; t < t_end; ++t) {
    const int slot = (int)(t % kMfHist);
#pragma unroll
    for (int i = 0; i < N; ++i) ring[(slot * N + i) * kMfB + tid] = nxt[i];
    if (t + 1 < t_end) {
#pragma unroll
      for (int i = 0; i < N; ++i)
        nxt[i] = *reinterpret_cast<const uint32_t*>(src + ((int64_t)i * T + t + 1) * d + c0);
    }
    if (t < t_begin) continue;  // warm-up rows of the history only

    // Ring offset of lag k for this token (slot of token t - k).
    int base[kMfHist];
#pragma unroll
    for (int k = 0; k < kMfHist; ++k) base[k] = ((slot - k + kMfHist) % kMfHist) * N * kMfB + tid;

    // The four streams of source i at this thread's two channels.
    auto streams = [&](int i, float2 (&x)[kMsarStreams]) {
      float2 win[kMfHist];
#pragma unroll
      for (int k = 0; k < kMfHist; ++k) win[k] = bf2_to_f2(ring[base[k] + i * kMfB]);
      x[0] = win[0];
#pragma unroll
      for (int r = 1; r < kMsarStreams; ++r) {
        const int K = msar_kernel(r), off = msar_offset(r);
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          acc.x = fmaf(tap[off + k].x, win[k].x, acc.x);
          acc.y = fmaf(tap[off + k].y, win[k].y, acc.y);
        }
        x[r] = acc;
      }
    };

    if constexpr (PASS == 0) {
      float v[NV];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float2 x[kMsarStreams];
        streams(i, x);
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          v[i * 8 + r] = fmaf(x[r].x, x[r].x, x[r].y * x[r].y);
          v[i * 8 + 4 + r] = fmaf(wq[r].x, x[r].x, wq[r].y * x[r].y);
        }
      }
      float tot[NG];
      wave_reduce_values<NV>(v, tot);
#pragma unroll
      for (int g = 0; g < NG; ++g) red[buf][wave][g * 64 + lane] = tot[g];
      lds_barrier();
      if (tid < NV) {
        const float s = (red[buf][0][tid] + red[buf][1][tid]) + (red[buf][2][tid] + red[buf][3][tid]);
        b.part[(t * S + slice) * NV + tid] = s;
      }
    } else {
      const float* al = b.alpha + t * (kMsarStreams * kMfAlphaRow);  // wave-uniform
      float2 z[kMsarStreams];
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) z[r] = make_float2(0.f, 0.f);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float2 x[kMsarStreams];
        streams(i, x);
#pragma unroll
        for (int r = 0; r < kMsarStreams; ++r) {
          const float w_ri = al[r * kMfAlphaRow + i];
          z[r].x = fmaf(w_ri, x[r].x, z[r].x);
          z[r].y = fmaf(w_ri, x[r].y, z[r].y);
        }
      }
      float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) {
        *reinterpret_cast<float2*>(b.zbuf + (t * kMsarStreams + r) * d + c0) = z[r];
        v[0] = fmaf(z[r].x, z[r].x, fmaf(z[r].y, z[r].y, v[0]));
        v[1] = fmaf(z[r].x, pm[r][0].x, fmaf(z[r].y, pm[r][1].x, v[1]));
        v[2] = fmaf(z[r].x, pm[r][0].y, fmaf(z[r].y, pm[r][1].y, v[2]));
        v[3] = fmaf(z[r].x, pm[r][0].z, fmaf(z[r].y, pm[r][1].z, v[3]));
        v[4] = fmaf(z[r].x, pm[r][0].w, fmaf(z[r].y, pm[r][1].w, v[4]));
      }
#pragma unroll
      for (int q = 0; q < 5; ++q) v[q] = wave_allsum(v[q]);
      if (lane < 5) {
        float mine = v[0];
#pragma unroll
        for (int q = 1; q < 5; ++q) mine = lane == q ? v[q] : mine;
        red[buf][wave][lane] = mine;
      }
      lds_barrier();
      if (tid < 5) {
        const float s = (red[buf][0][tid] + red[buf][1][tid]) + (red[buf][2][tid] + red[buf][3][tid]);
        b.part2[(t * S + slice) * kMfPart2 + tid] = s;
      }
    }
    buf ^= 1;
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
    float m = score;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    const float e = valid ? expf(score - m) : 0.f;
    float l = e;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, kWave);
    b.alpha[t * (kMsarStreams * kMfAlphaRow) + r * kMfAlphaRow + i] = e / l;
  }
}

// Per token: beta from the slices' sums, then h = sum_r beta_r Z^(r).
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
    const float* z = b.zbuf + t * kMsarStreams * d;
    for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += (int64_t)blockDim.x * 4) {
      float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < kMsarStreams; ++r) {
        const float4 zr = *reinterpret_cast<const float4*>(z + r * d + c);
        h.x = fmaf(beta[r], zr.x, h.x);
        h.y = fmaf(beta[r], zr.y, h.y);
        h.z = fmaf(beta[r], zr.z, h.z);
        h.w = fmaf(beta[r], zr.w, h.w);
      }
      *reinterpret_cast<uint2*>(out + t * d + c) = make_uint2(pack_bf2(h.x, h.y), pack_bf2(h.z, h.w));
    }
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
  b.zbuf = reinterpret_cast<float*>(p);
  return b;
}

template <int N>
hipError_t launch_n(const MsarArgs& a, hipStream_t st) {
  const MsarFastBufs b = carve(a);
  const dim3 grid((unsigned)(a.d / kMfSlice), (unsigned)((a.T + kMfRange - 1) / kMfRange));
  hipLaunchKernelGGL((k_msar_slice<N, 0>), grid, dim3(kMfB), 0, st, a, b);
  int64_t ablocks = (a.T + 3) / 4;
  if (ablocks > 8 * (int64_t)num_cus()) ablocks = 8 * (int64_t)num_cus();
  hipLaunchKernelGGL((k_msar_alpha<N>), dim3((unsigned)ablocks), dim3(256), 0, st, a, b);
  hipLaunchKernelGGL((k_msar_slice<N, 1>), grid, dim3(kMfB), 0, st, a, b);
  int64_t oblocks = a.T < 4 * (int64_t)num_cus() ? a.T : 4 * (int64_t)num_cus();
  hipLaunchKernelGGL(k_msar_out, dim3((unsigned)oblocks), dim3(256), 0, st, a, b);
  return hipGetLastError();
}

}  // namespace

size_t msar_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int dtype) {
  if (dtype != kBF16 || n_dst != 1 || n_src < 1 || n_src > kMsarFastMaxSources || T < 1 || d % kMfSlice != 0)
    return 0;
  const int64_t S = d / kMfSlice;
  return align256((size_t)(T * S * 8 * n_src) * 4) + align256((size_t)(T * kMsarStreams * kMfAlphaRow) * 4) +
         align256((size_t)(T * S * kMfPart2) * 4) + align256((size_t)(T * kMsarStreams * d) * 4);
}

bool msar_fast_ok(const MsarArgs& a) {
  const size_t need = msar_fast_workspace_bytes(a.n_src, a.n_dst, a.T, a.d, a.dtype);
  if (need == 0 || a.ws == nullptr || a.ws_bytes < need) return false;
  if (a.T > ((int64_t)1 << 30) || a.d > ((int64_t)1 << 20)) return false;
  return al16(a.src) && al16(a.out) && al16(a.w) && al16(a.conv) && al16(a.mix) && al16(a.ws);
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
