// General AttnRes kernels: any d, H, source count and dtype within the
// documented limits.  One wavefront processes one token at a time (grid-stride
// over tokens); per-source scalars live one per lane (lane i holds the value of
// source i), so a token may have at most 64 sources.  These kernels favour
// obviousness over speed: they re-read a token's sources from cache for every
// destination and head.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace attnres {
namespace {

constexpr int kGenWaves = 4;       // wavefronts per block
constexpr int kBwdTab = kBwdTable; // S*H*(N+1) table entries per wave (backward)

// Inverse RMS of sources row(0..n-1): lane i returns r_i = 1/sqrt(mean(v_i^2) + eps).
// (ai-systems-engineering explainer, learned-query section: RMS = root mean square.)
template <typename E, typename RowFn>
__device__ float inv_rms_lanes(RowFn row, int n, int d, float eps, float* max_ss = nullptr) {
  const int lane = lane_id();
  float r_lane = 0.f, mx = 0.f;
  for (int i = 0; i < n; ++i) {
    const E* v = row(i);
    float ss = 0.f;
    for (int k = lane; k < d; k += kWave) {
      const float x = ld(v + k);
      ss = fmaf(x, x, ss);
    }
    ss = wave_sum(ss);
    mx = fmaxf(mx, ss);
    if (lane == i) r_lane = 1.0f / sqrtf(ss / (float)d + eps);
  }
  if (max_ss) *max_ss = mx;
  return r_lane;
}

// One destination reading sources row(0..n-1) of one token:
//   s_i = r_i * (w * g) . v_i per head, alpha = softmax over i, out = sum alpha_i v_i
// (b-lab.team summary §1; chatpaper MHAR abstract for the per-head softmax).
// When lse != nullptr, lse[h * lse_stride] = max s + log sum exp(s - max s).
// Outputs are multiplied by out_mul before the store (a power of two for a
// scaled fp16 state, else 1).
template <typename E, typename O, typename RowFn>
__device__ void depth_read_wave(RowFn row, int n, float r_lane, int d, int H, const float* w,
                                const float* g, O* out, float* lse, int64_t lse_stride,
                                float out_mul = 1.0f) {
  const int lane = lane_id();
  const int hd = d / H;
  for (int h = 0; h < H; ++h) {
    const int c0 = h * hd, c1 = c0 + hd;
    float s_lane = -INFINITY;
    for (int i = 0; i < n; ++i) {
      const E* v = row(i);
      float acc = 0.f;
      for (int k = c0 + lane; k < c1; k += kWave) {
        const float gk = (g ? g : w)[k];  // unconditional load: no wait per channel
        const float q = g ? w[k] * gk : w[k];
        acc = fmaf(q, ld(v + k), acc);
      }
      acc = wave_sum(acc);
      const float ri = read_lane(r_lane, i);
      if (lane == i) s_lane = ri * acc;
    }
    const float m = wave_max(s_lane);
    const float e = (lane < n) ? expf(s_lane - m) : 0.f;
    const float l = wave_sum(e);
    const float a_lane = e / l;
    if (lse != nullptr && lane == 0) lse[h * lse_stride] = m + logf(l);
    // Uniform loop bounds: the cross-lane reads below must run with every lane
    // active, so the channel bound is a predicate on the loads and the store.
    for (int kb = c0; kb < c1; kb += kWave) {
      const int k = kb + lane;
      const bool in = k < c1;
      float acc = 0.f;
      for (int i = 0; i < n; ++i) {
        const float ai = read_lane(a_lane, i);
        acc = fmaf(ai, in ? ld(row(i) + k) : 0.f, acc);
      }
      if (in) st(out + k, acc * out_mul);
    }
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_full_generic(FullArgs a) {
  const E* src = static_cast<const E*>(a.src);
  E* out = static_cast<E*>(a.out);
  const int d = (int)a.d;
  const int64_t T = a.T, td = a.T * a.d;
  const int64_t wave = (int64_t)blockIdx.x * kGenWaves + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kGenWaves;
  for (int64_t t = wave; t < T; t += nw) {
    auto row = [&](int i) { return src + i * td + t * d; };
    const float r_lane = inv_rms_lanes<E>(row, (int)a.n_src, d, a.eps);
    for (int64_t j = 0; j < a.n_dst; ++j) {
      const int n = (int)(a.n_src - a.n_dst + j + 1);  // destination j reads sources 0..n-1
      const float* g = a.gain ? a.gain + j * a.gain_ld : nullptr;
      depth_read_wave<E, E>(row, n, r_lane, d, a.H, a.w + j * d, g, out + (j * T + t) * d,
                            nullptr, 0);
    }
  }
}

template <typename E, typename O0, typename OR>
__global__ __launch_bounds__(256) void k_phase1_generic(Phase1Args a) {
  const E* reps = static_cast<const E*>(a.reps);
  const int d = (int)a.d;
  const int64_t T = a.T, rs = a.rep_stride != 0 ? a.rep_stride : a.T * a.d;
  const int64_t os = a.orest_stride != 0 ? a.orest_stride : a.T * a.d;
  const int64_t wave = (int64_t)blockIdx.x * kGenWaves + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kGenWaves;
  for (int64_t t = wave; t < T; t += nw) {
    auto row = [&](int i) { return reps + i * rs + t * d; };
    float max_ss = 0.f;
    const float r_lane = inv_rms_lanes<E>(row, (int)a.N, d, a.eps, &max_ss);
    // A scaled fp16 state: |o| <= max_i ||v_i||_2 = sqrt(max_i ss_i) bounds every value.
    float inv_scale = 1.0f;
    if (a.orest_dtype == kF16) {
      const float scale = f16_state_scale(sqrtf(max_ss));
      inv_scale = 1.0f / scale;
      if (lane_id() == 0) a.oscale[t] = scale;
    }
    for (int64_t l = 0; l < a.S; ++l) {
      const float* g = a.gain ? a.gain + l * a.gain_ld : nullptr;
      float* lse = a.lse + l * a.H * T + t;
      if (l == 0)
        depth_read_wave<E, O0>(row, (int)a.N, r_lane, d, a.H, a.w, g,
                               static_cast<O0*>(a.o0) + t * d, lse, T);
      else
        depth_read_wave<E, OR>(row, (int)a.N, r_lane, d, a.H, a.w + l * d, g,
                               static_cast<OR*>(a.orest) + (l - 1) * os + t * d, lse, T, inv_scale);
    }
  }
}

// Phase 2 merge (dimensionstp Review §3-2 (4); b-lab.team summary §3 Inference).
template <typename E, typename O>
__global__ __launch_bounds__(256) void k_phase2_generic(Phase2Args a) {
  const int lane = lane_id();
  const int d = (int)a.d, hd = (int)(a.d / a.H);
  const int64_t T = a.T;
  const int64_t wave = (int64_t)blockIdx.x * kGenWaves + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kGenWaves;
  for (int64_t t = wave; t < T; t += nw) {
    const E* p = static_cast<const E*>(a.partial) + t * d;
    const O* o = static_cast<const O*>(a.o) + t * d;
    E* hout = static_cast<E*>(a.h) + t * d;
    if (a.f != nullptr) {
      // Fused update: the partial this sublayer reads is partial + f, rounded
      // once and stored; the passes below read the stored values.  Each lane
      // rereads only what it wrote, so in-place updates are consistent.
      const E* fp = static_cast<const E*>(a.f) + t * d;
      E* po = static_cast<E*>(a.partial_out) + t * d;
      for (int k = lane; k < d; k += kWave) st(po + k, (a.partial ? ld(p + k) : 0.f) + ld(fp + k));
      p = po;
    }
    float ss = 0.f;
    for (int k = lane; k < d; k += kWave) {
      const float x = ld(p + k);
      ss = fmaf(x, x, ss);
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + a.eps);
    for (int h = 0; h < a.H; ++h) {
      const int c0 = h * hd, c1 = c0 + hd;
      float acc = 0.f;
      for (int k = c0 + lane; k < c1; k += kWave) {
        const float gk = (a.gain ? a.gain : a.w)[k];  // unconditional load
        const float q = a.gain ? a.w[k] * gk : a.w[k];
        acc = fmaf(q, ld(p + k), acc);
      }
      const float s_p = r * wave_sum(acc);
      const float L = a.lse[h * T + t];
      const float m = fmaxf(L, s_p);
      const float wa = expf(L - m), wb = expf(s_p - m);
      const float inv = 1.0f / (wa + wb);
      const float ca = wa * inv * (a.o_dtype == kF16 ? a.oscale[t] : 1.0f), cb = wb * inv;
      for (int k = c0 + lane; k < c1; k += kWave)
        st(hout + k, ca * ld(o + k) + cb * ld(p + k));
    }
    if (a.h_inv_rms != nullptr) {
      // Inverse RMS of the stored h (this lane's own writes, read back).
      float sh = 0.f;
      for (int k = lane; k < d; k += kWave) {
        const float x = ld(hout + k);
        sh = fmaf(x, x, sh);
      }
      sh = wave_sum(sh);
      if (lane == 0) a.h_inv_rms[t] = 1.0f / sqrtf(sh / (float)d + a.norm_eps);
    }
  }
}

// Backward (analytic gradient of sum_j <dh_j, h_j>; see attnres.h).
// Source index i < N is rep i; i >= N is partial i - N, read only by destination
// j = i - N + 1.  Tables alpha, c, s are kept per wave in LDS, indexed
// [(j*H + h)*(N+1) + u] where u < N is a rep and u == N the partial.
template <typename E>
__global__ __launch_bounds__(256) void k_bwd_generic(BwdArgs a) {
  __shared__ float tab[kGenWaves][3][kBwdTab];
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  float* t_alpha = tab[wv][0];
  float* t_c = tab[wv][1];
  float* t_s = tab[wv][2];
  const int N = (int)a.N, S = (int)a.S, d = (int)a.d, H = a.H, hd = d / H, NS = N + 1;
  const int ns = N + S - 1;
  const int64_t T = a.T, td = a.T * a.d;
  const int64_t wave = (int64_t)blockIdx.x * kGenWaves + wv;
  const int64_t nw = (int64_t)gridDim.x * kGenWaves;
  const E* reps = static_cast<const E*>(a.reps);
  const E* parts = static_cast<const E*>(a.partials);
  const E* dh = static_cast<const E*>(a.dh);
  E* d_reps = static_cast<E*>(a.d_reps);
  E* d_parts = static_cast<E*>(a.d_partials);
  float* z = a.zslots + wave * (int64_t)S * d;
  for (int64_t k = lane; k < (int64_t)S * d; k += kWave) z[k] = 0.f;

  const float* gq = a.gain ? a.gain : a.w;  // unconditional loads in q()
  const int64_t gld = a.gain ? a.gain_ld : (int64_t)d;
  auto q = [&](int j, int k) {
    const float wq = a.w[(int64_t)j * d + k], gv = gq[j * gld + k];
    return a.gain ? wq * gv : wq;
  };
  for (int64_t t = wave; t < T; t += nw) {
    auto src = [&](int i) { return (i < N ? reps + i * td : parts + (i - N) * td) + t * d; };
    auto dsrc = [&](int i) { return (i < N ? d_reps + i * td : d_parts + (i - N) * td) + t * d; };
    const float r_lane = inv_rms_lanes<E>(src, ns, d, a.eps);

    for (int j = 0; j < S; ++j) {
      const int nj = N + (j >= 1 ? 1 : 0);
      const E* dhj = dh + j * td + t * d;
      for (int h = 0; h < H; ++h) {
        const int c0 = h * hd, c1 = c0 + hd;
        float s_lane = -INFINITY, a_lane = 0.f;
        for (int u = 0; u < nj; ++u) {
          const int i = u < N ? u : N + j - 1;
          const E* v = src(i);
          float aq = 0.f, ad = 0.f;
          for (int k = c0 + lane; k < c1; k += kWave) {
            const float x = ld(v + k);
            aq = fmaf(q(j, k), x, aq);
            ad = fmaf(ld(dhj + k), x, ad);
          }
          aq = wave_sum(aq);
          ad = wave_sum(ad);
          const float ri = read_lane(r_lane, i);
          if (lane == u) {
            s_lane = ri * aq;
            a_lane = ad;
          }
        }
        const float m = wave_max(s_lane);
        const float e = (lane < nj) ? expf(s_lane - m) : 0.f;
        const float al = e / wave_sum(e);
        const float sa = wave_sum(al * a_lane);
        if (lane < nj) {
          const int idx = (j * H + h) * NS + lane;
          t_alpha[idx] = al;
          t_c[idx] = al * (a_lane - sa);
          t_s[idx] = s_lane;
        }
      }
    }
    wave_lds_sync();

    for (int i = 0; i < ns; ++i) {
      const float ri = read_lane(r_lane, i);
      const int j0 = i < N ? 0 : i - N + 1;
      const int j1 = i < N ? S : i - N + 2;
      const int u = i < N ? i : N;
      float cs = 0.f;
      for (int j = j0; j < j1; ++j)
        for (int h = 0; h < H; ++h) {
          const int idx = (j * H + h) * NS + u;
          cs = fmaf(t_c[idx], t_s[idx], cs);
        }
      const float coef = ri * ri * cs / (float)d;
      const E* v = src(i);
      E* gout = dsrc(i);
      for (int k = lane; k < d; k += kWave) {
        const int hh = k / hd;
        float gk = 0.f;
        for (int j = j0; j < j1; ++j) {
          const int idx = (j * H + hh) * NS + u;
          gk = fmaf(t_alpha[idx], ld(dh + j * td + t * d + k), gk);
          gk = fmaf(ri * t_c[idx], q(j, k), gk);
        }
        gk = fmaf(-coef, ld(v + k), gk);
        if (a.accumulate) gk += ld(gout + k);
        st(gout + k, gk);
      }
    }

    for (int j = 0; j < S; ++j) {
      const int nj = N + (j >= 1 ? 1 : 0);
      for (int kb = 0; kb < d; kb += kWave) {  // uniform bounds around read_lane
        const int k = kb + lane;
        const bool in = k < d;
        const int hh = (in ? k : 0) / hd;
        float zz = 0.f;
        for (int u = 0; u < nj; ++u) {
          const int i = u < N ? u : N + j - 1;
          const float ri = read_lane(r_lane, i);
          if (in) zz = fmaf(t_c[(j * H + hh) * NS + u] * ri, ld(src(i) + k), zz);
        }
        if (in) z[(int64_t)j * d + k] += zz;
      }
    }
    wave_lds_sync();
  }
}

// Full AttnRes backward, one wavefront per token (any shape with
// n_dst * H * n_src <= kBwdTab).  Destination j reads sources 0 .. lim_j,
// lim_j = n_src - n_dst + j (b-lab.team summary §1).  With x_i = RMSNorm(v_i),
// r_i its inverse RMS, q_j = w_j * g_j and s = r_i q_j . v_i per head:
//   a_{j,i} = dout_j . v_i,  c_{j,i} = alpha_{j,i} (a_{j,i} - sum_m alpha_{j,m} a_{j,m})
//   dv_i = sum_{j: lim_j >= i} (alpha_{j,i} dout_j + r_i c_{j,i} q_j) - r_i^2 v_i sum_{j,h} c s / d
//   Z_j += sum_{i <= lim_j} c_{j,i} r_i v_i   (per head chunk; dw_j = g_j Z_j, dg_j = w_j Z_j)
// The pages give no backward; this is the chain rule through the forward.
template <typename E>
__global__ __launch_bounds__(256) void k_full_bwd_generic(FullBwdArgs a) {
  __shared__ float tab[kGenWaves][3][kBwdTab];
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  float* t_alpha = tab[wv][0];
  float* t_c = tab[wv][1];
  float* t_s = tab[wv][2];
  const int n_src = (int)a.n_src, n_dst = (int)a.n_dst, d = (int)a.d, H = a.H, hd = d / H;
  const int off = n_src - n_dst;  // destination j reads sources 0 .. off + j
  const int64_t T = a.T, td = a.T * a.d;
  const int64_t wave = (int64_t)blockIdx.x * kGenWaves + wv;
  const int64_t nw = (int64_t)gridDim.x * kGenWaves;
  const E* src = static_cast<const E*>(a.src);
  const E* dout = static_cast<const E*>(a.dout);
  E* d_src = static_cast<E*>(a.d_src);
  float* z = a.zslots + wave * (int64_t)n_dst * d;
  for (int64_t k = lane; k < (int64_t)n_dst * d; k += kWave) z[k] = 0.f;

  const float* gq = a.gain ? a.gain : a.w;  // unconditional loads in q()
  const int64_t gld = a.gain ? a.gain_ld : (int64_t)d;
  auto q = [&](int j, int k) {
    const float wq = a.w[(int64_t)j * d + k], gv = gq[j * gld + k];
    return a.gain ? wq * gv : wq;
  };
  for (int64_t t = wave; t < T; t += nw) {
    auto row = [&](int i) { return src + i * td + t * d; };
    const float r_lane = inv_rms_lanes<E>(row, n_src, d, a.eps);

    // alpha, c and s for every (destination, head, source) pair of this token.
    for (int j = 0; j < n_dst; ++j) {
      const int nj = off + j + 1;
      const E* dj = dout + j * td + t * d;
      for (int h = 0; h < H; ++h) {
        const int c0 = h * hd, c1 = c0 + hd;
        float s_lane = -INFINITY, a_lane = 0.f;
        for (int u = 0; u < nj; ++u) {
          const E* v = row(u);
          float aq = 0.f, ad = 0.f;
          for (int k = c0 + lane; k < c1; k += kWave) {
            const float x = ld(v + k);
            aq = fmaf(q(j, k), x, aq);
            ad = fmaf(ld(dj + k), x, ad);
          }
          aq = wave_sum(aq);
          ad = wave_sum(ad);
          const float ru = read_lane(r_lane, u);
          if (lane == u) {
            s_lane = ru * aq;
            a_lane = ad;
          }
        }
        const float m = wave_max(s_lane);
        const float e = (lane < nj) ? expf(s_lane - m) : 0.f;
        const float al = e / wave_sum(e);
        const float sa = wave_sum(al * a_lane);
        if (lane < nj) {
          const int idx = (j * H + h) * n_src + lane;
          t_alpha[idx] = al;
          t_c[idx] = al * (a_lane - sa);
          t_s[idx] = s_lane;
        }
      }
    }
    wave_lds_sync();

    // Source gradients: every destination whose prefix contains source i.
    for (int i = 0; i < n_src; ++i) {
      const float ri = read_lane(r_lane, i);
      const int j0 = i > off ? i - off : 0;
      float cs = 0.f;
      for (int j = j0; j < n_dst; ++j)
        for (int h = 0; h < H; ++h) {
          const int idx = (j * H + h) * n_src + i;
          cs = fmaf(t_c[idx], t_s[idx], cs);
        }
      const float coef = ri * ri * cs / (float)d;
      const E* v = row(i);
      E* gout = d_src + i * td + t * d;
      for (int k = lane; k < d; k += kWave) {
        const int hh = k / hd;
        float gk = 0.f;
        for (int j = j0; j < n_dst; ++j) {
          const int idx = (j * H + hh) * n_src + i;
          gk = fmaf(t_alpha[idx], ld(dout + j * td + t * d + k), gk);
          gk = fmaf(ri * t_c[idx], q(j, k), gk);
        }
        gk = fmaf(-coef, ld(v + k), gk);
        if (a.accumulate) gk += ld(gout + k);
        st(gout + k, gk);
      }
    }

    // Z_j partials for dw / dgain.
    for (int j = 0; j < n_dst; ++j) {
      const int nj = off + j + 1;
      for (int kb = 0; kb < d; kb += kWave) {  // uniform bounds around read_lane
        const int k = kb + lane;
        const bool in = k < d;
        const int hh = (in ? k : 0) / hd;
        float zz = 0.f;
        for (int u = 0; u < nj; ++u) {
          const float ru = read_lane(r_lane, u);
          if (in) zz = fmaf(t_c[(j * H + hh) * n_src + u] * ru, ld(row(u) + k), zz);
        }
        if (in) z[(int64_t)j * d + k] += zz;
      }
    }
    wave_lds_sync();
  }
}

// dw_j = g_j * Z_j, dg_j = w_j * Z_j (summed over j for a shared gain), with
// Z_j the fixed-order sum of the slot partials: slot s goes to group
// s % kRedGroups and, within it, to accumulator (s / kRedGroups) % 8; each
// group adds its eight accumulators pairwise, and the group sums are added
// pairwise in group order.  Sixteen groups of eight accumulators keep 128
// independent loads in flight per channel (a single running sum waits for
// each load in turn, and the calls with a thousand slabs were bound by that).
constexpr int kRedGroups = 16;

__device__ __forceinline__ float z_group_sum(const float* z, int64_t slots, int S, int j, int d, int k, int gi) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t stride = (int64_t)S * d;
  constexpr int kStep = 8 * kRedGroups;
  int64_t s = gi;
  for (; s + (kStep - kRedGroups) < slots; s += kStep) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += z[(s + kRedGroups * u) * stride + (int64_t)j * d + k];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (s + kRedGroups * u < slots) acc[u] += z[(s + kRedGroups * u) * stride + (int64_t)j * d + k];
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// The group sums of one channel, added pairwise in group order.
__device__ __forceinline__ float z_combine(const float (&g)[kRedGroups]) {
  float h[kRedGroups / 2];
#pragma unroll
  for (int i = 0; i < kRedGroups / 2; ++i) h[i] = g[2 * i] + g[2 * i + 1];
  float q4[kRedGroups / 4];
#pragma unroll
  for (int i = 0; i < kRedGroups / 4; ++i) q4[i] = h[2 * i] + h[2 * i + 1];
  return ((q4[0] + q4[1]) + (q4[2] + q4[3]));
}
static_assert(kRedGroups == 16, "z_combine adds 16 group sums");

// Block = kRedGroups groups of 64 lanes over 64 consecutive channels of one
// destination; group gi sums its slots, then the group sums are combined in
// a fixed order.  With one destination a shared gain's dg = w Z is written
// here too.
__global__ __launch_bounds__(64 * kRedGroups) void k_bwd_reduce(const float* z, int64_t slots, int S, int d,
                                                                const float* w, const float* gain,
                                                                int64_t gain_ld, float* dw, float* dgain,
                                                                int accumulate) {
  __shared__ float part[kRedGroups][64];
  const int lane = lane_id(), gi = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + lane;
  const int j = blockIdx.y;
  part[gi][lane] = k < d ? z_group_sum(z, slots, S, j, d, k, gi) : 0.f;
  __syncthreads();
  if (gi != 0 || k >= d) return;
  float g[kRedGroups];
#pragma unroll
  for (int i = 0; i < kRedGroups; ++i) g[i] = part[i][lane];
  const float Z = z_combine(g);
  const int64_t jk = (int64_t)j * d + k;
  const float gj = gain ? gain[j * gain_ld + k] : 1.0f;
  dw[jk] = accumulate ? dw[jk] + gj * Z : gj * Z;
  if (gain != nullptr && (gain_ld != 0 || S == 1))
    dgain[jk] = accumulate ? dgain[jk] + w[jk] * Z : w[jk] * Z;
}

// Shared gain over several destinations: dg = sum_j w_j * Z_j, summed over j
// in order (one thread per channel).
__global__ __launch_bounds__(256) void k_bwd_reduce_shared_gain(const float* z, int64_t slots,
                                                                int S, int d, const float* w,
                                                                float* dgain, int accumulate) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d) return;
  float total = 0.f;
  for (int j = 0; j < S; ++j) {
    // Same grouping and order as k_bwd_reduce, so Z matches it bit for bit.
    float g[kRedGroups];
    for (int gi = 0; gi < kRedGroups; ++gi) g[gi] = z_group_sum(z, slots, S, j, d, k, gi);
    total = fmaf(w[(int64_t)j * d + k], z_combine(g), total);
  }
  dgain[k] = accumulate ? dgain[k] + total : total;
}

int64_t gen_blocks(int64_t T) {
  int64_t b = (T + kGenWaves - 1) / kGenWaves;
  const int64_t cap = 8 * (int64_t)num_cus();
  return b < 1 ? 1 : (b > cap ? cap : b);
}

}  // namespace

hipError_t launch_full_generic(const FullArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)gen_blocks(a.T)), block(kGenWaves * kWave);
  if (a.dtype == kF32)
    hipLaunchKernelGGL(k_full_generic<float>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(k_full_generic<bf16_t>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_phase1_generic(const Phase1Args& a, hipStream_t st) {
  const dim3 grid((unsigned)gen_blocks(a.T)), block(kGenWaves * kWave);
  if (a.dtype == kF32) {
    hipLaunchKernelGGL((k_phase1_generic<float, float, float>), grid, block, 0, st, a);
  } else if (a.o0_dtype == kBF16 && a.orest_dtype == kF32) {
    hipLaunchKernelGGL((k_phase1_generic<bf16_t, bf16_t, float>), grid, block, 0, st, a);
  } else if (a.o0_dtype == kBF16 && a.orest_dtype == kF16) {
    hipLaunchKernelGGL((k_phase1_generic<bf16_t, bf16_t, f16_t>), grid, block, 0, st, a);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_phase2_generic(const Phase2Args& a, hipStream_t st) {
  const dim3 grid((unsigned)gen_blocks(a.T)), block(kGenWaves * kWave);
  if (a.dtype == kF32)
    hipLaunchKernelGGL((k_phase2_generic<float, float>), grid, block, 0, st, a);
  else if (a.o_dtype == kF32)
    hipLaunchKernelGGL((k_phase2_generic<bf16_t, float>), grid, block, 0, st, a);
  else if (a.o_dtype == kF16)
    hipLaunchKernelGGL((k_phase2_generic<bf16_t, f16_t>), grid, block, 0, st, a);
  else
    return hipErrorNotSupported;  // a bf16 state is refused before any launch
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const BwdArgs& a, hipStream_t st) {
  if (a.slots % kGenWaves != 0 || a.slots < kGenWaves) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.slots / kGenWaves)), block(kGenWaves * kWave);
  if (a.dtype == kF32)
    hipLaunchKernelGGL(k_bwd_generic<float>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(k_bwd_generic<bf16_t>, grid, block, 0, st, a);
  return hipGetLastError();
}

// Z slots [slots_used, rows, d] -> dw [rows, d] and dgain (rows or shared).
static hipError_t launch_z_reduce(const float* z, int64_t slots_used, int rows, int d, const float* w,
                                  const float* gain, int64_t gain_ld, float* dw, float* dgain,
                                  int accumulate, hipStream_t st) {
  const bool shared = gain != nullptr && gain_ld == 0;
  hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((d + 63) / 64), (unsigned)rows), dim3(64 * kRedGroups), 0, st, z,
                     slots_used, rows, d, w, gain, gain_ld, dw, dgain, accumulate);
  if (shared && rows > 1)
    hipLaunchKernelGGL(k_bwd_reduce_shared_gain, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, st, z,
                       slots_used, rows, d, w, dgain, accumulate);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdArgs& a, int64_t slots_used, hipStream_t st) {
  return launch_z_reduce(a.zslots, slots_used, (int)a.S, (int)a.d, a.w, a.gain, a.gain_ld, a.dw, a.dgain,
                         a.accumulate, st);
}

hipError_t launch_full_bwd_generic(const FullBwdArgs& a, hipStream_t st) {
  if (a.slots % kGenWaves != 0 || a.slots < kGenWaves) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.slots / kGenWaves)), block(kGenWaves * kWave);
  if (a.dtype == kF32)
    hipLaunchKernelGGL(k_full_bwd_generic<float>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(k_full_bwd_generic<bf16_t>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_full_bwd_reduce(const FullBwdArgs& a, const float* slabs, int64_t n_slabs, hipStream_t st) {
  return launch_z_reduce(slabs, n_slabs, (int)a.n_dst, (int)a.d, a.w, a.gain, a.gain_ld, a.dw, a.dgain,
                         a.accumulate, st);
}

}  // namespace attnres
