// Block AttnRes Phase 2 for gfx950 (bf16 I/O, fp32 arithmetic): the
// online-softmax merge of the intra-block partial sum into Phase 1's state
// (dimensionstp "Attention Residuals Review" §3-2 (4); b-lab.team summary §3,
// Inference), plain or fused with the partial-sum update.  One wavefront per
// token; lane owns CPL chunks of 8 channels at (c*64 + lane)*8; the sum of
// squares and the per-head dots reduce inside the wave, then each element is
// merged.  (Phase 1 is in p1_kernel.hpp.)
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

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

template <typename O> __device__ __forceinline__ void store8(O* p, const float (&x)[8]);
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&x)[8]) {
  uint4 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  u.z = pack_bf2(x[4], x[5]);
  u.w = pack_bf2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
// Compile-time tuning knobs.  The defaults are the fastest combination measured on
// MI355X for the d=4096 block (bf16 I/O, scaled fp16 state):
//   ATTNRES_P2_PREFETCH  issue the next token's partial and state loads before
//                        merging the current token
//   ATTNRES_P2_QLDS      q in LDS instead of registers
//   ATTNRES_P2_NT        nontemporal loads of the streamed-once inputs
//   ATTNRES_P2_MINWAVES  minimum waves per SIMD the register allocation must
//                        leave room for
#ifndef ATTNRES_P2_PREFETCH
#define ATTNRES_P2_PREFETCH 0
#endif
#ifndef ATTNRES_P2_QLDS
#define ATTNRES_P2_QLDS 1
#endif
#ifndef ATTNRES_P2_NT
#define ATTNRES_P2_NT 1
#endif
#ifndef ATTNRES_P2_MINWAVES
#define ATTNRES_P2_MINWAVES 2
#endif
constexpr bool kP2Nt = ATTNRES_P2_NT != 0;
constexpr bool kP2Prefetch = ATTNRES_P2_PREFETCH != 0;
constexpr bool kP2QLds = ATTNRES_P2_QLDS != 0;

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
  // The token's Phase 1 lse (per chunk's head) and state scale, loaded with
  // its rows: read where they are used, they would add a memory round trip
  // after the dot products.
  float lse_t[MH ? CPL : 1], osc_t = 1.0f;
  auto load_s = [&](int64_t tt) {
#pragma unroll
    for (int c = 0; c < (MH ? CPL : 1); ++c) lse_t[c] = a.lse[(int64_t)(MH ? c / segs_per_head : 0) * T + tt];
    if constexpr (__is_same(OT, f16_t)) osc_t = a.oscale[tt];
  };
  // q = w * g, one copy per workgroup in LDS (every wave uses the same lane ->
  // channel map).  Its loads go out first, unconditionally (w again when there
  // is no gain), and the first token's after them: the in-order load counter
  // then lets the fold finish while the token's loads are still in flight,
  // which is most of a call's time when T is small.  256 threads cover the
  // d / 4 = 128 CPL float4 of q in CPL / 2 each.
  constexpr int FQ = kP2QLds ? CPL / 2 : 1;
  float4 wq[FQ], gq[FQ];
  const bool has_gain = a.gain != nullptr;
  if constexpr (kP2QLds) {
    const float4* w4 = reinterpret_cast<const float4*>(a.w);
    const float4* g4 = reinterpret_cast<const float4*>(has_gain ? a.gain : a.w);
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      wq[j] = w4[threadIdx.x + j * 256];
      gq[j] = g4[threadIdx.x + j * 256];
    }
    keep_memory_order();  // the token's loads below go out after these
  }
  {
    // Unconditional (a wave past the last token loads that token's rows and
    // never uses them): a branch here would make the fold below wait for
    // these loads too.
    const int64_t t0 = t < T ? t : T - 1;
    load_p2<CPL, OT>(p, o, part, oin, t0, d, lane);
    load_f(t0);
    load_s(t0);
  }
  __shared__ float4 qs[kP2QLds ? CPL * 64 * 2 : 1];
  float qreg[QR][8];
  if constexpr (kP2QLds) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      float4 q = wq[j];
      q.x *= has_gain ? gq[j].x : 1.0f;
      q.y *= has_gain ? gq[j].y : 1.0f;
      q.z *= has_gain ? gq[j].z : 1.0f;
      q.w *= has_gain ? gq[j].w : 1.0f;
      qs[threadIdx.x + j * 256] = q;
    }
    lds_barrier();  // orders the LDS copy only: the token's loads stay in flight
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = (c * 64 + lane) * 8 + e;
        qreg[kP2QLds ? 0 : c][e] = a.gain ? a.w[col] * a.gain[col] : a.w[col];
      }
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
    const float oscale = osc_t;
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
      const float L = lse_t[MH ? c : 0];
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
      if (tn < T) load_s(tn);
    } else {
      if (tn < T) {
        load_p2<CPL, OT>(p, o, part, oin, tn, d, lane);
        load_f(tn);
        load_s(tn);
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
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
    return hipErrorNotSupported;  // a bf16 state is refused before any launch
  };
  if (a.f == nullptr) return by_state(std::integral_constant<int, 0>());
  if (a.partial != nullptr) return by_state(std::integral_constant<int, 1>());
  return by_state(std::integral_constant<int, 2>());
}

bool heads_fit_segments(int64_t d, int H) { return (d / H) % 512 == 0; }

// The specialised kernels use 16-byte vector loads and stores.
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

}  // namespace

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
