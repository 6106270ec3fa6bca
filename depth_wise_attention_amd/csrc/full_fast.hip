// Specialised Full AttnRes forward for gfx950 (bf16 I/O, H = 1, up to 32
// sources and destinations).
//
// Per token the routing is a dense contraction: scores S[j][i] = q_j . v_i over
// d channels for up to 32 x 32 (destination, source) pairs (b-lab.team summary
// §1: O(L^2 d) per token).  That part runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 with A = q (split into bf16 hi + lo parts, so the
// product carries about 16 significant bits of q) and B = the token's sources,
// read straight from HBM in the MFMA operand layout.  The same source registers
// also give G = V V^T, whose diagonal is each source's sum of squares.
//
// A workgroup of 4 waves owns one token at a time; wave w covers channels
// [w d/4, (w+1) d/4).  The four partial S tiles and diag(G) are summed through
// LDS, the causal softmax runs 8 threads per destination (4 sources each), and
// alpha^T goes to LDS.  The weighted sums h_j = sum_i alpha_ji v_i then run on
// the vector ALUs, one thread per 8 channels and 8 destinations at a time,
// reading the sources a second time (from cache) channel-contiguously.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace attnres {
namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef float f16acc __attribute__((ext_vector_type(16)));

constexpr int kFW = 4;          // waves per workgroup
constexpr int kFB = kFW * 64;   // threads per workgroup
constexpr int kTile = 32;       // MFMA tile: 32 destinations x 32 sources

__device__ __forceinline__ bf8v as_bf8(uint4 u) { return __builtin_bit_cast(bf8v, u); }

// q = w * g split into bf16 hi + lo parts, rows padded to 32 with zeros:
// qhi/qlo [32][d].
__global__ __launch_bounds__(256) void k_full_qsplit(FullArgs a, bf16_t* qhi, bf16_t* qlo) {
  const int64_t n = (int64_t)kTile * a.d;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = x / a.d, k = x % a.d;
    float q = 0.f;
    if (j < a.n_dst) {
      q = a.w[j * a.d + k];
      if (a.gain) q *= a.gain[j * a.gain_ld + k];
    }
    const bf16_t h = f2bf(q);
    qhi[x] = h;
    qlo[x] = f2bf(q - bf2f(h));
  }
}

__global__ __launch_bounds__(kFB, 2) void k_full_fast(FullArgs a, const bf16_t* qhi, const bf16_t* qlo) {
  __shared__ float sred[kFW][kTile * kTile];          // per-wave partial S
  __shared__ float gred[kFW][kTile];                   // per-wave partial diag(G)
  __shared__ __align__(16) float alphaT[kTile][kTile];  // alpha^T[i][j]
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T, Td = a.T * a.d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const int kw = d / kFW;             // channels per wave (multiple of 64)
  const int row = lane % 32;          // MFMA row (destination j for A, source i for B)
  const int kofs = 8 * (lane / 32);   // 8-channel half of each 16-channel step
  const bool src_ok = row < n_src;

  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    // ---------------- stage 1: S = Q V^T and G = V V^T over this wave's channels
    // Operands for step k0 + 64 are loaded while step k0 runs on the matrix cores.
    f16acc S = {}, G = {};
    const bf16_t* vrow = src + ((int64_t)(src_ok ? row : 0) * T + t) * d + wave * kw + kofs;
    const bf16_t* qh = qhi + (int64_t)row * d + wave * kw + kofs;
    const bf16_t* ql = qlo + (int64_t)row * d + wave * kw + kofs;
    uint4 vb[4], ah[4], al[4];
    auto load_step = [&](int k0, uint4* v, uint4* h, uint4* l) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = src_ok ? *reinterpret_cast<const uint4*>(vrow + k0 + 16 * u) : make_uint4(0, 0, 0, 0);
        h[u] = *reinterpret_cast<const uint4*>(qh + k0 + 16 * u);
        l[u] = *reinterpret_cast<const uint4*>(ql + k0 + 16 * u);
      }
    };
    load_step(0, vb, ah, al);
    for (int k0 = 0; k0 < kw; k0 += 64) {
      uint4 vn[4], hn[4], ln[4];
      if (k0 + 64 < kw) load_step(k0 + 64, vn, hn, ln);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(ah[u]), as_bf8(vb[u]), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(al[u]), as_bf8(vb[u]), S, 0, 0, 0);
        G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(vb[u]), as_bf8(vb[u]), G, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vb[u] = vn[u];
        ah[u] = hn[u];
        al[u] = ln[u];
      }
    }
    // D layout: element r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      sred[wave][m * kTile + row] = S[r];
      if (m == row) gred[wave][row] = G[r];
    }
    __syncthreads();

    // ---------------- softmax: thread -> destination j = tid / 8, sources 4*(tid % 8) .. +4
    {
      const int j = tid / 8, i0 = 4 * (tid % 8);
      const int lim = n_src - n_dst + j;  // destination j reads sources 0..lim
      float s[4];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q;
        float sv = 0.f, gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kFW; ++w2) {
          sv += sred[w2][j * kTile + i];
          gv += gred[w2][i];
        }
        const float r = 1.0f / sqrtf(gv / (float)d + a.eps);
        s[q] = (j < n_dst && i <= lim) ? r * sv : -INFINITY;
        m = fmaxf(m, s[q]);
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
      float e[4], l = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[q] = (s[q] == -INFINITY) ? 0.f : expf(s[q] - m);
        l += e[q];
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) l += __shfl_xor(l, off, kWave);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) alphaT[i0 + q][j] = e[q] * inv;
    }
    __syncthreads();

    // ---------------- stage 2: h_j = sum_i alpha_ji v_i, 4 channels per thread.
    // All source rows of the thread's channels are loaded first (one pass over
    // the sources), then destinations are produced 8 at a time from registers.
    // Row bases are wave-uniform; the per-thread offset t*d + col fits 32 bits.
    for (int col = tid * 4; col < d; col += kFB * 4) {
      const uint32_t voff = (uint32_t)t * (uint32_t)d + (uint32_t)col;
      uint2 vv[kTile];
      int64_t step = Td;
      asm volatile("" : "+s"(step));  // keeps 32 row offsets from being precomputed and held
      const bf16_t* rp = src + voff;
#pragma unroll
      for (int i = 0; i < kTile; ++i) {
        vv[i] = i < n_src ? *reinterpret_cast<const uint2*>(rp) : make_uint2(0, 0);
        rp += step;
      }
      for (int jb = 0; jb < n_dst; jb += 8) {
        const int i_end = min(n_src, n_src - n_dst + jb + 8);  // sources any of j in [jb, jb+8) reads
        // Keep the rows packed: without this the unpacked fp32 copies of all
        // rows are hoisted out of the jb loop (twice the registers).
#pragma unroll
        for (int i = 0; i < kTile; ++i) asm volatile("" : "+v"(vv[i].x), "+v"(vv[i].y));
        float acc[8][4];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[jj][e] = 0.f;
#pragma unroll
        for (int i = 0; i < kTile; ++i) {
          if (i < i_end) {
            const float x[4] = {bf_lo(vv[i].x), bf_hi(vv[i].x), bf_lo(vv[i].y), bf_hi(vv[i].y)};
            const float4 a0 = *reinterpret_cast<const float4*>(&alphaT[i][jb]);
            const float4 a1 = *reinterpret_cast<const float4*>(&alphaT[i][jb + 4]);
            const float al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[jj][e] = fmaf(al[jj], x[e], acc[jj][e]);
          }
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = jb + jj;
          if (j < n_dst) {
            uint2 o;
            o.x = pack_bf2(acc[jj][0], acc[jj][1]);
            o.y = pack_bf2(acc[jj][2], acc[jj][3]);
            *reinterpret_cast<uint2*>(out + (int64_t)j * Td + voff) = o;
          }
        }
      }
    }
    // No barrier needed here: the next token writes sred/gred only after every
    // thread passed this token's second barrier (all softmax reads done), and
    // alphaT only after its own first barrier (all stage-2 reads done).
  }
}

bool al16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

}  // namespace

size_t full_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t d, int H, int dtype) {
  if (dtype != kBF16 || H != 1 || n_src > kTile || n_dst > n_src) return 0;
  return (size_t)2 * kTile * (size_t)d * sizeof(bf16_t);
}

bool full_fast_ok(const FullArgs& a) {
  if (a.dtype != kBF16 || a.H != 1 || a.T < 1) return false;
  if (a.n_src > kTile || a.n_dst > a.n_src) return false;
  // Stage 1 steps 64 channels per wave; stage 2 moves 4 channels per thread
  // and addresses a source row with a 32-bit offset.
  if (a.d % (kFW * 64) != 0 || a.d > ((int64_t)1 << 16)) return false;
  if (a.T > (((int64_t)1 << 31) - 1) / a.d) return false;
  const size_t need = full_fast_workspace_bytes(a.n_src, a.n_dst, a.d, a.H, a.dtype);
  if (a.ws == nullptr || a.ws_bytes < need) return false;
  return al16(a.src) && al16(a.out) && al16(a.ws);
}

hipError_t launch_full_fast(const FullArgs& a, hipStream_t st) {
  bf16_t* qhi = static_cast<bf16_t*>(a.ws);
  bf16_t* qlo = qhi + (size_t)kTile * a.d;
  hipLaunchKernelGGL(k_full_qsplit, dim3(64), dim3(256), 0, st, a, qhi, qlo);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_full_fast, kFB, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL(k_full_fast, dim3((unsigned)grid), dim3(kFB), 0, st, a, (const bf16_t*)qhi,
                     (const bf16_t*)qlo);
  return hipGetLastError();
}

}  // namespace attnres
