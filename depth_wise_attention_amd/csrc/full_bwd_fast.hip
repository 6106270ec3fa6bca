// Specialised Full AttnRes backward for gfx950 (bf16 I/O, up to 32 sources
// and destinations): the register-resident kernel (d = 1024 .. 2048 in steps
// of 256, one head or H = 2, 4, 8), the query packing and the Z kernel shared
// with the staged kernel of full_bwd_wide.hip (one head, d a multiple of 512,
// one or two 32-source tiles), and the dispatch between them.
//
// The pages give no backward; these kernels evaluate the chain rule through
// the Full forward (b-lab.team summary §1) for L = sum_j <dout_j, out_j>.  Per
// token, with x_i = RMSNorm(v_i), r_i its inverse RMS, q_j = w_j * g_j and
// destination j reading sources 0 .. lim_j:
//   s_ji = r_i q_j . v_i,  a_ji = dout_j . v_i,  alpha_j = softmax_i(s_j)
//   c_ji = alpha_ji (a_ji - sum_m alpha_jm a_jm)
//   dv_i = sum_j alpha_ji dout_j + r_i sum_j c_ji q_j - (r_i^2 / d) (sum_j c_ji s_ji) v_i
//   Z_j  = sum over tokens of sum_i (r_i c_ji) v_i,  dw_j = g_j Z_j,  dg_j = w_j Z_j
// Every contraction runs on the matrix cores (v_mfma_f32_32x32x16_bf16):
//   stage 1  S = Q V^T (q split into bf16 high + low parts), G = V V^T (its
//            diagonal gives the sums of squares), A = dOut V^T;
//   stage 2  dV^T = dOut^T alpha^T + Q^T (r c)^T - V^T diag(coef): the source
//            and upstream-gradient tiles are transposed by an MFMA against the
//            identity (exact), alpha, r c and coef are split into bf16 high +
//            low parts, and Q^T is packed once per call in operand order;
//   Z        a second kernel forms (r c) V per token and sums it over token
//            groups into fixed slabs, summed in order by the shared reduction.
// The resident kernel keeps each token's sources and dout in registers
// through both stages; the staged kernel streams 64-channel chunks through LDS
// and reads them again in the second stage (from cache).
#include <math.h>

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"
#include "mfma_tiles.hpp"

namespace attnres {
namespace {

constexpr int kBW = 4;            // waves per workgroup of the staged kernel
constexpr int kZGroups = 64;      // token groups of the Z kernel (slabs)

// Channel position (0..31 within a 32-channel block) that row m of a
// transposed tile holds when the transpose multiplies by the permuted
// identity of res_ident (below); the identity is res_ident's without PERM.
__host__ __device__ constexpr int res_pos(int m) { return 16 * ((m & 7) >> 2) + 4 * (m >> 3) + (m & 3); }

// Q^T in A-operand order with the destination index inside the lane: for
// 32-channel tile c, k-step b and part p (0 = bf16 high, 1 = low), lane (h, n)
// holds q_p[transposed_row(b, h, e)][32 c + pos(n)], e = 0..7, at
// qt[((c * 2 + b) * 2 + p) * 64 + lane], with pos(n) = n, or res_pos(n) for
// the register-resident kernel's permuted transposes (PERM).  Rows past n_dst
// are zero.
template <bool PERM>
__global__ __launch_bounds__(256) void k_full_qtsplit(FullBwdArgs a, uint4* qt) {
  const int64_t units = a.d / 32 * 2 * 64;  // (tile, b, lane)
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < units;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(x % 64), h = lane >> 5, n = lane & 31;
    const int b = (int)((x / 64) % 2);
    const int64_t c = x / 128;
    const int64_t k = 32 * c + (PERM ? res_pos(n) : n);
    // Unconditional loads (rows past n_dst read row n_dst - 1, then store zero)
    // so the 16 loads are in flight together.
    const bool has_g = a.gain != nullptr;
    const float* gsrc = has_g ? a.gain : a.w;
    const int64_t gld = has_g ? a.gain_ld : a.d;
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = transposed_row(b, h, e);
      const int jc = j < a.n_dst ? j : (int)a.n_dst - 1;
      const float wv = a.w[jc * a.d + k], gv = gsrc[jc * gld + k];
      const float q = j < a.n_dst ? (has_g ? wv * gv : wv) : 0.f;
      hi[e] = bf2f(f2bf(q));
      lo[e] = q - hi[e];
    }
    qt[((c * 2 + b) * 2 + 0) * 64 + lane] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
    qt[((c * 2 + b) * 2 + 1) * 64 + lane] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
  }
}

// q = w * g in the A-operand order of the forward's score contraction (same
// layout as the forward's split query).
__global__ __launch_bounds__(256) void k_full_bwd_qsplit(FullBwdArgs a, uint4* qpk) {
  const int64_t units = a.d / kChunk * 4 * 64;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < units;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(x % 64);
    const int64_t gs = x / 64;
    const int j = lane % 32;
    const int64_t k0 = gs * 16 + 8 * (lane / 32);
    const bool has_g = a.gain != nullptr;
    const int jc = j < a.n_dst ? j : (int)a.n_dst - 1;
    float q[8], hi[8], lo[8];
    if (has_g)
      fold_q8<true>(a.w + jc * a.d + k0, a.gain + jc * a.gain_ld + k0, q);
    else
      fold_q8<false>(a.w + jc * a.d + k0, nullptr, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qe = j < a.n_dst ? q[e] : 0.f;
      hi[e] = bf2f(f2bf(qe));
      lo[e] = qe - hi[e];
    }
    qpk[gs * 2 * 64 + lane] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
    qpk[gs * 2 * 64 + 64 + lane] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
  }
}

// Z_j = sum over tokens of sum_i (r_i c_ji) v_i for one 64-channel tile and one
// token group: one wave, D[j][c'] = (r c)[j][i] V[i][c'] with (r c) split hi + lo
// as the A operand and the identity-transposed source tile as B.  The group's
// sum goes to slab grp ([groups, n_dst, d] fp32).
__global__ __launch_bounds__(64) void k_full_bwd_z(FullBwdArgs a, const float* cws, float* zs, int groups) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kTile * kVRow];
  const int lane = lane_id(), h = lane >> 5, n = lane & 31;
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T;
  // The token group is the fast grid index: workgroups go to the XCDs round
  // robin, so every channel tile of a group runs on one XCD and that L2 holds
  // the group's (r c) rows once (each wave reads the whole row of its token).
  const int grp = blockIdx.x;
  const int ch0 = blockIdx.y * kChunk;
  const int zhead = ch0 / (d / a.H);  // the head of this tile's channels (r c is per head)
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const uint4 ident0 = ident_operand(0), ident1 = ident_operand(1);
  uint32_t vmask[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) vmask[u] = 8 * u + (lane >> 3) < n_src ? 0xFFFFFFFFu : 0u;
  f16acc Z0 = {}, Z1 = {};
  // One token ahead: the next token's source rows and (r c) row are loaded
  // while this token's products run (the last token reloads itself, so every
  // iteration has the same loads outstanding).
  auto load_token = [&](int64_t t, uint4 (&v)[4], float4 (&x)[4]) {
    const bf16_t* vrow[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 8 * u + (lane >> 3);
      vrow[u] = src + ((int64_t)(r < n_src ? r : 0) * T + t) * d + ch0;
    }
    load_chunk(vrow, 0, v);
    // A operands: lane (h, j = n) holds (r c)[j][transposed_row(b, h, e)].
    const float* cj = cws + (t * a.H + zhead) * (kTile * kTile) + n * kTile + 4 * h;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      x[2 * b] = *reinterpret_cast<const float4*>(cj + 16 * b);
      x[2 * b + 1] = *reinterpret_cast<const float4*>(cj + 16 * b + 8);
    }
  };
  uint4 v[4];
  float4 x[4];
  if (grp < T) load_token(grp, v, x);
  for (int64_t t = grp; t < T; t += groups) {
    uint4 cA[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float xs[8] = {x[2 * b].x, x[2 * b].y, x[2 * b].z, x[2 * b].w,
                           x[2 * b + 1].x, x[2 * b + 1].y, x[2 * b + 1].z, x[2 * b + 1].w};
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = bf2f(f2bf(xs[e]));
        lo[e] = xs[e] - hi[e];
      }
      cA[b][0] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
      cA[b][1] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
    }
    wave_lds_sync();
    stage_chunk(tile, v, vmask);
    const int64_t tn = t + groups < T ? t + groups : t;
    load_token(tn, v, x);
    wave_lds_sync();
    uint4 op[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) op[s] = tile_operand(tile, s);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f16acc D1 = {};
      D1 = mfma(op[2 * half], ident0, D1);
      D1 = mfma(op[2 * half + 1], ident1, D1);
      const uint4 tv0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
      const uint4 tv1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
      f16acc& Z = half ? Z1 : Z0;
      Z = mfma(cA[0][0], tv0, Z);
      Z = mfma(cA[0][1], tv0, Z);
      Z = mfma(cA[1][0], tv1, Z);
      Z = mfma(cA[1][1], tv1, Z);
    }
  }
  // Z[j][c']: element r of lane (h, c' = n) is destination 8 (r/4) + 4 h + r%4.
  float* slab = zs + (int64_t)grp * n_dst * d;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f16acc& Z = half ? Z1 : Z0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 8 * (r / 4) + 4 * h + (r % 4);
      if (j < n_dst) slab[(int64_t)j * d + ch0 + 32 * half + n] = Z[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Register-resident variant (d = 1024 .. 2048 in steps of 256): a workgroup of
// d / 256 waves owns one token at a time, wave w channels 256 w .. 256 w + 255.
// Lane (h, r) holds, for each of the wave's 16 k-steps s, channels
// 256 w + 16 s + 8 h .. + 7 of source row r and of upstream-gradient row r in
// registers: exactly the stage-1 B operand of V^T and A operand of dOut.  Stage
// 1 runs from them, and stage 2 transposes them from the same registers, so
// each byte of the sources and of dout crosses HBM once.  After stage 2 the
// registers are refilled with the next token's rows.
//
// Stage 2 transposes with a permuted identity: row m of a transposed tile is
// channel position res_pos(m) of its block, so that the 16 accumulator rows of
// lane (h, i), m = 8 (r / 4) + 4 h + r % 4, are the 16 consecutive channels
// 16 h .. 16 h + 15 of the block, and dV leaves the accumulators as two
// 16-byte stores per lane.

constexpr int kRK = 16;            // k-steps per wave
constexpr int kRCh = 16 * kRK;     // channels per wave

// res_ident(a2): the B operand of k-step a2 of the permuted transpose,
// I[k][n] = 1 when n is the row that holds channel position 16 a2 + k, i.e.
// res_pos(n) == 16 a2 + k.
__device__ __forceinline__ uint4 res_ident(int a2) {
  const int lane = lane_id(), hb = lane >> 5, n = lane & 31;
  const int p = res_pos(n) - 16 * a2 - 8 * hb;  // element holding the one, if in 0..7
  uint32_t wds[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo16 = p == 2 * q ? 0x3F80u : 0u;
    const uint32_t hi16 = p == 2 * q + 1 ? 0x3F80u : 0u;
    wds[q] = lo16 | (hi16 << 16);
  }
  return make_uint4(wds[0], wds[1], wds[2], wds[3]);
}

// LDS of the resident kernel for W waves: per-wave partials of S and A
// (32 x 32 each) and of the sums of squares, then the per-token tables.
struct ResLds {
  int W;
  __device__ float* sred(char* base, int w) const { return reinterpret_cast<float*>(base) + w * kTile * kTile; }
  __device__ float* ared(char* base, int w) const {
    return reinterpret_cast<float*>(base) + (W + w) * kTile * kTile;
  }
  // The whole 32 x 32 partial of G = V V^T (its diagonal holds the sums of squares).
  __device__ float* gred(char* base, int w) const {
    return reinterpret_cast<float*>(base) + (2 * W + w) * kTile * kTile;
  }
  __device__ float* table(char* base, int k) const {  // alpha (0), r c (1), c s (2): [32][kARow]
    return reinterpret_cast<float*>(base) + 3 * W * kTile * kTile + k * kTile * kARow;
  }
  static size_t bytes(int W) { return (size_t)4 * (3 * W * kTile * kTile + 3 * kTile * kARow + kTile); }
};

// LDS of the resident kernel with H heads (MH): per wave a V tile (staging,
// then the S partial, then the dV output tile) and a dout tile (staging, then
// the A partial), the diagonal of each wave's G partial, each head's stage-2
// operands (alpha and r c, 8 x 64 uint4), the diag(-coef) operands shared by
// the heads (4 x 64 uint4) and each head's partial coef sums.
struct ResLdsMH {
  int W, H;
  __device__ float* tile_v(char* base, int w) const { return reinterpret_cast<float*>(base) + w * kTile * kTile; }
  __device__ float* tile_d(char* base, int w) const {
    return reinterpret_cast<float*>(base) + (W + w) * kTile * kTile;
  }
  __device__ float* gdiag(char* base, int w) const {
    return reinterpret_cast<float*>(base) + 2 * W * kTile * kTile + w * kTile;
  }
  __device__ uint4* bpk(char* base, int hh) const {
    return reinterpret_cast<uint4*>(gdiag(base, W)) + hh * 8 * 64;
  }
  __device__ uint4* cdiag(char* base) const { return bpk(base, H); }
  __device__ float* cpart(char* base, int hh) const {
    return reinterpret_cast<float*>(cdiag(base) + 4 * 64) + hh * kTile;
  }
  static size_t bytes(int W, int H) {
    return (size_t)4 * (2 * W * kTile * kTile + W * kTile) + (size_t)16 * 64 * (8 * H + 4) + (size_t)4 * H * kTile;
  }
};

// 16-byte load at byte voff + soff of a buffer whose base is uniform over the
// wave: the base and the (constant) soff live in scalar registers.
__device__ __forceinline__ uint4 res_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t res_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferWord3);
}

// MH: H = 2, 4 or 8 heads of whole waves (W / H waves each, d / H channels),
// each with its own depth softmax (MHAR abstract); the RMS and its term in dv
// stay over the whole d.  The first wave of each head sums the head's S and A
// partials and forms alpha, c, r c and c s in registers: its accumulators
// already hold one source per lane and the destinations in stage 2's operand
// order, so the operands are written as they are.  r c goes to the Z kernel
// per head ([T][H][32][32]).
template <bool ACC, bool MH>
__global__ __launch_bounds__(512, 1) void k_full_bwd_res(FullBwdArgs a, const uint4* qpk, const uint4* qt,
                                                          float* cws) {
  extern __shared__ __attribute__((aligned(16))) char res_smem[];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: the wave's buffer bases stay scalar
  const int W = (int)blockDim.x >> 6;
  const ResLds L{W};
  const ResLdsMH M{W, MH ? a.H : 1};
  const int gw = MH ? W / a.H : W;        // waves per head
  const int head = MH ? wave / gw : 0;
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const bf16_t* dout = static_cast<const bf16_t*>(a.dout);
  bf16_t* dsrc = static_cast<bf16_t*>(a.d_src);
  const int ch0 = wave * kRCh;
  const int h = lane >> 5, n = lane & 31;
  // Whole-row loads: instruction u of lane l reads 16-byte piece l % 8 of
  // row 8 u + l / 8 of a 64-channel chunk (8 rows x 128 bytes per
  // instruction).  Rows past n_src (n_dst) repeat the last real row; the
  // tables give them zero weight and their gradients are not stored.  The
  // token's rows start at a scalar base (src + t d); the per-lane byte offsets
  // below fit 32 bits (checked when the kernel is chosen).
  // Row 8 u + l / 8 is at voff0 + u * row8 bytes, or at the clamped row's
  // offset when past the last real row.
  const int r0 = lane >> 3;
  const int64_t cbase = ch0 + 8 * (lane & 7);
  const uint32_t row8 = (uint32_t)(8 * T * d * 2);
  const uint32_t voff0 = (uint32_t)(((int64_t)r0 * T * d + cbase) * 2);
  const uint32_t vclamp = (uint32_t)(((int64_t)(n_src - 1) * T * d + cbase) * 2);
  const uint32_t dclamp = (uint32_t)(((int64_t)(n_dst - 1) * T * d + cbase) * 2);
  // Recomputed at each use from an opaque copy of the base, so that the
  // compiler does not keep all eight offsets live (and spill them) across the
  // token loop.
  auto voff = [&](int u) {
    uint32_t b = voff0;
    asm volatile("" : "+v"(b));
    return 8 * u + r0 < n_src ? b + (uint32_t)u * row8 : vclamp;
  };
  auto doff = [&](int u) {
    uint32_t b = voff0;
    asm volatile("" : "+v"(b));
    return 8 * u + r0 < n_dst ? b + (uint32_t)u * row8 : dclamp;
  };
  // Query operands of this wave's k-steps and 32-channel blocks: k-step s at
  // byte 2048 s (+ 1024 for the low part), block b2 at 4096 b2 (+ 1024 per
  // operand), lane at 16 lane.
  const __amdgpu_buffer_rsrc_t qrs = res_rsrc(qpk + (int64_t)(ch0 / 16) * 2 * 64);
  const __amdgpu_buffer_rsrc_t qtrs = res_rsrc(qt + (int64_t)(ch0 / 32) * 4 * 64);
  const uint32_t loff = (uint32_t)lane * 16u;
  const uint4 ip0 = res_ident(0), ip1 = res_ident(1);

  // vr / dr hold the token's rows: as loaded (chunk c in registers 4 c .. 4 c
  // + 3, instruction order) until stage 1 re-lays each chunk, through this
  // wave's LDS tiles, into operand order (register 4 c + s = k-step s).
  uint4 vr[kRK], dr[kRK];
  auto load_rows = [&](int64_t t) {
    const __amdgpu_buffer_rsrc_t vrs = res_rsrc(src + t * d), drs = res_rsrc(dout + t * d);
#pragma unroll
    for (int c = 0; c < kRK / 4; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vr[4 * c + u] = res_ld(vrs, voff(u), 128 * c);
        dr[4 * c + u] = res_ld(drs, doff(u), 128 * c);
      }
  };
  if ((int64_t)blockIdx.x < T) load_rows(blockIdx.x);

  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int64_t tn = t + gridDim.x;
    const bool more = tn < T;

    // ---------------- stage 1: S = Q V^T, G = V V^T, A = dOut V^T over this wave's channels
    // The query operands stream from L2 two k-steps ahead; fences keep the
    // compiler from issuing all of them at once (they would need 128 registers
    // beside the resident rows).
    f16acc S = {}, G = {}, A = {};
    {
      uint4 qh[kRK], ql[kRK];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        qh[s] = res_ld(qrs, loff, 2048 * s);
        ql[s] = res_ld(qrs, loff, 2048 * s + 1024);
      }
      // This wave's staging tiles: the partial-sum rows of S and G, unused
      // until the partials are written (after a barrier).
      unsigned char* vt = reinterpret_cast<unsigned char*>(MH ? M.tile_v(res_smem, wave) : L.sred(res_smem, wave));
      unsigned char* dt = reinterpret_cast<unsigned char*>(MH ? M.tile_d(res_smem, wave) : L.gred(res_smem, wave));
#pragma unroll
      for (int s = 0; s < kRK; ++s) {
        if (s % 4 == 0) {
          // Re-lay chunk s / 4 into operand order.  The swizzled addresses come
          // from an opaque lane id, so they are recomputed here rather than
          // held (spilled) across the token loop.
          const int c = s / 4;
          int ol = lane;
          asm volatile("" : "+v"(ol));
          const int wb = vpos(ol >> 3, ol & 7);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            *reinterpret_cast<uint4*>(vt + wb + u * 8 * kVRow) = vr[4 * c + u];
            *reinterpret_cast<uint4*>(dt + wb + u * 8 * kVRow) = dr[4 * c + u];
          }
          wave_lds_sync();
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rb = vpos(ol & 31, 2 * k + (ol >> 5));
            vr[4 * c + k] = *reinterpret_cast<const uint4*>(vt + rb);
            dr[4 * c + k] = *reinterpret_cast<const uint4*>(dt + rb);
          }
          wave_lds_sync();
        }
        if (s + 2 < kRK) {
          qh[s + 2] = res_ld(qrs, loff, 2048 * (s + 2));
          ql[s + 2] = res_ld(qrs, loff, 2048 * (s + 2) + 1024);
        }
        S = mfma(qh[s], vr[s], S);
        S = mfma(ql[s], vr[s], S);
        G = mfma(vr[s], vr[s], G);
        A = mfma(dr[s], vr[s], A);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The A partials share LDS with nothing, but the tables below are read by
    // the previous token's stage 2: every wave must be past it.
    lds_barrier();
    {
      // Element r of lane (h, n) is row 8 (r / 4) + 4 h + r % 4, column n: one
      // per-lane base (row 4 h, column n) plus constant offsets.
      int rl = lane;
      asm volatile("" : "+v"(rl));
      const int base = 4 * (rl >> 5) * kTile + (rl & 31);
      if constexpr (MH) {
        float* sr = M.tile_v(res_smem, wave) + base;
        float* ar = M.tile_d(res_smem, wave) + base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = (8 * (r / 4) + (r % 4)) * kTile;
          sr[off] = S[r];
          ar[off] = A[r];
          if (8 * (r / 4) + 4 * (rl >> 5) + (r % 4) == (rl & 31)) M.gdiag(res_smem, wave)[rl & 31] = G[r];
        }
      } else {
        float* sr = L.sred(res_smem, wave) + base;
        float* ar = L.ared(res_smem, wave) + base;
        float* gr = L.gred(res_smem, wave) + base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = (8 * (r / 4) + (r % 4)) * kTile;
          sr[off] = S[r];
          ar[off] = A[r];
          gr[off] = G[r];
        }
      }
    }
    lds_barrier();

    if constexpr (MH) {
      // ---------------- each head's first wave: alpha, c, r c, c s from its accumulators' layout
      if (wave % gw == 0) {
        int rl = lane;
        asm volatile("" : "+v"(rl));
        const int base = 4 * (rl >> 5) * kTile + (rl & 31);
        float gv = 0.f;
        for (int w2 = 0; w2 < W; ++w2) gv += M.gdiag(res_smem, w2)[n];
        const float ri = 1.0f / sqrtf(gv / (float)d + a.eps);
        // Lane (h, i = n), element r: destination j = 8 (r / 4) + 4 h + r % 4.
        float al[16], rcv[16], csum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // The head's S and A at (destination j, source n): the sum of its waves' partials.
          float sv = 0.f, av = 0.f;
          for (int w2 = head * gw; w2 < head * gw + gw; ++w2) {
            sv += M.tile_v(res_smem, w2)[base + (8 * (r / 4) + (r % 4)) * kTile];
            av += M.tile_d(res_smem, w2)[base + (8 * (r / 4) + (r % 4)) * kTile];
          }
          const int j = 8 * (r / 4) + 4 * h + (r % 4);
          const bool ok = j < n_dst && n <= n_src - n_dst + j;
          const float sc = ok ? ri * sv : -INFINITY;
          const float m = group_max<32>(sc);
          const float e = ok ? expf(sc - m) : 0.f;
          const float l = group_sum<32>(e);
          al[r] = l > 0.f ? e / l : 0.f;
          const float sa = group_sum<32>(al[r] * av);
          const float cc = al[r] * (av - sa);
          rcv[r] = ok ? ri * cc : 0.f;
          csum += ok ? cc * sc : 0.f;
        }
        // Operands: k-step b, element e is destination transposed_row(b, h, e) = element 8 b + e.
        uint4* bp = M.bpk(res_smem, head);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const float* x = k2 == 0 ? al : rcv;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              hi[e] = bf2f(f2bf(x[8 * b + e]));
              lo[e] = x[8 * b + e] - hi[e];
            }
            bp[(4 * k2 + 2 * b) * 64 + lane] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
            bp[(4 * k2 + 2 * b + 1) * 64 + lane] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
          }
        }
        // r c for the Z kernel: [T][H][32][32] fp32, row j, column i = n.
        float* cw = cws + ((t * a.H + head) * kTile) * kTile + n;
#pragma unroll
        for (int r = 0; r < 16; ++r) cw[(8 * (r / 4) + 4 * h + (r % 4)) * kTile] = rcv[r];
        // sum over the destinations of c s for source n: this half's 16, then the other half's.
        csum += __shfl_xor(csum, 32);
        if (h == 0) M.cpart(res_smem, head)[n] = csum;
      }
      lds_barrier();
      if (wave == 0) {
        // coef_i = r_i^2 (sum over heads and destinations of c s) / d, as diag(-coef) operands.
        float cs = 0.f, gv = 0.f;
        for (int hh = 0; hh < a.H; ++hh) cs += M.cpart(res_smem, hh)[n];
        for (int w2 = 0; w2 < W; ++w2) gv += M.gdiag(res_smem, w2)[n];
        const float r2 = 1.0f / (gv / (float)d + a.eps);
        const float cn = n < n_src ? -(r2 * cs / (float)d) : 0.f;
        uint4* cd = M.cdiag(res_smem);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float hi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = transposed_row(b, h, e) == n ? cn : 0.f;
            hi[e] = bf2f(f2bf(x));
            lo[e] = x - hi[e];
          }
          cd[(2 * b) * 64 + lane] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
          cd[(2 * b + 1) * 64 + lane] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
        }
      }
      lds_barrier();
    } else {
    // ---------------- per (destination, source): alpha, c, r c, c s (threads 0..255)
    float* t_alpha = L.table(res_smem, 0);
    float* t_rc = L.table(res_smem, 1);
    float* t_cs = L.table(res_smem, 2);
    if (tid < 256) {
      const int j = tid / 8, i0 = 4 * (tid % 8);
      const int lim = n_src - n_dst + j;
      float sc[4], av[4], rr[4];
      bool ok[4];
      float m = -INFINITY;
      // The waves' partials, four sources at a time.
      float4 sv4 = make_float4(0.f, 0.f, 0.f, 0.f), av4 = sv4, gv4 = sv4;
      for (int w2 = 0; w2 < W; ++w2) {
        const float4 x = *reinterpret_cast<const float4*>(L.sred(res_smem, w2) + j * kTile + i0);
        const float4 y = *reinterpret_cast<const float4*>(L.ared(res_smem, w2) + j * kTile + i0);
        const float* g = L.gred(res_smem, w2) + i0 * (kTile + 1);
        sv4.x += x.x; sv4.y += x.y; sv4.z += x.z; sv4.w += x.w;
        av4.x += y.x; av4.y += y.y; av4.z += y.z; av4.w += y.w;
        gv4.x += g[0]; gv4.y += g[kTile + 1]; gv4.z += g[2 * (kTile + 1)]; gv4.w += g[3 * (kTile + 1)];
      }
      const float svs[4] = {sv4.x, sv4.y, sv4.z, sv4.w}, avs[4] = {av4.x, av4.y, av4.z, av4.w};
      const float gvs[4] = {gv4.x, gv4.y, gv4.z, gv4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q;
        rr[q] = 1.0f / sqrtf(gvs[q] / (float)d + a.eps);
        ok[q] = j < n_dst && i <= lim;
        sc[q] = ok[q] ? rr[q] * svs[q] : -INFINITY;
        av[q] = avs[q];
        m = fmaxf(m, sc[q]);
      }
      m = group_max<8>(m);
      float e[4], l = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[q] = ok[q] ? expf(sc[q] - m) : 0.f;
        l += e[q];
      }
      l = group_sum<8>(l);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float al[4], sa = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        al[q] = e[q] * inv;
        sa = fmaf(al[q], av[q], sa);
      }
      sa = group_sum<8>(sa);
      float rcv[4], csv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float cc = al[q] * (av[q] - sa);
        rcv[q] = ok[q] ? rr[q] * cc : 0.f;
        csv[q] = ok[q] ? cc * sc[q] : 0.f;
      }
      *reinterpret_cast<float4*>(&t_alpha[j * kARow + i0]) = make_float4(al[0], al[1], al[2], al[3]);
      *reinterpret_cast<float4*>(&t_rc[j * kARow + i0]) = make_float4(rcv[0], rcv[1], rcv[2], rcv[3]);
      *reinterpret_cast<float4*>(&t_cs[j * kARow + i0]) = make_float4(csv[0], csv[1], csv[2], csv[3]);
      // r c for the Z kernel: [T][32][32] fp32.
      *reinterpret_cast<float4*>(cws + t * (kTile * kTile) + j * kTile + i0) =
          make_float4(rcv[0], rcv[1], rcv[2], rcv[3]);
    }
    lds_barrier();

    // ---------------- stage 2 B operands, built once per token (into the A
    // partials' space, dead now): lane (h, n = source i), element e <-> row
    // k = transposed_row(b, h, e) of alpha[k][i] (slots 0..3), (r c)[k][i]
    // (4..7) and diag(-coef) (8..11), each split into bf16 high and low parts.
    uint4* bpk = reinterpret_cast<uint4*>(L.ared(res_smem, 0));
    {
      auto store_split = [&](const float (&x)[8], int slot) {
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = bf2f(f2bf(x[e]));
          lo[e] = x[e] - hi[e];
        }
        bpk[slot * 64 + lane] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
        bpk[(slot + 1) * 64 + lane] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
      };
      if (wave < 2) {
        const float* base = (wave == 0 ? t_alpha : t_rc) + 4 * h * kARow + n;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = base[(16 * b + 8 * (e / 4) + (e % 4)) * kARow];
          store_split(x, 4 * wave + 2 * b);
        }
      } else if (wave == 2) {
        // coef_i = r_i^2 (sum_j c_ji s_ji) / d for source i = n.
        float cs = 0.f, gv = 0.f;
        for (int j = 0; j < kTile; ++j) cs += t_cs[j * kARow + n];
        for (int w2 = 0; w2 < W; ++w2) gv += L.gred(res_smem, w2)[n * (kTile + 1)];
        const float r2 = 1.0f / (gv / (float)d + a.eps);
        const float cn = n < n_src ? -(r2 * cs / (float)d) : 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = transposed_row(b, h, e) == n ? cn : 0.f;
          store_split(x, 8 + 2 * b);
        }
      }
    }
    lds_barrier();

    }  // one head

    // ---------------- stage 2: dV^T = dOut^T alpha^T + Q^T (r c)^T - V^T diag(coef), per 32 channels
    // Block b uses the rows in registers 2 b, 2 b + 1 of vr and dr.  Every L2
    // load (the Q^T operands) is issued before the first load of the next
    // token's rows: the vector-memory counter retires in order, so a Q^T load
    // issued after such a prefetch would wait for an HBM round trip.  Blocks
    // 0..3 load the next block's Q^T after their own last use of it and park
    // the Q^T of blocks 4..7 in their own freed registers; after each of
    // blocks 4..7 the
    // registers of that block and of the block four earlier are free, and the
    // next token's rows go into them (register x of vr / dr holds instruction
    // x % 4 of chunk x / 4, so the refill needs no other bookkeeping).
    // dV is staged through this wave's LDS tile (a 64-channel chunk at a
    // time) and leaves as whole-row stores.
    {
      unsigned char* ot = reinterpret_cast<unsigned char*>(MH ? M.tile_v(res_smem, wave) : L.sred(res_smem, wave));
      // alpha and r c operands (slots 0..7) and diag(-coef) (slots 8..11).
      const uint4* opa = MH ? M.bpk(res_smem, head) : reinterpret_cast<const uint4*>(L.ared(res_smem, 0));
      const uint4* opc = MH ? M.cdiag(res_smem) : reinterpret_cast<const uint4*>(L.ared(res_smem, 0)) + 8 * 64;
      const __amdgpu_buffer_rsrc_t ors = res_rsrc(dsrc + t * d);
      const __amdgpu_buffer_rsrc_t nvrs = res_rsrc(src + (more ? tn : t) * d);
      const __amdgpu_buffer_rsrc_t ndrs = res_rsrc(dout + (more ? tn : t) * d);
      auto refill = [&](int x) {
        // the chunk's 128-byte step as the scalar offset: only the row offsets
        // (voff, doff) take vector registers
        vr[x] = res_ld(nvrs, voff(x % 4), 128 * (x / 4));
        dr[x] = res_ld(ndrs, doff(x % 4), 128 * (x / 4));
      };
      uint4 qc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) qc[k] = res_ld(qtrs, loff, 1024 * k);
#pragma unroll
      for (int b2 = 0; b2 < kRK / 2; ++b2) {
        const int s0 = 2 * b2, s1 = 2 * b2 + 1;
        // The tables are the same for every block: an opaque offset keeps the
        // compiler from loading them once and holding 48 registers.
        int boff = lane;
        asm volatile("" : "+v"(boff));
        const uint4* bl = opa + boff;
        const uint4* blc = opc + boff - 8 * 64;  // blc[k * 64] for slots k = 8 .. 11
        f16acc D = {};
        {
          f16acc D3 = {};
          D3 = mfma(dr[s0], ip0, D3);
          D3 = mfma(dr[s1], ip1, D3);
          const uint4 td0 = pack8(D3[0], D3[1], D3[2], D3[3], D3[4], D3[5], D3[6], D3[7]);
          const uint4 td1 = pack8(D3[8], D3[9], D3[10], D3[11], D3[12], D3[13], D3[14], D3[15]);
          D = mfma(td0, bl[0 * 64], D);   // alpha, b = 0, hi
          D = mfma(td0, bl[1 * 64], D);   //               lo
          D = mfma(td1, bl[2 * 64], D);   // alpha, b = 1, hi
          D = mfma(td1, bl[3 * 64], D);   //               lo
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          f16acc D1 = {};
          D1 = mfma(vr[s0], ip0, D1);
          D1 = mfma(vr[s1], ip1, D1);
          const uint4 tv0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
          const uint4 tv1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
          D = mfma(tv0, blc[8 * 64], D);   // -coef, b = 0
          D = mfma(tv0, blc[9 * 64], D);
          D = mfma(tv1, blc[10 * 64], D);  // -coef, b = 1
          D = mfma(tv1, blc[11 * 64], D);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          // Q^T of this block: in flight (blocks 0..3) or parked in the
          // registers of block b2 - 4 (blocks 4..7).
          uint4 q0h, q0l, q1h, q1l;
          if (b2 < 4) {
            q0h = qc[0]; q0l = qc[1]; q1h = qc[2]; q1l = qc[3];
          } else {
            const int p = b2 - 4;
            q0h = dr[2 * p]; q0l = dr[2 * p + 1]; q1h = vr[2 * p]; q1l = vr[2 * p + 1];
          }
          D = mfma(q0h, bl[4 * 64], D);   // r c, b = 0: (q_hi + q_lo)(rc_hi + rc_lo) less lo * lo
          D = mfma(q0h, bl[5 * 64], D);
          D = mfma(q0l, bl[4 * 64], D);
          D = mfma(q1h, bl[6 * 64], D);   // r c, b = 1
          D = mfma(q1h, bl[7 * 64], D);
          D = mfma(q1l, bl[6 * 64], D);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (b2 < 4) {
          // The next block's Q^T (its other products cover the latency), and
          // the Q^T of block b2 + 4 parked in this block's freed registers.
          if (b2 + 1 < 4) {
#pragma unroll
            for (int k = 0; k < 4; ++k) qc[k] = res_ld(qtrs, loff, 4096 * (b2 + 1) + 1024 * k);
          }
          dr[s0] = res_ld(qtrs, loff, 4096 * (b2 + 4));
          dr[s1] = res_ld(qtrs, loff, 4096 * (b2 + 4) + 1024);
          vr[s0] = res_ld(qtrs, loff, 4096 * (b2 + 4) + 2048);
          vr[s1] = res_ld(qtrs, loff, 4096 * (b2 + 4) + 3072);
        } else if (more) {
          refill(2 * (b2 - 4));
          refill(2 * (b2 - 4) + 1);
          refill(s0);
          refill(s1);
        }
        // Element r of lane (h, i) is channel 32 (b2 % 2) + 16 h + r of the
        // chunk: two 16-byte pieces of tile row i.
        int ol = lane;
        asm volatile("" : "+v"(ol));
        {
          const int on = ol & 31, piece = 4 * (b2 & 1) + 2 * (ol >> 5);
          *reinterpret_cast<uint4*>(ot + vpos(on, piece)) = pack8(D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7]);
          *reinterpret_cast<uint4*>(ot + vpos(on, piece + 1)) =
              pack8(D[8], D[9], D[10], D[11], D[12], D[13], D[14], D[15]);
        }
        if (b2 & 1) {
          // The chunk's tile is complete: whole-row stores, instruction u of
          // lane l writing piece l % 8 of row 8 u + l / 8 (rows past n_src
          // are not stored).
          const int c = b2 >> 1;
          wave_lds_sync();
          const int rb = vpos(ol >> 3, ol & 7);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int row = 8 * u + (ol >> 3);
            uint4 y = *reinterpret_cast<const uint4*>(ot + rb + u * 8 * kVRow);
            if (row < n_src) {
              const uint32_t off = voff(u);
              if constexpr (ACC) {
                const uint4 o = res_ld(ors, off, 128 * c);
                const uint32_t yw[4] = {y.x, y.y, y.z, y.w}, ow[4] = {o.x, o.y, o.z, o.w};
                uint32_t rw[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  rw[k] = pack_bf2(bf_lo(yw[k]) + bf_lo(ow[k]), bf_hi(yw[k]) + bf_hi(ow[k]));
                y = make_uint4(rw[0], rw[1], rw[2], rw[3]);
              }
              __builtin_amdgcn_raw_buffer_store_b128(v4u{y.x, y.y, y.z, y.w}, ors, (int)off, 128 * c, 0);
            }
          }
          wave_lds_sync();  // the tile is rewritten by the next chunk
        }
      }
    }
  }
}

bool al16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

int64_t z_groups(int64_t T) { return T < kZGroups ? T : kZGroups; }

}  // namespace

// Sources per row of the (r c) table: 32, or 64 for the two-tile kernel.
int64_t rc_cols(int64_t n_src) { return n_src > kTile ? 2 * kTile : kTile; }

size_t full_bwd_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int H) {
  // qpk [128 d] + qt [128 d] + (r c) [T][H][32][rc_cols] fp32 + Z slabs [groups][n_dst][d] fp32
  const size_t mfma =
      (size_t)256 * (size_t)d + (size_t)T * H * kTile * rc_cols(n_src) * 4 + (size_t)z_groups(T) * n_dst * d * 4;
  return std::max(mfma, full_bwd_one_workspace_bytes(n_src, n_dst, T, d, H));
}

// The register-resident kernel: d = 1024 .. 2048 in steps of 256 (d / 256
// waves of 256 channels each).
bool full_bwd_res_ok(const FullBwdArgs& a) {
  // Per-lane byte offsets of the rows from a token's base are 32-bit.
  const int64_t span = std::max(a.n_src, a.n_dst) * a.T * a.d * 2;
  if (a.d < 1024 || a.d > 2048 || a.d % 256 != 0 || span >= ((int64_t)1 << 31)) return false;
  // Heads: H = 2, 4 or 8 runs of whole waves (d / 256 waves).
  return a.H == 1 || ((a.H == 2 || a.H == 4 || a.H == 8) && (a.d / kRCh) % a.H == 0);
}

bool full_bwd_fast_ok(const FullBwdArgs& a) {
  if (a.dtype != kBF16 || a.T < 1) return false;
  if (full_bwd_one_ok(a)) return true;
  if (full_bwd_wide_shape(a)) {
    if (a.zslots == nullptr || a.ws_bytes < full_bwd_fast_workspace_bytes(a.n_src, a.n_dst, a.T, a.d, a.H))
      return false;
    return al16(a.src) && al16(a.dout) && al16(a.d_src) && al16(a.zslots) && al16(a.w) && al16(a.gain);
  }
  if (a.H != 1 && !full_bwd_res_ok(a)) return false;  // heads: the resident kernel only
  if (a.n_src > kTile || a.n_dst > a.n_src) return false;
  if ((!full_bwd_res_ok(a) && a.d % (2 * kBW * kChunk) != 0) || a.d > ((int64_t)1 << 16)) return false;
  if (a.zslots == nullptr || a.ws_bytes < full_bwd_fast_workspace_bytes(a.n_src, a.n_dst, a.T, a.d, a.H))
    return false;
  return al16(a.src) && al16(a.dout) && al16(a.d_src) && al16(a.zslots) && al16(a.w) && al16(a.gain);
}

const char* full_bwd_fast_variant(const FullBwdArgs& a) {
  if (!full_bwd_fast_ok(a)) return nullptr;
  if (full_bwd_one_ok(a)) return "full_bwd_one";
  if (full_bwd_wide_shape(a)) return "full_bwd_wide";
  return full_bwd_res_ok(a) ? "full_bwd_res" : "full_bwd_fast";
}

hipError_t launch_full_bwd_fast(const FullBwdArgs& a, const float** slabs, int64_t* n_slabs, hipStream_t st) {
  if (full_bwd_one_ok(a)) return launch_full_bwd_one(a, slabs, n_slabs, st);
  char* ws = reinterpret_cast<char*>(a.zslots);
  uint4* qpk = reinterpret_cast<uint4*>(ws);
  uint4* qt = reinterpret_cast<uint4*>(ws + 128 * a.d);
  float* cws = reinterpret_cast<float*>(ws + 256 * a.d);
  float* zs = cws + a.T * a.H * kTile * rc_cols(a.n_src);  // (r c) is [T][H][32][rc_cols]
  hipLaunchKernelGGL(k_full_bwd_qsplit, dim3(64), dim3(256), 0, st, a, qpk);
  if (full_bwd_wide_shape(a)) {
    hipLaunchKernelGGL(k_full_qtsplit<false>, dim3(64), dim3(256), 0, st, a, qt);
    const int groups = (int)z_groups(a.T);
    hipError_t e = launch_full_bwd_staged(a, qpk, qt, cws, st);
    if (e == hipSuccess) e = launch_full_bwd_zw(a, cws, zs, groups, st);
    *slabs = zs;
    *n_slabs = groups;
    return e;
  }
  if (full_bwd_res_ok(a)) {
    hipLaunchKernelGGL(k_full_qtsplit<true>, dim3(64), dim3(256), 0, st, a, qt);
    const int W = (int)(a.d / kRCh);
    const bool mh = a.H > 1;
    const size_t lds = mh ? ResLdsMH::bytes(W, (int)a.H) : ResLds::bytes(W);
    const int which = (a.accumulate ? 1 : 0) + (mh ? 2 : 0);
    auto kern = a.accumulate ? (mh ? k_full_bwd_res<true, true> : k_full_bwd_res<true, false>)
                             : (mh ? k_full_bwd_res<false, true> : k_full_bwd_res<false, false>);
    static std::atomic<bool> allowed[4] = {false, false, false, false};
    if (!allowed[which].load(std::memory_order_relaxed)) {
      const size_t most = std::max(ResLds::bytes(2048 / kRCh), ResLdsMH::bytes(2048 / kRCh, 8));
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
      if (e != hipSuccess) return e;
      allowed[which].store(true, std::memory_order_relaxed);
    }
    int per_cu = 0;
    const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), W * 64, &per_cu, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    if (grid > a.T) grid = a.T;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(W * 64), lds, st, a, (const uint4*)qpk, (const uint4*)qt,
                       cws);
    const int groups = (int)z_groups(a.T);
    hipLaunchKernelGGL(k_full_bwd_z, dim3((unsigned)groups, (unsigned)(a.d / kChunk)), dim3(64), 0, st, a,
                       (const float*)cws, zs, groups);
    *slabs = zs;
    *n_slabs = groups;
    return hipGetLastError();
  }
  // The staged kernel with one source tile (d outside the resident range).
  hipLaunchKernelGGL(k_full_qtsplit<false>, dim3(64), dim3(256), 0, st, a, qt);
  const hipError_t e = launch_full_bwd_staged(a, qpk, qt, cws, st);
  if (e != hipSuccess) return e;
  const int groups = (int)z_groups(a.T);
  hipLaunchKernelGGL(k_full_bwd_z, dim3((unsigned)groups, (unsigned)(a.d / kChunk)), dim3(64), 0, st, a,
                     (const float*)cws, zs, groups);
  *slabs = zs;
  *n_slabs = groups;
  return hipGetLastError();
}

}  // namespace attnres
