// Full AttnRes backward for 33 .. 64 sources on the matrix cores (gfx950, bf16
// I/O, one head, up to 32 destinations): the per-sublayer backward of a model
// deeper than 32 sublayers (b-lab.team summary §1; dimensionstp "Attention
// Residuals Review" §3 (2) runs 54).  The chain rule is the one of
// full_bwd_fast.hip: per token, with x_i = RMSNorm(v_i), r_i its inverse RMS,
// q_j = w_j * g_j and destination j reading sources 0 .. lim_j,
//   s_ji = r_i q_j . v_i,  a_ji = dout_j . v_i,  alpha_j = softmax_i(s_j)
//   c_ji = alpha_ji (a_ji - sum_m alpha_jm a_jm)
//   dv_i = sum_j alpha_ji dout_j + r_i sum_j c_ji q_j - (r_i^2 / d) (sum_j c_ji s_ji) v_i
//   Z_j  = sum over tokens of sum_i (r_i c_ji) v_i,  dw_j = g_j Z_j,  dg_j = w_j Z_j
// over two 32-source tiles:
//   stage 1  S = Q V^T (q split into bf16 high + low parts), G = V V^T (its
//            diagonal: the sums of squares), A = dOut V^T, per source tile;
//   stage 2  per source tile, dV^T = dOut^T alpha^T + Q^T (r c)^T - V^T
//            diag(coef), the source and dout tiles transposed by an MFMA
//            against the identity (exact), alpha, r c and coef split into
//            bf16 high + low parts;
//   Z        a second kernel forms (r c) V per token over both tiles and sums
//            it over token groups into fixed slabs.
// A workgroup of 4 waves owns one token at a time; wave w covers channels
// [w d/4, (w+1) d/4) in 64-channel chunks, staged through per-wave LDS tiles
// with whole-row loads, one chunk in flight; stage 2 reads the rows again
// (from cache).  The LDS regions of the tiles, the per-wave partials, the
// per-token tables and the stage-2 operands overlap where their lifetimes do
// not (workgroup barriers between), so two workgroups fit on a compute unit.
#include <math.h>

#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kXW = 4;                        // waves per workgroup
constexpr int kXB = kXW * 64;                 // threads per workgroup

// Sizes and LDS layout for TS 32-source tiles.  The regions of the tiles, the
// per-wave partials, the per-token tables and the stage-2 operands overlap
// where their lifetimes do not.
template <int TS>
struct XL {
  static constexpr int S = TS * kTile;                 // source rows
  static constexpr int Row = S + 4;                    // floats per table row (16-byte aligned)
  static constexpr int TileV = S * kVRow;              // a wave's staged source tile (then its dV tile)
  static constexpr int TileD = kTile * kVRow;          // a wave's staged dout tile
  static constexpr int Ops = kXW * (TileV + TileD);    // stage-2 operands follow the tiles
  static constexpr int OpsBytes = TS * 12 * 64 * 16;   // per source tile 12 slots of 64 lanes x 16 bytes
  static constexpr int Part = kXW * kTile * S * 4;     // one array of per-wave partials ([wave][j][i])
  static constexpr int Union = Ops + OpsBytes > 2 * Part ? Ops + OpsBytes : 2 * Part;
  static constexpr int Gred = Union;                   // [wave][i] partial sums of squares
  static constexpr int Coef = Gred + kXW * S * 4;      // coef_i
  static constexpr int Lds = Coef + S * 4;
  static_assert(3 * kTile * Row * 4 <= Ops, "the tables must not reach the operands");
  static_assert(2 * Lds <= 160 * 1024, "two workgroups per compute unit");
};
constexpr int kXS = XL<2>::S;  // the two-tile Z pass

__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferWord3);
}
__device__ __forceinline__ uint4 x_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ROWS rows of one 64-channel chunk (tok: the token's row of plane 0 at this
// wave's first channel): instruction u of lane ol reads piece ol % 8 of row
// 8 u + ol / 8; rows at or past nreal read row 0 (no branch: exact wait
// counts) and are zeroed when staged.
template <int ROWS>
__device__ __forceinline__ void x_load(const bf16_t* tok, int64_t plane, int nreal, int ch, int ol,
                                       uint4 (&v)[ROWS / 8]) {
  const bf16_t* base = tok + ch + 8 * (ol & 7);
#pragma unroll
  for (int u = 0; u < ROWS / 8; ++u) {
    const int r = 8 * u + (ol >> 3);
    v[u] = *reinterpret_cast<const uint4*>(base + (int64_t)(r < nreal ? r : 0) * plane);
  }
}
template <int ROWS>
__device__ __forceinline__ void x_stage(unsigned char* tile, const uint4 (&v)[ROWS / 8], int nreal, int ol) {
  unsigned char* base = tile + vpos(ol >> 3, ol & 7);
#pragma unroll
  for (int u = 0; u < ROWS / 8; ++u) {
    const uint32_t m = 8 * u + (ol >> 3) < nreal ? 0xFFFFFFFFu : 0u;
    *reinterpret_cast<uint4*>(base + u * 8 * kVRow) = make_uint4(v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m);
  }
}
__device__ __forceinline__ uint4 x_operand(const unsigned char* tile, int ol, int s) {
  return *reinterpret_cast<const uint4*>(tile + vpos(ol & 31, 2 * s + (ol >> 5)));
}

template <bool ACC, int TS>
__global__ __launch_bounds__(kXB, 2) void k_full_bwd_wide(FullBwdArgs a, const uint4* qpk, const uint4* qt,
                                                          float* cws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char xsm[];
  using L = XL<TS>;
  constexpr int kS = L::S;                 // source rows of the tiles
  constexpr int SPT = kS / 8;              // softmax sources per thread (8 threads per destination)
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T, plane = T * d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const bf16_t* dout = static_cast<const bf16_t*>(a.dout);
  bf16_t* dsrc = static_cast<bf16_t*>(a.d_src);
  const int kw = d / kXW;
  const int nch = kw / kChunk;
  const int ch_base = wave * kw;
  unsigned char* vt = xsm + wave * (L::TileV + L::TileD);
  unsigned char* dt = vt + L::TileV;
  float* sred = reinterpret_cast<float*>(xsm);            // [wave][j][i], after stage 1
  float* ared = reinterpret_cast<float*>(xsm + L::Part);   // [wave][j][i]
  float* t_alpha = reinterpret_cast<float*>(xsm);         // [j][L::Row], after the partials are read
  float* t_rc = t_alpha + kTile * L::Row;
  float* t_cs = t_rc + kTile * L::Row;
  uint4* bpk = reinterpret_cast<uint4*>(xsm + L::Ops);     // [ts][slot][lane]
  float* gred = reinterpret_cast<float*>(xsm + L::Gred);
  float* coef = reinterpret_cast<float*>(xsm + L::Coef);
  const int h = lane >> 5, n = lane & 31;
  // Query operands of this wave's chunks: chunk c at byte 8 KiB c, k-step s
  // and part p at (2 s + p) KiB, lane at 16 lane.  Q^T operands: 32-channel
  // tile c32 at 4 KiB c32, k-step b and part p at (2 b + p) KiB.
  const __amdgpu_buffer_rsrc_t qrs = x_rsrc(qpk + (int64_t)(ch_base / kChunk) * 8 * 64);
  const __amdgpu_buffer_rsrc_t qtrs = x_rsrc(qt + (int64_t)(ch_base / 32) * 4 * 64);
  const uint4 ident0 = ident_operand(0), ident1 = ident_operand(1);

  // One chunk in flight, in the order stage 1 (chunks 0 .. nch - 1), stage 2
  // (0 .. nch - 1), the next token's stage 1, ...
  int64_t t = blockIdx.x;
  uint4 v[kS / 8], g[4];
  if (t < T) {
    int ol = lane;
    asm volatile("" : "+v"(ol));
    x_load<kS>(src + t * d + ch_base, plane, n_src, 0, ol, v);
    x_load<kTile>(dout + t * d + ch_base, plane, n_dst, 0, ol, g);
  }
  for (; t < T; t += gridDim.x) {
    const bf16_t* tv_ = src + t * d + ch_base;
    const bf16_t* td_ = dout + t * d + ch_base;
    const int64_t tn = t + gridDim.x < T ? t + gridDim.x : t;  // this token again after the last
    const bf16_t* tvn = src + tn * d + ch_base;
    const bf16_t* tdn = dout + tn * d + ch_base;

    // ---------------- stage 1: S = Q V^T, G = V V^T, A = dOut V^T, per source tile
    f16acc S[TS], G[TS], A[TS];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) S[ts] = G[ts] = A[ts] = f16acc{};
    for (int c = 0; c < nch; ++c) {
      int ol = lane;
      asm volatile("" : "+v"(ol));
      const uint32_t qoff = (uint32_t)ol * 16u + (uint32_t)c * 8192u;
      x_stage<kS>(vt, v, n_src, ol);
      x_stage<kTile>(dt, g, n_dst, ol);
      const int cn = c + 1 < nch ? c + 1 : 0;  // after the last chunk: stage 2's first
      x_load<kS>(tv_, plane, n_src, cn * kChunk, ol, v);
      x_load<kTile>(td_, plane, n_dst, cn * kChunk, ol, g);
      wave_lds_sync();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 qh = x_ld(qrs, qoff, (2 * s) * 1024), ql = x_ld(qrs, qoff, (2 * s + 1) * 1024);
        const uint4 bd = x_operand(dt, ol, s);
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
          const uint4 bv = x_operand(vt + ts * kTile * kVRow, ol, s);
          S[ts] = mfma(qh, bv, S[ts]);
          S[ts] = mfma(ql, bv, S[ts]);
          G[ts] = mfma(bv, bv, G[ts]);
          A[ts] = mfma(bd, bv, A[ts]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();  // operand reads done before the tiles are rewritten
    }
    lds_barrier();  // every wave is done with its tiles (and the previous token's operands)
    {
      int rl = lane;
      asm volatile("" : "+v"(rl));
      const int rh = rl >> 5, rn = rl & 31;
      // Element r of lane (h, n) is row 8 (r/4) + 4 h + r%4 (destination, or
      // source for G), column n (source of the tile).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r / 4) + 4 * rh + (r % 4);
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
          sred[(wave * kTile + m) * kS + ts * kTile + rn] = S[ts][r];
          ared[(wave * kTile + m) * kS + ts * kTile + rn] = A[ts][r];
          if (m == rn) gred[wave * kS + ts * kTile + rn] = G[ts][r];
        }
      }
    }
    lds_barrier();

    // ---------------- per (destination, source): alpha, c, r c, c s
    {
      const int j = tid / 8, i0 = SPT * (tid % 8);
      const int lim = n_src - n_dst + j;
      float sc[SPT], av[SPT], rr[SPT];
      bool ok[SPT];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const int i = i0 + q;
        float sv = 0.f, aa = 0.f, gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kXW; ++w2) {
          sv += sred[(w2 * kTile + j) * kS + i];
          aa += ared[(w2 * kTile + j) * kS + i];
          gv += gred[w2 * kS + i];
        }
        rr[q] = 1.0f / sqrtf(gv / (float)d + a.eps);
        ok[q] = j < n_dst && i <= lim;
        sc[q] = ok[q] ? rr[q] * sv : -INFINITY;
        av[q] = aa;
        m = fmaxf(m, sc[q]);
      }
      m = group_max<8>(m);
      float e[SPT], l = 0.f;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        e[q] = ok[q] ? expf(sc[q] - m) : 0.f;
        l += e[q];
      }
      l = group_sum<8>(l);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float al[SPT], sa = 0.f;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        al[q] = e[q] * inv;
        sa = fmaf(al[q], av[q], sa);
      }
      sa = group_sum<8>(sa);
      float rcv[SPT], csv[SPT];
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const float cc = al[q] * (av[q] - sa);
        rcv[q] = ok[q] ? rr[q] * cc : 0.f;
        csv[q] = ok[q] ? cc * sc[q] : 0.f;
      }
      lds_barrier();  // every partial has been read: the tables overwrite them
#pragma unroll
      for (int q = 0; q < SPT; q += 4) {
        *reinterpret_cast<float4*>(&t_alpha[j * L::Row + i0 + q]) = make_float4(al[q], al[q + 1], al[q + 2], al[q + 3]);
        *reinterpret_cast<float4*>(&t_rc[j * L::Row + i0 + q]) = make_float4(rcv[q], rcv[q + 1], rcv[q + 2], rcv[q + 3]);
        *reinterpret_cast<float4*>(&t_cs[j * L::Row + i0 + q]) = make_float4(csv[q], csv[q + 1], csv[q + 2], csv[q + 3]);
        // r c for the Z kernel: [T][32][32 TS] fp32.
        *reinterpret_cast<float4*>(cws + (t * kTile + j) * kS + i0 + q) =
            make_float4(rcv[q], rcv[q + 1], rcv[q + 2], rcv[q + 3]);
      }
    }
    lds_barrier();
    if (tid < kS) {
      // coef_i = r_i^2 (sum_j c_ji s_ji) / d
      const int i = tid;
      float cs = 0.f, gv = 0.f;
      for (int j = 0; j < kTile; ++j) cs += t_cs[j * L::Row + i];
#pragma unroll
      for (int w2 = 0; w2 < kXW; ++w2) gv += gred[w2 * kS + i];
      const float r2 = 1.0f / (gv / (float)d + a.eps);
      coef[i] = i < n_src ? r2 * cs / (float)d : 0.f;
    }
    lds_barrier();

    // ---------------- stage 2 B operands, per source tile ts: lane (h, n = source
    // 32 ts + n), element e <-> destination k = transposed_row(b, h, e) of
    // alpha[k][i] (slots 0..3), (r c)[k][i] (4..7) and diag(-coef) (8..11),
    // slot type * 4 + 2 b + part, bf16 high (part 0) and low (1).
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
      if (wave < 2) {  // wave 0: alpha, wave 1: r c
        const float* tab = wave == 0 ? t_alpha : t_rc;
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = tab[transposed_row(b, h, e) * L::Row + ts * kTile + n];
            store_split(x, ts * 12 + 4 * wave + 2 * b);
          }
      } else if (wave == 2) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
          const float cn = -coef[ts * kTile + n];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = transposed_row(b, h, e) == n ? cn : 0.f;
            store_split(x, ts * 12 + 8 + 2 * b);
          }
        }
      }
    }
    lds_barrier();  // the operands are built: the tiles overwrite the tables

    // ---------------- stage 2: dV^T = dOut^T alpha^T + Q^T (r c)^T - V^T diag(coef), per source tile
    for (int c = 0; c < nch; ++c) {
      int ol = lane;
      asm volatile("" : "+v"(ol));
      const int oh = ol >> 5, on = ol & 31;
      const uint32_t qtoff = (uint32_t)ol * 16u + (uint32_t)(c * 2) * 4096u;
      // Q^T of both halves, issued before the next chunk's loads (the
      // vector-memory counter retires in order).
      uint4 qq[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int k = 0; k < 4; ++k) qq[half][k] = x_ld(qtrs, qtoff, half * 4096 + k * 1024);
      x_stage<kS>(vt, v, n_src, ol);
      x_stage<kTile>(dt, g, n_dst, ol);
      // The next chunk, or after the last one the next token's first.
      const bool last = c + 1 == nch;
      x_load<kS>(last ? tvn : tv_, plane, n_src, last ? 0 : (c + 1) * kChunk, ol, v);
      x_load<kTile>(last ? tdn : td_, plane, n_dst, last ? 0 : (c + 1) * kChunk, ol, g);
      wave_lds_sync();
      uint4 ov[TS][4];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts)
#pragma unroll
        for (int s = 0; s < 4; ++s) ov[ts][s] = x_operand(vt + ts * kTile * kVRow, ol, s);
      wave_lds_sync();  // the source tile becomes the output tile below
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f16acc D3 = {};
        D3 = mfma(x_operand(dt, ol, 2 * half), ident0, D3);
        D3 = mfma(x_operand(dt, ol, 2 * half + 1), ident1, D3);
        const uint4 td0 = pack8(D3[0], D3[1], D3[2], D3[3], D3[4], D3[5], D3[6], D3[7]);
        const uint4 td1 = pack8(D3[8], D3[9], D3[10], D3[11], D3[12], D3[13], D3[14], D3[15]);
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
          f16acc D1 = {};
          D1 = mfma(ov[ts][2 * half], ident0, D1);
          D1 = mfma(ov[ts][2 * half + 1], ident1, D1);
          const uint4 tv0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
          const uint4 tv1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
          const uint4* bl = bpk + ts * 12 * 64 + ol;
          f16acc D = {};
          D = mfma(td0, bl[0 * 64], D);   // alpha, b = 0, hi
          D = mfma(td0, bl[1 * 64], D);   //               lo
          D = mfma(td1, bl[2 * 64], D);   // alpha, b = 1, hi
          D = mfma(td1, bl[3 * 64], D);   //               lo
          D = mfma(qq[half][0], bl[4 * 64], D);  // r c, b = 0: (q_hi + q_lo)(rc_hi + rc_lo) less lo * lo
          D = mfma(qq[half][0], bl[5 * 64], D);
          D = mfma(qq[half][1], bl[4 * 64], D);
          D = mfma(qq[half][2], bl[6 * 64], D);  // r c, b = 1
          D = mfma(qq[half][2], bl[7 * 64], D);
          D = mfma(qq[half][3], bl[6 * 64], D);
          D = mfma(tv0, bl[8 * 64], D);   // -coef, b = 0
          D = mfma(tv0, bl[9 * 64], D);
          D = mfma(tv1, bl[10 * 64], D);  // -coef, b = 1
          D = mfma(tv1, bl[11 * 64], D);
          // D[c'][i]: lane (h, i = n) holds channels 8 q + 4 h .. + 3 (of this
          // half) of source 32 ts + n in elements 4 q .. 4 q + 3 -> bf16 tile
          // row 32 ts + n, 8 bytes at offset 8 h of 16-byte piece 4 half + q.
          const int row = ts * kTile + on;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float y0 = D[4 * q], y1 = D[4 * q + 1], y2 = D[4 * q + 2], y3 = D[4 * q + 3];
            if constexpr (ACC) {
              const int i = row < n_src ? row : n_src - 1;
              const uint2 old = *reinterpret_cast<const uint2*>(
                  dsrc + ((int64_t)i * T + t) * d + ch_base + c * kChunk + 32 * half + 8 * q + 4 * oh);
              y0 += bf_lo(old.x); y1 += bf_hi(old.x); y2 += bf_lo(old.y); y3 += bf_hi(old.y);
            }
            *reinterpret_cast<uint2*>(vt + vpos(row, 4 * half + q) + 8 * oh) =
                make_uint2(pack_bf2(y0, y1), pack_bf2(y2, y3));
          }
          __builtin_amdgcn_sched_barrier(0);  // one source tile's registers at a time
        }
      }
      wave_lds_sync();
      // Whole-row stores; rows past n_src store row n_src - 1 again (identical bytes).
      const int chn = ch_base + c * kChunk + 8 * (ol & 7);
#pragma unroll
      for (int u = 0; u < kS / 8; ++u) {
        const int ir = min(8 * u + (ol >> 3), n_src - 1);
        const uint4 o = *reinterpret_cast<const uint4*>(vt + vpos(ir, ol & 7));
        __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w},
                                    reinterpret_cast<v4u*>(dsrc + ((int64_t)ir * T + t) * d + chn));
      }
      wave_lds_sync();  // the tiles are rewritten by the next chunk
    }
    // The next token writes its partials only after a barrier that every wave
    // reaches after finishing this stage; the tables and operands after later
    // ones.
  }
}

// Z_j = sum over tokens of sum_i (r_i c_ji) v_i over both source tiles, for
// one 64-channel tile and one token group per wave: D[j][c'] = (r c)[j][i]
// V[i][c'] with (r c) split hi + lo as the A operand and the identity-
// transposed source tiles as B.  The group's sum goes to slab grp
// ([groups, n_dst, d] fp32).
__global__ __launch_bounds__(64) void k_full_bwd_zw(FullBwdArgs a, const float* cws, float* zs, int groups) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kXS * kVRow];
  const int lane = lane_id(), h = lane >> 5, n = lane & 31;
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T, plane = T * d;
  // The token group is the fast grid index: workgroups go to the XCDs round
  // robin, so every channel tile of a group runs on one XCD and that L2 holds
  // the group's (r c) rows once (each wave reads the whole row of its token).
  const int grp = blockIdx.x;
  const int ch0 = blockIdx.y * kChunk;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const uint4 ident0 = ident_operand(0), ident1 = ident_operand(1);
  f16acc Z0 = {}, Z1 = {};
  // One token ahead: its source rows and (r c) row load while this token's
  // products run (the last token reloads itself: the same loads every time).
  // x[ts][b][k]: lane (h, j = n) holds (r c)[j][32 ts + transposed_row(b, h, e)].
  auto load_token = [&](int64_t t, uint4 (&v)[8], float4 (&x)[2][2][2]) {
    int ol = lane;
    asm volatile("" : "+v"(ol));
    x_load<kXS>(src + t * d + ch0, plane, n_src, 0, ol, v);
    const float* cj = cws + (t * kTile + (ol & 31)) * kXS + 4 * (ol >> 5);
#pragma unroll
    for (int ts = 0; ts < 2; ++ts)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        x[ts][b][0] = *reinterpret_cast<const float4*>(cj + ts * kTile + 16 * b);
        x[ts][b][1] = *reinterpret_cast<const float4*>(cj + ts * kTile + 16 * b + 8);
      }
  };
  uint4 v[8];
  float4 x[2][2][2];
  if (grp < T) load_token(grp, v, x);
  for (int64_t t = grp; t < T; t += groups) {
    uint4 cA[2][2][2];  // [ts][b][part]
#pragma unroll
    for (int ts = 0; ts < 2; ++ts)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float xs[8] = {x[ts][b][0].x, x[ts][b][0].y, x[ts][b][0].z, x[ts][b][0].w,
                             x[ts][b][1].x, x[ts][b][1].y, x[ts][b][1].z, x[ts][b][1].w};
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = bf2f(f2bf(xs[e]));
          lo[e] = xs[e] - hi[e];
        }
        cA[ts][b][0] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
        cA[ts][b][1] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
      }
    int ol = lane;
    asm volatile("" : "+v"(ol));
    wave_lds_sync();
    x_stage<kXS>(tile, v, n_src, ol);
    const int64_t tn = t + groups < T ? t + groups : t;
    load_token(tn, v, x);
    wave_lds_sync();
    uint4 op[2][4];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts)
#pragma unroll
      for (int s = 0; s < 4; ++s) op[ts][s] = x_operand(tile + ts * kTile * kVRow, ol, s);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f16acc& Z = half ? Z1 : Z0;
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        f16acc D1 = {};
        D1 = mfma(op[ts][2 * half], ident0, D1);
        D1 = mfma(op[ts][2 * half + 1], ident1, D1);
        const uint4 tv0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
        const uint4 tv1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
        Z = mfma(cA[ts][0][0], tv0, Z);
        Z = mfma(cA[ts][0][1], tv0, Z);
        Z = mfma(cA[ts][1][0], tv1, Z);
        Z = mfma(cA[ts][1][1], tv1, Z);
      }
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

template <int TS>
hipError_t launch_staged(const FullBwdArgs& a, const uint4* qpk, const uint4* qt, float* cws, hipStream_t st) {
  auto kern = a.accumulate ? k_full_bwd_wide<true, TS> : k_full_bwd_wide<false, TS>;
  constexpr int lds = XL<TS>::Lds;
  if constexpr (lds > 64 * 1024) {
    static std::atomic<bool> allowed[2] = {false, false};  // dynamic LDS above 64 KiB, once per kernel
    const int which = a.accumulate ? 1 : 0;
    if (!allowed[which].load(std::memory_order_relaxed)) {
      const hipError_t e =
          hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      allowed[which].store(true, std::memory_order_relaxed);
    }
  }
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), kXB, &per_cu, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kXB), lds, st, a, qpk, qt, cws);
  return hipGetLastError();
}

}  // namespace

bool full_bwd_wide_shape(const FullBwdArgs& a) {
  return a.dtype == kBF16 && a.H == 1 && a.n_src > kTile && a.n_src <= kXS && a.n_dst >= 1 && a.n_dst <= kTile &&
         a.n_dst <= a.n_src && a.d % (2 * kXW * kChunk) == 0 && a.d <= ((int64_t)1 << 16);
}

hipError_t launch_full_bwd_staged(const FullBwdArgs& a, const uint4* qpk, const uint4* qt, float* cws,
                                  hipStream_t st) {
  return a.n_src > kTile ? launch_staged<2>(a, qpk, qt, cws, st) : launch_staged<1>(a, qpk, qt, cws, st);
}

hipError_t launch_full_bwd_zw(const FullBwdArgs& a, const float* cws, float* zs, int groups, hipStream_t st) {
  hipLaunchKernelGGL(k_full_bwd_zw, dim3((unsigned)groups, (unsigned)(a.d / kChunk)), dim3(64), 0, st, a, cws, zs,
                     groups);
  return hipGetLastError();
}

}  // namespace attnres
