// Specialised Full AttnRes forward for gfx950 (bf16 I/O, H = 1, up to 32
// sources and destinations).
//
// Per token the routing is two dense contractions (b-lab.team summary §1:
// O(L^2 d) per token), and both run on the matrix cores with
// v_mfma_f32_32x32x16_bf16:
//   stage 1  S = Q V^T (32 destinations x 32 sources over d channels), with
//            q = w * g split into bf16 high + low parts so the product keeps
//            about 16 significant bits of q; G = V V^T on the same operands
//            gives each source's sum of squares on its diagonal;
//   stage 2  H = alpha V, with alpha split the same way.
// A workgroup of 4 waves owns one token at a time; wave w covers channels
// [w d/4, (w+1) d/4) in chunks of 64.
//
// Operand staging.  Each chunk of the token's sources (32 rows x 128 bytes)
// is read with coalesced 16-byte loads (8 whole rows per wave instruction) and
// written to a per-wave LDS tile whose 16-byte pieces are XOR-swizzled by row,
// so the MFMA operand reads (one row per lane) hit distinct banks.  The query
// parts are packed once per call in exact operand-register order, so each
// lane's 16 bytes of a k-step are one contiguous 1 KiB block per wave.
//
// Stage 2 needs the sources with the source index inside a lane (the
// contraction dimension); the staged operands have one source per lane.  An
// MFMA against an identity matrix moves the channel index into the lanes
// (exact: every output is one bf16 value times 1).  Outputs are staged through
// a second LDS tile and written as whole rows with 16-byte stores.
#include <math.h>
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"
#include "mfma_tiles.hpp"

namespace attnres {
namespace {

constexpr int kFW = 4;            // waves per workgroup
constexpr int kFB = kFW * 64;     // threads per workgroup

// Packs q = w * g into MFMA A-operand order: for chunk g (64 channels), k-step
// s (16 channels) and part (0 = bf16 high, 1 = low), lane l's 8 values are
// q_part[l % 32][64 g + 16 s + 8 (l / 32) + e], stored at
// qpk[((g * 4 + s) * 2 + part) * 512 + l * 8 + e].  Rows past n_dst are zero.
__global__ __launch_bounds__(256) void k_full_qsplit(FullArgs a, bf16_t* qpk) {
  const int64_t units = a.d / kChunk * 4 * 64;  // (g, s, lane) triples
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < units;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(x % 64);
    const int64_t gs = x / 64;  // g * 4 + s
    const int j = lane % 32;
    const int64_t k0 = gs * 16 + 8 * (lane / 32);
    // Rows past n_dst load row n_dst - 1 (in bounds, no branch) and store zeros.
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
    uint4* dst = reinterpret_cast<uint4*>(qpk) + gs * 2 * 64 + lane;
    dst[0] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
    dst[64] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
  }
}

struct FullSmem {
  float sred[kFW][kTile * kTile];                   // per-wave partial S[j][i]
  float gred[kFW][kTile];                           // per-wave partial sum of squares
  __attribute__((aligned(16))) float alpha[kTile][kARow];  // alpha[j][i]
  __attribute__((aligned(16))) unsigned char vtile[kFW][kTile * kVRow];
  __attribute__((aligned(16))) unsigned char otile[kFW][kTile * kORow];
};

__global__ __launch_bounds__(kFB, 2) void k_full_fast(FullArgs a, const bf16_t* qpk) {
  __shared__ FullSmem sm;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const int kw = d / kFW;                  // channels per wave
  const int nch = kw / kChunk;             // chunks per wave
  const int ch_base = wave * kw;
  unsigned char* vt = sm.vtile[wave];
  unsigned char* ot = sm.otile[wave];
  const int h = lane >> 5;                 // MFMA half (k offset 8)
  const int n = lane & 31;                 // MFMA column
  const uint4* qv = reinterpret_cast<const uint4*>(qpk) + lane;

  // Identity operands for the transpose: I_a[k][n] = 1 when 16 a + k == n,
  // with k = 8 h + e held by lane (h, n).
  uint4 ident[2];
#pragma unroll
  for (int a2 = 0; a2 < 2; ++a2) {
    uint32_t wds[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e0 = 2 * q, e1 = 2 * q + 1;
      const uint32_t lo16 = (16 * a2 + 8 * h + e0 == n) ? 0x3F80u : 0u;
      const uint32_t hi16 = (16 * a2 + 8 * h + e1 == n) ? 0x3F80u : 0u;
      wds[q] = lo16 | (hi16 << 16);
    }
    ident[a2] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  }

  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const bf16_t* rowp[4];
    uint32_t rowmask[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 8 * u + (lane >> 3);
      rowmask[u] = r < n_src ? 0xFFFFFFFFu : 0u;
      rowp[u] = src + ((int64_t)(r < n_src ? r : 0) * T + t) * d + ch_base;
    }

    // ---------------- stage 1: S = Q V^T and G = V V^T over this wave's channels
    // Two chunks of sources are in flight while one is consumed (ping-pong
    // buffers, no register copies of loads in flight); the query operands of a
    // chunk come from L2 and are loaded when its turn comes.
    f16acc S = {}, G = {};
    {
      auto chunk1 = [&](int c, uint4 (&v)[4]) {
        const uint4* qc = qv + (int64_t)(ch_base / kChunk + c) * 8 * 64;
        uint4 q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = qc[k * 64];
        stage_chunk(vt, v, rowmask);
        load_chunk(rowp, min(c + 2, nch - 1) * kChunk, v);  // unconditional: exact wait counts
        wave_lds_sync();
        uint4 b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = tile_operand(vt, s);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          S = mfma(q[2 * s], b[s], S);
          S = mfma(q[2 * s + 1], b[s], S);
          G = mfma(b[s], b[s], G);
        }
        wave_lds_sync();  // operand reads done before the tile is rewritten
      };
      uint4 va[4], vb[4];
      load_chunk(rowp, 0, va);
      __builtin_amdgcn_sched_barrier(0);  // keep the loop's load order (va, then vb)
      load_chunk(rowp, kChunk, vb);
      // nch is even and >= 2.  The first pair is peeled so that the loop head
      // sees the same outstanding loads and stores on entry as on the back edge
      // (the wait counts are then exact, not the minimum over both paths).
      chunk1(0, va);
      chunk1(1, vb);
      for (int c = 2; c < nch; c += 2) {
        chunk1(c, va);
        chunk1(c + 1, vb);
      }
    }
    // D layout: element r of lane l is D[8 (r/4) + 4 (l/32) + r%4][l%32].
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r / 4) + 4 * h + (r % 4);
      sm.sred[wave][m * kTile + n] = S[r];
      if (m == n) sm.gred[wave][n] = G[r];
    }
    lds_barrier();

    // ---------------- softmax: thread -> destination j = tid / 8, sources 4 (tid % 8) .. + 3
    {
      const int j = tid / 8, i0 = 4 * (tid % 8);
      const int lim = n_src - n_dst + j;  // destination j reads sources 0..lim
      float sc[4];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q;
        float sv = 0.f, gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kFW; ++w2) {
          sv += sm.sred[w2][j * kTile + i];
          gv += sm.gred[w2][i];
        }
        const float r = 1.0f / sqrtf(gv / (float)d + a.eps);
        sc[q] = (j < n_dst && i <= lim) ? r * sv : -INFINITY;
        m = fmaxf(m, sc[q]);
      }
      m = group_max<8>(m);
      float e[4], l = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[q] = (sc[q] == -INFINITY) ? 0.f : expf(sc[q] - m);
        l += e[q];
      }
      l = group_sum<8>(l);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      *reinterpret_cast<float4*>(&sm.alpha[j][i0]) = make_float4(e[0] * inv, e[1] * inv, e[2] * inv, e[3] * inv);
    }
    lds_barrier();

    // ---------------- stage 2: H = alpha V
    // A operands: lane (h, j = l%32) holds alpha_part[j][src(b, h, e)] with
    // src(b, h, e) = 16 b + 8 (e/4) + 4 h + e%4, the source order the
    // transpose leaves in the B operand.
    uint4 ahi[2], alo[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const float4 x0 = *reinterpret_cast<const float4*>(&sm.alpha[n][16 * b2 + 4 * h]);
      const float4 x1 = *reinterpret_cast<const float4*>(&sm.alpha[n][16 * b2 + 8 + 4 * h]);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = bf2f(f2bf(x[e]));
        lo[e] = x[e] - hi[e];
      }
      ahi[b2] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
      alo[b2] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
    }
    {
      // Output tile addresses: row j = 8 (r/4) + 4 h + r%4 and channel 32 half + n
      // are one per-lane base plus compile-time offsets.
      unsigned char* obase = ot + 4 * h * kORow + 2 * n;
      auto chunk2 = [&](int c, uint4 (&v)[4]) {
        stage_chunk(vt, v, rowmask);
        load_chunk(rowp, min(c + 2, nch - 1) * kChunk, v);
        wave_lds_sync();
        uint4 op[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) op[s] = tile_operand(vt, s);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // D1[i][n'] = V[i][32 half + n']: lane (h, n') element r holds source 8 (r/4) + 4 h + r%4.
          f16acc D1 = {};
          D1 = mfma(op[2 * half], ident[0], D1);
          D1 = mfma(op[2 * half + 1], ident[1], D1);
          const uint4 b0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
          const uint4 b1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
          f16acc D2 = {};
          D2 = mfma(ahi[0], b0, D2);
          D2 = mfma(alo[0], b0, D2);
          D2 = mfma(ahi[1], b1, D2);
          D2 = mfma(alo[1], b1, D2);
          // D2[j][n'] -> output tile row j, channel 32 half + n'.
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *reinterpret_cast<bf16_t*>(obase + (8 * (r / 4) + (r % 4)) * kORow + 64 * half) = f2bf(D2[r]);
        }
        wave_lds_sync();
        const int ch = ch_base + c * kChunk + 8 * (lane & 7);
        // Rows past n_dst store row n_dst - 1 again (identical bytes), so the
        // stores need no branch.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = min(8 * u + (lane >> 3), n_dst - 1);
          const uint4 o = *reinterpret_cast<const uint4*>(ot + j * kORow + ((lane & 7) << 4));
          __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(out + ((int64_t)j * T + t) * d + ch));
        }
        wave_lds_sync();  // tiles are rewritten by the next chunk
      };
      uint4 va[4], vb[4];
      load_chunk(rowp, 0, va);
      __builtin_amdgcn_sched_barrier(0);  // keep the loop's load order (va, then vb)
      load_chunk(rowp, kChunk, vb);
      // nch is even and >= 2.  The first pair is peeled so that the loop head
      // sees the same outstanding loads and stores on entry as on the back edge
      // (the wait counts are then exact, not the minimum over both paths).
      chunk2(0, va);
      chunk2(1, vb);
      for (int c = 2; c < nch; c += 2) {
        chunk2(c, va);
        chunk2(c + 1, vb);
      }
    }
    // No barrier needed here: the next token writes sred/gred only after every
    // thread passed this token's second barrier (all softmax reads done), and
    // alpha only after its own first barrier (all operand reads done).
  }
}

// ---------------------------------------------------------------------------
// Resident variant for d <= 2048: 8 waves, one workgroup per CU.  Wave w owns
// channels [w d/8, (w+1) d/8) as NCH 64-channel chunks and keeps its whole
// slice of the token's sources (NCH x 4 KiB) in its own LDS slots through
// both contractions, so the sources are read from HBM exactly once.  The next
// token's slice is loaded into registers while the current token's reductions
// and weighted sums run, and each slot doubles as the output tile once its
// operands have been read.
constexpr int kRW = 8;            // waves per workgroup
constexpr int kRB = kRW * 64;     // threads per workgroup
constexpr int kRMaxCh = 4;        // chunks per wave at d = 2048

struct ResidentSmem {
  __attribute__((aligned(16))) unsigned char slots[kRW][kRMaxCh][kTile * kVRow];
  float sred[kRW / 2][kTile * kTile];                      // pairwise-summed partial S
  float gred[kRW][kTile];                                  // partial sums of squares
  __attribute__((aligned(16))) float alpha[kTile][kARow];  // alpha[j][i]
};

// The query operand of chunk g, k-step s and part p (0 = bf16 high, 1 =
// low) for this lane, formed from w and g exactly as k_full_qsplit forms it
// (used when each workgroup has a single token, so no packing launch runs).
__device__ __forceinline__ void full_q_operand(const FullArgs& a, int64_t g, int s, uint4& hi4, uint4& lo4) {
  const int lane = lane_id(), j = lane % 32;
  const int64_t k0 = (g * 4 + s) * 16 + 8 * (lane / 32);
  const int jc = j < a.n_dst ? j : (int)a.n_dst - 1;
  float q[8], hi[8], lo[8];
  if (a.gain != nullptr)
    fold_q8<true>(a.w + jc * a.d + k0, a.gain + jc * a.gain_ld + k0, q);
  else
    fold_q8<false>(a.w + jc * a.d + k0, nullptr, q);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float qe = j < a.n_dst ? q[e] : 0.f;
    hi[e] = bf2f(f2bf(qe));
    lo[e] = qe - hi[e];
  }
  hi4 = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
  lo4 = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
}

// FQ: form the query operands in the kernel (one token per workgroup) instead
// of reading them from the packed workspace.
// MH: H = 2, 4 or 8 heads (MHAR abstract), a head being 8 / H consecutive
// waves (d / H channels), each with its own depth softmax.  Each head's score
// partials are summed into its first wave through LDS, halving the waves per
// round; that wave forms the head's softmax in registers (a max and a sum
// over the 32 lanes holding one destination's sources), transposes alpha
// (bf16 high and low parts, exact) with a permuted identity into stage 2's
// operand order, and hands the operands to the head's other waves.  The sums
// of squares stay over the whole d.
template <int NCH, bool FQ, bool MH>
__global__ __launch_bounds__(kRB, 1) void k_full_resident(FullArgs a, const bf16_t* qpk) {
  __shared__ ResidentSmem sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: buffer offsets from it stay scalar
  const int d = (int)a.d, n_src = (int)a.n_src, n_dst = (int)a.n_dst;
  const int64_t T = a.T;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const int ch_base = wave * NCH * kChunk;
  const int h = lane >> 5, n = lane & 31;
  const uint4* qv = reinterpret_cast<const uint4*>(qpk) + lane;

  uint4 ident[2];
#pragma unroll
  for (int a2 = 0; a2 < 2; ++a2) {
    uint32_t wds[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo16 = (16 * a2 + 8 * h + 2 * q == n) ? 0x3F80u : 0u;
      const uint32_t hi16 = (16 * a2 + 8 * h + 2 * q + 1 == n) ? 0x3F80u : 0u;
      wds[q] = lo16 | (hi16 << 16);
    }
    ident[a2] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  }
  uint32_t rowmask[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) rowmask[u] = 8 * u + (lane >> 3) < n_src ? 0xFFFFFFFFu : 0u;

  // Loads of one token's slice: P[c][u] = row 8u + l/8, piece l%8 of chunk c.
  // Rows >= n_src read row 0 (masked when staged); the token index is clamped,
  // so every load is unconditional and the wait counts stay exact.
  uint4 P[NCH][4];
  auto load_slice = [&](int64_t tt) {
    // Addresses from an opaque lane id: recomputed per token instead of held
    // (and spilled) across the token loop.
    int ol = lane;
    asm volatile("" : "+v"(ol));
    const int piece = ol & 7;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 8 * u + (ol >> 3);
      const bf16_t* rp = src + ((int64_t)(r < n_src ? r : 0) * T + tt) * d + ch_base + 8 * piece;
#pragma unroll
      for (int c = 0; c < NCH; ++c) P[c][u] = *reinterpret_cast<const uint4*>(rp + c * kChunk);
    }
  };
  load_slice(blockIdx.x < T ? blockIdx.x : 0);

  auto token = [&](int64_t t) {
    // ---------------- stage the slice, then start loading the next token's
    wave_lds_sync();  // previous token's reads of the slots are done
#pragma unroll
    for (int c = 0; c < NCH; ++c) stage_chunk(sm.slots[wave][c], P[c], rowmask);
    wave_lds_sync();

    // ---------------- stage 1: S = Q V^T, G = V V^T over this wave's channels
    f16acc S = {}, G = {};
    // The query operands of chunk c + 1 are loaded while chunk c runs (the
    // next-token registers are free during this stage).
    {
      uint4 q[2][8];
      auto load_q = [&](int c, uint4 (&dst)[8]) {
        const int64_t g = ch_base / kChunk + c;
        if constexpr (FQ) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) full_q_operand(a, g, s2, dst[2 * s2], dst[2 * s2 + 1]);
        } else {
          // Buffer loads: the packed operands' base and offsets are scalar, so no
          // per-lane 64-bit address is held across the token loop.
          const __amdgpu_buffer_rsrc_t qr =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(qpk), 0, 0x7fffffff, kBufferWord3);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(qr, lane * 16, (int)((g * 8 + k) * 1024), 0);
            dst[k] = make_uint4(v.x, v.y, v.z, v.w);
          }
        }
      };
      load_q(0, q[0]);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (c + 1 < NCH) load_q(c + 1, q[(c + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // issue them now, not next to their use
        uint4 b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = tile_operand(sm.slots[wave][c], s);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          S = mfma(q[c & 1][2 * s], b[s], S);
          S = mfma(q[c & 1][2 * s + 1], b[s], S);
          G = mfma(b[s], b[s], G);
        }
        __builtin_amdgcn_sched_barrier(0);  // bound the live ranges to one chunk
      }
    }
    // The next token's slice is requested only now: the wait counter retires
    // loads in order, so loads issued before the query loads above would have
    // delayed stage 1.  From here on nothing loads from memory until the next
    // token is staged, so these loads overlap the reductions and stage 2.
    {
      const int64_t tn = t + gridDim.x;
      load_slice(tn < T ? tn : t);
    }
    uint4 ahi[2], alo[2];
    if constexpr (MH) {
      const int g = kRW / a.H;  // waves per head
      const int wh = wave % g, head = wave / g;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + 4 * h + (r % 4) == n) sm.gred[wave][n] = G[r];
      // Head partials: round with `half` moves waves [half, 2 half) of each head
      // onto waves [0, half) through slot head * half + (wh - half).
      for (int half = g / 2; half >= 1; half /= 2) {
        if (wh >= half && wh < 2 * half) {
          float* sl = sm.sred[head * half + (wh - half)];
#pragma unroll
          for (int r = 0; r < 16; ++r) sl[(8 * (r / 4) + 4 * h + (r % 4)) * kTile + n] = S[r];
        }
        lds_barrier();
        if (wh < half) {
          const float* sl = sm.sred[head * half + wh];
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] += sl[(8 * (r / 4) + 4 * h + (r % 4)) * kTile + n];
        }
        lds_barrier();
      }
      if (g == 1) lds_barrier();  // the sums of squares
      uint4* share = reinterpret_cast<uint4*>(sm.sred[head]);  // a head's operands: 4 x 64 uint4
      if (wh == 0) {
        float gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kRW; ++w2) gv += sm.gred[w2][n];
        const float ri = 1.0f / sqrtf(gv / (float)d + a.eps);
        // Lane (h, i = n), element r: destination j = 8 (r / 4) + 4 h + r % 4.
        float al[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 8 * (r / 4) + 4 * h + (r % 4);
          const bool valid = j < n_dst && n <= n_src - n_dst + j;
          const float sc = valid ? ri * S[r] : -INFINITY;
          const float m = group_max<32>(sc);
          const float e = valid ? expf(sc - m) : 0.f;
          const float l = group_sum<32>(e);
          al[r] = l > 0.f ? e / l : 0.f;
        }
        // alpha^T as A operands (row i = n, k-step b holding destinations
        // transposed_row(b, h, e)), times I[k][j] = 1 when transposed_row
        // maps k to j: D[i][j] = alpha[j][i] with lane (h, j) holding the
        // sources transposed_row(b2, h, e) of destination j.
        uint4 ip[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          uint32_t wds[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo16 = transposed_row(b, h, 2 * q) == n ? 0x3F80u : 0u;
            const uint32_t hi16 = transposed_row(b, h, 2 * q + 1) == n ? 0x3F80u : 0u;
            wds[q] = lo16 | (hi16 << 16);
          }
          ip[b] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        }
        // part 0: bf16(alpha); part 1: alpha - bf16(alpha), one at a time.
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          f16acc D = {};
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float hi = bf2f(f2bf(al[8 * b + e]));
              x[e] = part == 0 ? hi : al[8 * b + e] - hi;
            }
            D = mfma(pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]), ip[b], D);
          }
          uint4* dst = part == 0 ? ahi : alo;
          dst[0] = pack8(D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7]);
          dst[1] = pack8(D[8], D[9], D[10], D[11], D[12], D[13], D[14], D[15]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (g > 1) {
          share[0 * 64 + lane] = ahi[0];
          share[1 * 64 + lane] = ahi[1];
          share[2 * 64 + lane] = alo[0];
          share[3 * 64 + lane] = alo[1];
        }
      }
      if (g > 1) {
        lds_barrier();
        if (wh != 0) {
          ahi[0] = share[0 * 64 + lane];
          ahi[1] = share[1 * 64 + lane];
          alo[0] = share[2 * 64 + lane];
          alo[1] = share[3 * 64 + lane];
        }
      }
    } else {
    // ---------------- cross-wave sums: waves 4..7 hand their partials to waves 0..3
    if (wave >= kRW / 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.sred[wave - kRW / 2][(8 * (r / 4) + 4 * h + (r % 4)) * kTile + n] = S[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r / 4) + 4 * h + (r % 4) == n) sm.gred[wave][n] = G[r];
    lds_barrier();
    if (wave < kRW / 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* p = &sm.sred[wave][(8 * (r / 4) + 4 * h + (r % 4)) * kTile + n];
        *p = *p + S[r];
      }
    }
    lds_barrier();

    // ---------------- softmax (waves 0..3): destination j = tid / 8, sources 4 (tid % 8) .. + 3
    if (wave < kRW / 2) {
      const int j = tid / 8, i0 = 4 * (tid % 8);
      const int lim = n_src - n_dst + j;
      float sc[4];
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q;
        float sv = 0.f, gv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kRW / 2; ++w2) sv += sm.sred[w2][j * kTile + i];
#pragma unroll
        for (int w2 = 0; w2 < kRW; ++w2) gv += sm.gred[w2][i];
        const float r = 1.0f / sqrtf(gv / (float)d + a.eps);
        sc[q] = (j < n_dst && i <= lim) ? r * sv : -INFINITY;
        m = fmaxf(m, sc[q]);
      }
      m = group_max<8>(m);
      float e[4], l = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[q] = (sc[q] == -INFINITY) ? 0.f : expf(sc[q] - m);
        l += e[q];
      }
      l = group_sum<8>(l);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      *reinterpret_cast<float4*>(&sm.alpha[j][i0]) = make_float4(e[0] * inv, e[1] * inv, e[2] * inv, e[3] * inv);
    }
    lds_barrier();

    // ---------------- stage 2 operands: alpha in operand order, split hi + lo
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const float4 x0 = *reinterpret_cast<const float4*>(&sm.alpha[n][16 * b2 + 4 * h]);
      const float4 x1 = *reinterpret_cast<const float4*>(&sm.alpha[n][16 * b2 + 8 + 4 * h]);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = bf2f(f2bf(x[e]));
        lo[e] = x[e] - hi[e];
      }
      ahi[b2] = pack8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
      alo[b2] = pack8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
    }
    }  // H == 1

    // ---------------- stage 2: H = alpha V from the resident slots
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      unsigned char* slot = sm.slots[wave][c];
      uint4 op[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) op[s] = tile_operand(slot, s);
      wave_lds_sync();  // the slot becomes the output tile below
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f16acc D1 = {};
        D1 = mfma(op[2 * half], ident[0], D1);
        D1 = mfma(op[2 * half + 1], ident[1], D1);
        const uint4 b0 = pack8(D1[0], D1[1], D1[2], D1[3], D1[4], D1[5], D1[6], D1[7]);
        const uint4 b1 = pack8(D1[8], D1[9], D1[10], D1[11], D1[12], D1[13], D1[14], D1[15]);
        // H^T = V^T alpha^T: the transposed sources are the A operand and alpha
        // the B operand, so D[c'][j] leaves lane (h, j) with channels
        // 8q + 4h .. + 3 of destination j in elements 4q .. 4q + 3.
        f16acc D2 = {};
        D2 = mfma(b0, ahi[0], D2);
        D2 = mfma(b0, alo[0], D2);
        D2 = mfma(b1, ahi[1], D2);
        D2 = mfma(b1, alo[1], D2);
        // Tile row j = n, channels 32 half + 8q + 4h .. + 3: 8 bytes at offset 8h of
        // 16-byte piece 4 half + q (same swizzle as the sources).
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(slot + vpos(n, 4 * half + q) + 8 * h) =
              make_uint2(pack_bf2(D2[4 * q], D2[4 * q + 1]), pack_bf2(D2[4 * q + 2], D2[4 * q + 3]));
      }
      wave_lds_sync();
      const int ch = ch_base + c * kChunk + 8 * (lane & 7);
      uint4 o[4];
      int jr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        jr[u] = min(8 * u + (lane >> 3), n_dst - 1);  // rows past n_dst repeat row n_dst - 1
        o[u] = *reinterpret_cast<const uint4*>(slot + vpos(jr[u], lane & 7));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_nontemporal_store(v4u{o[u].x, o[u].y, o[u].z, o[u].w},
                                    reinterpret_cast<v4u*>(out + ((int64_t)jr[u] * T + t) * d + ch));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The first token is peeled so that the loop head sees the same outstanding
  // loads and stores on entry as on the back edge; the wait for the staged
  // slice then leaves the previous token's stores in flight.
  int64_t t = blockIdx.x;
  if (t < T) token(t);
  for (t += gridDim.x; t < T; t += gridDim.x) token(t);
}

bool al16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Shapes the resident kernel takes: d = 512 .. 2048 in steps of 512 (whole
// 64-channel chunks for each of the 8 waves); with heads, H = 2, 4 or 8 so
// that a head is a run of whole waves.
bool resident_shape(int64_t d, int H) {
  if (d % (kRW * kChunk) != 0 || d > kRW * kRMaxCh * kChunk) return false;
  return H == 1 || H == 2 || H == 4 || H == 8;
}

}  // namespace

size_t full_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t d, int H, int dtype) {
  if (full_wide_shape(n_src, n_dst, d, H, dtype)) return full_wide_workspace_bytes(n_dst, d);
  if (dtype != kBF16 || n_src > kTile || n_dst > n_src) return 0;
  if (H != 1 && !resident_shape(d, H)) return 0;
  return (size_t)2 * kTile * (size_t)d * sizeof(bf16_t);
}

bool full_fast_ok(const FullArgs& a) {
  if (a.dtype != kBF16 || a.T < 1) return false;
  if (full_one_ok(a)) return true;  // needs no workspace
  if (full_wide_shape(a.n_src, a.n_dst, a.d, a.H, a.dtype)) {
    if (a.ws == nullptr || a.ws_bytes < full_wide_workspace_bytes(a.n_dst, a.d)) return false;
    return al16(a.src) && al16(a.out) && al16(a.ws) && al16(a.w) && al16(a.gain);
  }
  if (a.H != 1 && !resident_shape(a.d, a.H)) return false;  // heads: the resident kernel only
  if (a.n_src > kTile || a.n_dst > a.n_src) return false;
  // Each wave streams an even number of whole 64-channel chunks.
  if (a.d % (2 * kFW * kChunk) != 0 || a.d > ((int64_t)1 << 16)) return false;
  const size_t need = full_fast_workspace_bytes(a.n_src, a.n_dst, a.d, a.H, a.dtype);
  if (a.ws == nullptr || a.ws_bytes < need) return false;
  return al16(a.src) && al16(a.out) && al16(a.ws) && al16(a.w) && al16(a.gain);
}

// With at most one token per workgroup the resident kernel forms the query
// operands itself and the packing launch is skipped (one launch per call).
template <int NCH, bool MH>
hipError_t launch_resident(const FullArgs& a, const bf16_t* qpk, hipStream_t st) {
  int64_t grid = num_cus();
  if (grid >= a.T) {
    hipLaunchKernelGGL((k_full_resident<NCH, true, MH>), dim3((unsigned)a.T), dim3(kRB), 0, st, a, qpk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_full_qsplit, dim3(64), dim3(256), 0, st, a, const_cast<bf16_t*>(qpk));
  hipLaunchKernelGGL((k_full_resident<NCH, false, MH>), dim3((unsigned)grid), dim3(kRB), 0, st, a, qpk);
  return hipGetLastError();
}

template <int NCH>
hipError_t launch_resident_h(const FullArgs& a, const bf16_t* qpk, hipStream_t st) {
  return a.H > 1 ? launch_resident<NCH, true>(a, qpk, st) : launch_resident<NCH, false>(a, qpk, st);
}

const char* full_fast_variant(const FullArgs& a) {
  if (full_one_ok(a)) return "full_one";
  return full_wide_shape(a.n_src, a.n_dst, a.d, a.H, a.dtype) ? "full_wide" : "full_fast";
}

hipError_t launch_full_fast(const FullArgs& a, hipStream_t st) {
  if (full_one_ok(a)) return launch_full_one(a, st);
  if (full_wide_shape(a.n_src, a.n_dst, a.d, a.H, a.dtype)) return launch_full_wide(a, st);
  bf16_t* qpk = static_cast<bf16_t*>(a.ws);
  if (resident_shape(a.d, a.H)) {
    switch (a.d / (kRW * kChunk)) {
      case 1: return launch_resident_h<1>(a, qpk, st);
      case 2: return launch_resident_h<2>(a, qpk, st);
      case 3: return launch_resident_h<3>(a, qpk, st);
      case 4: return launch_resident_h<4>(a, qpk, st);
      default: break;
    }
  }
  hipLaunchKernelGGL(k_full_qsplit, dim3(64), dim3(256), 0, st, a, qpk);
  int per_cu = 0;
  hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(k_full_fast), kFB, &per_cu);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)num_cus() * per_cu;
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL(k_full_fast, dim3((unsigned)grid), dim3(kFB), 0, st, a, (const bf16_t*)qpk);
  return hipGetLastError();
}

}  // namespace attnres
