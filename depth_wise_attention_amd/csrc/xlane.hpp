// Cross-lane reductions for wave64 on gfx950, built from v_permlane32_swap,
// v_permlane16_swap and DPP row/quad/bank controls (no LDS traffic).
#pragma once

#include "common.hpp"

namespace attnres {

namespace dpp {
constexpr int kXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRor4 = 0x124;  // row_ror:4  (lane L reads lane (L - 4) mod 16 of its row)
constexpr int kRor8 = 0x128;  // row_ror:8  (lane L reads lane L ^ 8)
constexpr int kRor12 = 0x12C; // row_ror:12 (lane L reads lane (L + 4) mod 16 of its row)
}  // namespace dpp

template <int Ctrl, int BankMask = 0xF>
__device__ __forceinline__ float dpp_move(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), Ctrl, 0xF,
                                                    BankMask, false));
}

// Value of lane (lane ^ 4).  row_ror:n gives lane L the value of lane (L - n)
// mod 16 within its row.  Lanes whose bit 2 is set (DPP banks 1 and 3) need
// lane L - 4 (row_ror:4); the others (banks 0 and 2) need L + 4 (row_ror:12).
__device__ __forceinline__ float xor4(float v) {
  const float t = dpp_move<dpp::kRor4, 0xA>(0.f, v);
  return dpp_move<dpp::kRor12, 0x5>(t, v);
}

// {a + a[lane ^ 32] in lanes 0..31, b + b[lane ^ 32] in lanes 32..63}.
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// {a + a[lane ^ 16] in rows 0 and 2, b + b[lane ^ 16] in rows 1 and 3} (rows of 16 lanes).
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over all 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_allsum(float v) {
  v += dpp_move<dpp::kXor1>(0.f, v);
  v += dpp_move<dpp::kXor2>(0.f, v);
  v += xor4(v);
  v += dpp_move<dpp::kRor8>(0.f, v);
  v = swap16_add(v, v);
  v = swap32_add(v, v);
  return v;
}

// op(v, v of lane ^ OFF) for OFF in {1, 2, 4, 8, 16, 32}, without LDS.  For 16
// and 32 the permlane swap of v with itself leaves {v, v[lane ^ OFF]} in its
// two results (in some order), so the op must be symmetric.
template <int OFF, typename Op>
__device__ __forceinline__ float xor_combine(float v, Op op) {
  if constexpr (OFF == 1) {
    return op(v, dpp_move<dpp::kXor1>(0.f, v));
  } else if constexpr (OFF == 2) {
    return op(v, dpp_move<dpp::kXor2>(0.f, v));
  } else if constexpr (OFF == 4) {
    return op(v, xor4(v));
  } else if constexpr (OFF == 8) {
    return op(v, dpp_move<dpp::kRor8>(0.f, v));
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    static_assert(OFF == 32, "offset must be a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

struct SumOp {
  __device__ __forceinline__ float operator()(float x, float y) const { return x + y; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float x, float y) const { return fmaxf(x, y); }
};

// Butterfly over lane offsets LO, 2 LO, ..., < HI: with LO = 1 every lane of a
// group of HI consecutive lanes ends with the group's total; with LO = G, HI =
// 64 every lane ends with the total over the lanes congruent to it mod G.
template <int LO, int HI, typename Op>
__device__ __forceinline__ float butterfly(float v, Op op) {
  if constexpr (LO < HI) {
    v = xor_combine<LO>(v, op);
    return butterfly<2 * LO, HI>(v, op);
  } else {
    return v;
  }
}

template <int G> __device__ __forceinline__ float group_sum(float v) { return butterfly<1, G>(v, SumOp()); }
template <int G> __device__ __forceinline__ float group_max(float v) { return butterfly<1, G>(v, MaxOp()); }

// Transpose-reduce of 64 values per lane: on return, lane L holds the sum over
// all 64 lanes of value index L.  Each halving stage keeps, per lane, the half
// of the values selected by one lane bit and adds the partner lane's copy.
__device__ __forceinline__ float transpose_reduce64(const float (&v)[64]) {
  const int lane = lane_id();
  float a[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) a[m] = swap32_add(v[m], v[m + 32]);  // lane bit 5 -> index bit 5
  float b[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) b[m] = swap16_add(a[m], a[m + 16]);  // lane bit 4 -> index bit 4
  float c[8];
  const bool hi8 = (lane & 8) != 0;
#pragma unroll
  for (int m = 0; m < 8; ++m) {                                      // lane bit 3 -> index bit 3
    const float send = hi8 ? b[m] : b[m + 8];
    const float keep = hi8 ? b[m + 8] : b[m];
    c[m] = keep + dpp_move<dpp::kRor8>(0.f, send);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {                                      // full sums over lane bits 0..2
    c[m] += dpp_move<dpp::kXor1>(0.f, c[m]);
    c[m] += dpp_move<dpp::kXor2>(0.f, c[m]);
    c[m] += xor4(c[m]);
  }
  const int sel = lane & 7;
  float r = c[0];
#pragma unroll
  for (int m = 1; m < 8; ++m) r = (sel == m) ? c[m] : r;
  return r;
}

// One halving stage of a transposing reduction over lane bit OFF (8, 4, 2 or
// 1): the lane keeps the value selected by its own bit and adds its partner's
// copy of that value.
template <int OFF>
__device__ __forceinline__ float exchange_add(float lo, float hi) {
  const bool up = (lane_id() & OFF) != 0;
  const float keep = up ? hi : lo, send = up ? lo : hi;
  float got;
  if constexpr (OFF == 8) {
    got = dpp_move<dpp::kRor8>(0.f, send);
  } else if constexpr (OFF == 4) {
    got = xor4(send);
  } else if constexpr (OFF == 2) {
    got = dpp_move<dpp::kXor2>(0.f, send);
  } else {
    static_assert(OFF == 1, "lane bit below 16");
    got = dpp_move<dpp::kXor1>(0.f, send);
  }
  return keep + got;
}

// Transpose-reduce of P = 2^k values per lane (P = 8, 32; 16 and 64 have their
// own forms below): on return, lane L holds the sum over all 64 lanes of value
// index L >> (6 - k).  Lane bits 5, 4, ... select index bits k-1, k-2, ... in k
// halving stages; the 6 - k lowest lane bits are summed out.
template <int P>
__device__ __forceinline__ float transpose_reduce_pow2(const float (&v)[P]) {
  static_assert(P == 8 || P == 32, "8 or 32 values");
  float a[P / 2];
#pragma unroll
  for (int m = 0; m < P / 2; ++m) a[m] = swap32_add(v[m], v[m + P / 2]);      // lane bit 5
  float b[P / 4];
#pragma unroll
  for (int m = 0; m < P / 4; ++m) b[m] = swap16_add(a[m], a[m + P / 4]);      // lane bit 4
  if constexpr (P == 8) {
    float e = exchange_add<8>(b[0], b[1]);                                     // lane bit 3
    e += xor4(e);                                                              // sum bits 2..0
    e += dpp_move<dpp::kXor2>(0.f, e);
    e += dpp_move<dpp::kXor1>(0.f, e);
    return e;
  } else {
    float c[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) c[m] = exchange_add<8>(b[m], b[m + 4]);       // lane bit 3
    float e2[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) e2[m] = exchange_add<4>(c[m], c[m + 2]);      // lane bit 2
    float e = exchange_add<2>(e2[0], e2[1]);                                   // lane bit 1
    e += dpp_move<dpp::kXor1>(0.f, e);                                         // sum bit 0
    return e;
  }
}

// Transpose-reduce of 16 values per lane: on return, lane L holds the sum over
// all 64 lanes of value index L >> 2.  Lane bits 5, 4, 3 and 2 select index
// bits 3, 2, 1 and 0 in four halving stages; the last two lane bits are
// summed out.
__device__ __forceinline__ float transpose_reduce16(const float (&v)[16]) {
  const int lane = lane_id();
  float a[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) a[m] = swap32_add(v[m], v[m + 8]);    // lane bit 5 -> index bit 3
  float b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = swap16_add(a[m], a[m + 4]);    // lane bit 4 -> index bit 2
  float c[2];
  const bool hi8 = (lane & 8) != 0;
#pragma unroll
  for (int m = 0; m < 2; ++m) {                                      // lane bit 3 -> index bit 1
    const float send = hi8 ? b[m] : b[m + 2];
    const float keep = hi8 ? b[m + 2] : b[m];
    c[m] = keep + dpp_move<dpp::kRor8>(0.f, send);
  }
  const bool hi4 = (lane & 4) != 0;                                  // lane bit 2 -> index bit 0
  float e = (hi4 ? c[1] : c[0]) + xor4(hi4 ? c[0] : c[1]);
  e += dpp_move<dpp::kXor1>(0.f, e);
  e += dpp_move<dpp::kXor2>(0.f, e);
  return e;
}

// Reduce P values per lane over the wave.  out[g] in lane L is the total of
// value 64*g + L (zero for indices >= P).
template <int P>
__device__ __forceinline__ void wave_reduce_values(const float (&v)[P], float (&out)[(P + 63) / 64]) {
#pragma unroll
  for (int g = 0; g < (P + 63) / 64; ++g) {
    float t[64];
#pragma unroll
    for (int m = 0; m < 64; ++m) t[m] = (64 * g + m < P) ? v[64 * g + m] : 0.f;
    out[g] = transpose_reduce64(t);
  }
}

}  // namespace attnres
