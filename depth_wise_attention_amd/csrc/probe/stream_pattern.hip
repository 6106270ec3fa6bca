// Streaming-pattern probe: the HBM ceiling of a kernel's access pattern with
// no arithmetic.  Not part of the routing library: it is built into its own
// libattnres_probe.so and used only by bench.py --ceilings, which reports
// what each routing kernel's read/write mix can reach on the device at hand.
//
// Per token t and 16-byte piece c of a d-wide bf16 row, the probe reads row t
// of each of n_read source planes ([n_read][T][d]) and writes row t of each of
// n_write destination planes ([n_write][T][d]) -- the per-token traffic of a
// routing kernel (for example 8 rows read and 4 written for Block Phase 1).
// Consecutive threads take consecutive pieces of a row, as the routing
// kernels do.  `mode` selects the flavour of the memory operations:
//   bit 0  plain loads instead of nontemporal ones
//   bit 1  plain stores instead of nontemporal ones
//   bit 2  each thread takes two adjacent 16-byte pieces (32 bytes) per row
// The written value depends on every loaded value, so no load is dead.  With
// n_write == 0 the combination is written only when it equals an improbable
// constant.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 64;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <bool PlainLd, bool PlainSt, int K>
__global__ __launch_bounds__(kThreads) void k_stream_pattern(const uint16_t* src, int n_read, uint16_t* dst,
                                                             int n_write, int64_t T, int64_t d, uint32_t* sink) {
  const int64_t pieces = d / (8 * K);
  const int64_t units = T * pieces;
  const int64_t plane = T * d;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += (int64_t)gridDim.x * kThreads) {
    const int64_t off = (u / pieces) * d + (u % pieces) * 8 * K;
    v4u acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = (v4u){0u, 0u, 0u, 0u};
    for (int r = 0; r < n_read; ++r)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const v4u* p = reinterpret_cast<const v4u*>(src + r * plane + off) + k;
        acc[k] ^= PlainLd ? *p : __builtin_nontemporal_load(p);
      }
    for (int w = 0; w < n_write; ++w)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const v4u val = acc[k] ^ (v4u){(uint32_t)w, 0u, 0u, 0u};
        v4u* p = reinterpret_cast<v4u*>(dst + w * plane + off) + k;
        if constexpr (PlainSt)
          *p = val;
        else
          __builtin_nontemporal_store(val, p);
      }
    if (n_write == 0 && acc[0].x == 0x9E3779B9u && acc[K - 1].y == 0x7F4A7C15u) sink[0] = acc[0].z;
  }
}

template <bool PlainLd, bool PlainSt, int K>
void launch(int64_t blocks, hipStream_t stream, const uint16_t* src, int n_read, uint16_t* dst, int n_write,
            int64_t T, int64_t d, uint32_t* sink) {
  hipLaunchKernelGGL((k_stream_pattern<PlainLd, PlainSt, K>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, src,
                     n_read, dst, n_write, T, d, sink);
}

}  // namespace

extern "C" {

// Runs the pattern once on `stream`.  src holds n_read planes and dst n_write
// planes of T x d bf16 (16-byte aligned, d a multiple of 8, of 16 with mode
// bit 2); sink is one 4-byte device word; mode as above (0..7).  Returns 0,
// -1 for invalid arguments (nothing is enqueued), -3 for a launch error.
int attnres_probe_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, int64_t T, int64_t d,
                         void* sink, int64_t blocks, int32_t mode, hipStream_t stream) {
  if (n_read < 0 || n_write < 0 || n_read + n_write < 1 || n_read > kMaxRows || n_write > kMaxRows || T < 1 ||
      d < 8 || d % 8 != 0 || blocks < 1 || blocks > (1 << 20) || sink == nullptr || mode < 0 || mode > 7)
    return -1;
  if ((mode & 4) != 0 && d % 16 != 0) return -1;
  if ((n_read > 0 && (src == nullptr || ((uintptr_t)src & 15u) != 0)) ||
      (n_write > 0 && (dst == nullptr || ((uintptr_t)dst & 15u) != 0)))
    return -1;
  const uint16_t* s16 = static_cast<const uint16_t*>(src);
  uint16_t* d16 = static_cast<uint16_t*>(dst);
  uint32_t* k32 = static_cast<uint32_t*>(sink);
  const int nr = (int)n_read, nw = (int)n_write;
  switch (mode) {
    case 0: launch<false, false, 1>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 1: launch<true, false, 1>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 2: launch<false, true, 1>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 3: launch<true, true, 1>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 4: launch<false, false, 2>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 5: launch<true, false, 2>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    case 6: launch<false, true, 2>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
    default: launch<true, true, 2>(blocks, stream, s16, nr, d16, nw, T, d, k32); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
