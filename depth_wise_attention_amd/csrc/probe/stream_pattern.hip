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
// kernels do, and the loads are nontemporal like theirs.  The written value
// depends on every loaded value, so no load is dead.  With n_write == 0 the
// combination is written only when it equals an improbable constant.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 64;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_stream_pattern(const uint16_t* src, int n_read, uint16_t* dst,
                                                             int n_write, int64_t T, int64_t d, uint32_t* sink) {
  const int64_t pieces = d / 8;
  const int64_t units = T * pieces;
  const int64_t plane = T * d;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += (int64_t)gridDim.x * kThreads) {
    const int64_t off = (u / pieces) * d + (u % pieces) * 8;
    v4u acc = {0u, 0u, 0u, 0u};
    for (int r = 0; r < n_read; ++r)
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src + r * plane + off));
    for (int w = 0; w < n_write; ++w) {
      const v4u val = acc ^ (v4u){(uint32_t)w, 0u, 0u, 0u};
      __builtin_nontemporal_store(val, reinterpret_cast<v4u*>(dst + w * plane + off));
    }
    if (n_write == 0 && acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[0] = acc.z;
  }
}

}  // namespace

extern "C" {

// Runs the pattern once on `stream`.  src holds n_read planes and dst n_write
// planes of T x d bf16 (16-byte aligned, d a multiple of 8); sink is one
// 4-byte device word.  Returns 0, -1 for invalid arguments (nothing is
// enqueued), -3 for a launch error.
int attnres_probe_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, int64_t T, int64_t d,
                         void* sink, int64_t blocks, hipStream_t stream) {
  if (n_read < 0 || n_write < 0 || n_read + n_write < 1 || n_read > kMaxRows || n_write > kMaxRows || T < 1 ||
      d < 8 || d % 8 != 0 || blocks < 1 || blocks > (1 << 20) || sink == nullptr)
    return -1;
  if ((n_read > 0 && (src == nullptr || ((uintptr_t)src & 15u) != 0)) ||
      (n_write > 0 && (dst == nullptr || ((uintptr_t)dst & 15u) != 0)))
    return -1;
  hipLaunchKernelGGL(k_stream_pattern, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(src), (int)n_read, static_cast<uint16_t*>(dst), (int)n_write, T, d,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
