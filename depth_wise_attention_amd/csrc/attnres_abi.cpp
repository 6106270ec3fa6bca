// C ABI of libattnres.so: argument validation, error reporting and kernel
// dispatch.  Every check runs before the first HIP call, so a rejected call
// enqueues nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdint>

#include "../../include/attnres.h"
#include "launch.hpp"

using namespace attnres;

namespace {

thread_local char g_err[1024] = "";
std::atomic<int> g_policy{0};

constexpr int kMaxSources = 64;
constexpr int64_t kMaxD = int64_t(1) << 22;
constexpr size_t kAlign = 256;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTNRES_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// a * b * c without int64 overflow; false on overflow or negative operands.
bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  if (a < 0 || b < 0 || c < 0) return false;
  int64_t ab;
  if (__builtin_mul_overflow(a, b, &ab)) return false;
  return !__builtin_mul_overflow(ab, c, out);
}

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& x, const Range& y) {
  if (x.p == nullptr || y.p == nullptr || x.bytes == 0 || y.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)x.p, a1 = a0 + x.bytes;
  const uintptr_t b0 = (uintptr_t)y.p, b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

// Each output must not overlap any input or any other output.
int check_aliasing(const Range* ins, int nin, const Range* outs, int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], ins[i]))
        return fail(ATTNRES_ERR_INVALID, "output %s overlaps input %s", outs[o].name, ins[i].name);
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p]))
        return fail(ATTNRES_ERR_INVALID, "outputs %s and %s overlap", outs[o].name, outs[p].name);
  }
  return ATTNRES_OK;
}

// Checks shared by every call.  elems = T*d (validated for overflow).
int check_common(int64_t T, int64_t d, int32_t H, int32_t dtype, float eps, const float* gain,
                 int64_t gain_ld, int64_t* td) {
  if (dtype != ATTNRES_F32 && dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "dtype %d is not ATTNRES_F32 (0) or ATTNRES_BF16 (1)", dtype);
  if (T < 0) return fail(ATTNRES_ERR_INVALID, "T = %lld is negative", (long long)T);
  if (d < 1) return fail(ATTNRES_ERR_INVALID, "d = %lld must be >= 1", (long long)d);
  if (d > kMaxD) return fail(ATTNRES_ERR_UNSUPPORTED, "d = %lld exceeds %lld", (long long)d, (long long)kMaxD);
  if (H < 1) return fail(ATTNRES_ERR_INVALID, "H = %d must be >= 1", H);
  if (d % H != 0) return fail(ATTNRES_ERR_INVALID, "d = %lld is not divisible by H = %d", (long long)d, H);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(ATTNRES_ERR_INVALID, "eps must be finite and >= 0");
  if (gain != nullptr && gain_ld != 0 && gain_ld != d)
    return fail(ATTNRES_ERR_INVALID, "gain_ld = %lld must be 0 (shared) or d = %lld", (long long)gain_ld,
                (long long)d);
  if (!mul3(T, d, 4, td)) return fail(ATTNRES_ERR_INVALID, "T * d overflows");
  *td = T * d;
  return ATTNRES_OK;
}

// Phase-1 state: fp32, or with bf16 I/O the scaled fp16 state.  A bf16 state
// keeps 8 significant bits, and the merge's second rounding then exceeds the
// bf16 tolerance at full size, so it is refused.
int check_state_dtype(int32_t o_dtype, int32_t dtype) {
  if (o_dtype == ATTNRES_F32) return ATTNRES_OK;
  if (o_dtype == ATTNRES_F16 && dtype == ATTNRES_BF16) return ATTNRES_OK;
  if (o_dtype == ATTNRES_BF16 && dtype == ATTNRES_BF16)
    return fail(ATTNRES_ERR_UNSUPPORTED,
                "a bf16 Phase-1 state is not supported (use ATTNRES_F16, the scaled fp16 state, or ATTNRES_F32)");
  return fail(ATTNRES_ERR_INVALID, "o_dtype %d must be ATTNRES_F32, or ATTNRES_F16 with bf16 I/O", o_dtype);
}

int check_count(int64_t n, int64_t td, int64_t es, const char* name, size_t* bytes) {
  int64_t b;
  if (!mul3(n, td, es, &b)) return fail(ATTNRES_ERR_INVALID, "%s size overflows", name);
  *bytes = (size_t)b;
  return ATTNRES_OK;
}

#define RETURN_IF(x)          \
  do {                        \
    const int rc_ = (x);      \
    if (rc_ != ATTNRES_OK) return rc_; \
  } while (0)

#define REQUIRE_PTR(p, name) \
  if ((p) == nullptr) return fail(ATTNRES_ERR_INVALID, "%s is NULL", name)

bool use_fast() { return g_policy.load(std::memory_order_relaxed) == 0; }

int run_phase1(const Phase1Args& a, hipStream_t st) {
  const hipError_t e = (use_fast() && phase1_fast_ok(a)) ? launch_phase1_fast(a, st)
                                                         : launch_phase1_generic(a, st);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "phase 1 launch");
}

int run_phase2(const Phase2Args& a, hipStream_t st) {
  const hipError_t e = (use_fast() && phase2_fast_ok(a)) ? launch_phase2_fast(a, st)
                                                         : launch_phase2_generic(a, st);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "phase 2 launch");
}

int64_t bwd_slots(int64_t T) {
  const int64_t s = (T + 3) / 4 * 4;
  return s < kMaxBwdSlots ? s : kMaxBwdSlots;
}

int64_t full_bwd_slots(int64_t T) {
  const int64_t s = (T + 3) / 4 * 4;
  return s < kMaxFullBwdSlots ? s : kMaxFullBwdSlots;
}

}  // namespace

namespace attnres {
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// The occupancy query is a host call that costs microseconds; at decode sizes
// a launch is itself a few microseconds, so the answer is kept per device,
// kernel and block size.
hipError_t blocks_per_cu(const void* kern, int block, int* out, size_t dyn_lds) {
  struct Entry {
    int dev;
    const void* kern;
    int block;
    size_t lds;
    int value;
  };
  static std::mutex mu;
  static Entry table[512];
  static int used = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (table[i].dev == dev && table[i].kern == kern && table[i].block == block && table[i].lds == dyn_lds) {
        *out = table[i].value;
        return hipSuccess;
      }
  }
  int v = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, block, dyn_lds);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 512) table[used++] = Entry{dev, kern, block, dyn_lds, v};
  *out = v;
  return hipSuccess;
}
}  // namespace attnres

extern "C" {

const char* attnres_last_error(void) { return g_err; }

size_t attnres_msar_fwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int32_t dtype) {
  if (n_src < 1 || n_src > kMaxSources || n_dst < 1 || n_dst > n_src || T < 1 || d < 1 || d > kMaxD) return 0;
  return msar_fast_workspace_bytes(n_src, n_dst, T, d, dtype);
}

int attnres_msar_fwd(const void* src, int64_t n_src, int64_t T, int64_t d, const float* w, const float* conv,
                     const float* mix, int64_t n_dst, float eps, int32_t dtype, void* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, 1, dtype, eps, nullptr, 0, &td));
  if (n_src < 1 || n_src > kMaxSources)
    return fail(ATTNRES_ERR_INVALID, "n_src = %lld must be in [1, %d]", (long long)n_src, kMaxSources);
  if (n_dst < 1 || n_dst > n_src)
    return fail(ATTNRES_ERR_INVALID, "n_dst = %lld must be in [1, n_src = %lld]", (long long)n_dst,
                (long long)n_src);
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(src, "src");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(conv, "conv");
  REQUIRE_PTR(mix, "mix");
  REQUIRE_PTR(out, "out");
  const size_t need = attnres_msar_fwd_workspace_size(n_src, n_dst, T, d, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0,
                need);
  const int64_t es = (int64_t)dt_size(dtype);
  size_t b_src, b_out, b_w, b_mix;
  RETURN_IF(check_count(n_src, td, es, "src", &b_src));
  RETURN_IF(check_count(n_dst, td, es, "out", &b_out));
  RETURN_IF(check_count(n_dst * kMsarStreams, d, 4, "w", &b_w));
  RETURN_IF(check_count(n_dst * kMsarStreams * kMsarStreams, d, 4, "mix", &b_mix));
  const Range ins[] = {{src, b_src, "src"},
                       {w, b_w, "w"},
                       {conv, (size_t)(kMsarTaps * d * 4), "conv"},
                       {mix, b_mix, "mix"}};
  const Range outs[] = {{out, b_out, "out"}, {need > 0 ? ws : nullptr, need, "ws"}};
  RETURN_IF(check_aliasing(ins, 4, outs, 2));
  MsarArgs a{src, n_src, T, d, w, conv, mix, n_dst, eps, dtype, out, need > 0 ? ws : nullptr, need};
  const hipError_t e = (use_fast() && msar_fast_ok(a)) ? launch_msar_fast(a, stream) : launch_msar_generic(a, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "MSAR forward launch");
}

namespace {
int check_bmsar_shape(int64_t T, int64_t d, int32_t dtype, float eps) {
  if (dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_UNSUPPORTED, "Block MSAR takes bf16 activations (dtype %d)", dtype);
  if (T < 0) return fail(ATTNRES_ERR_INVALID, "T = %lld is negative", (long long)T);
  if (d < 1 || d % 512 != 0 || d > ((int64_t)1 << 20))
    return fail(ATTNRES_ERR_UNSUPPORTED, "Block MSAR needs d a multiple of 512 up to 2^20 (d = %lld)", (long long)d);
  if (T > ((int64_t)1 << 30)) return fail(ATTNRES_ERR_UNSUPPORTED, "T = %lld exceeds 2^30", (long long)T);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(ATTNRES_ERR_INVALID, "eps must be finite and >= 0");
  return ATTNRES_OK;
}

bool aligned16p(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
}  // namespace

size_t attnres_block_msar_phase1_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d) {
  return bmsar_phase1_workspace_bytes(N, S, T, d);
}

int attnres_block_msar_phase1(const void* reps, int64_t N, int64_t T, int64_t d, const float* w, int64_t S,
                              const float* conv, const float* mix1, float eps, int32_t dtype, void* h1,
                              void* o_state, float* o_scale, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  clear_error();
  RETURN_IF(check_bmsar_shape(T, d, dtype, eps));
  if (N < 1) return fail(ATTNRES_ERR_INVALID, "N = %lld must be >= 1", (long long)N);
  if (N > kMsarFastMaxSources)
    return fail(ATTNRES_ERR_UNSUPPORTED, "Block MSAR takes at most %d reps (N = %lld)", kMsarFastMaxSources,
                (long long)N);
  if (S < 1) return fail(ATTNRES_ERR_INVALID, "S = %lld must be >= 1", (long long)S);
  if (S > 4) return fail(ATTNRES_ERR_UNSUPPORTED, "Block MSAR takes at most 4 sublayers (S = %lld)", (long long)S);
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(reps, "reps");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(conv, "conv");
  REQUIRE_PTR(mix1, "mix1");
  REQUIRE_PTR(h1, "h1");
  REQUIRE_PTR(o_scale, "o_scale");
  if (S > 1) {
    REQUIRE_PTR(o_state, "o_state");
    REQUIRE_PTR(lse, "lse");
  }
  const size_t need = attnres_block_msar_phase1_workspace_size(N, S, T, d);
  if (ws == nullptr || ws_bytes < need)
    return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0, need);
  for (const void* q : {reps, (const void*)w, (const void*)conv, (const void*)mix1, (const void*)h1,
                        (const void*)o_state, (const void*)o_scale, (const void*)lse, (const void*)ws})
    if (!aligned16p(q)) return fail(ATTNRES_ERR_INVALID, "Block MSAR pointers must be 16-byte aligned");
  const size_t td = (size_t)(T * d);
  const Range ins[] = {{reps, (size_t)N * td * 2, "reps"},
                       {w, (size_t)(S * kMsarStreams * d * 4), "w"},
                       {conv, (size_t)(kMsarTaps * d * 4), "conv"},
                       {mix1, (size_t)(kMsarStreams * d * kMsarStreams * 4), "mix1"}};
  const Range outs[] = {{h1, td * 2, "h1"},
                        {S > 1 ? o_state : nullptr, (size_t)(S - 1) * kMsarStreams * td * 2, "o_state"},
                        {o_scale, (size_t)T * 4, "o_scale"},
                        {S > 1 ? lse : nullptr, (size_t)((S - 1) * kMsarStreams * T * 4), "lse"},
                        {ws, need, "ws"}};
  RETURN_IF(check_aliasing(ins, 4, outs, 5));
  BmsarCall c{reps, N, T, d, w, S, conv, mix1, eps, h1, o_state, o_scale, lse, ws};
  const hipError_t e = launch_bmsar_phase1(c, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "Block MSAR phase 1 launch");
}

size_t attnres_block_msar_phase2_workspace_size(int64_t T, int64_t d) { return bmsar_phase2_workspace_bytes(T, d); }

int attnres_block_msar_phase2(const void* o_i, const float* o_scale, const float* lse_i, const void* partial,
                              int64_t T, int64_t d, const float* w_i, const float* conv, const float* mix_i, float eps,
                              int32_t dtype, void* h_i, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  RETURN_IF(check_bmsar_shape(T, d, dtype, eps));
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(o_i, "o_i");
  REQUIRE_PTR(o_scale, "o_scale");
  REQUIRE_PTR(lse_i, "lse_i");
  REQUIRE_PTR(partial, "partial");
  REQUIRE_PTR(w_i, "w_i");
  REQUIRE_PTR(conv, "conv");
  REQUIRE_PTR(mix_i, "mix_i");
  REQUIRE_PTR(h_i, "h_i");
  const size_t need = attnres_block_msar_phase2_workspace_size(T, d);
  if (ws == nullptr || ws_bytes < need)
    return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0, need);
  for (const void* q : {o_i, (const void*)o_scale, (const void*)lse_i, partial, (const void*)w_i,
                        (const void*)conv, (const void*)mix_i, (const void*)h_i, (const void*)ws})
    if (!aligned16p(q)) return fail(ATTNRES_ERR_INVALID, "Block MSAR pointers must be 16-byte aligned");
  const size_t td = (size_t)(T * d);
  const Range ins[] = {{o_i, kMsarStreams * td * 2, "o_i"},
                       {o_scale, (size_t)T * 4, "o_scale"},
                       {lse_i, (size_t)(kMsarStreams * T * 4), "lse_i"},
                       {partial, td * 2, "partial"},
                       {w_i, (size_t)(kMsarStreams * d * 4), "w_i"},
                       {conv, (size_t)(kMsarTaps * d * 4), "conv"},
                       {mix_i, (size_t)(kMsarStreams * d * kMsarStreams * 4), "mix_i"}};
  const Range outs[] = {{h_i, td * 2, "h_i"}, {ws, need, "ws"}};
  RETURN_IF(check_aliasing(ins, 7, outs, 2));
  Bmsar2Call c{o_i, o_scale, lse_i, partial, T, d, w_i, conv, mix_i, eps, h_i, ws};
  const hipError_t e = launch_bmsar_phase2(c, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "Block MSAR phase 2 launch");
}

int attnres_version(void) { return (2 << 16) | 6; }

int attnres_kernel_variant(int32_t op, int64_t N, int64_t S, int64_t T, int64_t d, int32_t H, int32_t dtype,
                           int32_t o_dtype, char* buf, size_t len) {
  clear_error();
  if (buf == nullptr || len == 0) return fail(ATTNRES_ERR_INVALID, "buf is NULL or empty");
  buf[0] = '\0';
  // Any 16-byte-aligned address: the predicates below only test alignment.
  void* p = reinterpret_cast<void*>((uintptr_t)4096);
  const float* fp = static_cast<const float*>(p);
  const bool fast = use_fast();
  switch (op) {
    case ATTNRES_OP_PHASE1: {
      Phase1Args a{p, N, T, d, fp, S, fp, d, 1e-6f, H, dtype, p, dtype, p, o_dtype, static_cast<float*>(p),
                   static_cast<float*>(p)};
      if (fast) phase1_fast_variant(a, buf, len);
      if (buf[0] == '\0') snprintf(buf, len, "phase1_generic");
      return ATTNRES_OK;
    }
    case ATTNRES_OP_PHASE2: {
      Phase2Args a{p, o_dtype, fp, fp, p, T, d, fp, fp, 1e-6f, H, dtype, p};
      snprintf(buf, len, fast && phase2_fast_ok(a) ? "phase2_fast<CPL=%lld,MH=%d>" : "phase2_generic",
               (long long)(d / 512), H > 1 ? 1 : 0);
      return ATTNRES_OK;
    }
    case ATTNRES_OP_BWD: {
      BwdArgs a{p, N, p, S, T, d, fp, fp, d, 1e-6f, H, dtype, p, p, p, static_cast<float*>(p),
                static_cast<float*>(p), 0, static_cast<float*>(p), T > 0 ? bwd_slots(T) : 0};
      if (fast) bwd_fast_variant(a, buf, len);
      if (buf[0] == '\0') snprintf(buf, len, "bwd_generic");
      return ATTNRES_OK;
    }
    case ATTNRES_OP_FULL_FWD: {
      FullArgs a{p, N, T, d, fp, S, fp, d, 1e-6f, H, dtype, p, p,
                 attnres_full_fwd_workspace_size(N, S, d, H, dtype)};
      snprintf(buf, len, "%s", fast && full_fast_ok(a) ? full_fast_variant(a) : "full_generic");
      return ATTNRES_OK;
    }
    case ATTNRES_OP_FULL_BWD: {
      FullBwdArgs a{p, N, T, d, fp, S, fp, d, 1e-6f, H, dtype, p, p, static_cast<float*>(p),
                    static_cast<float*>(p), 0, static_cast<float*>(p), T > 0 ? full_bwd_slots(T) : 0,
                    attnres_full_bwd_workspace_size(N, S, T, d, H)};
      const char* v = fast ? full_bwd_fast_variant(a) : nullptr;
      snprintf(buf, len, "%s", v ? v : "full_bwd_generic");
      return ATTNRES_OK;
    }
    default:
      return fail(ATTNRES_ERR_INVALID, "unknown op %d", op);
  }
}

int attnres_set_kernel_policy(int32_t policy) {
  if (policy != 0 && policy != 1) return fail(ATTNRES_ERR_INVALID, "unknown kernel policy %d", policy);
  return g_policy.exchange(policy);
}

size_t attnres_full_fwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t d, int32_t H,
                                       int32_t dtype) {
  if (n_src < 1 || n_dst < 1 || n_dst > n_src || d < 1 || d > kMaxD || H < 1) return 0;
  return full_fast_workspace_bytes(n_src, n_dst, d, H, dtype);
}

int attnres_full_fwd(const void* src, int64_t n_src, int64_t T, int64_t d, const float* w,
                     int64_t n_dst, const float* gain, int64_t gain_ld, float eps, int32_t H,
                     int32_t dtype, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, gain, gain_ld, &td));
  if (n_src < 1 || n_src > kMaxSources)
    return fail(ATTNRES_ERR_INVALID, "n_src = %lld must be in [1, %d]", (long long)n_src, kMaxSources);
  if (n_dst < 1 || n_dst > n_src)
    return fail(ATTNRES_ERR_INVALID, "n_dst = %lld must be in [1, n_src = %lld]", (long long)n_dst,
                (long long)n_src);
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(src, "src");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(out, "out");
  const int64_t es = (int64_t)dt_size(dtype);
  size_t b_src, b_out;
  RETURN_IF(check_count(n_src, td, es, "src", &b_src));
  RETURN_IF(check_count(n_dst, td, es, "out", &b_out));
  const Range ins[] = {{src, b_src, "src"},
                       {w, (size_t)(n_dst * d * 4), "w"},
                       {gain, gain ? (size_t)((gain_ld ? n_dst : 1) * d * 4) : 0, "gain"}};
  const size_t need = attnres_full_fwd_workspace_size(n_src, n_dst, d, H, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0,
                need);
  const Range outs[] = {{out, b_out, "out"}, {need > 0 ? ws : nullptr, need, "ws"}};
  RETURN_IF(check_aliasing(ins, 3, outs, 2));

  FullArgs a{src, n_src, T, d, w, n_dst, gain, gain ? gain_ld : 0, eps, H, dtype, out,
             need > 0 ? ws : nullptr, need};
  const hipError_t e = (use_fast() && full_fast_ok(a)) ? launch_full_fast(a, stream)
                                                       : launch_full_generic(a, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "full forward launch");
}

int attnres_block_phase1(const void* reps, int64_t N, int64_t T, int64_t d, const float* w,
                         int64_t S, const float* gain, int64_t gain_ld, float eps, int32_t H,
                         int32_t dtype, void* h_first, void* o_state, int32_t o_dtype, float* lse,
                         float* o_scale, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, gain, gain_ld, &td));
  if (N < 1 || N > kMaxSources - 1)
    return fail(ATTNRES_ERR_INVALID, "N = %lld must be in [1, %d]", (long long)N, kMaxSources - 1);
  if (S < 1) return fail(ATTNRES_ERR_INVALID, "S = %lld must be >= 1", (long long)S);
  RETURN_IF(check_state_dtype(o_dtype, dtype));
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(reps, "reps");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(h_first, "h_first");
  if (S > 1) REQUIRE_PTR(o_state, "o_state");
  REQUIRE_PTR(lse, "lse");
  if (o_dtype == ATTNRES_F16 && S > 1) REQUIRE_PTR(o_scale, "o_scale");
  const int64_t es = (int64_t)dt_size(dtype), eo = (int64_t)dt_size(o_dtype);
  size_t b_reps, b_h, b_o, b_lse;
  RETURN_IF(check_count(N, td, es, "reps", &b_reps));
  RETURN_IF(check_count(1, td, es, "h_first", &b_h));
  RETURN_IF(check_count(S - 1, td, eo, "o_state", &b_o));
  RETURN_IF(check_count(S * H, T, 4, "lse", &b_lse));
  const Range ins[] = {{reps, b_reps, "reps"},
                       {w, (size_t)(S * d * 4), "w"},
                       {gain, gain ? (size_t)((gain_ld ? S : 1) * d * 4) : 0, "gain"}};
  const bool scaled = o_dtype == ATTNRES_F16 && S > 1;
  const Range outs[] = {{h_first, b_h, "h_first"},
                        {o_state, b_o, "o_state"},
                        {lse, b_lse, "lse"},
                        {scaled ? o_scale : nullptr, (size_t)T * 4, "o_scale"}};
  RETURN_IF(check_aliasing(ins, 3, outs, 4));

  Phase1Args a{reps, N, T, d, w, S, gain, gain ? gain_ld : 0, eps, H, dtype,
               h_first, dtype, o_state, o_dtype, lse, scaled ? o_scale : nullptr};
  return run_phase1(a, stream);
}

int attnres_block_phase2_merge(const void* o_i, int32_t o_dtype, const float* o_scale,
                               const float* lse_i, const void* partial, int64_t T, int64_t d,
                               const float* w_i, const float* gain_i, float eps, int32_t H,
                               int32_t dtype, void* h_i, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, nullptr, 0, &td));
  RETURN_IF(check_state_dtype(o_dtype, dtype));
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(o_i, "o_i");
  if (o_dtype == ATTNRES_F16) REQUIRE_PTR(o_scale, "o_scale");
  REQUIRE_PTR(lse_i, "lse_i");
  REQUIRE_PTR(partial, "partial");
  REQUIRE_PTR(w_i, "w_i");
  REQUIRE_PTR(h_i, "h_i");
  const int64_t es = (int64_t)dt_size(dtype), eo = (int64_t)dt_size(o_dtype);
  size_t b_p, b_o, b_lse;
  RETURN_IF(check_count(1, td, es, "partial", &b_p));
  RETURN_IF(check_count(1, td, eo, "o_i", &b_o));
  RETURN_IF(check_count(H, T, 4, "lse_i", &b_lse));
  const bool in_place = (h_i == o_i);
  if (in_place && dt_size(o_dtype) != dt_size(dtype))
    return fail(ATTNRES_ERR_INVALID, "in-place merge needs a state of the I/O element size");
  const Range ins[] = {{in_place ? nullptr : o_i, b_o, "o_i"},
                       {lse_i, b_lse, "lse_i"},
                       {partial, b_p, "partial"},
                       {w_i, (size_t)(d * 4), "w_i"},
                       {gain_i, gain_i ? (size_t)(d * 4) : 0, "gain_i"},
                       {o_dtype == ATTNRES_F16 ? o_scale : nullptr, (size_t)T * 4, "o_scale"}};
  const Range outs[] = {{h_i, b_p, "h_i"}};
  RETURN_IF(check_aliasing(ins, 6, outs, 1));
  Phase2Args a{o_i, o_dtype, o_dtype == ATTNRES_F16 ? o_scale : nullptr, lse_i, partial, T, d,
               w_i, gain_i, eps, H, dtype, h_i};
  return run_phase2(a, stream);
}

int attnres_block_phase2_merge_update(const void* o_i, int32_t o_dtype, const float* o_scale,
                                      const float* lse_i, const void* partial_prev, const void* f_prev,
                                      int64_t T, int64_t d, const float* w_i, const float* gain_i,
                                      float eps, int32_t H, int32_t dtype, void* partial_out, void* h_i,
                                      float norm_eps, float* h_inv_rms, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, nullptr, 0, &td));
  RETURN_IF(check_state_dtype(o_dtype, dtype));
  if (h_inv_rms != nullptr && (!(norm_eps >= 0.0f) || !std::isfinite(norm_eps)))
    return fail(ATTNRES_ERR_INVALID, "norm_eps must be finite and >= 0");
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(o_i, "o_i");
  if (o_dtype == ATTNRES_F16) REQUIRE_PTR(o_scale, "o_scale");
  REQUIRE_PTR(lse_i, "lse_i");
  REQUIRE_PTR(f_prev, "f_prev");
  REQUIRE_PTR(w_i, "w_i");
  REQUIRE_PTR(partial_out, "partial_out");
  REQUIRE_PTR(h_i, "h_i");
  const int64_t es = (int64_t)dt_size(dtype), eo = (int64_t)dt_size(o_dtype);
  size_t b_p, b_o, b_lse;
  RETURN_IF(check_count(1, td, es, "partial_out", &b_p));
  RETURN_IF(check_count(1, td, eo, "o_i", &b_o));
  RETURN_IF(check_count(H, T, 4, "lse_i", &b_lse));
  const bool o_in_place = (h_i == o_i);
  if (o_in_place && dt_size(o_dtype) != dt_size(dtype))
    return fail(ATTNRES_ERR_INVALID, "in-place merge needs a state of the I/O element size");
  const bool p_in_place = (partial_out == partial_prev);
  const Range ins[] = {{o_in_place ? nullptr : o_i, b_o, "o_i"},
                       {lse_i, b_lse, "lse_i"},
                       {p_in_place ? nullptr : partial_prev, partial_prev ? b_p : 0, "partial_prev"},
                       {f_prev, b_p, "f_prev"},
                       {w_i, (size_t)(d * 4), "w_i"},
                       {gain_i, gain_i ? (size_t)(d * 4) : 0, "gain_i"},
                       {o_dtype == ATTNRES_F16 ? o_scale : nullptr, (size_t)T * 4, "o_scale"}};
  const Range outs[] = {{partial_out, b_p, "partial_out"},
                        {h_i, b_p, "h_i"},
                        {h_inv_rms, h_inv_rms ? (size_t)T * 4 : 0, "h_inv_rms"}};
  RETURN_IF(check_aliasing(ins, 7, outs, 3));
  Phase2Args a{o_i, o_dtype, o_dtype == ATTNRES_F16 ? o_scale : nullptr, lse_i, partial_prev, T, d,
               w_i, gain_i, eps, H, dtype, h_i};
  a.f = f_prev;
  a.partial_out = partial_out;
  a.norm_eps = norm_eps;
  a.h_inv_rms = h_inv_rms;
  return run_phase2(a, stream);
}

size_t mhar_fwd_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d, int32_t H) {
  (void)N;
  (void)d;
  int64_t ls, sc;
  if (S < 1 || T < 0 || d < 1 || H < 1) return 0;
  if (!mul3(S, H, T, &ls) || !mul3(ls, 4, 1, &ls)) return 0;
  if (!mul3(T, 4, 1, &sc)) return 0;
  return align_up((size_t)ls) + align_up((size_t)sc);
}

namespace {

// One block over tokens [t0, t0 + C) of a T-token sequence: Phase 1, then the
// S - 1 merges, with the state and statistics of those C tokens in ws.
int run_block_chunk(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t t0,
                    int64_t C, int64_t d, const float* w, const float* gain, int64_t gain_ld, float eps,
                    int32_t H, int32_t dtype, void* h, void* ws, hipStream_t stream) {
  (void)N;
  const int64_t es = (int64_t)dt_size(dtype), td = T * d;
  // State between the phases: the scaled fp16 state for bf16 I/O, fp32 for
  // fp32 I/O -- the I/O element size either way, so Phase 1 writes sublayer
  // i's state into h[i - 1] itself and merge i overwrites it in place.  The
  // workspace holds only the statistics and the per-token scales.
  const int sdt = dtype == ATTNRES_BF16 ? ATTNRES_F16 : ATTNRES_F32;
  float* lse = static_cast<float*>(ws);                                                         // [S, H, C]
  float* oscale = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)(S * H * C * 4)));  // [C]
  const char* r0 = static_cast<const char*>(reps) + t0 * d * es;
  char* h0 = static_cast<char*>(h) + t0 * d * es;
  const int64_t gld = gain ? gain_ld : 0;
  // h is [S, T, d]: the chunk's rows of sublayers 2..S start T*d elements apart,
  // which Phase 1 addresses as a state of stride T*d (orest_stride).
  Phase1Args p1{r0, N, C, d, w, S, gain, gld, eps, H, dtype, h0, dtype, h0 + td * es, sdt, lse,
                sdt == ATTNRES_F16 ? oscale : nullptr};
  p1.rep_stride = td;
  p1.orest_stride = td;
  RETURN_IF(run_phase1(p1, stream));
  for (int64_t i = 2; i <= S; ++i) {
    Phase2Args p2{h0 + (i - 1) * td * es,
                  sdt,
                  sdt == ATTNRES_F16 ? oscale : nullptr,
                  lse + (i - 1) * H * C,
                  static_cast<const char*>(partials) + ((i - 2) * td + t0 * d) * es,
                  C,
                  d,
                  w + (i - 1) * d,
                  gain ? gain + (i - 1) * gld : nullptr,
                  eps,
                  H,
                  dtype,
                  h0 + (i - 1) * td * es};
    RETURN_IF(run_phase2(p2, stream));
  }
  return ATTNRES_OK;
}

// Validation shared by mhar_fwd and mhar_fwd_chunked; chunk tokens per pass.
// The static scratch of mhar_fwd_noalloc: one array per device (each GPU
// holds its own copy).  Host code never passes the array's name to a kernel --
// in host code it only stands in for the symbol -- but the device address
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kNoallocScratchBytes = (size_t)ATTNRES_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

static int noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(ATTNRES_ERR_UNSUPPORTED, "device %d is beyond the 64 the library tracks", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(ATTNRES_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return ATTNRES_OK;
}

// Validation shared by mhar_fwd, mhar_fwd_chunked and mhar_fwd_noalloc; chunk
// tokens per pass.  With use_scratch the workspace is the device's static
// scratch, resolved only after every argument has been checked.
int mhar_common(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H, int32_t dtype,
                void* h, int64_t chunk, void* ws, size_t ws_bytes, hipStream_t stream, bool use_scratch = false) {
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, gain, gain_ld, &td));
  if (N < 1 || N > kMaxSources - 1)
    return fail(ATTNRES_ERR_INVALID, "N = %lld must be in [1, %d]", (long long)N, kMaxSources - 1);
  if (S < 1) return fail(ATTNRES_ERR_INVALID, "S = %lld must be >= 1", (long long)S);
  if (chunk < 1) return fail(ATTNRES_ERR_INVALID, "chunk_T = %lld must be >= 1", (long long)chunk);
  if (T == 0) return ATTNRES_OK;
  REQUIRE_PTR(reps, "reps");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(h, "h");
  if (S > 1) REQUIRE_PTR(partials, "partials");
  const int64_t C = chunk < T ? chunk : T;
  const size_t need = mhar_fwd_workspace_size(N, S, C, d, H);
  if (need == 0) return fail(ATTNRES_ERR_INVALID, "workspace size overflows");
  if (use_scratch) {
    if (need > kNoallocScratchBytes)
      return fail(ATTNRES_ERR_UNSUPPORTED,
                  "mhar_fwd_noalloc needs %zu bytes of scratch for S = %lld, H = %d, T = %lld, beyond its %zu; "
                  "use mhar_fwd with a workspace",
                  need, (long long)S, H, (long long)T, kNoallocScratchBytes);
  } else if (ws == nullptr || ws_bytes < need) {
    return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0,
                need);
  }
  const int64_t es = (int64_t)dt_size(dtype);
  size_t b_reps, b_parts, b_h;
  RETURN_IF(check_count(N, td, es, "reps", &b_reps));
  RETURN_IF(check_count(S - 1, td, es, "partials", &b_parts));
  RETURN_IF(check_count(S, td, es, "h", &b_h));
  const Range ins[] = {{reps, b_reps, "reps"},
                       {partials, b_parts, "partials"},
                       {w, (size_t)(S * d * 4), "w"},
                       {gain, gain ? (size_t)((gain_ld ? S : 1) * d * 4) : 0, "gain"}};
  const Range outs[] = {{h, b_h, "h"}, {use_scratch ? nullptr : ws, need, "ws"}};
  RETURN_IF(check_aliasing(ins, 4, outs, 2));
  if (use_scratch) RETURN_IF(noalloc_scratch(&ws));
  for (int64_t t0 = 0; t0 < T; t0 += C) {
    const int64_t c = T - t0 < C ? T - t0 : C;
    RETURN_IF(run_block_chunk(reps, N, partials, S, T, t0, c, d, w, gain, gain_ld, eps, H, dtype, h, ws,
                              stream));
  }
  return ATTNRES_OK;
}

}  // namespace

int mhar_fwd(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
             const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H, int32_t dtype,
             void* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  return mhar_common(reps, N, partials, S, T, d, w, gain, gain_ld, eps, H, dtype, h, T > 0 ? T : 1, ws,
                     ws_bytes, stream);
}

int mhar_fwd_noalloc(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                     const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H, int32_t dtype,
                     void* h, hipStream_t stream) {
  clear_error();
  return mhar_common(reps, N, partials, S, T, d, w, gain, gain_ld, eps, H, dtype, h, T > 0 ? T : 1, nullptr, 0,
                     stream, true);
}

int mhar_fwd_chunked(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                     const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H,
                     int32_t dtype, void* h, int64_t chunk_T, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  return mhar_common(reps, N, partials, S, T, d, w, gain, gain_ld, eps, H, dtype, h, chunk_T, ws, ws_bytes,
                     stream);
}

size_t attnres_bwd_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d, int32_t H) {
  (void)H;
  int64_t b, r = 0;
  if (S < 1 || T < 0 || d < 1) return 0;
  if (!mul3(bwd_slots(T), S, d, &b) || !mul3(b, 4, 1, &b)) return 0;
  // A block of more than kBwdChunkMax destinations also keeps the first
  // chunk's rep gradients in fp32 ([N, T, d]).
  if (S > kBwdChunkMax && (N < 1 || !mul3(N, T, d, &r) || !mul3(r, 4, 1, &r) || b > INT64_MAX - r)) return 0;
  return (size_t)(b + r);
}

int attnres_bwd(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H,
                int32_t dtype, const void* dh, void* d_reps, void* d_partials, float* dw,
                float* dgain, int32_t accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, gain, gain_ld, &td));
  if (N < 1) return fail(ATTNRES_ERR_INVALID, "N = %lld must be >= 1", (long long)N);
  if (S < 1) return fail(ATTNRES_ERR_INVALID, "S = %lld must be >= 1", (long long)S);
  if (N + S - 1 > kMaxSources)
    return fail(ATTNRES_ERR_UNSUPPORTED, "N + S - 1 = %lld exceeds %d sources", (long long)(N + S - 1),
                kMaxSources);
  if (accumulate != 0 && accumulate != 1)
    return fail(ATTNRES_ERR_INVALID, "accumulate = %d must be 0 or 1", accumulate);
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(dw, "dw");
  if (gain != nullptr) REQUIRE_PTR(dgain, "dgain");
  const int64_t es = (int64_t)dt_size(dtype);
  size_t b_reps, b_parts;
  RETURN_IF(check_count(N, td, es, "reps", &b_reps));
  RETURN_IF(check_count(S - 1, td, es, "partials", &b_parts));
  const size_t b_dh = (size_t)(S * td * es);
  const size_t b_dw = (size_t)(S * d * 4);
  const size_t b_dg = gain ? (size_t)((gain_ld ? S : 1) * d * 4) : 0;
  const size_t need = attnres_bwd_workspace_size(N, S, T, d, H);
  if (T > 0) {
    REQUIRE_PTR(reps, "reps");
    REQUIRE_PTR(dh, "dh");
    REQUIRE_PTR(d_reps, "d_reps");
    if (S > 1) {
      REQUIRE_PTR(partials, "partials");
      REQUIRE_PTR(d_partials, "d_partials");
    }
    if (need == 0) return fail(ATTNRES_ERR_INVALID, "workspace size overflows");
    if (ws == nullptr || ws_bytes < need)
      return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  ws ? ws_bytes : 0, need);
  }
  const Range ins[] = {{reps, T ? b_reps : 0, "reps"},
                       {partials, T ? b_parts : 0, "partials"},
                       {w, b_dw, "w"},
                       {gain, b_dg, "gain"},
                       {dh, T ? b_dh : 0, "dh"}};
  const Range outs[] = {{d_reps, T ? b_reps : 0, "d_reps"},
                        {d_partials, T ? b_parts : 0, "d_partials"},
                        {dw, b_dw, "dw"},
                        {dgain, b_dg, "dgain"},
                        {ws, T ? need : 0, "ws"}};
  RETURN_IF(check_aliasing(ins, 5, outs, 5));
  BwdArgs a{reps,  N,    partials, S,         T,    d,        w,          gain,
            gain ? gain_ld : 0, eps, H,  dtype,    dh,   d_reps, d_partials, dw,
            dgain, accumulate, static_cast<float*>(ws), T ? bwd_slots(T) : 0};
  const bool fast = use_fast() && bwd_fast_ok(a);
  if (!fast && S * (int64_t)H * (N + 1) > 1024)
    return fail(ATTNRES_ERR_UNSUPPORTED, "S * H * (N + 1) = %lld exceeds 1024 on the general path",
                (long long)(S * H * (N + 1)));
  int64_t used = 0;
  if (T > 0) {
    const hipError_t e = fast ? launch_bwd_fast(a, &used, stream) : launch_bwd_generic(a, stream);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    if (!fast) used = a.slots;
  }
  const hipError_t e = launch_bwd_reduce(a, used, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "backward reduction launch");
}

size_t attnres_full_bwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int32_t H) {
  int64_t b, c;
  if (n_src < 1 || n_dst < 1 || T < 1 || d < 1 || d > kMaxD || H < 1 || H > d) return 0;  // T == 0 needs none
  if (!mul3(full_bwd_slots(T), n_dst, d, &b) || !mul3(b, 4, 1, &b)) return 0;  // general path
  if (!mul3(T, 8192, H, &c)) return 0;                                      // matrix-core path
  const size_t fast = full_bwd_fast_workspace_bytes(n_src, n_dst, T, d, H);
  return (size_t)b > fast ? (size_t)b : fast;
}

int attnres_full_bwd(const void* src, int64_t n_src, int64_t T, int64_t d, const float* w, int64_t n_dst,
                     const float* gain, int64_t gain_ld, float eps, int32_t H, int32_t dtype, const void* dout,
                     void* d_src, float* dw, float* dgain, int32_t accumulate, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  clear_error();
  int64_t td = 0;
  RETURN_IF(check_common(T, d, H, dtype, eps, gain, gain_ld, &td));
  if (n_src < 1 || n_src > kMaxSources)
    return fail(ATTNRES_ERR_INVALID, "n_src = %lld must be in [1, %d]", (long long)n_src, kMaxSources);
  if (n_dst < 1 || n_dst > n_src)
    return fail(ATTNRES_ERR_INVALID, "n_dst = %lld must be in [1, n_src = %lld]", (long long)n_dst,
                (long long)n_src);
  if (accumulate != 0 && accumulate != 1)
    return fail(ATTNRES_ERR_INVALID, "accumulate = %d must be 0 or 1", accumulate);
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(dw, "dw");
  if (gain != nullptr) REQUIRE_PTR(dgain, "dgain");
  const int64_t es = (int64_t)dt_size(dtype);
  size_t b_src, b_dout;
  RETURN_IF(check_count(n_src, td, es, "src", &b_src));
  RETURN_IF(check_count(n_dst, td, es, "dout", &b_dout));
  const size_t b_dw = (size_t)(n_dst * d * 4);
  const size_t b_dg = gain ? (size_t)((gain_ld ? n_dst : 1) * d * 4) : 0;
  const size_t need = attnres_full_bwd_workspace_size(n_src, n_dst, T, d, H);
  if (T > 0) {
    REQUIRE_PTR(src, "src");
    REQUIRE_PTR(dout, "dout");
    REQUIRE_PTR(d_src, "d_src");
    if (need == 0) return fail(ATTNRES_ERR_INVALID, "workspace size overflows");
    if (ws == nullptr || ws_bytes < need)
      return fail(ATTNRES_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0, need);
  }
  const Range ins[] = {{src, T ? b_src : 0, "src"},
                       {w, b_dw, "w"},
                       {gain, b_dg, "gain"},
                       {dout, T ? b_dout : 0, "dout"}};
  const Range outs[] = {{d_src, T ? b_src : 0, "d_src"},
                        {dw, b_dw, "dw"},
                        {dgain, b_dg, "dgain"},
                        {ws, T ? need : 0, "ws"}};
  RETURN_IF(check_aliasing(ins, 4, outs, 4));
  FullBwdArgs a{src,   n_src, T,    d,     w,     n_dst,      gain,    gain ? gain_ld : 0, eps,
                H,     dtype, dout, d_src, dw,    dgain,      accumulate, static_cast<float*>(ws),
                T ? full_bwd_slots(T) : 0, T ? ws_bytes : 0};
  const bool fast = T > 0 && use_fast() && full_bwd_fast_ok(a);
  // The general kernel keeps a per-wave table of (destination, head, source)
  // entries; the matrix-core kernels have no such limit.
  if (T > 0 && !fast && n_dst * (int64_t)H * n_src > kBwdTable)
    return fail(ATTNRES_ERR_UNSUPPORTED, "n_dst * H * n_src = %lld exceeds %d on the general path",
                (long long)(n_dst * H * n_src), kBwdTable);
  const float* slabs = static_cast<const float*>(ws);
  int64_t n_slabs = 0;
  if (T > 0) {
    hipError_t e;
    if (fast) {
      e = launch_full_bwd_fast(a, &slabs, &n_slabs, stream);
    } else {
      e = launch_full_bwd_generic(a, stream);
      n_slabs = a.slots;
    }
    if (e != hipSuccess) return hip_fail(e, "full backward launch");
  }
  const hipError_t e = launch_full_bwd_reduce(a, slabs, n_slabs, stream);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "full backward reduction launch");
}

}  // extern "C"
