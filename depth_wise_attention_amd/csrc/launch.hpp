// Internal launch interface between the C ABI (attnres_abi.cpp) and the
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attnres {

// kF16 is only a Phase-1 -> Phase-2 state format: fp16 values scaled per token
// by a power of two (see Phase1Args::oscale).
enum Dt : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

inline size_t dt_size(int dt) { return dt == kF32 ? 4 : 2; }

struct FullArgs {
  const void* src;
  int64_t n_src, T, d;
  const float* w;
  int64_t n_dst;
  const float* gain;
  int64_t gain_ld;
  float eps;
  int H;
  int dtype;
  void* out;
  void* ws;  // scratch for the specialised kernel (may be null)
  size_t ws_bytes;
};

// Phase 1: layer 0 is written to o0 (o0_dtype), layers 1..S-1 to
// orest + (l-1)*orest_stride (orest_dtype; orest_stride 0 means T*d).
struct Phase1Args {
  const void* reps;
  int64_t N, T, d;
  const float* w;
  int64_t S;
  const float* gain;
  int64_t gain_ld;
  float eps;
  int H;
  int dtype;
  void* o0;
  int o0_dtype;
  void* orest;
  int orest_dtype;
  float* lse;     // [S, H, T]
  float* oscale;  // [T], written when orest_dtype == kF16: orest = o * (1 / oscale[t])
  // Elements between consecutive reps (0: T * d).  A T-chunk of a longer
  // sequence passes the full sequence's T * d with reps at the chunk's first token.
  int64_t rep_stride = 0;
  // Elements between consecutive state rows (0: T * d).  mhar_fwd keeps the
  // state of sublayer i in h[i - 1], whose rows are the whole sequence apart.
  int64_t orest_stride = 0;
};

struct Phase2Args {
  const void* o;
  int o_dtype;
  const float* oscale;  // [T] when o_dtype == kF16 (o = stored * oscale[t])
  const float* lse;  // [H, T]
  const void* partial;
  int64_t T, d;
  const float* w;
  const float* gain;  // [d] or null
  float eps;
  int H;
  int dtype;
  void* h;
  // Fused update (null f: plain merge).  The merged partial is
  // partial + f (partial null: f alone), rounded to dtype once and written to
  // partial_out (which may equal partial).  h_inv_rms[t] (may be null) is
  // 1 / sqrt(mean(h_t^2) + norm_eps) over the stored h.
  const void* f = nullptr;
  void* partial_out = nullptr;
  float norm_eps = 0.f;
  float* h_inv_rms = nullptr;
};

// MSAR: four streams per source (identity, then causal depthwise convolutions
// with kernel sizes 4, 8, 12 along the tokens); taps packed as [24, d].
constexpr int kMsarStreams = 4;
constexpr int kMsarMaxTaps = 12;
constexpr int kMsarTaps = 24;
__host__ __device__ constexpr int msar_kernel(int r) { return r == 1 ? 4 : (r == 2 ? 8 : 12); }  // r = 1..3
__host__ __device__ constexpr int msar_offset(int r) { return r == 1 ? 0 : (r == 2 ? 4 : 12); }

struct MsarArgs {
  const void* src;     // [n_src, T, d]
  int64_t n_src, T, d;
  const float* w;      // [n_dst, 4, d]
  const float* conv;   // [24, d]
  const float* mix;    // [n_dst, 4 d, 4]
  int64_t n_dst;
  float eps;
  int dtype;
  void* out;           // [n_dst, T, d]
  void* ws;            // specialised kernels' partial sums (may be null)
  size_t ws_bytes;
};

struct BwdArgs {
  const void* reps;
  int64_t N;
  const void* partials;
  int64_t S, T, d;
  const float* w;
  const float* gain;
  int64_t gain_ld;
  float eps;
  int H;
  int dtype;
  const void* dh;
  void* d_reps;
  void* d_partials;
  float* dw;
  float* dgain;
  int accumulate;
  float* zslots;  // [slots, S, d] fp32
  int64_t slots;
  // Set by the specialised kernel's launcher for each destination chunk:
  // floats between Z slabs; rep gradients to d_reps (rep_mode 0), to the fp32
  // buffer rep32 [N, T, d] (1), or added to rep32's before the store (2).
  int64_t zld = 0;
  float* rep32 = nullptr;
  int rep_mode = 0;
};

// Maximum number of [S, d] partial-gradient slabs in the backward workspace.
constexpr int64_t kMaxBwdSlots = 1024;
// Destinations one specialised backward kernel holds; a larger block runs as
// two chunks.
constexpr int kBwdChunkMax = 4;

// Full AttnRes backward: gradients of sum_j <dout_j, out_j> for the Full forward.
struct FullBwdArgs {
  const void* src;
  int64_t n_src, T, d;
  const float* w;
  int64_t n_dst;
  const float* gain;
  int64_t gain_ld;
  float eps;
  int H;
  int dtype;
  const void* dout;
  void* d_src;
  float* dw;
  float* dgain;
  int accumulate;
  float* zslots;  // workspace: [slots, n_dst, d] fp32 on the general path
  int64_t slots;
  size_t ws_bytes;
};

// Maximum number of [n_dst, d] slabs in the Full backward workspace (one per
// wavefront of the general kernel).
constexpr int64_t kMaxFullBwdSlots = 1024;
// Per-wave table entries (alpha, c, s) of the general backward kernels.
constexpr int kBwdTable = 1024;

// General kernels: any shape within the documented limits.
hipError_t launch_full_generic(const FullArgs& a, hipStream_t st);
hipError_t launch_phase1_generic(const Phase1Args& a, hipStream_t st);
hipError_t launch_phase2_generic(const Phase2Args& a, hipStream_t st);
hipError_t launch_bwd_generic(const BwdArgs& a, hipStream_t st);  // uses a.slots waves

// Fixed-order reduction of the slot partials into dw / dgain.
hipError_t launch_bwd_reduce(const BwdArgs& a, int64_t slots_used, hipStream_t st);
hipError_t launch_full_bwd_generic(const FullBwdArgs& a, hipStream_t st);  // uses a.slots waves
// Fixed-order sum of n_slabs [n_dst, d] slabs at `slabs` into dw / dgain.
hipError_t launch_full_bwd_reduce(const FullBwdArgs& a, const float* slabs, int64_t n_slabs, hipStream_t st);
// Matrix-core Full backward (bf16, H = 1, n_src <= 32, d % 512 == 0); leaves
// its Z slabs at *slabs (n_slabs of them) inside the workspace.
bool full_bwd_fast_ok(const FullBwdArgs& a);
// Name of the specialised Full backward variant a call runs (nullptr: the general kernel).
const char* full_bwd_fast_variant(const FullBwdArgs& a);
size_t full_bwd_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int H);
// Staged matrix-core Full backward (full_bwd_wide.hip), one or two 32-source
// tiles: the shapes that need two (33 .. 64 sources, up to 32 destinations),
// the main kernel after the query packing (qpk, qt; writes the (r c) table
// cws, [T][32][32 tiles]), and the two-tile Z pass over cws into slabs zs.
bool full_bwd_wide_shape(const FullBwdArgs& a);
hipError_t launch_full_bwd_staged(const FullBwdArgs& a, const uint4* qpk, const uint4* qt, float* cws,
                                  hipStream_t st);
hipError_t launch_full_bwd_zw(const FullBwdArgs& a, const float* cws, float* zs, int groups, hipStream_t st);
hipError_t launch_full_bwd_fast(const FullBwdArgs& a, const float** slabs, int64_t* n_slabs, hipStream_t st);
// Vector Full backward for one destination over up to 64 sources
// (full_bwd_one.hip; d <= 4096 for up to 32 sources, d <= 2048 above): its Z
// slabs ([slabs, d] fp32, one per workgroup) are the whole workspace.
size_t full_bwd_one_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int H);
bool full_bwd_one_ok(const FullBwdArgs& a);
hipError_t launch_full_bwd_one(const FullBwdArgs& a, const float** slabs, int64_t* n_slabs, hipStream_t st);

// Specialised gfx950 kernels.  The *_ok predicates are pure functions of the
// arguments (no HIP calls); a launcher may only be called when its predicate
// holds.
bool phase1_fast_ok(const Phase1Args& a);
// Name of the Phase 1 kernel variant a call would run ("" when not eligible).
void phase1_fast_variant(const Phase1Args& a, char* buf, size_t len);
bool phase2_fast_ok(const Phase2Args& a);
bool bwd_fast_ok(const BwdArgs& a);
// Name of the Block backward kernel variant a call would run ("" when not eligible).
void bwd_fast_variant(const BwdArgs& a, char* buf, size_t len);
bool full_fast_ok(const FullArgs& a);
size_t full_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t d, int H, int dtype);
hipError_t launch_phase1_fast(const Phase1Args& a, hipStream_t st);
hipError_t launch_phase2_fast(const Phase2Args& a, hipStream_t st);
hipError_t launch_bwd_fast(const BwdArgs& a, int64_t* slots_used, hipStream_t st);
hipError_t launch_full_fast(const FullArgs& a, hipStream_t st);
// Name of the specialised Full forward kernel a call runs ("full_one" for one
// destination over up to 64 sources with d <= 4096 and heads of whole waves,
// else "full_fast" for up to 32 sources and "full_wide" for 33 .. 64); only
// meaningful when full_fast_ok.
const char* full_fast_variant(const FullArgs& a);
// Matrix-core Full forward over 33 .. 64 sources (full_wide.hip): the shapes
// it takes, its workspace (the packed query) and its launch.
bool full_wide_shape(int64_t n_src, int64_t n_dst, int64_t d, int H, int dtype);
size_t full_wide_workspace_bytes(int64_t n_dst, int64_t d);
hipError_t launch_full_wide(const FullArgs& a, hipStream_t st);
// Vector Full forward for one destination over up to 64 sources (full_one.hip):
// reads each source row once and needs no workspace.
bool full_one_ok(const FullArgs& a);
hipError_t launch_full_one(const FullArgs& a, hipStream_t st);

hipError_t launch_msar_generic(const MsarArgs& a, hipStream_t st);
constexpr int kMsarFastMaxSources = 12;
size_t msar_fast_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int dtype);
bool msar_fast_ok(const MsarArgs& a);
hipError_t launch_msar_fast(const MsarArgs& a, hipStream_t st);

// Block MSAR two-phase (bf16, N <= 12 reps, SB <= 4 sublayers, d % 512 == 0).
struct BmsarCall {
  const void* reps;
  int64_t N, T, d;
  const float* w;      // [SB][4][d]
  int64_t SB;
  const float* conv;   // [24][d]
  const float* mix1;   // [4 d][4]
  float eps;
  void* h1;            // [T][d] bf16
  void* o_state;       // [SB-1][4][T][d] fp16, scaled per token
  float* o_scale;      // [T]
  float* lse;          // [SB-1][4][T]
  void* ws;
};
struct Bmsar2Call {
  const void* o_i;     // [4][T][d] fp16, scaled per token
  const float* o_scale;  // [T]
  const float* lse_i;  // [4][T]
  const void* partial; // [T][d] bf16
  int64_t T, d;
  const float* w_i;    // [4][d]
  const float* conv;
  const float* mix_i;  // [4 d][4]
  float eps;
  void* h_i;           // [T][d] bf16
  void* ws;
};
size_t bmsar_phase1_workspace_bytes(int64_t N, int64_t SB, int64_t T, int64_t d);
hipError_t launch_bmsar_phase1(const BmsarCall& c, hipStream_t st);
size_t bmsar_phase2_workspace_bytes(int64_t T, int64_t d);
hipError_t launch_bmsar_phase2(const Bmsar2Call& c, hipStream_t st);

int num_cus();  // compute units of the current device (cached per device)
// Resident blocks per compute unit for a kernel and block size (cached).
// dyn_lds: bytes of dynamic LDS per workgroup of the launch.
hipError_t blocks_per_cu(const void* kern, int block, int* out, size_t dyn_lds = 0);

}  // namespace attnres
