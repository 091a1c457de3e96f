// Host-side launchers for the NF4 kernels.  Arguments are validated by the
// C-ABI layer (nf4_abi.hip) before any of these is called: shapes are
// non-negative, K % 64 == 0, every size fits the kernels' index types and
// every pointer is 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

hipError_t launch_dequant(const float* scales, const uint8_t* codes, float* out, int64_t N, int64_t K,
                          hipStream_t stream);

hipError_t launch_pack(const float* w, float* scales, uint8_t* codes, int64_t N, int64_t K,
                       hipStream_t stream);

// grad_a[M][K] = grad_out[M][N] . dequant(codes, scales)[N][K]; M, K > 0, N >= 0.
hipError_t launch_grad_a(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                         int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Launch plan chosen for a shape (exposed for tests and the benchmark).
struct GradAPlan {
  int kernel;    // 0 = tile (BM = 128 * rb), 1 = skinny (M <= 16), 2 = zero-fill (N == 0),
                 // 3 = wide (8 waves, tile 512 x 128, fp32 grad_out converted in the loop),
                 // 4 = stream (M <= 16),
                 // 5 = wide fed by fp16 A fragments from a conversion pass (tile 512 x 128),
                 // 6 = unfused comparison path (fp16 weight pass, then a fragment-copy GEMM),
                 // 8 = line streaming (M <= 16, 256-column strips),
                 // 9 = mid-size tiles (256 x 128, four waves, two workgroups per CU) fed by kernel 5's pass,
                 // 10 = small tiles (128 x 128, four waves, three workgroups per CU) fed by the same pass
  int rb;        // tile: 32-row blocks per wave; wide: 1; line streaming: rows decoded in registers;
                 // mid-size and small: k-steps of A fragments in flight
  int splits;    // number of N-chunks (1 = no workspace, no reduce launch)
  int n_chunk;   // rows of N per chunk
  int grid;      // workgroups of the main kernel
};
GradAPlan plan_grad_a(int64_t M, int64_t N, int64_t K);

// Complete a forced plan (kernel, rb, splits) for a shape; returns false if
// the combination is not valid for it.
bool make_plan(int64_t M, int64_t N, int64_t K, int kernel, int rb, int splits, GradAPlan* out);

// Split-N workspace of at least `bytes` for calls on `stream` (cached per
// device and stream, grown with a stream-ordered allocation); and the release
// of every cached workspace (drains the devices that hold one).  `counters`
// (optional) receives the buffer's kWsCounters 32-bit arrival counters: zero
// between calls on the stream, and a kernel that counts on them must leave
// them at zero.
constexpr int kWsCounters = 4096;
hipError_t stream_workspace(hipStream_t stream, size_t bytes, void** out, uint32_t** counters = nullptr);
hipError_t release_workspaces();

// Caller-provided scratch in place of the stream's workspace: `bytes` at
// `base` for the plan's partials and fragments, and kWsCounters arrival
// counters (zero between calls).
struct FixedScratch {
  char* base;
  size_t bytes;
  uint32_t* counters;
};

// Launch a given plan; its partials and fragments go to the stream's
// workspace, or to `fixed` when given (nothing is allocated then).
hipError_t launch_grad_a_plan(const GradAPlan& p, const float* grad_out, const float* scales, const uint8_t* codes,
                              float* grad_a, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                              const FixedScratch* fixed = nullptr);
// Bytes of workspace a plan needs beyond the arrival counters.
size_t grad_a_workspace_bytes(const GradAPlan& p, int64_t M, int64_t N, int64_t K);

// nf4_grad_a without any allocation: nf4_grad_a's plan with its scratch in a
// static device array of kNoallocScratchBytes per GPU (the arrival counters,
// then noalloc_scratch_capacity() bytes).  hipErrorOutOfMemory (nothing
// enqueued) when the plan needs more.
constexpr size_t kNoallocScratchBytes = (size_t)128 << 20;
size_t noalloc_scratch_capacity();
hipError_t launch_grad_a_noalloc(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Wide tile kernel (nf4_grad_a_wide.hip): usable when N % 64 == 0 and the
// operands have 32-bit byte offsets; its tile is wide_tile_rows() x
// wide_tile_cols() (512 x 128).
bool wide_kernel_supported(int64_t M, int64_t N, int64_t K);
int wide_tile_rows();
int wide_tile_cols();
hipError_t launch_grad_a_wide(int grid, const float* grad_out, const float* scales, const uint32_t* codes, float* dst,
                              int M, int N, int K, int n_chunk, int tiles_m, int tiles_k, hipStream_t stream);

// Fragment-fed wide kernel: grad_out converted once to fp16 A fragments in a
// workspace of wide_frag_bytes(M, N) bytes, then the wide kernel (tile 512 x
// 128) reads them.  Same preconditions as the wide kernel.
size_t wide_frag_bytes(int64_t M, int64_t N);
// Mid-size tiles from the same fragments (four waves; bitwise the same
// results): `rows` = 256 (two workgroups per CU, `af` 1 or 3 k-steps of A
// fragments in flight) or 128 (three per CU, af 1), x 128 columns.
inline int mid_tile_rows() { return 256; }
inline int small_tile_rows() { return 128; }
hipError_t launch_grad_a_mid_frag(int af, int rows, int grid, const float* grad_out, void* frags,
                                  const float* scales, const uint32_t* codes, float* dst, int M, int N, int K,
                                  int n_chunk, int tiles_m, int tiles_k, hipStream_t stream);
hipError_t launch_grad_a_wide_frag(int grid, const float* grad_out, void* frags, const float* scales,
                                   const uint32_t* codes, float* dst, int M, int N, int K, int n_chunk, int tiles_m,
                                   int tiles_k, hipStream_t stream);

// Grouped launch of the fragment-fed wide kernel (512 x 128 tiles, no N split)
// over several problems sharing M; problems[i].tile_begin is the index of its
// first tile in the group's tile order (prefix sums of tiles_m * tiles_k).
constexpr int kWideGroupMax = 8;
struct WideProblem {
  const void* frags;  // fp16 A fragments of this problem's grad_out
  const float* scales;
  const uint32_t* codes;
  float* out;
  int N, K, tiles_k, tile_begin;
};
struct WideGroup {
  WideProblem p[kWideGroupMax];
  int count, M, tiles_m, total;
};
hipError_t launch_grad_a_wide_grouped(const WideGroup& g, hipStream_t stream);
hipError_t launch_grad_a_grouped(const float* const* grad_out, const float* const* scales,
                                 const uint8_t* const* codes, float* const* grad_a, const int64_t* N,
                                 const int64_t* K, int count, int64_t M, hipStream_t stream);

// RMSNorm backward (rms_norm_bwd.hip): H % 4 == 0, H <= 8192; uses
// rms_norm_workspace_bytes(H) of the stream's workspace for dgamma partials.
bool rms_norm_supported(int64_t rows, int64_t H);
size_t rms_norm_workspace_bytes(int64_t H);
hipError_t launch_rms_norm_backward(const float* x, const float* gamma, const float* rms, const float* dy, float* dx,
                                    float* dgamma, int64_t rows, int64_t H, hipStream_t stream);

// Unfused comparison path (kernel 6): the weights dequantised to fp16 once
// into B fragments (unfused_bfrag_bytes(N, K) bytes), then the fragment-fed
// wide kernel copying them into LDS instead of decoding.  Same preconditions
// as the wide kernel.
size_t unfused_bfrag_bytes(int64_t N, int64_t K);
hipError_t launch_grad_a_unfused(int grid, const float* grad_out, void* afrags, void* bfrags, const float* scales,
                                 const uint32_t* codes, float* dst, int M, int N, int K, int n_chunk, int tiles_m,
                                 int tiles_k, hipStream_t stream);

// fp32 [rows][cols] -> fp16 MFMA A fragments (reduction along cols, cols % 32
// == 0), rows padded to 16 with zeros: the backward wide kernel's permuted
// reduction order, or natural order for the forward kernel.
hipError_t launch_frag_pass(const float* src, void* frags, int rows, int cols, bool natural, hipStream_t stream);

// kernel: -1 picks (streaming for M <= 16 where supported, else a tile kernel), 0 tiles of 512 x 128,
// 1 streaming, 2 tiles of 256 x 128 (two workgroups per CU), 3 tiles of 128 x 128 (three per CU).
constexpr int kForwardAuto = -1, kForwardTile = 0, kForwardStream = 1, kForwardMid = 2, kForwardSmall = 3;
// Forward product C[M][N] = A[M][K] . dequant(W)^T (nf4_forward.hip): tiles of
// forward_tile_rows(kernel) x 128 (kernel 0, 2 or 3; bitwise the same
// results), K split into chunks of whole 64-wide stages; A converted first
// into fragments (forward_frag_bytes(M, K) bytes of workspace).
bool forward_supported(int64_t M, int64_t N, int64_t K);
size_t forward_frag_bytes(int64_t M, int64_t K);
int forward_tile_rows(int kernel);
hipError_t launch_forward(int kernel, int grid, const float* a, void* frags, const float* scales,
                          const uint32_t* codes, float* dst, int M, int N, int K, int k_chunk, int tiles_m,
                          int tiles_n, hipStream_t stream);
// The tile kernel alone, on fragments a conversion pass already wrote.
hipError_t launch_forward_tiles(int kernel, int grid, const void* frags, const float* scales, const uint32_t* codes,
                                float* dst, int M, int N, int K, int k_chunk, int tiles_m, int tiles_n,
                                hipStream_t stream);
// Streaming forward kernel for M <= 16 (nf4_forward_skinny.hip): 128-column
// strips (16 per wave) x K chunks of whole 128-wide steps.
bool forward_stream_supported(int64_t M, int64_t N, int64_t K);
int forward_stream_strips(int64_t N);
// With splits > 1, dst holds the chunks' partials and, when `counters` (one
// per strip, zero on entry and on exit) is given, the last workgroup of each
// strip to finish sums them in chunk order into c; without counters the
// caller runs the reduction.
hipError_t launch_forward_stream(int grid, const float* a, const float* scales, const uint32_t* codes, float* dst,
                                 float* c, uint32_t* counters, int M, int N, int K, int k_chunk, int strips,
                                 int splits, hipStream_t stream);
// splits <= 0 picks the K chunk count.
hipError_t launch_nf4_forward(const float* a, const float* scales, const uint8_t* codes, float* c, int64_t M,
                              int64_t N, int64_t K, int kernel, int splits, hipStream_t stream);

// Grouped launch of the streaming forward kernel: problems sharing M, each
// with its own plan's strips and K-chunks (bitwise the result of its own
// launch).  Problem p owns blocks [begin, begin + padded), padded = strips x
// splits rounded up to a multiple of 8; part = its chunk partials (c itself
// when splits == 1), counters = its strips' arrival counters (null when
// splits == 1).
constexpr int kStreamGroupMax = 8;  // problems per grouped streaming launch
struct ForwardStreamProblem {
  const float* A;
  const float* S;
  const uint32_t* C32;
  float* part;
  float* c;
  uint32_t* counters;
  int N, K, k_chunk, strips, splits, begin, padded;
};
struct ForwardStreamGroup {
  ForwardStreamProblem p[kStreamGroupMax];
  int count;
  int M;
};
hipError_t launch_forward_stream_grouped(const ForwardStreamGroup& g, int grid, hipStream_t stream);
// Grouped forward: M <= 16 problems on the streaming kernel in one grid, the
// others through their own nf4_forward plans.
hipError_t launch_nf4_forward_grouped(const float* const* a, const float* const* scales, const uint8_t* const* codes,
                                      float* const* c, const int64_t* N, const int64_t* K, int count, int64_t M,
                                      hipStream_t stream);

// Streaming kernel for M <= 16 (nf4_grad_a_skinny.hip): 128-column strips,
// N-chunks of whole 32-row k-steps, two 8-wave workgroups per CU; needs
// 32-bit byte offsets.
constexpr int kStreamBK = 128;
bool stream_kernel_supported(int64_t M, int64_t N, int64_t K);
// Grouped launch of the streaming kernel (nf4_grad_a_skinny.hip): problems
// sharing M, each with its own plan's strips and N-chunks (bitwise the result
// of its own launch).  Problem p owns blocks [begin, begin + padded), padded =
// its workgroup count rounded up to a multiple of 8; part = its split
// partials (grad_a itself when splits == 1), counters = its strips' arrival
// counters (null when splits == 1).  Requires N % 4 == 0.
struct StreamProblem {
  const float* G;
  const float* S;
  const uint32_t* C32;
  float* part;
  float* grad_a;
  uint32_t* counters;
  int N, K, n_chunk, tiles_k, splits, begin, padded;
};
struct StreamGroup {
  StreamProblem p[kStreamGroupMax];
  int count;
  int M;
};
hipError_t launch_grad_a_stream_grouped(const StreamGroup& g, int grid, hipStream_t stream);

// With splits > 1, dst holds the splits' partials and, when `counters` (one
// per strip, zero on entry and on exit) is given, the last workgroup of each
// strip to finish sums them in split order into grad_a; without counters the
// caller runs the split reduction.
hipError_t launch_grad_a_stream(int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                                float* dst, float* grad_a, uint32_t* counters, int M, int N, int K, int n_chunk,
                                int tiles_k, int splits, hipStream_t stream);

// Line-streaming kernel for M <= 16 (nf4_grad_a_lines.hip): 256-column strips
// (whole 128-byte code lines), N-chunks of whole 16-row k-steps, one 8-wave
// workgroup per CU; `vr` (0..4) of each lane's 4 rows are decoded
// through the shared fp32 codebook, the rest through per-k-step fp16 tables.
// Needs N % 4 == 0 (16-byte grad_out
// rows) and 32-bit byte offsets.  With
// splits > 1, dst holds the partials and, when `counters` is given, the last
// workgroup of each strip sums them in split order into grad_a.
constexpr int kLinesBK = 256;
bool lines_kernel_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_grad_a_lines(int vr, int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                               float* dst, float* grad_a, uint32_t* counters, int M, int N, int K, int n_chunk,
                               int tiles_k, int splits, hipStream_t stream);

// Kernel launchers of nf4_grad_a.hip (tile, skinny, split reduction, zero fill).
hipError_t launch_grad_a_tile(int rb, int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                              float* dst, int M, int N, int K, int n_chunk, int tiles_m, int tiles_k,
                              hipStream_t stream);
hipError_t launch_grad_a_skinny(int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                                float* dst, int M, int N, int K, int n_chunk, int tiles_k, hipStream_t stream);
hipError_t launch_grad_a_reduce(int grid, const float* ws, float* out, int64_t n4, int splits, hipStream_t stream);
hipError_t launch_fill_zero(int grid, float* out, int64_t n4, hipStream_t stream);

}  // namespace nf4
