/*
 * nf4bwd.h -- C ABI of the NF4-dequant-fused input-gradient GEMM for one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (aprender-gpu 0.32.0, src/kernels/backward/nf4_tensor_core.rs,
 * doc comment of Nf4TensorCoreGemmBackwardAKernel):
 *
 *     grad_A[M x K] = grad_out[M x N] . dequant(B_nf4[K x N])^T
 *
 * the input gradient of a frozen 4-bit (NF4) linear layer.  K is the layer's
 * in-features (the output dimension here), N its out-features (the reduction
 * dimension), M the token count.
 *
 * Packed-weight format (same page, Phase 2, "NF4 addressing"): the stored
 * array is W = B^T, N x K.  For every out-feature n its K codes are
 * contiguous, two per byte, the even k in the low nibble:
 *
 *     codes  : uint8_t [N][K/2]      code(n,k) = (codes[n][k/2] >> 4*(k%2)) & 0xF
 *     scales : float   [N][K/64]     one fp32 scale per (n, 64-wide block of k)
 *
 * so w[n][k] = fl32(scales[n][k/64] * NF4[code(n,k)]), one fp32 multiply
 * (Phase 2, "NF4 LUT lookup + dequant").  NF4 is the 16-level NormalFloat-4
 * codebook of QLoRA (Dettmers et al., 2023): level 7 is 0.0, level 15 is 1.0,
 * level 0 is -1.0.  K must be a multiple of 64 (the page's block size).
 *
 * Shared rules for every entry point below:
 *   - All array pointers are DEVICE pointers on the current HIP device; all
 *     arrays are dense row-major with the shapes stated.  The caller owns every
 *     buffer; the library never frees caller memory.
 *   - Calls are asynchronous on `stream` (0 = the default stream).  They
 *     return once the work is enqueued; the caller synchronises.
 *   - Outputs must not alias inputs.
 *   - Every pointer must be 16-byte aligned (128-bit loads and stores).
 *   - Return value is an nf4_status; on any error other than NF4_ERR_HIP
 *     nothing has been enqueued.  NF4_ERR_HIP reports a failed launch or a
 *     failed stream-ordered allocation (hipGetLastError); the stream's later
 *     work is then undefined.
 *   - State kept across calls: the workspace of nf4_grad_a / nf4_forward /
 *     nf4_rms_norm_backward, one device buffer per (device, stream) that has
 *     needed one, grown on demand and held until nf4_release_workspaces().
 *     (A stream-ordered allocate/free pair per call costs more host time than
 *     a skinny call's kernels take, so the buffer is cached rather than
 *     allocated per call.)  Calls on one stream share it (they run in order);
 *     concurrent calls on different streams use different buffers and are
 *     safe.  Calls on one stream must be issued from one host thread at a time
 *     (a call that grows the buffer frees the old one in stream order, before
 *     work another thread enqueues later).  A stream handle that is destroyed
 *     while its calls are still running must not be reused by a new stream
 *     before they finish (the new stream would inherit the buffer).  The
 *     buffer starts with per-strip arrival counters, zeroed when it is
 *     allocated; the streaming kernels count their split workgroups on them
 *     and leave them at zero.
 *   - HIP graphs: the calls can be captured on a stream and replayed, as long
 *     as the stream's workspace already holds what they need (an eager call
 *     of the same shapes on that stream before capture).  A call that would
 *     have to grow the workspace while its stream is capturing returns
 *     NF4_ERR_CAPTURE and enqueues nothing.  A captured graph keeps the
 *     address of the capture stream's workspace: growing that workspace later
 *     (a larger call on the stream) or nf4_release_workspaces() frees it and
 *     invalidates the graph.  A replay uses the capture stream's workspace
 *     wherever it is launched, so it must not overlap other work that uses it
 *     (eager calls on the capture stream, or another replay of a graph
 *     captured there).  No call issues hipMemset (buffers are cleared by
 *     kernels).
 */
#ifndef NF4BWD_H
#define NF4BWD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,   /* a required pointer is NULL while its array is non-empty */
  NF4_ERR_SHAPE = 2,  /* negative size, K % 64 != 0, or a size over 2^31-1 */
  NF4_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned */
  NF4_ERR_HIP = 4,    /* a HIP launch, allocation or synchronisation failed */
  NF4_ERR_CAPTURE = 5, /* the stream's workspace would have to grow during graph capture */
  NF4_ERR_SCRATCH = 6  /* nf4_grad_a_noalloc: the call needs more than its static scratch */
} nf4_status;

/*
 * nf4_grad_a -- the fused input gradient (the page's four phases: grad_out
 * fp32 -> fp16 operand, NF4 decode -> fp16 operand, fp16 products accumulated
 * in fp32 over N, fp32 store).
 *
 *   grad_out : const float   [M][N]
 *   scales   : const float   [N][K/64]
 *   codes    : const uint8_t [N][K/2]
 *   grad_a   : float         [M][K], OVERWRITTEN (no accumulate), as the
 *              page's Phase 4 store does.
 *
 *   grad_a[m][k] = sum_n fp16(grad_out[m][n]) * fp16(w[n][k]), accumulated in
 *   fp32, with fp16() round-to-nearest-even and w the fp32 dequantised weight.
 *   Any M >= 0 and N >= 0 are accepted (tails are masked); N == 0 writes
 *   zeros; M == 0 or K == 0 enqueues nothing.  Results are bitwise
 *   deterministic for a given (M, N, K): no atomics, fixed summation order.
 *   Large N may use the split-N workspace of `stream` (see the shared rules):
 *   the first call that needs it, or a larger one, grows it with a
 *   stream-ordered allocation (hipMallocAsync on `stream`).
 */
int nf4_grad_a(const float* grad_out, const float* scales, const uint8_t* codes,
               float* grad_a, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * nf4_grad_a_noalloc -- nf4_grad_a for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, layout, contract and launch plan as
 * nf4_grad_a, and bitwise the same results; it allocates nothing (no
 * hipMalloc, hipMallocAsync or hipFree, and no stream workspace).  Its
 * kernels' scratch -- split partials, arrival counters, fp16 A fragments --
 * lives in one static device array of NF4_NOALLOC_SCRATCH_BYTES (128 MiB),
 * which every GPU the library runs on holds until the process ends; the first
 * call on a GPU looks up its address there and clears its counters with a
 * kernel on `stream`.  A shape whose plan needs more than that (the plan's
 * partials and fragments, e.g. 2 * 16*ceil(M/16) * N bytes of fragments for
 * large M) returns NF4_ERR_SCRATCH and enqueues nothing.  Every call on one
 * GPU shares the array and leaves it as the next call needs it: calls that
 * overlap on one GPU (on different streams, or a graph replay beside another
 * call) race and must not be issued.
 */
#define NF4_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int nf4_grad_a_noalloc(const float* grad_out, const float* scales, const uint8_t* codes,
                       float* grad_a, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * nf4_dequant -- w_out[n][k] = fl32(scales[n][k/64] * NF4[code(n,k)]), fp32
 * [N][K] (= W = B^T).  Bit-exact: one IEEE fp32 multiply per element.
 */
int nf4_dequant(const float* scales, const uint8_t* codes, float* w_out,
                int64_t N, int64_t K, hipStream_t stream);

/*
 * nf4_pack -- quantise fp32 weights w[N][K] (= B^T, the nn.Linear layout) to
 * NF4.  Per (n, 64-block): scales[n][kb] = max |w| over the block, stored as
 * is; code = the level nearest to w/absmax, ties to the lower code, decided
 * exactly as #{i : w > absmax * mid_i} in fp64 with mid_i the midpoint of
 * levels i and i+1.  An all-zero block gets scale 0 and code 7.  Non-finite
 * weights are outside the contract.
 */
int nf4_pack(const float* w, float* scales, uint8_t* codes,
             int64_t N, int64_t K, hipStream_t stream);

/* Human-readable text for an nf4_status value (static storage). */
const char* nf4_status_string(int status);

/*
 * nf4_grad_a_plan -- host-only introspection of the launch plan nf4_grad_a
 * uses for a shape (no device work).  out5 receives, in order: kernel
 * (0 = tiled, 1 = skinny M <= 16, 2 = zero fill for N == 0, 3 = wide tiled
 * 512 x 128 converting fp32 grad_out in its loop, 4 = streaming M <= 16 with
 * 128-column strips, 5 = wide tiled 512 x 128 fed by an fp16 A-fragment
 * conversion pass of grad_out, 9 = mid-size tiles of 256 x 128 fed by the
 * same pass, two workgroups per CU, 10 = small tiles of 128 x 128 fed by the
 * same pass, three workgroups per CU), the kernel's tile parameter (tiled:
 * 32-row blocks per wave; wide: 1; mid-size and small: k-steps of A
 * fragments in flight; 0 for the others), number of N-chunks (1 = no split partials),
 * rows per N-chunk, workgroups of the main launch.
 * Returns NF4_ERR_SHAPE / NF4_ERR_NULL like nf4_grad_a.
 */
int nf4_grad_a_plan(int64_t M, int64_t N, int64_t K, int* out5);

/*
 * nf4_grad_a_forced -- nf4_grad_a with the launch plan forced, for tests and
 * tuning: kernel 0 = tiled with `rb` (1 or 2) 32-row blocks per wave, kernel
 * 1 = skinny (requires M <= 16), kernel 3 = wide tiled 512 x 128 (requires
 * N % 64 == 0 and grad_out and the codes below 2 GiB; `rb` ignored), kernel
 * 4 = streaming (requires M <= 16 and grad_out and the codes below 2 GiB;
 * `rb` ignored), kernel 5 = wide tiled 512 x 128 fed by the fp16 A-fragment
 * pass (same requirements as kernel 3; `rb` ignored; the fragments take
 * 2 * 16*ceil(M/16) * N bytes of the split-N workspace), kernel 6 = the
 * unfused comparison path: the weights dequantised to fp16 by a separate pass
 * (2 * N * 128*ceil(K/128) bytes of workspace), then the kernel-5 GEMM
 * reading them instead of decoding (same requirements, bitwise the same
 * result as kernel 5), kernel 8 = line streaming for M <= 16 (requires
 * N % 4 == 0 and grad_out and the codes below 2 GiB; 256-column strips of
 * whole code lines; `rb` 0..4 = rows of each lane's 4 decoded in registers
 * from byte planes, the rest by 16-bit table reads, 5 = one row through the
 * shared codebook: every `rb` gives bitwise the same result), kernel 9 =
 * mid-size tiles of 256 x 128 fed by the kernel-5 fragment pass (same
 * requirements and workspace as kernel 5; `rb` 1 or 3 = k-steps of A
 * fragments in flight; bitwise the same result as kernel 5), kernel 10 =
 * small tiles of 128 x 128 (as kernel 9 with `rb` 1 only); `splits` =
 * requested number of N-chunks (rounded so
 * that every chunk but the last is a whole number of stages).  Same contract
 * and results-to-bound as nf4_grad_a; NF4_ERR_SHAPE if the forced plan does
 * not fit the shape.
 */
int nf4_grad_a_forced(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                      int64_t M, int64_t N, int64_t K, int kernel, int rb, int splits, hipStream_t stream);

/*
 * nf4_grad_a_grouped -- up to NF4_GROUP_MAX grad_A problems that share M (for
 * example a layer's projections) in as few launches as possible.  For M > 16,
 * every problem the large-M wide kernel takes (N % 64 == 0, grad_out and
 * codes below 2 GiB) runs in one grid, the tiles of the longest reductions
 * first, which keeps the CUs busy where separate launches end in a part-full
 * round; results are bitwise equal to nf4_grad_a_forced with kernel 5 and one
 * N-chunk.  For M <= 16, every problem nf4_grad_a would run on the streaming
 * kernel (N % 4 == 0) runs in one grid of that kernel with its own plan's
 * strips and N-chunks, the largest chunks first; results are bitwise equal to
 * nf4_grad_a.  Any other problem runs as nf4_grad_a would run it.  Each
 * problem's fields mean what nf4_grad_a's arguments mean, with the same
 * layout, ownership and bound.  The grad_a arrays must not alias each other
 * or any input.  The fp16 fragments of all grouped grad_outs (M > 16: sum of
 * 2 * 16*ceil(M/16) * N bytes) or the split partials (M <= 16) share the
 * stream's workspace.  NF4_ERR_SHAPE if count is outside 0..NF4_GROUP_MAX or
 * a problem's shape is invalid; nothing is enqueued on any argument error.
 */
#define NF4_GROUP_MAX 8
typedef struct nf4_grad_a_problem {
  const float* grad_out;  /* [M][N] */
  const float* scales;    /* [N][K/64] */
  const uint8_t* codes;   /* [N][K/2] */
  float* grad_a;          /* [M][K], overwritten */
  int64_t N;
  int64_t K;
} nf4_grad_a_problem;
int nf4_grad_a_grouped(const nf4_grad_a_problem* problems, int count, int64_t M, hipStream_t stream);

/*
 * nf4_forward -- the forward product of the same frozen layer (the subject
 * page's header comment: the backward kernel is the analog of the forward
 * C = A @ B over the shared dimension K, B_nf4 being K x N):
 *
 *   a      : const float   [M][K]    activations
 *   scales : const float   [N][K/64]  } the same packed weight as nf4_grad_a
 *   codes  : const uint8_t [N][K/2]   }
 *   c      : float         [M][N], OVERWRITTEN
 *
 *   c[m][n] = sum_k fp16(a[m][k]) * fp16(w[n][k]), accumulated in fp32, with
 *   fp16() round-to-nearest-even and w the fp32 dequantised weight.  Requires
 *   K % 64 == 0 and N % 8 == 0 (NF4_ERR_SHAPE otherwise), and a, codes below
 *   2 GiB.  M == 0 or N == 0 enqueues nothing; K == 0 writes zeros.  Bitwise
 *   deterministic for a given (M, N, K).  1 <= M <= 16 runs a streaming
 *   kernel (256-column strips of C, the weight read once); larger M runs
 *   512 x 128, 256 x 128 or 128 x 128 tiles, as the launch planner picks
 *   for the shape.  Uses the stream's workspace (see the shared rules) for
 *   an fp16 copy of `a` (tiles: 2 * 16*ceil(M/16) * K bytes) and, when K is
 *   split, fp32 partials.
 */
int nf4_forward(const float* a, const float* scales, const uint8_t* codes, float* c,
                int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * nf4_forward_grouped -- up to NF4_GROUP_MAX forward products that share M
 * (for example a layer's projections at decode size) in as few launches as
 * possible: for 1 <= M <= 16, every problem nf4_forward would run on its
 * streaming kernel runs in one grid of that kernel, each with its own plan's
 * strips and K-chunks, the largest chunks first; results are bitwise equal to
 * nf4_forward.  Any other problem (larger M, or limits of the in-kernel chunk
 * sum) runs with the plan nf4_forward gives it, and problems among those with
 * the same `a` pointer and K (a layer's q, k and v, or gate and up) share one
 * conversion of `a` into fp16 fragments; results are again bitwise those of
 * nf4_forward.  Each problem's fields mean what
 * nf4_forward's arguments mean, with the same layout, ownership, requirements
 * and bound; the c arrays must not alias each other or any input.  The chunk
 * partials share the stream's workspace.  NF4_ERR_SHAPE if count is outside
 * 0..NF4_GROUP_MAX or a problem's shape is invalid; nothing is enqueued on
 * any argument error.
 */
typedef struct nf4_forward_problem {
  const float* a;         /* [M][K] */
  const float* scales;    /* [N][K/64] */
  const uint8_t* codes;   /* [N][K/2] */
  float* c;               /* [M][N], overwritten */
  int64_t N;
  int64_t K;
} nf4_forward_problem;
int nf4_forward_grouped(const nf4_forward_problem* problems, int count, int64_t M, hipStream_t stream);

/*
 * nf4_forward_forced -- nf4_forward with the kernel and the number of K
 * chunks forced, for tests and tuning: kernel NF4_FORWARD_TILE (512 x 128
 * tiles, eight waves, any M), NF4_FORWARD_MID (256 x 128 tiles, four waves,
 * two workgroups per CU), NF4_FORWARD_SMALL (128 x 128 tiles, four waves,
 * three per CU) -- the three tile kernels give bitwise the same result for
 * the same `splits` -- or NF4_FORWARD_STREAM (the streaming kernel
 * nf4_forward picks for 1 <= M <= 16; NF4_ERR_SHAPE for other M); `splits`
 * >= 1, rounded so that every chunk is a whole number of 64-wide blocks.
 * Same contract as nf4_forward otherwise (the streaming kernel needs no fp16
 * copy of `a`).
 */
#define NF4_FORWARD_TILE 0
#define NF4_FORWARD_STREAM 1
#define NF4_FORWARD_MID 2
#define NF4_FORWARD_SMALL 3
int nf4_forward_forced(const float* a, const float* scales, const uint8_t* codes, float* c,
                       int64_t M, int64_t N, int64_t K, int kernel, int splits, hipStream_t stream);

/*
 * nf4_rms_norm_backward -- the RMSNorm backward of the same training step
 * (trueno-gpu 0.4.17, src/kernels/backward/rms_norm.rs, module documentation),
 * fp32 throughout:
 *
 *   x      : const float [rows][H]   the forward pass's input
 *   gamma  : const float [H]         the learned scale
 *   rms    : const float [rows]      the forward pass's sqrt(mean(x^2) + eps)
 *   dy     : const float [rows][H]   gradient of the output
 *   dx     : float       [rows][H]   OVERWRITTEN:
 *            dx_i = (gamma_i dy_i - x_i m / rms^2) / rms, m = mean_j(x_j dy_j gamma_j)
 *   dgamma : float       [H]         OVERWRITTEN: sum over rows of dy_i x_i / rms
 *
 * dx is the exact derivative of the page's forward y_i = x_i / rms * gamma_i
 * (the page's finite-difference prediction; its printed dx formula scales the
 * correction term by gamma_i too, which agrees only at gamma = 1).  rms is used
 * as stored.  Requires H % 4 == 0 and H <= 8192 (NF4_ERR_SHAPE otherwise);
 * rows == 0 writes dgamma = 0.  Every pointer 16-byte aligned.  Bitwise
 * deterministic (fixed summation orders, no atomics).  Uses 512 * H * 4 bytes
 * of the stream's workspace for dgamma partials.
 */
int nf4_rms_norm_backward(const float* x, const float* gamma, const float* rms, const float* dy, float* dx,
                          float* dgamma, int64_t rows, int64_t H, hipStream_t stream);

/*
 * nf4_release_workspaces -- frees every cached split-N workspace.  It first
 * waits for all work on each device that holds one (hipDeviceSynchronize),
 * since the owning streams may no longer exist.  Host-blocking; not for use
 * while another thread is calling nf4_grad_a.  Later calls allocate again as
 * needed.  Returns NF4_OK or NF4_ERR_HIP.
 */
int nf4_release_workspaces(void);

#ifdef __cplusplus
}
#endif

#endif /* NF4BWD_H */
