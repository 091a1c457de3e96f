// C ABI of the NF4 input-gradient library: argument validation, then the
// launchers.  Declarations and the contract are in include/nf4bwd.h.
#include <stdint.h>

#include "nf4_launch.h"
#include "nf4bwd.h"

namespace {

constexpr int64_t kMaxDim = 0x7fffffffLL;        // every dimension fits an int
constexpr int64_t kMaxElems = (1LL << 40);       // any one array: at most 2^40 elements

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_ok(int64_t a, int64_t b) {
  if (a < 0 || b < 0 || a > kMaxDim || b > kMaxDim) return false;
  return a == 0 || b <= kMaxElems / a;
}

int from_hip(hipError_t e) {
  if (e == hipSuccess) return NF4_OK;
  return e == hipErrorStreamCaptureUnsupported ? NF4_ERR_CAPTURE : NF4_ERR_HIP;
}

int forward_checked(const float* a, const float* scales, const uint8_t* codes, float* c, int64_t M, int64_t N,
                    int64_t K, int kernel, int splits, hipStream_t stream) {
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N) || (K % 64) != 0 || (N % 8) != 0) return NF4_ERR_SHAPE;
  if (M == 0 || N == 0) return NF4_OK;
  if (c == nullptr) return NF4_ERR_NULL;
  if (K > 0 && (a == nullptr || scales == nullptr || codes == nullptr)) return NF4_ERR_NULL;
  if (!aligned16(c) || (K > 0 && (!aligned16(a) || !aligned16(scales) || !aligned16(codes)))) return NF4_ERR_ALIGN;
  if (K > 0 && !nf4::forward_supported(M, N, K)) return NF4_ERR_SHAPE;
  if (splits < 0 || splits > 4096) return NF4_ERR_SHAPE;
  if (kernel == nf4::kForwardStream && K > 0 && !nf4::forward_stream_supported(M, N, K)) return NF4_ERR_SHAPE;
  return from_hip(nf4::launch_nf4_forward(a, scales, codes, c, M, N, K, kernel, splits, stream));
}

}  // namespace

extern "C" {

int nf4_grad_a(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a, int64_t M,
               int64_t N, int64_t K, hipStream_t stream) {
  if (!dims_ok(M, N) || !dims_ok(N, K) || !dims_ok(M, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  if (M == 0 || K == 0) return NF4_OK;
  if (grad_a == nullptr) return NF4_ERR_NULL;
  if (N > 0 && (grad_out == nullptr || scales == nullptr || codes == nullptr)) return NF4_ERR_NULL;
  if (!aligned16(grad_a) || (N > 0 && (!aligned16(grad_out) || !aligned16(scales) || !aligned16(codes))))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_grad_a(grad_out, scales, codes, grad_a, M, N, K, stream));
}

int nf4_grad_a_noalloc(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  static_assert(nf4::kNoallocScratchBytes == (size_t)NF4_NOALLOC_SCRATCH_BYTES, "scratch size as declared");
  if (!dims_ok(M, N) || !dims_ok(N, K) || !dims_ok(M, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  if (M == 0 || K == 0) return NF4_OK;
  if (grad_a == nullptr) return NF4_ERR_NULL;
  if (N > 0 && (grad_out == nullptr || scales == nullptr || codes == nullptr)) return NF4_ERR_NULL;
  if (!aligned16(grad_a) || (N > 0 && (!aligned16(grad_out) || !aligned16(scales) || !aligned16(codes))))
    return NF4_ERR_ALIGN;
  if (nf4::grad_a_workspace_bytes(nf4::plan_grad_a(M, N, K), M, N, K) > nf4::noalloc_scratch_capacity())
    return NF4_ERR_SCRATCH;
  return from_hip(nf4::launch_grad_a_noalloc(grad_out, scales, codes, grad_a, M, N, K, stream));
}

int nf4_dequant(const float* scales, const uint8_t* codes, float* w_out, int64_t N, int64_t K, hipStream_t stream) {
  if (!dims_ok(N, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  if (N == 0 || K == 0) return NF4_OK;
  if (scales == nullptr || codes == nullptr || w_out == nullptr) return NF4_ERR_NULL;
  if (!aligned16(scales) || !aligned16(codes) || !aligned16(w_out)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_dequant(scales, codes, w_out, N, K, stream));
}

int nf4_pack(const float* w, float* scales, uint8_t* codes, int64_t N, int64_t K, hipStream_t stream) {
  if (!dims_ok(N, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  if (N * (K / 64) * 8 / 256 > kMaxDim) return NF4_ERR_SHAPE;  // one thread per 8 weights
  if (N == 0 || K == 0) return NF4_OK;
  if (w == nullptr || scales == nullptr || codes == nullptr) return NF4_ERR_NULL;
  if (!aligned16(w) || !aligned16(scales) || !aligned16(codes)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_pack(w, scales, codes, N, K, stream));
}

int nf4_grad_a_forced(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                      int64_t M, int64_t N, int64_t K, int kernel, int rb, int splits, hipStream_t stream) {
  if (!dims_ok(M, N) || !dims_ok(N, K) || !dims_ok(M, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  if (M == 0 || K == 0) return NF4_OK;
  if (grad_a == nullptr) return NF4_ERR_NULL;
  if (N > 0 && (grad_out == nullptr || scales == nullptr || codes == nullptr)) return NF4_ERR_NULL;
  if (!aligned16(grad_a) || (N > 0 && (!aligned16(grad_out) || !aligned16(scales) || !aligned16(codes))))
    return NF4_ERR_ALIGN;
  nf4::GradAPlan p{};
  if (!nf4::make_plan(M, N, K, kernel, rb, splits, &p)) return NF4_ERR_SHAPE;
  return from_hip(nf4::launch_grad_a_plan(p, grad_out, scales, codes, grad_a, M, N, K, stream));
}

int nf4_grad_a_plan(int64_t M, int64_t N, int64_t K, int* out5) {
  if (out5 == nullptr) return NF4_ERR_NULL;
  if (!dims_ok(M, N) || !dims_ok(N, K) || !dims_ok(M, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
  const nf4::GradAPlan p = nf4::plan_grad_a(M, N, K);
  out5[0] = p.kernel;
  out5[1] = p.rb;
  out5[2] = p.splits;
  out5[3] = p.n_chunk;
  out5[4] = p.grid;
  return NF4_OK;
}


int nf4_forward(const float* a, const float* scales, const uint8_t* codes, float* c, int64_t M, int64_t N, int64_t K,
                hipStream_t stream) {
  return forward_checked(a, scales, codes, c, M, N, K, nf4::kForwardAuto, 0, stream);
}

int nf4_forward_forced(const float* a, const float* scales, const uint8_t* codes, float* c, int64_t M, int64_t N,
                       int64_t K, int kernel, int splits, hipStream_t stream) {
  if (splits < 1 || kernel < nf4::kForwardTile || kernel > nf4::kForwardSmall) return NF4_ERR_SHAPE;
  return forward_checked(a, scales, codes, c, M, N, K, kernel, splits, stream);
}

int nf4_grad_a_grouped(const nf4_grad_a_problem* problems, int count, int64_t M, hipStream_t stream) {
  if (count < 0 || count > NF4_GROUP_MAX) return NF4_ERR_SHAPE;
  if (count > 0 && problems == nullptr) return NF4_ERR_NULL;
  if (M < 0) return NF4_ERR_SHAPE;
  const float* g[NF4_GROUP_MAX];
  const float* sc[NF4_GROUP_MAX];
  const uint8_t* cd[NF4_GROUP_MAX];
  float* out[NF4_GROUP_MAX];
  int64_t n[NF4_GROUP_MAX], k[NF4_GROUP_MAX];
  for (int i = 0; i < count; ++i) {
    const nf4_grad_a_problem& p = problems[i];
    const int64_t N = p.N, K = p.K;
    if (!dims_ok(M, N) || !dims_ok(N, K) || !dims_ok(M, K) || (K % 64) != 0) return NF4_ERR_SHAPE;
    if (M > 0 && K > 0) {
      if (p.grad_a == nullptr) return NF4_ERR_NULL;
      if (N > 0 && (p.grad_out == nullptr || p.scales == nullptr || p.codes == nullptr)) return NF4_ERR_NULL;
      if (!aligned16(p.grad_a) || (N > 0 && (!aligned16(p.grad_out) || !aligned16(p.scales) || !aligned16(p.codes))))
        return NF4_ERR_ALIGN;
    }
    g[i] = p.grad_out;
    sc[i] = p.scales;
    cd[i] = p.codes;
    out[i] = p.grad_a;
    n[i] = N;
    k[i] = K;
  }
  if (M == 0 || count == 0) return NF4_OK;
  return from_hip(nf4::launch_grad_a_grouped(g, sc, cd, out, n, k, count, M, stream));
}

int nf4_forward_grouped(const nf4_forward_problem* problems, int count, int64_t M, hipStream_t stream) {
  if (count < 0 || count > NF4_GROUP_MAX) return NF4_ERR_SHAPE;
  if (count > 0 && problems == nullptr) return NF4_ERR_NULL;
  if (M < 0) return NF4_ERR_SHAPE;
  const float* a[NF4_GROUP_MAX];
  const float* sc[NF4_GROUP_MAX];
  const uint8_t* cd[NF4_GROUP_MAX];
  float* out[NF4_GROUP_MAX];
  int64_t n[NF4_GROUP_MAX], k[NF4_GROUP_MAX];
  for (int i = 0; i < count; ++i) {
    const nf4_forward_problem& p = problems[i];
    const int64_t N = p.N, K = p.K;
    if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N) || (K % 64) != 0 || (N % 8) != 0) return NF4_ERR_SHAPE;
    if (M > 0 && N > 0) {
      if (p.c == nullptr) return NF4_ERR_NULL;
      if (K > 0 && (p.a == nullptr || p.scales == nullptr || p.codes == nullptr)) return NF4_ERR_NULL;
      if (!aligned16(p.c) || (K > 0 && (!aligned16(p.a) || !aligned16(p.scales) || !aligned16(p.codes))))
        return NF4_ERR_ALIGN;
      if (K > 0 && !nf4::forward_supported(M, N, K)) return NF4_ERR_SHAPE;
    }
    a[i] = p.a;
    sc[i] = p.scales;
    cd[i] = p.codes;
    out[i] = p.c;
    n[i] = N;
    k[i] = K;
  }
  if (M == 0 || count == 0) return NF4_OK;
  return from_hip(nf4::launch_nf4_forward_grouped(a, sc, cd, out, n, k, count, M, stream));
}

int nf4_rms_norm_backward(const float* x, const float* gamma, const float* rms, const float* dy, float* dx,
                          float* dgamma, int64_t rows, int64_t H, hipStream_t stream) {
  if (!dims_ok(rows, H) || !nf4::rms_norm_supported(rows, H)) return NF4_ERR_SHAPE;
  if (gamma == nullptr || dgamma == nullptr) return NF4_ERR_NULL;
  if (rows > 0 && (x == nullptr || rms == nullptr || dy == nullptr || dx == nullptr)) return NF4_ERR_NULL;
  if (!aligned16(gamma) || !aligned16(dgamma) ||
      (rows > 0 && (!aligned16(x) || !aligned16(rms) || !aligned16(dy) || !aligned16(dx))))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_rms_norm_backward(x, gamma, rms, dy, dx, dgamma, rows, H, stream));
}

int nf4_release_workspaces(void) { return from_hip(nf4::release_workspaces()); }

const char* nf4_status_string(int status) {
  switch (status) {
    case NF4_OK: return "ok";
    case NF4_ERR_NULL: return "null pointer for a non-empty array";
    case NF4_ERR_SHAPE: return "bad shape (negative size, K not a multiple of 64, or size too large)";
    case NF4_ERR_ALIGN: return "pointer not 16-byte aligned";
    case NF4_ERR_HIP: return "HIP launch, allocation or synchronisation failed";
    case NF4_ERR_CAPTURE: return "the stream's workspace would have to grow during HIP graph capture";
    case NF4_ERR_SCRATCH: return "the call needs more scratch than nf4_grad_a_noalloc's static buffer holds";
    default: return "unknown nf4 status";
  }
}

}  // extern "C"
