// RMSNorm backward (trueno-gpu 0.4.17, src/kernels/backward/rms_norm.rs, the
// module documentation's specification), fp32.  Per row of x (hidden size H),
// with the forward pass's stored rms = sqrt(mean(x^2) + eps):
//
//   m        = mean_j(x_j dy_j gamma_j)
//   dx_i     = (gamma_i dy_i - x_i m / rms^2) / rms
//   dgamma_i = sum over rows of dy_i x_i / rms
//
// dx is the exact derivative of the stated forward (the page's own
// finite-difference prediction; its printed formula also scales the
// correction term by gamma_i, which agrees only at gamma = 1).
//
// HBM-bound: x and dy are read once and dx written once (12 bytes per
// element).  A workgroup of 256 threads works on one row at a time, rows
// dealt to the workgroups round-robin (two workgroups per CU); thread t owns
// the float4 columns t + 256 c (c < C) and keeps its gamma chunks and its
// dgamma accumulators in registers for all its rows.  The x and dy of the
// next rows (two for H <= 4096, else one) are loaded before the current row
// is reduced, so loads stay in flight across the row's barrier.  The row sum
// is formed per thread in chunk order, across the wave by a fixed butterfly
// and across the four waves in wave order through LDS (one slot set per row
// parity, so one barrier per row).  dx leaves with non-temporal stores.  The
// workgroup's dgamma partial (its rows' sum, in row order) goes to a
// workspace; a second kernel adds the partials in workgroup order.  No
// atomics: bitwise deterministic.
#include "nf4_kernel_util.h"
#include "nf4_launch.h"

namespace nf4 {

constexpr int kRmsThreads = 256;
constexpr int kRmsWgPerCu = 2;                        // row workers per CU; also sets the dgamma partial count
constexpr int kRmsMaxParts = 256 * kRmsWgPerCu;    // 256 CUs
constexpr int kRmsDepth = 2;                          // rows in flight ahead of the one worked on (H <= 4096)
constexpr int kRmsMaxChunks = 8;                      // H <= 4 * 256 * 8
constexpr int kRmsRedWaves = 16;                      // dgamma reduce: waves per workgroup (64 columns each)
constexpr int kRmsRedBatch = 32;                      // dgamma reduce: loads in flight per thread

template <int C, int D>
__global__ __launch_bounds__(kRmsThreads) void rms_norm_bwd_kernel(const float* __restrict__ x,
                                                                   const float* __restrict__ gamma,
                                                                   const float* __restrict__ rms,
                                                                   const float* __restrict__ dy,
                                                                   float* __restrict__ dx, float* __restrict__ part,
                                                                   int rows, int H) {
  __shared__ float wsum[2][kRmsThreads / 64];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int H4 = H / 4;
  const int step = gridDim.x;
  const float invH = 1.0f / (float)H;
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  const floatx4* x4 = reinterpret_cast<const floatx4*>(x);
  const floatx4* dy4 = reinterpret_cast<const floatx4*>(dy);

  floatx4 g[C], dg[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = t + kRmsThreads * c;
    g[c] = j < H4 ? reinterpret_cast<const floatx4*>(gamma)[j] : zero;
    dg[c] = zero;
  }
  int row = blockIdx.x;
  if (row >= rows) return;  // uniform over the workgroup (the grid never exceeds rows)
  // rows row, row + step, ..., row + (D-1) step in flight; slot 0 is the one being worked on
  floatx4 xs[D][C], ds[D][C];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int rr = row + d * step;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = t + kRmsThreads * c;
      const bool ok = rr < rows && j < H4;
      const size_t o = (size_t)rr * (size_t)H4 + (size_t)j;
      xs[d][c] = ok ? x4[o] : zero;
      ds[d][c] = ok ? dy4[o] : zero;
    }
  }
  for (int it = 0; row < rows; row += step, ++it) {
    const int next = row + D * step;
    floatx4 xn[C], dn[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = t + kRmsThreads * c;
      const bool ok = next < rows && j < H4;
      const size_t o = (size_t)next * (size_t)H4 + (size_t)j;
      xn[c] = ok ? x4[o] : zero;
      dn[c] = ok ? dy4[o] : zero;
    }
    const float r = rms[row];
    const float inv_r = 1.0f / r;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += xs[0][c][e] * ds[0][c][e] * g[c][e];
        dg[c][e] += ds[0][c][e] * xs[0][c][e] * inv_r;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) wsum[it & 1][w] = s;
    __syncthreads();
    float tot = wsum[it & 1][0];
#pragma unroll
    for (int v = 1; v < kRmsThreads / 64; ++v) tot += wsum[it & 1][v];
    const float k = tot * invH / (r * r);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = t + kRmsThreads * c;
      if (j < H4) {
        floatx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (g[c][e] * ds[0][c][e] - xs[0][c][e] * k) * inv_r;
        // streamed out: dx is not read again here
        __builtin_nontemporal_store(o, &reinterpret_cast<floatx4*>(dx)[(size_t)row * (size_t)H4 + (size_t)j]);
      }
    }
#pragma unroll
    for (int d = 0; d + 1 < D; ++d) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        xs[d][c] = xs[d + 1][c];
        ds[d][c] = ds[d + 1][c];
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      xs[D - 1][c] = xn[c];
      ds[D - 1][c] = dn[c];
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = t + kRmsThreads * c;
    if (j < H4) reinterpret_cast<floatx4*>(part)[(size_t)blockIdx.x * (size_t)H4 + (size_t)j] = dg[c];
  }
}

// dgamma[j] = sum over partials b = 0 .. nparts-1 (in order) of part[b][j].  A workgroup covers 64
// columns; wave v adds the v-th contiguous run of partials (loads issued kRmsRedBatch at a time,
// added in order), then wave 0 adds the runs in wave order.
__global__ __launch_bounds__(64 * kRmsRedWaves) void rms_norm_dgamma_kernel(const float* __restrict__ part,
                                                                            float* __restrict__ dgamma, int nparts,
                                                                            int H) {
  __shared__ float run[kRmsRedWaves][64];
  const int lane = threadIdx.x & 63;
  const int v = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int per = (nparts + kRmsRedWaves - 1) / kRmsRedWaves;
  const int b0 = v * per;
  const int b1 = min(nparts, b0 + per);
  float s = 0.f;
  if (j < H) {
    for (int b = b0; b < b1; b += kRmsRedBatch) {
      float u[kRmsRedBatch];
#pragma unroll
      for (int q = 0; q < kRmsRedBatch; ++q) u[q] = b + q < b1 ? part[(size_t)(b + q) * (size_t)H + j] : 0.f;
#pragma unroll
      for (int q = 0; q < kRmsRedBatch; ++q)
        if (b + q < b1) s += u[q];
    }
  }
  run[v][lane] = s;
  __syncthreads();
  if (v == 0 && j < H) {
    float tot = run[0][lane];
#pragma unroll
    for (int q = 1; q < kRmsRedWaves; ++q) tot += run[q][lane];
    dgamma[j] = tot;
  }
}

bool rms_norm_supported(int64_t rows, int64_t H) {
  return H > 0 && H % 4 == 0 && H <= 4 * kRmsThreads * kRmsMaxChunks && rows >= 0;
}

size_t rms_norm_workspace_bytes(int64_t H) { return (size_t)kRmsMaxParts * (size_t)H * sizeof(float); }

hipError_t launch_rms_norm_backward(const float* x, const float* gamma, const float* rms, const float* dy, float* dx,
                                    float* dgamma, int64_t rows, int64_t H, hipStream_t stream) {
  float* part = nullptr;
  hipError_t e = stream_workspace(stream, rms_norm_workspace_bytes(H), reinterpret_cast<void**>(&part));
  if (e != hipSuccess) return e;
  const int nparts = (int)(rows < kRmsMaxParts ? rows : kRmsMaxParts);
  const int h = (int)H;
  if (nparts > 0) {
    const int chunks = (int)((H / 4 + kRmsThreads - 1) / kRmsThreads);
    const int r = (int)rows;
#define RMS_CASE(C)                                                                                        \
  case C:                                                                                                  \
    hipLaunchKernelGGL((rms_norm_bwd_kernel<C, (C <= 4 ? kRmsDepth : 1)>), dim3(nparts), dim3(kRmsThreads), 0, \
                       stream, x, gamma, rms, dy, dx, part, r, h);                                         \
    break
    switch (chunks) {
      RMS_CASE(1);
      RMS_CASE(2);
      RMS_CASE(3);
      RMS_CASE(4);
      RMS_CASE(5);
      RMS_CASE(6);
      RMS_CASE(7);
      RMS_CASE(8);
      default:
        return hipErrorInvalidValue;
    }
#undef RMS_CASE
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(rms_norm_dgamma_kernel, dim3((h + 63) / 64), dim3(64 * kRmsRedWaves), 0, stream, part, dgamma,
                     nparts, h);
  return hipGetLastError();
}

}  // namespace nf4
