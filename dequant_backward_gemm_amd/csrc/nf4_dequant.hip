// nf4_dequant: standalone NF4 -> fp32 decode, w[n][k] = fl32(s[n][k/64] * NF4[code]).
//
// This is the decode step of the subject page's Phase 2 (aprender-gpu
// nf4_tensor_core.rs, "NF4 LUT lookup + dequant") on its own: one fp32
// multiply per element, so the output is bit-exact.  It is HBM-bound: per
// element it reads half a byte of code and 1/16 of a scale and writes 4
// bytes.  The arrays are walked flat: since K % 64 == 0, element e = n K + k
// has its code in byte e / 2 and its scale at e / 64.  A thread takes groups
// of four elements (two code bytes, one scale, one 16-byte store) with the
// groups of a wave contiguous, so every load and store instruction covers
// one contiguous span; four groups per thread are loaded before any is
// written, and the stores stream (the weights are not read back here).
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

constexpr int kDqUnroll = 4;

__global__ __launch_bounds__(256) void dequant_kernel(const float* __restrict__ scales,
                                                      const uint16_t* __restrict__ codes16,
                                                      floatx4* __restrict__ out, int64_t groups) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = kLevels[threadIdx.x];
  __syncthreads();

  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g0 < groups; g0 += kDqUnroll * stride) {
    uint32_t c[kDqUnroll];
    float s[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t g = g0 + u * stride;  // group g: elements 4g .. 4g + 3
      c[u] = g < groups ? codes16[g] : 0u;
      s[u] = g < groups ? scales[g / 16] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t g = g0 + u * stride;
      if (g < groups) {
        floatx4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = s[u] * lut[(c[u] >> (4 * e)) & 15u];
        __builtin_nontemporal_store(w, out + g);
      }
    }
  }
}

hipError_t launch_dequant(const float* scales, const uint8_t* codes, float* out, int64_t N, int64_t K,
                          hipStream_t stream) {
  const int64_t groups = N * (K / 4);
  int64_t blocks = (groups + 255) / 256;
  const int64_t cap = 256 * 64;  // grid-stride beyond this
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scales,
                     reinterpret_cast<const uint16_t*>(codes), reinterpret_cast<floatx4*>(out), groups);
  return hipGetLastError();
}

}  // namespace nf4
