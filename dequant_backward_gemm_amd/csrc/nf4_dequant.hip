// nf4_dequant: standalone NF4 -> fp32 decode, w[n][k] = fl32(s[n][k/64] * NF4[code]).
//
// This is the decode step of the subject page's Phase 2 (aprender-gpu
// nf4_tensor_core.rs, "NF4 LUT lookup + dequant") on its own: one fp32
// multiply per element, so the output is bit-exact.  It is HBM-bound: per
// element it reads half a byte of code and 1/16 of a scale and writes 4
// bytes.  Each thread turns one dword of codes (8 elements of one row, all in
// one 64-block) into two 128-bit stores.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

__global__ __launch_bounds__(256) void dequant_kernel(const float* __restrict__ scales,
                                                      const uint32_t* __restrict__ codes32,
                                                      float* __restrict__ out, int64_t N, int64_t K) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = kLevels[threadIdx.x];
  __syncthreads();

  const int64_t words_per_row = K / 8;
  const int64_t total = N * words_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t n = idx / words_per_row;
    const int64_t wk = idx - n * words_per_row;  // word index within the row: k = 8*wk .. 8*wk+7
    const uint32_t x = codes32[idx];
    const float s = scales[n * (K / kBlock) + wk / 8];
    floatx4 lo, hi;
    lo[0] = s * lut[x & 15u];
    lo[1] = s * lut[(x >> 4) & 15u];
    lo[2] = s * lut[(x >> 8) & 15u];
    lo[3] = s * lut[(x >> 12) & 15u];
    hi[0] = s * lut[(x >> 16) & 15u];
    hi[1] = s * lut[(x >> 20) & 15u];
    hi[2] = s * lut[(x >> 24) & 15u];
    hi[3] = s * lut[x >> 28];
    floatx4* o = reinterpret_cast<floatx4*>(out + n * K + wk * 8);
    o[0] = lo;
    o[1] = hi;
  }
}

hipError_t launch_dequant(const float* scales, const uint8_t* codes, float* out, int64_t N, int64_t K,
                          hipStream_t stream) {
  const int64_t words = N * (K / 8);
  int64_t blocks = (words + 255) / 256;
  const int64_t cap = 256 * 64;  // grid-stride beyond this
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scales,
                     reinterpret_cast<const uint32_t*>(codes), out, N, K);
  return hipGetLastError();
}

}  // namespace nf4
