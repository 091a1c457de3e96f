// nf4_pack: fp32 weights [N][K] -> NF4 codes [N][K/2] + fp32 absmax scales [N][K/64].
//
// The subject page stores one fp32 scale per (n, 64-block) and decodes
// w = scale * level (aprender-gpu nf4_tensor_core.rs, Phase 2).  The
// quantiser producing that format is not on the page; this follows the
// reading documented with the library: scale = absmax of the block; code =
// the nearest level to w/absmax with ties to the lower code.  The decision is
// exact: code = #{i : w > absmax * mid_i} with mid_i = (level_i +
// level_{i+1}) / 2, all in fp64, where the midpoints are exact (at most 25
// significant bits) and absmax * mid_i is exact (at most 49 bits).  An
// all-zero block gets scale 0 and code 7 (level 0.0).
//
// Mapping: 8 lanes per 64-block, 8 consecutive elements per lane (two
// 128-bit loads); the block absmax is a max over the 8 lanes by xor-shuffles;
// each lane emits one dword of 8 codes.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ w, float* __restrict__ scales,
                                                   uint32_t* __restrict__ codes32, int64_t N, int64_t K) {
  const int64_t nblocks = N * (K / kBlock);
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gtid >> 3;  // (n, kb) block handled by this group of 8 lanes
  const int sub = threadIdx.x & 7;
  // Groups of 8 lanes never straddle a block boundary; a whole group is in or out.
  const bool active = blk < nblocks;

  floatx4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const floatx4* p = reinterpret_cast<const floatx4*>(w + blk * kBlock + sub * 8);
    v0 = p[0];
    v1 = p[1];
  }
  float a = fmaxf(fmaxf(fmaxf(fabsf(v0[0]), fabsf(v0[1])), fmaxf(fabsf(v0[2]), fabsf(v0[3]))),
                  fmaxf(fmaxf(fabsf(v1[0]), fabsf(v1[1])), fmaxf(fabsf(v1[2]), fabsf(v1[3]))));
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));

  // Thresholds absmax * mid_i, exact in fp64.
  double thr[15];
  const double ad = (double)a;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    const double mid = ((double)kLevels[i] + (double)kLevels[i + 1]) * 0.5;
    thr[i] = ad * mid;
  }
  const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t c = 0;
    const double xd = (double)x[e];
#pragma unroll
    for (int i = 0; i < 15; ++i) c += (xd > thr[i]) ? 1u : 0u;
    if (a == 0.f) c = 7u;
    word |= c << (4 * e);
  }
  if (active) {
    codes32[blk * 8 + sub] = word;
    if (sub == 0) scales[blk] = a;
  }
}

hipError_t launch_pack(const float* w, float* scales, uint8_t* codes, int64_t N, int64_t K,
                       hipStream_t stream) {
  const int64_t threads = N * (K / kBlock) * 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, scales,
                     reinterpret_cast<uint32_t*>(codes), N, K);
  return hipGetLastError();
}

}  // namespace nf4
