// Device-side definitions shared by the NF4 kernels (gfx950, wave64).
//
// The 16 NormalFloat-4 levels (QLoRA, Dettmers et al. 2023) as exact fp32
// hex literals: level 7 is 0.0, level 0 is -1.0, level 15 is 1.0.  The
// subject page (aprender-gpu nf4_tensor_core.rs) imports this table as its
// NF4 LUT without printing it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;  // scale block along K

__device__ constexpr float kLevels[16] = {
    -0x1.000000p+0f, -0x1.647362p-1f, -0x1.0cd660p-1f, -0x1.946540p-2f,
    -0x1.23449ap-2f, -0x1.7a6a7ep-3f, -0x1.74f0e2p-4f, 0x0p+0f,
    0x1.45f5fep-4f,  0x1.4995c6p-3f,  0x1.f809bap-3f,  0x1.5a0674p-2f,
    0x1.c34970p-2f,  0x1.200f56p-1f,  0x1.722766p-1f,  0x1.000000p+0f,
};

// Two fp32 values -> two fp16 (round to nearest even) packed in one dword,
// `lo` in bits 0..15.  Lowers to v_cvt_pk_f16_f32, which honours the IEEE
// rounding mode (never the round-toward-zero v_cvt_pkrtz form).
__device__ __forceinline__ uint32_t pack_half2_rne(float lo, float hi) {
  float2v f = {lo, hi};
  half2v h = __builtin_convertvector(f, half2v);
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace nf4
