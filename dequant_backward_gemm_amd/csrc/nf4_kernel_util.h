// Device helpers shared by the grad_A tile kernels (gfx950, wave64).
#pragma once

#include <type_traits>
#include <utility>

#include "nf4_device.h"

// Race-check build (NF4_EXTRA_BARRIERS defined): every kernel separates each
// of its LDS phases with an extra barrier, so that no wave starts a phase
// before all have finished the previous one; its results must equal the
// release build's bit for bit.  NF4_PHASE_BARRIER() is a workgroup barrier and
// sits only where every wave of the workgroup passes the same number of
// times; NF4_WAVE_DRAIN() completes a wave's own LDS accesses (for phases on a
// wave's private LDS area, in loops whose trip count differs between waves).
#ifdef NF4_EXTRA_BARRIERS
#define NF4_PHASE_BARRIER() __syncthreads()
#define NF4_WAVE_DRAIN()                                                 \
  do {                                                                   \
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");               \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0) */                 \
    __builtin_amdgcn_wave_barrier();                                     \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");               \
  } while (0)
#else
#define NF4_PHASE_BARRIER() \
  do {                      \
  } while (0)
#define NF4_WAVE_DRAIN() \
  do {                   \
  } while (0)
#endif

namespace nf4 {

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs.
// Map them so that the ids one XCD receives are consecutive in logical order.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }

// LDS accessors.  One LDS array is viewed with several element types (levels
// or tables, code words, packed fp16 fragments), so every access goes through
// a may_alias type: without it, type-based alias analysis would let the
// compiler reorder a read of one type above a write of another.
typedef float f32_alias __attribute__((may_alias));
typedef uint16_t u16_alias __attribute__((may_alias));
typedef uint32_t u32_alias __attribute__((may_alias));
typedef u32x2 u32x2_alias __attribute__((may_alias));
typedef u32x4 u32x4_alias __attribute__((may_alias));

__device__ __forceinline__ float lds_load_f32(const uint32_t* smem, uint32_t byte_addr) {
  return *reinterpret_cast<const f32_alias*>(reinterpret_cast<const char*>(smem) + byte_addr);
}
__device__ __forceinline__ uint32_t lds_load_u16(const uint32_t* smem, uint32_t byte_addr) {
  return *reinterpret_cast<const u16_alias*>(reinterpret_cast<const char*>(smem) + byte_addr);
}
__device__ __forceinline__ uint32_t lds_load_u32(const uint32_t* smem, uint32_t byte_addr) {
  return *reinterpret_cast<const u32_alias*>(reinterpret_cast<const char*>(smem) + byte_addr);
}
__device__ __forceinline__ void lds_store_u32(uint32_t* smem, uint32_t byte_addr, uint32_t v) {
  *reinterpret_cast<u32_alias*>(reinterpret_cast<char*>(smem) + byte_addr) = v;
}
__device__ __forceinline__ void lds_store_u32x2(uint32_t* smem, uint32_t byte_addr, u32x2 v) {
  *reinterpret_cast<u32x2_alias*>(reinterpret_cast<char*>(smem) + byte_addr) = v;
}
__device__ __forceinline__ u32x4 lds_load_u32x4(const uint32_t* smem, uint32_t byte_addr) {
  return *reinterpret_cast<const u32x4_alias*>(reinterpret_cast<const char*>(smem) + byte_addr);
}
__device__ __forceinline__ void lds_store_u32x4(uint32_t* smem, uint32_t byte_addr, u32x4 v) {
  *reinterpret_cast<u32x4_alias*>(reinterpret_cast<char*>(smem) + byte_addr) = v;
}

// Calls f(std::integral_constant<int, K>{}) for K = 0, 1, ... in order, fully
// expanded at compile time (each call sees K as a constant expression).
template <class F, int... Ks>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, Ks...>, F&& f) {
  (f(std::integral_constant<int, Ks>{}), ...);
}

// Instruction order inside one tick of the tile kernels (N MFMAs plus their
// share of LDS reads and stores, buffer loads and VALU work): each MFMA is
// followed by one memory instruction and two VALU instructions, so that a
// wave issues its own decode and operand traffic while its MFMAs run instead
// of in a run before or after them (measured 2-2.5% faster for the eight-wave
// grad_A tiles and 1-1.4% for the forward's on the full-step shapes than the
// compiler's own order).  Masks: 0x008 MFMA, 0x100 LDS read,
// 0x200 LDS write, 0x020 buffer load, 0x002 VALU.
template <int N>
__device__ __forceinline__ void interleave_tick() {
  for_each_index(std::make_integer_sequence<int, N>{}, [](auto) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100 | 0x200 | 0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  });
}

// The four-wave 256-row tiles (grad_A and forward) hold their accumulators
// and two decode lanes' state per lane; pinning their VALU work as well pushes
// them past the register budget, so there only the memory instructions are
// spread out: each MFMA is followed by one of them (measured 0.6-4% faster on
// the k/v projection and short-reduction shapes; the 128-row tiles were up to
// 4% slower with it and keep the compiler's order).
template <int N>
__device__ __forceinline__ void interleave_tick_memory() {
  for_each_index(std::make_integer_sequence<int, N>{}, [](auto) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100 | 0x200 | 0x020, 1, 0);
  });
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): offsets are byte offsets, reads past `bytes` return 0
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// base + byte B of y, one VALU instruction (SDWA operand select).  Written
// out because the compiler otherwise splits the byte extract into a shift and
// a mask before the add.
template <int B>
__device__ __forceinline__ uint32_t add_byte(uint32_t base, uint32_t y) {
  static_assert(B >= 0 && B < 4, "byte index");
  uint32_t r;
  if constexpr (B == 0)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(base), "v"(y));
  else if constexpr (B == 1)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(base), "v"(y));
  else if constexpr (B == 2)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(base), "v"(y));
  else
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(base), "v"(y));
  return r;
}

// Lane-bit exchanges.  Data held as registers x lanes is permuted by
// exchanging one lane-index bit with one register-index bit: for a register
// pair (a, b) that differs in that register bit,
//   a'[l] = (l & m) ? b[l ^ m] : a[l],   b'[l] = (l & m) ? b[l] : a[l ^ m],
// with m the lane bit.  Lane bits 0 and 1 use a DPP quad permutation fused
// into v_cndmask (one instruction per output dword, written out because the
// compiler does not fuse the two), lane bits 4 and 5 the gfx950 permlane swaps.
//
// Four pairs per call; LB is the lane bit (0 or 1).  The leading s_nop covers
// the VALU-write -> DPP-read hazard on the inputs, the others the VCC writes.
template <int LB>
__device__ __forceinline__ void xchg_lane_lo4(uint32_t (&a)[4], uint32_t (&b)[4]) {
  static_assert(LB == 0 || LB == 1, "lane bit 0 or 1");
  uint32_t na[4], nb[4];
  if constexpr (LB == 0)
    asm("s_nop 1\n\t"
        "s_mov_b32 vcc_lo, 0x55555555\n\t"
        "s_mov_b32 vcc_hi, 0x55555555\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_dpp %0, %12, %8, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %1, %13, %9, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %2, %14, %10, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %3, %15, %11, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_mov_b32 vcc_lo, 0xaaaaaaaa\n\t"
        "s_mov_b32 vcc_hi, 0xaaaaaaaa\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_dpp %4, %8, %12, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %5, %9, %13, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %6, %10, %14, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %7, %11, %15, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=&v"(na[0]), "=&v"(na[1]), "=&v"(na[2]), "=&v"(na[3]), "=&v"(nb[0]), "=&v"(nb[1]), "=&v"(nb[2]),
          "=&v"(nb[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
        : "vcc");
  else
    asm("s_nop 1\n\t"
        "s_mov_b32 vcc_lo, 0x33333333\n\t"
        "s_mov_b32 vcc_hi, 0x33333333\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_dpp %0, %12, %8, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %1, %13, %9, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %2, %14, %10, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %3, %15, %11, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_mov_b32 vcc_lo, 0xcccccccc\n\t"
        "s_mov_b32 vcc_hi, 0xcccccccc\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_dpp %4, %8, %12, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %5, %9, %13, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %6, %10, %14, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_cndmask_b32_dpp %7, %11, %15, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=&v"(na[0]), "=&v"(na[1]), "=&v"(na[2]), "=&v"(na[3]), "=&v"(nb[0]), "=&v"(nb[1]), "=&v"(nb[2]),
          "=&v"(nb[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
        : "vcc");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = na[i];
    b[i] = nb[i];
  }
}

// Exchange of lane bit 4 (16-lane rows) or 5 (32-lane halves) with a register
// bit, same convention as xchg_lane_lo4.
template <int LB>
__device__ __forceinline__ void xchg_lane_hi(uint32_t& a, uint32_t& b) {
  static_assert(LB == 4 || LB == 5, "lane bit 4 or 5");
  if constexpr (LB == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  }
}

}  // namespace nf4
