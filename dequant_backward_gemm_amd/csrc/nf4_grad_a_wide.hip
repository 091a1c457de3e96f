// Wide tile kernel for grad_A = grad_out . dequant(W) at large M, N % 64 == 0.
//
// Same arithmetic as the other grad_A kernels (grad_out rounded fp32 -> fp16,
// weights fp16(fl32(scale * level)), fp16 MFMA products accumulated in fp32
// over N), organised for two waves per SIMD:
//
// * A workgroup is 8 waves (512 threads).  Each wave owns 64 rows x 128
//   columns of grad_A: four 16-row blocks x eight 16x16x32 MFMA tiles, 128
//   fp32 accumulators per lane, so two waves fit one SIMD and one wave's MFMAs
//   run while the other waits on memory or decodes.  The waves are arranged
//   WR x WC over the tile: BM = 64 * WR rows by BK = 128 * WC columns.
// * grad_out reaches the MFMA A operand through coalesced loads and an
//   in-register transpose.  The A layout wants one grad_out row per lane
//   (lanes i, i+16, i+32, i+48 share row i), and loads in that pattern touch a
//   different cache line in every lane, which the vector memory pipe serves at
//   a third of its rate.  So each group of four lanes loads 64 contiguous
//   bytes of one row, the values are rounded to fp16, and four lane-bit
//   exchanges (DPP selects for lane bits 0 and 1, permlane swaps for 4 and 5)
//   move the two low lane bits (the 16-byte chunk within the 64) up to lane
//   bits 4..5 and bring row bits down, ending in the A layout.
// * The reduction is walked in stages of 64 rows of N (two k-steps of 32).
//   Per stage every lane of the workgroup does a slice of three jobs:
//     - tables: for each (row n, 64-column scale block) of a stage, the 16
//       weights a code can stand for, fp16(fl32(scale * level)), are computed
//       once and written to LDS (32 bytes per table).  Decoding a weight is then
//       one table read -- no multiply and no conversion per weight;
//     - decode: a lane takes one dword of codes (8 columns) from each of two
//       adjacent rows n, n+1 and, per column, reads both rows' fp16 weights
//       from their tables and packs them into one dword, which is exactly one
//       register of an MFMA B operand (consecutive reduction indices at one
//       column), and stores it into the fragment buffer in LDS;
//     - MFMA: a wave multiplies its grad_out rows (converted on load) by the
//       B fragments of the current stage.
//   Tables are built two stages ahead and fragments one stage ahead, each in a
//   double buffer, with one barrier per stage.
// * Columns are permuted inside a tile so that every lane owns 8 consecutive
//   outputs per row: column c of MFMA tile t (t = 0..7) in column group wc is
//   k = k0 + 128*wc + 8*c + t.  A decoding lane's 8 columns are one code dword,
//   and each goes to a different tile at the same lane column.  Inside a
//   stage, k-step s, lane quarter q and element e is reduction row
//   n = n0 + 32*s + 16*(e/4) + 4*q + e%4 for both operands (what the transpose
//   of grad_out produces; consecutive pairs of n stay in one register).
// * Table slots are permuted so that the tables a half-wave reads at once
//   (random codes) fall in distinct 8-bank groups, and the decode lanes are
//   assigned so that a half-wave's fragment stores are consecutive dwords:
//   no LDS access has bank conflicts.
//
// Fragment variant (AF): grad_out is first rounded to fp16 by a separate pass
// (grad_out_frag_kernel) that writes it already in A-fragment order -- per
// 16-row block and 32-row k-step, 64 lanes x 16 bytes, the same reduction
// order as above -- so the main loop loads each A fragment with one 128-bit
// load per lane (1 KiB contiguous per wave), with no rounding or exchange work
// and half the bytes, and keeps AF k-steps of fragments in flight.
//
// Every global load is in bounds by clamping (rows of grad_out past M, code
// columns past K, stages past the end of a chunk) or by the buffer range
// (fragment rows past the padded M read zero); such values only reach outputs
// that are never stored or buffers that are never read.
#include "nf4_kernel_util.h"
#include "nf4_launch.h"

#include <algorithm>

#ifndef WIDE_FRAG_DEPTH
#define WIDE_FRAG_DEPTH 3
#endif

namespace nf4 {

typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int WC>
struct WideCfg {
  static constexpr int WR = 8 / WC;
  static constexpr int BM = 64 * WR;
  static constexpr int BK = 128 * WC;
  static constexpr int KB = BK / 64;                      // scale blocks per tile row
  static constexpr int kTabStage = 64 * KB * 32;          // 64 rows x KB tables x 16 fp16
  static constexpr int kFragStage = 2 * WC * 8 * 64 * 16; // [k-step][wc][tile][lane] x 16 B
  static constexpr int kTabBase = 0;
  static constexpr int kFragBase = 2 * kTabStage;
  static constexpr int kLds = kFragBase + 2 * kFragStage;
};

// Table slot (row n * KB + block) -> position in units of 32 bytes.  Slots are
// permuted inside aligned groups of four so that the tables a half-wave reads
// at once -- rows r, r + 2, r + 16, r + 18 of the stage at one block -- sit in
// four different 8-bank groups (rows differing in bits 1 and 4 are rotated
// apart).
template <int KB>
__device__ __forceinline__ uint32_t table_pos(uint32_t slot) {
  const uint32_t row = slot / KB;
  const uint32_t g = ((row >> 1) & 1u) + 2u * ((row >> 4) & 1u);
  return (slot & ~3u) | (((slot & 3u) + g) & 3u);
}

// fp32 [M][N] -> fp16 MFMA A fragments (the A operand of a product whose
// reduction runs along N).  Fragment (mb, ks) is 64 lanes x 16 bytes at
// ((mb * N/32 + ks) * 64 + lane) * 16: lane (ci, q) holds row 16mb + ci at
// reduction rows 32ks + 16*(e/4) + 4q + e%4 for e = 0..7 (the order the wide
// kernel's register transpose produces) or, NATURAL, 32ks + 8q + e.  Rows
// past M are zero.
template <bool NATURAL>
__global__ __launch_bounds__(256) void grad_out_frag_kernel(const float* __restrict__ G, u32x4* __restrict__ F,
                                                            int M, int N, int64_t total) {
  const int ksn = N / 32;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x; f < total; f += stride) {
    const int lane = (int)(f & 63);
    const int64_t blk = f >> 6;
    const int ks = (int)(blk % ksn);
    const int64_t mb = blk / ksn;
    const int64_t m = 16 * mb + (lane & 15);
    const int n = 32 * ks + (NATURAL ? 8 : 4) * (lane >> 4);
    u32x4 r = {0u, 0u, 0u, 0u};
    if (m < M) {
      const float* g = G + m * (int64_t)N + n;
      const floatx4 a = *reinterpret_cast<const floatx4*>(g);
      const floatx4 b = *reinterpret_cast<const floatx4*>(g + (NATURAL ? 4 : 16));
      r[0] = pack_half2_rne(a[0], a[1]);
      r[1] = pack_half2_rne(a[2], a[3]);
      r[2] = pack_half2_rne(b[0], b[1]);
      r[3] = pack_half2_rne(b[2], b[3]);
    }
    F[f] = r;
  }
}

// Unfused comparison path, first pass: the weights dequantised to fp16 once,
// written in exactly the LDS fragment layout the wide kernel's decode role
// produces for a stage (tile width 128): block (k-tile kt, stage of 64 rows
// st) is 16 KiB at (kt * N/64 + st) * 16 KiB.  Same decode arithmetic,
// fp16(fl32(scale * level)), computed per weight; columns past K are zero.
__global__ __launch_bounds__(512) void dequant_bfrag_kernel(const float* __restrict__ S,
                                                            const uint32_t* __restrict__ C32,
                                                            uint32_t* __restrict__ F, int N, int K) {
  __shared__ float lv[16];
  const int tid = threadIdx.x;
  if (tid < 16) lv[tid] = kLevels[tid];
  __syncthreads();
  const int nstg = N / 64;
  const int kt = blockIdx.x / nstg, st = blockIdx.x % nstg;
  const int wave = tid >> 6, lane = tid & 63;
  const int p = lane & 3, dl = lane >> 2;
  const int nr0 = 64 * st + 32 * (wave >> 2) + 16 * (p >> 1) + 4 * (wave & 3) + 2 * (p & 1);
  const int col0 = 128 * kt + 8 * dl;
  uint32_t x[2] = {0u, 0u};
  float sc[2] = {0.f, 0.f};
  if (col0 < K) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      x[r] = C32[((size_t)(nr0 + r) * (size_t)K + (size_t)col0) / 8];
      sc[r] = S[(size_t)(nr0 + r) * (size_t)(K / 64) + (size_t)(col0 / 64)];
    }
  }
  uint32_t* dst = F + ((size_t)kt * nstg + st) * 4096 + (size_t)(wave >> 2) * 2048 +
                  (size_t)(dl + 16 * (wave & 3)) * 4 + (size_t)p;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float w0 = sc[0] * lv[(x[0] >> (4 * c)) & 15u];
    const float w1 = sc[1] * lv[(x[1] >> (4 * c)) & 15u];
    dst[c * 256] = pack_half2_rne(w0, w1);
  }
}

// One workgroup's tile of the wide kernel over the reduction rows [nb, ne)
// (whole 64-row stages): tile `tile` in (k-tile fastest, then m-tile) order.
// Output element (row, col) of the tile goes to dst[(row - row0) * ld + col -
// col0] (rows < M and columns < K only).
template <int WC, int AF, bool BCOPY>
__device__ __forceinline__ void wide_tile(const void* __restrict__ Gv, const float* __restrict__ S,
                                          const uint32_t* __restrict__ C32, int M, int N, int K, int tiles_k,
                                          int tile, int nb, int ne, float* __restrict__ dst, int ld, int row0,
                                          int col0) {
  // AF == 0: Gv is grad_out (fp32 [M][N]); AF > 0: Gv holds the fp16 A
  // fragments of grad_out_frag_kernel and AF k-steps of them are in flight.
  // BCOPY: C32 holds the fp16 B fragments of dequant_bfrag_kernel, which are
  // copied into the LDS fragment buffers instead of decoded (S is unused).
  static_assert(AF == 0 || AF == 1 || AF == 3, "fragment prefetch depth 1 or 3");
  static_assert(!BCOPY || (WC == 1 && AF > 0), "fragment copy: 128-column tiles, A fragments");
  const float* __restrict__ G = static_cast<const float*>(Gv);
  using Cfg = WideCfg<WC>;
  constexpr int WR = Cfg::WR, BM = Cfg::BM, BK = Cfg::BK, KB = Cfg::KB;
  constexpr uint32_t kTabStage = Cfg::kTabStage, kFragStage = Cfg::kFragStage;
  __shared__ __attribute__((aligned(16))) uint32_t smem[Cfg::kLds / 4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ci = lane & 15, q = lane >> 4;  // MFMA lane: row / column index, quarter
  const int wr = wave % WR, wc = wave / WR;

  const int kt = tile % tiles_k;
  const int mt = tile / tiles_k;
  const int m0 = mt * BM, k0 = kt * BK;
  const int nst = (ne - nb) >> 6;

  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(C32, BCOPY ? (uint32_t)((size_t)tiles_k * (size_t)(N / 64) * 16384u) : (uint32_t)((size_t)N * (size_t)K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (uint32_t)((size_t)N * (size_t)(K / 64) * 4));
  const int mpad = (M + 15) & ~15;
  const __amdgpu_buffer_rsrc_t rg =
      make_rsrc(G, (uint32_t)((size_t)(AF ? mpad : M) * (size_t)N * (AF ? 2 : 4)));
  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row
  auto stage_row = [&](int st) { return (uint32_t)(nb + 64 * min(st, nst - 1)); };

  // ---- MFMA role: rows 64*wr + 16*rb + ci of the tile, reduction quarter q ----
  // grad_out load v (0..7) of a k-step: row 16*(lane/16) + 4*((lane/4)%4) + v/2
  // of the wave's 64, 16-byte chunk 4*(v%2) + lane%4 of the k-step's 128 bytes.
  uint32_t voff_g[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = min(m0 + 64 * wr + 16 * (lane >> 4) + 4 * ((lane >> 2) & 3) + u, M - 1);
    voff_g[u] = (uint32_t)row * (uint32_t)N * 4u + 16u * (uint32_t)(lane & 3);
  }
  const uint32_t rbase = Cfg::kFragBase + (uint32_t)wc * 8192u + 16u * lane;
  // fragment role (AF): fragment (mb, ks) of row block rb at
  // ((mb * N/32 + ks) * 64 + lane) * 16, mb = (m0 + 64 wr) / 16 + rb; blocks
  // past the padded M read zero through the buffer range
  uint32_t voff_f[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    voff_f[rb] = ((uint32_t)((m0 + 64 * wr) / 16 + rb) * (uint32_t)(N / 32) * 64u + (uint32_t)lane) * 16u;

  // ---- decode role: rows (nr0, nr0 + 1) of a stage, code dword 16*v + dl ----
  // Wave w takes the 8 stage rows that fill lane quarter q = w%4 of k-step
  // w/4 -- rows 16*(p/2) + 4q + 2*(p%2) (+1) of the k-step for its lane pair p,
  // which are B-operand register p -- so that a half-wave's fragment stores
  // are 32 consecutive dwords.
  const int p = lane & 3, dl = lane >> 2;
  const int nr0 = 32 * (wave >> 2) + 16 * (p >> 1) + 4 * (wave & 3) + 2 * (p & 1);
  // Code columns past K (last tile) read the next row, or zero past the end of
  // the array; they only reach columns that are never stored.
  const uint32_t cvoff = (uint32_t)nr0 * crow + (uint32_t)(k0 / 2 + 4 * dl);
  uint32_t tb[WC][2];
#pragma unroll
  for (int v = 0; v < WC; ++v) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t slot = (uint32_t)((nr0 + r) * KB + 2 * v + (dl >> 3));
      tb[v][r] = Cfg::kTabBase + table_pos<KB>(slot) * 32u;
    }
  }
  // fragment dword written for column c of code dword 16*v + dl: k-step wave/4,
  // group v, tile c, lane dl + 16*(wave%4), register p
  const uint32_t wb = Cfg::kFragBase + (uint32_t)(wave >> 2) * WC * 8192u +
                      (uint32_t)(dl + 16 * (wave & 3)) * 16u + 4u * (uint32_t)p;

  // ---- table role: slot (tid / 4) + 128 * u, levels 4 * (tid % 4) .. + 3 ----
  // (slot + 128 is row + 128 / KB of the same block, and its table sits 4 KiB
  // further; scale blocks past K read like code columns past K.)
  const int qq = tid & 3;
  const int sl0 = tid >> 2;
  const uint32_t svoff = (uint32_t)(sl0 / KB) * srow + 4u * (uint32_t)(k0 / 64 + sl0 % KB);
  const uint32_t twaddr = Cfg::kTabBase + table_pos<KB>((uint32_t)sl0) * 32u + 8u * qq;
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = kLevels[4 * qq + i];

  floatx4_t acc[4][8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[rb][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto load_codes = [&](int st, uint32_t (&x)[WC][2]) {
    const uint32_t r0 = stage_row(st);
#pragma unroll
    for (int v = 0; v < WC; ++v) {
      x[v][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff + 64u * v, r0 * crow, 0);
      x[v][1] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff + 64u * v, (r0 + 1) * crow, 0);
    }
  };
  auto load_scales = [&](int st, float (&sc)[WC]) {
    const uint32_t r0 = stage_row(st);
#pragma unroll
    for (int u = 0; u < WC; ++u)
      sc[u] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, svoff, (r0 + (uint32_t)(u * 128 / KB)) * srow, 0));
  };
  auto build_tables = [&](const float (&sc)[WC], uint32_t toff) {
#pragma unroll
    for (int u = 0; u < WC; ++u) {
      u32x2 w;
      w[0] = pack_half2_rne(sc[u] * lv[0], sc[u] * lv[1]);
      w[1] = pack_half2_rne(sc[u] * lv[2], sc[u] * lv[3]);
      lds_store_u32x2(smem, twaddr + toff + 4096u * u, w);
    }
  };
  // grad_out of k-step s of a stage, loaded coalesced (see voff_g)
  auto load_a = [&](int st, int s, float (&a)[8][4]) {
    const uint32_t soff = stage_row(st) * 4u;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const floatx4 x = __builtin_bit_cast(
          floatx4, __builtin_amdgcn_raw_buffer_load_b128(rg, voff_g[v >> 1] + (uint32_t)(128 * s + 64 * (v & 1)), soff, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) a[v][e] = x[e];
    }
  };
  // fp16 rounding, then the lane-bit exchanges that turn the load layout into
  // the A layout.  Register index v = (v2 v1 v0) and lane = (l5 .. l0): loaded,
  // l1 l0 = chunk bits C1 C0, v0 = C2, (l3 l2 v2 v1) = row bits R3..R0 and
  // l5 l4 = R5 R4.  Exchanging l0 <-> v1, l1 <-> v2, l4 <-> v1, l5 <-> v2 gives
  // lane = (C1 C0 R3 R2 R1 R0) = (q, i) and v = (R5 R4 C2) = (row block, half).
  auto round_a = [&](const float (&a)[8][4], uint32_t (&r)[8][2]) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      r[v][0] = pack_half2_rne(a[v][0], a[v][1]);
      r[v][1] = pack_half2_rne(a[v][2], a[v][3]);
    }
  };
  auto to_a_frags = [&](uint32_t (&r)[8][2], u32x4 (&af)[4]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // l0 <-> v1: pairs (v, v + 2), v in {4g, 4g + 1}
      uint32_t lo[4] = {r[4 * g][0], r[4 * g][1], r[4 * g + 1][0], r[4 * g + 1][1]};
      uint32_t hi[4] = {r[4 * g + 2][0], r[4 * g + 2][1], r[4 * g + 3][0], r[4 * g + 3][1]};
      xchg_lane_lo4<0>(lo, hi);
      r[4 * g][0] = lo[0]; r[4 * g][1] = lo[1]; r[4 * g + 1][0] = lo[2]; r[4 * g + 1][1] = lo[3];
      r[4 * g + 2][0] = hi[0]; r[4 * g + 2][1] = hi[1]; r[4 * g + 3][0] = hi[2]; r[4 * g + 3][1] = hi[3];
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // l1 <-> v2: pairs (v, v + 4), v in {2g, 2g + 1}
      uint32_t lo[4] = {r[2 * g][0], r[2 * g][1], r[2 * g + 1][0], r[2 * g + 1][1]};
      uint32_t hi[4] = {r[2 * g + 4][0], r[2 * g + 4][1], r[2 * g + 5][0], r[2 * g + 5][1]};
      xchg_lane_lo4<1>(lo, hi);
      r[2 * g][0] = lo[0]; r[2 * g][1] = lo[1]; r[2 * g + 1][0] = lo[2]; r[2 * g + 1][1] = lo[3];
      r[2 * g + 4][0] = hi[0]; r[2 * g + 4][1] = hi[1]; r[2 * g + 5][0] = hi[2]; r[2 * g + 5][1] = hi[3];
    }
#pragma unroll
    for (int v = 0; v < 8; ++v)  // l4 <-> v1
      if ((v & 2) == 0) {
        xchg_lane_hi<4>(r[v][0], r[v + 2][0]);
        xchg_lane_hi<4>(r[v][1], r[v + 2][1]);
      }
#pragma unroll
    for (int v = 0; v < 8; ++v)  // l5 <-> v2
      if ((v & 4) == 0) {
        xchg_lane_hi<5>(r[v][0], r[v + 4][0]);
        xchg_lane_hi<5>(r[v][1], r[v + 4][1]);
      }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      af[rb][0] = r[2 * rb][0];
      af[rb][1] = r[2 * rb][1];
      af[rb][2] = r[2 * rb + 1][0];
      af[rb][3] = r[2 * rb + 1][1];
    }
  };

  uint32_t y[WC][2], z[WC][2];  // code nibbles times two: low nibbles (even columns), high (odd)
  auto prep = [&](const uint32_t (&x)[WC][2]) {
#pragma unroll
    for (int v = 0; v < WC; ++v)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        y[v][r] = (x[v][r] << 1) & 0x1E1E1E1Eu;
        z[v][r] = (x[v][r] >> 3) & 0x1E1E1E1Eu;
      }
  };
  // Decode of column c: the two table reads, then (after other work) the pack
  // of both rows into one B-operand dword and its store.
  auto lookup_col = [&](auto cc, uint32_t toff, uint32_t (&lk)[WC][2]) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int v = 0; v < WC; ++v) {
      const uint32_t s0 = (c & 1) ? z[v][0] : y[v][0];
      const uint32_t s1 = (c & 1) ? z[v][1] : y[v][1];
      lk[v][0] = lds_load_u16(smem, add_byte<(c >> 1)>(tb[v][0], s0) + toff);
      lk[v][1] = lds_load_u16(smem, add_byte<(c >> 1)>(tb[v][1], s1) + toff);
    }
  };
  auto store_col = [&](auto cc, uint32_t foff, const uint32_t (&lk)[WC][2]) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int v = 0; v < WC; ++v)
      lds_store_u32(smem, wb + foff + (uint32_t)(v * 8192 + c * 1024), lk[v][0] | (lk[v][1] << 16));
  };

  // fp16 A fragments of k-step j of the chunk (j = 2 * stage + s), 4 row blocks
  auto load_af = [&](int j, u32x4 (&af)[4]) {
    const uint32_t soff = (stage_row(j >> 1) / 32u + (uint32_t)(j & 1)) * 1024u;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) af[rb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, voff_f[rb], soff, 0));
  };
  constexpr int NAB = AF ? AF + 1 : 1;  // fragment buffers in the ring
  // buffer (2 P + s) % NAB must hold k-step 2 st + s for either stage parity P = st % 2
  static_assert(4 % NAB == 0, "fragment ring of 1, 2 or 4 buffers");
  u32x4 afr[NAB][4];

  // fragment copy (BCOPY): thread tid moves bytes 16 tid and 8192 + 16 tid of a stage's 16 KiB
  auto load_bf = [&](int st, u32x4 (&x)[2]) {
    const uint32_t off = ((uint32_t)kt * (uint32_t)(N / 64) + stage_row(st) / 64u) * 16384u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      x[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, 16u * (uint32_t)tid + 8192u * h, off, 0));
  };
  auto store_bf = [&](uint32_t foff, const u32x4 (&x)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) lds_store_u32x4(smem, Cfg::kFragBase + foff + 16u * (uint32_t)tid + 8192u * h, x[h]);
  };
  u32x4 bfx[2];  // B fragments of the stage copied during the current one (BCOPY)

  float ar[8][4];       // grad_out of the next k-step, as loaded
  uint32_t xc[WC][2];   // codes of the stage decoded during the current one
  float sc[WC];         // scales of the tables built during the current stage

  // Prologue: tables of stages 0 and 1, stage 0 decoded into fragment buffer 0
  // (or, BCOPY, stage 0 copied into it and stage 1 loaded).
  if constexpr (BCOPY) {
    u32x4 b0[2];
    load_bf(0, b0);
    load_bf(1, bfx);
#pragma unroll
    for (int j = 0; j < AF; ++j) load_af(j, afr[j]);
    store_bf(0u, b0);
    __syncthreads();
  } else {
    float s0[WC], s1[WC];
    uint32_t x0[WC][2];
    load_scales(0, s0);
    load_scales(1, s1);
    load_codes(0, x0);
    load_codes(1, xc);
    if constexpr (AF) {
#pragma unroll
      for (int j = 0; j < AF; ++j) load_af(j, afr[j]);
    } else {
      load_a(0, 0, ar);
    }
    load_scales(2, sc);
    build_tables(s0, 0);
    build_tables(s1, kTabStage);
    __syncthreads();
    prep(x0);
    for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto cc) {
      uint32_t lk[WC][2];
      lookup_col(cc, 0u, lk);
      NF4_PHASE_BARRIER();
      store_col(cc, 0u, lk);
    });
    __syncthreads();
  }

  // One stage: MFMAs on fragment buffer P, decode of stage st+1 into buffer
  // P^1 with tables P^1, tables of stage st+2 into table buffer P.
  auto stage = [&](int st, auto par) {
    constexpr uint32_t P = decltype(par)::value;
    constexpr uint32_t toff_dec = (P ^ 1u) * kTabStage, toff_build = P * kTabStage;
    constexpr uint32_t frd = P * kFragStage, fwr = (P ^ 1u) * kFragStage;
    uint32_t xn[WC][2];
    float scn[WC];
    u32x4 bfn[2];
    if constexpr (!BCOPY) prep(xc);
    // k-step s: convert grad_out of s and issue the loads of the next k-step,
    // then 8 ticks, one per MFMA tile t (4 MFMAs, one per row block).  B
    // fragments are read three ticks ahead through a ring of four, across the
    // two k-steps of the stage (the stage's buffer is complete since its
    // barrier), so only the stage's first MFMAs wait on a fresh read; the decode
    // of columns 4s .. 4s+3 of the next stage (table reads, then two ticks
    // later the pack and fragment store) and the per-stage extras are spread
    // over the ticks.  Scheduling barriers between ticks keep every load where
    // it is issued (the compiler would otherwise sink loads to their uses).
    u32x4 bf[4];
    for_each_index(std::make_integer_sequence<int, 2>{}, [&](auto sc_) {
      constexpr int s = decltype(sc_)::value;
      constexpr int c0 = 4 * s;  // decode columns c0 .. c0 + 3 in this k-step
      u32x4 af[4];
      if constexpr (AF) {
        // fragments of this k-step were loaded AF k-steps ago; issue the
        // loads of k-step + AF into the buffer the previous k-step used
        constexpr int b = (2 * (int)P + s) % NAB;
        load_af(2 * st + s + AF, afr[(b + AF) % NAB]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) af[rb] = afr[b][rb];
      } else {
        // round this k-step's grad_out (freeing the load registers), issue the
        // next k-step's loads, then transpose: the loads do not wait for the
        // transpose, and its temporaries never coexist with the raw values
        uint32_t rr[8][2];
        round_a(ar, rr);
        __builtin_amdgcn_sched_barrier(0);
        load_a(s == 0 ? st : st + 1, s ^ 1, ar);
        __builtin_amdgcn_sched_barrier(0);
        to_a_frags(rr, af);
      }
      // B fragments of tick g = 8 k-step + tile of the stage
      auto read_b = [&](int g) { return lds_load_u32x4(smem, rbase + frd + (uint32_t)(((g / 8) * WC * 8 + g % 8) * 1024)); };
      if constexpr (s == 0) {
        bf[0] = read_b(0);
        bf[1] = read_b(1);
        bf[2] = read_b(2);
      }
      uint32_t lk[2][WC][2];
      __builtin_amdgcn_sched_barrier(0);
      for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto tc) {
        constexpr int t = decltype(tc)::value;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(af[rb]), as_half8(bf[t % 4]), acc[rb][t], 0, 0, 0);
        if constexpr (8 * s + t + 3 < 16) bf[(t + 3) % 4] = read_b(8 * s + t + 3);
        if constexpr (BCOPY) {
          if constexpr (t == 2 && s == 0) store_bf(fwr, bfx);
          if constexpr (t == 6 && s == 0) load_bf(st + 2, bfn);
        } else {
          if constexpr (t >= 2 && t < 6) store_col(std::integral_constant<int, c0 + t - 2>{}, fwr, lk[t & 1]);
          if constexpr (t < 4) lookup_col(std::integral_constant<int, c0 + t>{}, toff_dec, lk[t & 1]);
          if constexpr (t == 6 && s == 0) load_codes(st + 2, xn);
          if constexpr (t == 6 && s == 1) load_scales(st + 3, scn);
          if constexpr (t == 7 && s == 0) build_tables(sc, toff_build);
          // (not for the fp32-fed variant, whose registers do not fit the fixed
          // order; the four-wave tiles, which hold two decode slots per lane,
          // spill or run slower with it)
          if constexpr (AF > 0) interleave_tick<4>();
        }
        __builtin_amdgcn_sched_barrier(0);
        NF4_PHASE_BARRIER();  // race-check build: every tick's LDS accesses complete before the next
      });
    });
    __syncthreads();
    if constexpr (BCOPY) {
      bfx[0] = bfn[0];
      bfx[1] = bfn[1];
    } else {
#pragma unroll
      for (int v = 0; v < WC; ++v) {
        xc[v][0] = xn[v][0];
        xc[v][1] = xn[v][1];
        sc[v] = scn[v];
      }
    }
  };

  int st = 0;
  for (; st + 1 < nst; st += 2) {
    stage(st, std::integral_constant<uint32_t, 0>{});
    stage(st + 1, std::integral_constant<uint32_t, 1>{});
  }
  if (st < nst) stage(st, std::integral_constant<uint32_t, 0>{});

  // 16x16 accumulator layout: lane (ci, q), register r -> row 4*q + r, column ci.
  const int col = k0 + 128 * wc + 8 * ci;
  if (col < K) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * wr + 16 * rb + 4 * q + r;
        if (row < M) {
          const floatx4 lo = {acc[rb][0][r], acc[rb][1][r], acc[rb][2][r], acc[rb][3][r]};
          const floatx4 hi = {acc[rb][4][r], acc[rb][5][r], acc[rb][6][r], acc[rb][7][r]};
          floatx4* o = reinterpret_cast<floatx4*>(dst + (size_t)(row - row0) * (size_t)ld + (col - col0));
          o[0] = lo;
          o[1] = hi;
        }
      }
    }
  }
}

// Mid-size tiles: 64 RB x 128 with four waves (256 threads), for problems
// whose 512 x 128 tiles leave CUs idle or end in a thin last round.  RB = 4:
// 256 x 128, wave w owns rows 64w .. 64w + 63 (four 16-row blocks x eight
// MFMA tiles, 128 accumulators per lane, as in the eight-wave kernel), two
// workgroups per CU.  RB = 2: 128 x 128, 32 rows per wave, three workgroups
// per CU, for problems small enough that one round of these tiles covers
// them without splitting N.  Both are fed by the same fp16 A fragments.  The
// decode and table roles and every LDS layout are those of the eight-wave
// kernel, each lane playing two of its lanes (waves w and w + 4), so the B
// operands and the reduction order are the same and the results are bitwise
// equal to the 512 x 128 kernel's.
template <int AF, int RB>
__device__ __forceinline__ void mid_tile(const void* __restrict__ Gv, const float* __restrict__ S,
                                         const uint32_t* __restrict__ C32, int M, int N, int K, int tiles_k, int tile,
                                         int nb, int ne, float* __restrict__ dst, int ld) {
  // buffer (2 P + s) % (AF + 1) must hold k-step 2 st + s for either stage parity P = st % 2
  static_assert(AF == 1 || AF == 3, "fragment prefetch depth 1 or 3");
  static_assert(RB == 2 || RB == 4, "16-row blocks per wave: 2 or 4");
  using Cfg = WideCfg<1>;
  constexpr int BK = Cfg::BK, KB = Cfg::KB;
  constexpr uint32_t kTabStage = Cfg::kTabStage, kFragStage = Cfg::kFragStage;
  constexpr int BM = 64 * RB;  // tile rows: four waves of 16 RB rows
  __shared__ __attribute__((aligned(16))) uint32_t smem[Cfg::kLds / 4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  const int kt = tile % tiles_k;
  const int mt = tile / tiles_k;
  const int m0 = mt * BM, k0 = kt * BK;
  const int nst = (ne - nb) >> 6;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(C32, (uint32_t)((size_t)N * (size_t)K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (uint32_t)((size_t)N * (size_t)(K / 64) * 4));
  const int mpad = (M + 15) & ~15;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gv, (uint32_t)((size_t)mpad * (size_t)N * 2));
  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row
  auto stage_row = [&](int st) { return (uint32_t)(nb + 64 * min(st, nst - 1)); };

  // ---- MFMA role: rows 128*wave + 16*rb + ci of the tile ----
  const uint32_t rbase = Cfg::kFragBase + 16u * lane;
  // fragment (mb, ks) of row block rb at ((mb * N/32 + ks) * 64 + lane) * 16,
  // mb = (m0 + 128 wave) / 16 + rb; blocks past the padded M read zero
  const uint32_t fstride = (uint32_t)(N / 32) * 1024u;  // bytes between row blocks
  const uint32_t voff_f = ((uint32_t)((m0 + 16 * RB * wave) / 16) * (uint32_t)(N / 32) * 64u + (uint32_t)lane) * 16u;

  // ---- decode role: the eight-wave kernel's waves w and w + 4 (k-steps 0 and 1) ----
  const int p = lane & 3, dl = lane >> 2;
  uint32_t cvoff[2], tb[2][2], wb[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int vw = wave + 4 * v;
    const int nr0 = 32 * (vw >> 2) + 16 * (p >> 1) + 4 * (vw & 3) + 2 * (p & 1);
    cvoff[v] = (uint32_t)nr0 * crow + (uint32_t)(k0 / 2 + 4 * dl);
#pragma unroll
    for (int r = 0; r < 2; ++r) tb[v][r] = Cfg::kTabBase + table_pos<KB>((uint32_t)((nr0 + r) * KB + (dl >> 3))) * 32u;
    wb[v] = Cfg::kFragBase + (uint32_t)(vw >> 2) * 8192u + (uint32_t)(dl + 16 * (vw & 3)) * 16u + 4u * (uint32_t)p;
  }
  // ---- table role: slots tid / 4 and tid / 4 + 64, levels 4 * (tid % 4) .. + 3 ----
  const int qq = tid & 3;
  uint32_t svoff[2], twaddr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = (tid >> 2) + 64 * u;
    svoff[u] = (uint32_t)(sl / KB) * srow + 4u * (uint32_t)(k0 / 64 + sl % KB);
    twaddr[u] = Cfg::kTabBase + table_pos<KB>((uint32_t)sl) * 32u + 8u * qq;
  }
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = kLevels[4 * qq + i];

  floatx4_t acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[rb][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto load_codes = [&](int st, uint32_t (&x)[2][2]) {
    const uint32_t r0 = stage_row(st);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      x[v][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff[v], r0 * crow, 0);
      x[v][1] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff[v], (r0 + 1) * crow, 0);
    }
  };
  auto load_scales = [&](int st, float (&sc)[2]) {
    const uint32_t r0 = stage_row(st);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      sc[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, svoff[u], r0 * srow, 0));
  };
  auto build_tables = [&](const float (&sc)[2], uint32_t toff) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x2 w;
      w[0] = pack_half2_rne(sc[u] * lv[0], sc[u] * lv[1]);
      w[1] = pack_half2_rne(sc[u] * lv[2], sc[u] * lv[3]);
      lds_store_u32x2(smem, twaddr[u] + toff, w);
    }
  };
  uint32_t y[2][2], z[2][2];
  auto prep = [&](const uint32_t (&x)[2][2]) {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        y[v][r] = (x[v][r] << 1) & 0x1E1E1E1Eu;
        z[v][r] = (x[v][r] >> 3) & 0x1E1E1E1Eu;
      }
  };
  // decode of column c for both roles: four table reads, then (later) two packed stores
  auto lookup_col = [&](auto cc, uint32_t toff, uint32_t (&lk)[2][2]) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const uint32_t s0 = (c & 1) ? z[v][0] : y[v][0];
      const uint32_t s1 = (c & 1) ? z[v][1] : y[v][1];
      lk[v][0] = lds_load_u16(smem, add_byte<(c >> 1)>(tb[v][0], s0) + toff);
      lk[v][1] = lds_load_u16(smem, add_byte<(c >> 1)>(tb[v][1], s1) + toff);
    }
  };
  auto store_col = [&](auto cc, uint32_t foff, const uint32_t (&lk)[2][2]) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int v = 0; v < 2; ++v) lds_store_u32(smem, wb[v] + foff + (uint32_t)(c * 1024), lk[v][0] | (lk[v][1] << 16));
  };
  // fp16 A fragments of k-step j of the chunk (j = 2 * stage + s), 8 row blocks
  auto load_af = [&](int j, u32x4 (&af)[RB]) {
    const uint32_t soff = (stage_row(j >> 1) / 32u + (uint32_t)(j & 1)) * 1024u;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      af[rb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, voff_f, soff + (uint32_t)rb * fstride, 0));
  };
  constexpr int NAB = AF + 1;  // fragment buffers in the ring
  u32x4 afr[NAB][RB];

  uint32_t xc[2][2];  // codes of the stage decoded during the current one
  float sc[2];        // scales of the tables built during the current stage

  // Prologue: tables of stages 0 and 1, stage 0 decoded into fragment buffer 0.
  {
    float s0[2], s1[2];
    uint32_t x0[2][2];
    load_scales(0, s0);
    load_scales(1, s1);
    load_codes(0, x0);
    load_codes(1, xc);
#pragma unroll
    for (int j = 0; j < AF; ++j) load_af(j, afr[j]);
    load_scales(2, sc);
    build_tables(s0, 0);
    build_tables(s1, kTabStage);
    __syncthreads();
    prep(x0);
    for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto cc) {
      uint32_t lk[2][2];
      lookup_col(cc, 0u, lk);
      NF4_PHASE_BARRIER();
      store_col(cc, 0u, lk);
    });
    __syncthreads();
  }

  // One stage: MFMAs on fragment buffer P, decode of stage st+1 into buffer
  // P^1 with tables P^1, tables of stage st+2 into table buffer P.  Per
  // k-step, eight ticks (one MFMA tile each, four row blocks): B fragments
  // read three ticks ahead through a ring of four across the stage's two
  // k-steps; the decode of columns 4s .. 4s+3 of the next stage and the
  // per-stage extras spread over them.
  auto stage = [&](int st, auto par) {
    constexpr uint32_t P = decltype(par)::value;
    constexpr uint32_t toff_dec = (P ^ 1u) * kTabStage, toff_build = P * kTabStage;
    constexpr uint32_t frd = P * kFragStage, fwr = (P ^ 1u) * kFragStage;
    uint32_t xn[2][2];
    float scn[2];
    prep(xc);
    u32x4 bf[4];
    for_each_index(std::make_integer_sequence<int, 2>{}, [&](auto sc_) {
      constexpr int s = decltype(sc_)::value;
      constexpr int c0 = 4 * s;
      constexpr int b = (2 * (int)P + s) % NAB;
      load_af(2 * st + s + AF, afr[(b + AF) % NAB]);
      __builtin_amdgcn_sched_barrier(0);
      auto read_b = [&](int g) { return lds_load_u32x4(smem, rbase + frd + (uint32_t)(g * 1024)); };
      if constexpr (s == 0) {
        bf[0] = read_b(0);
        bf[1] = read_b(1);
        bf[2] = read_b(2);
      }
      uint32_t lk[2][2][2];
      __builtin_amdgcn_sched_barrier(0);
      for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto tc) {
        constexpr int t = decltype(tc)::value;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(afr[b][rb]), as_half8(bf[t % 4]), acc[rb][t], 0, 0, 0);
        if constexpr (8 * s + t + 3 < 16) bf[(t + 3) % 4] = read_b(8 * s + t + 3);
        if constexpr (t >= 2 && t < 6) store_col(std::integral_constant<int, c0 + t - 2>{}, fwr, lk[t & 1]);
        if constexpr (t < 4) lookup_col(std::integral_constant<int, c0 + t>{}, toff_dec, lk[t & 1]);
        if constexpr (t == 6 && s == 0) load_codes(st + 2, xn);
        if constexpr (t == 6 && s == 1) load_scales(st + 3, scn);
        if constexpr (t == 7 && s == 0) build_tables(sc, toff_build);
        if constexpr (RB == 4) interleave_tick_memory<RB>();
        __builtin_amdgcn_sched_barrier(0);
        NF4_PHASE_BARRIER();  // race-check build: every tick's LDS accesses complete before the next
      });
    });
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      xc[v][0] = xn[v][0];
      xc[v][1] = xn[v][1];
      sc[v] = scn[v];
    }
  };

  int st = 0;
  for (; st + 1 < nst; st += 2) {
    stage(st, std::integral_constant<uint32_t, 0>{});
    stage(st + 1, std::integral_constant<uint32_t, 1>{});
  }
  if (st < nst) stage(st, std::integral_constant<uint32_t, 0>{});

  // 16x16 accumulator layout: lane (ci, q), register r -> row 4*q + r, column ci.
  const int ci = lane & 15, q = lane >> 4;
  const int col = k0 + 8 * ci;
  if (col < K) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * RB * wave + 16 * rb + 4 * q + r;
        if (row < M) {
          const floatx4 lo = {acc[rb][0][r], acc[rb][1][r], acc[rb][2][r], acc[rb][3][r]};
          const floatx4 hi = {acc[rb][4][r], acc[rb][5][r], acc[rb][6][r], acc[rb][7][r]};
          floatx4* o = reinterpret_cast<floatx4*>(dst + (size_t)row * (size_t)ld + col);
          o[0] = lo;
          o[1] = hi;
        }
      }
    }
  }
}

template <int AF>
__global__ __launch_bounds__(256, 2) void grad_a_mid_kernel(const void* __restrict__ frags, const float* __restrict__ S,
                                                            const uint32_t* __restrict__ C32, float* __restrict__ out,
                                                            int M, int N, int K, int n_chunk, int tiles_m,
                                                            int tiles_k) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = tiles_m * tiles_k;
  const int split = logical / tiles;
  const int nb = split * n_chunk;
  mid_tile<AF, 4>(frags, S, C32, M, N, K, tiles_k, logical % tiles, nb, min(N, nb + n_chunk),
                  out + (size_t)split * (size_t)M * (size_t)K, K);
}

// 128 x 128 tiles (two 16-row blocks per wave), three workgroups per CU.
__global__ __launch_bounds__(256, 3) void grad_a_small_kernel(const void* __restrict__ frags,
                                                              const float* __restrict__ S,
                                                              const uint32_t* __restrict__ C32,
                                                              float* __restrict__ out, int M, int N, int K,
                                                              int n_chunk, int tiles_m, int tiles_k) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = tiles_m * tiles_k;
  const int split = logical / tiles;
  const int nb = split * n_chunk;
  mid_tile<1, 2>(frags, S, C32, M, N, K, tiles_k, logical % tiles, nb, min(N, nb + n_chunk),
                 out + (size_t)split * (size_t)M * (size_t)K, K);
}

// One tile over one N-chunk per workgroup; the chunk index is the slowest
// part of the logical index and selects the partial-sum matrix it writes.
template <int WC, int AF, bool BCOPY = false>
__global__ __launch_bounds__(512, 1) void grad_a_wide_kernel(
    const void* __restrict__ Gv, const float* __restrict__ S, const uint32_t* __restrict__ C32,
    float* __restrict__ out, int M, int N, int K, int n_chunk, int tiles_m, int tiles_k) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = tiles_m * tiles_k;
  const int split = logical / tiles;
  const int nb = split * n_chunk;
  wide_tile<WC, AF, BCOPY>(Gv, S, C32, M, N, K, tiles_k, logical % tiles, nb, min(N, nb + n_chunk),
                           out + (size_t)split * (size_t)M * (size_t)K, K, 0, 0);
}

// Grouped launch: the tiles of up to kWideGroupMax problems sharing M (each
// fed by its fp16 A fragments, no N split) in one grid.  The host orders the
// problems longest reduction first.  Tiles are dealt to the 8 XCDs in groups
// of 8 consecutive tiles (8 k-tiles of one m-tile, which share grad_out
// fragments in that XCD's L2), group g to XCD g % 8, so that every XCD works
// through its share in the same longest-first order and gets a balanced mix.
// Workgroups past the last tile (the grid is padded to whole rounds of
// groups) return at once.
__global__ __launch_bounds__(512, 1) void grad_a_wide_grouped_kernel(WideGroup g) {
  const int b = blockIdx.x;
  const int x = b & 7, slot = b >> 3;
  const int tile = ((slot >> 3) * 8 + x) * 8 + (slot & 7);
  if (tile >= g.total) return;
  const void* frags = g.p[0].frags;
  const float* scales = g.p[0].scales;
  const uint32_t* codes = g.p[0].codes;
  float* out = g.p[0].out;
  int N = g.p[0].N, K = g.p[0].K, tiles_k = g.p[0].tiles_k, begin = 0;
#pragma unroll
  for (int j = 1; j < kWideGroupMax; ++j)
    if (j < g.count && tile >= g.p[j].tile_begin) {
      frags = g.p[j].frags;
      scales = g.p[j].scales;
      codes = g.p[j].codes;
      out = g.p[j].out;
      N = g.p[j].N;
      K = g.p[j].K;
      tiles_k = g.p[j].tiles_k;
      begin = g.p[j].tile_begin;
    }
  wide_tile<1, WIDE_FRAG_DEPTH, false>(frags, scales, codes, g.M, N, K, tiles_k, tile - begin, 0, N, out, K, 0, 0);
}

bool wide_kernel_supported(int64_t M, int64_t N, int64_t K) {
  return N > 0 && (N % 64) == 0 && (uint64_t)M * (uint64_t)N * 4 < (1ull << 31) &&
         (uint64_t)N * (uint64_t)K / 2 < (1ull << 31);
}

int wide_tile_rows() { return WideCfg<1>::BM; }
int wide_tile_cols() { return WideCfg<1>::BK; }

hipError_t launch_grad_a_wide(int grid, const float* grad_out, const float* scales, const uint32_t* codes, float* dst,
                              int M, int N, int K, int n_chunk, int tiles_m, int tiles_k, hipStream_t stream) {
  hipLaunchKernelGGL((grad_a_wide_kernel<1, 0>), dim3(grid), dim3(512), 0, stream, grad_out, scales, codes, dst, M, N,
                     K, n_chunk, tiles_m, tiles_k);
  return hipGetLastError();
}

size_t wide_frag_bytes(int64_t M, int64_t N) { return (size_t)((M + 15) / 16) * 16 * (size_t)N * 2; }

size_t unfused_bfrag_bytes(int64_t N, int64_t K) { return (size_t)((K + 127) / 128) * (size_t)(N / 64) * 16384; }

hipError_t launch_grad_a_wide_grouped(const WideGroup& g, hipStream_t stream) {
  const int groups = (g.total + 7) / 8;
  const int grid = ((groups + 7) / 8) * 64;
  hipLaunchKernelGGL(grad_a_wide_grouped_kernel, dim3(grid), dim3(512), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_grad_a_unfused(int grid, const float* grad_out, void* afrags, void* bfrags, const float* scales,
                                 const uint32_t* codes, float* dst, int M, int N, int K, int n_chunk, int tiles_m,
                                 int tiles_k, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_bfrag_kernel, dim3(((K + 127) / 128) * (N / 64)), dim3(512), 0, stream, scales, codes,
                     static_cast<uint32_t*>(bfrags), N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_frag_pass(grad_out, afrags, M, N, /*natural=*/false, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grad_a_wide_kernel<1, WIDE_FRAG_DEPTH, true>), dim3(grid), dim3(512), 0, stream, afrags, scales,
                     static_cast<const uint32_t*>(bfrags), dst, M, N, K, n_chunk, tiles_m, tiles_k);
  return hipGetLastError();
}

hipError_t launch_frag_pass(const float* src, void* frags, int rows, int cols, bool natural, hipStream_t stream) {
  const int64_t total = (int64_t)((rows + 15) / 16) * (cols / 32) * 64;
  const int pgrid = (int)std::min<int64_t>((total + 255) / 256, 16384);
  if (natural)
    hipLaunchKernelGGL(grad_out_frag_kernel<true>, dim3(pgrid), dim3(256), 0, stream, src, static_cast<u32x4*>(frags),
                       rows, cols, total);
  else
    hipLaunchKernelGGL(grad_out_frag_kernel<false>, dim3(pgrid), dim3(256), 0, stream, src, static_cast<u32x4*>(frags),
                       rows, cols, total);
  return hipGetLastError();
}

hipError_t launch_grad_a_mid_frag(int af, int rows, int grid, const float* grad_out, void* frags,
                                  const float* scales, const uint32_t* codes, float* dst, int M, int N, int K,
                                  int n_chunk, int tiles_m, int tiles_k, hipStream_t stream) {
  if (rows != 256 && !(rows == 128 && af == 1)) return hipErrorInvalidValue;
  hipError_t e = launch_frag_pass(grad_out, frags, M, N, /*natural=*/false, stream);
  if (e != hipSuccess) return e;
  if (rows == 128)
    hipLaunchKernelGGL(grad_a_small_kernel, dim3(grid), dim3(256), 0, stream, frags, scales, codes, dst, M, N, K,
                       n_chunk, tiles_m, tiles_k);
  else if (af == 1)
    hipLaunchKernelGGL(grad_a_mid_kernel<1>, dim3(grid), dim3(256), 0, stream, frags, scales, codes, dst, M, N, K,
                       n_chunk, tiles_m, tiles_k);
  else
    hipLaunchKernelGGL(grad_a_mid_kernel<3>, dim3(grid), dim3(256), 0, stream, frags, scales, codes, dst, M, N, K,
                       n_chunk, tiles_m, tiles_k);
  return hipGetLastError();
}

hipError_t launch_grad_a_wide_frag(int grid, const float* grad_out, void* frags, const float* scales,
                                   const uint32_t* codes, float* dst, int M, int N, int K, int n_chunk, int tiles_m,
                                   int tiles_k, hipStream_t stream) {
  hipError_t e = launch_frag_pass(grad_out, frags, M, N, /*natural=*/false, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grad_a_wide_kernel<1, WIDE_FRAG_DEPTH>), dim3(grid), dim3(512), 0, stream, frags, scales, codes,
                     dst, M, N, K, n_chunk, tiles_m, tiles_k);
  return hipGetLastError();
}

}  // namespace nf4
