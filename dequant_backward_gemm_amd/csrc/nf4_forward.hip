// Forward product of the same frozen NF4 layer: C[M x N] = A[M x K] . W^T,
// W = dequant(codes, scales) [N x K] (the subject page's header comment: the
// backward kernel is the analog of the forward C = A @ B over the shared
// dimension K, B_nf4 being K x N, stored as W = B^T).
//
// Same arithmetic as the backward kernels: A rounded fp32 -> fp16 (RNE),
// weights fp16(fl32(scale * level)), fp16 MFMA products accumulated in fp32
// over K, C overwritten.  Here the reduction runs along K, which is the
// contiguous direction of the packed codes, so no operand needs a transpose:
//
// * A goes through the fragment pass in natural order: fragment (16-row block
//   mb, 32-wide k-step ks) is 64 lanes x 16 bytes, lane (ci, q) holding row
//   16mb + ci at k = 32ks + 8q + e (e = 0..7).  The main loop loads each
//   fragment with one 128-bit load per lane, three k-steps ahead.
// * A workgroup (8 waves) owns a 512 x 128 tile of C; each wave owns 64 rows
//   (four 16-row blocks) x all 128 columns (eight 16x16x32 MFMA tiles, column
//   c of tile t being n = n0 + 8c + t), 128 fp32 accumulators per lane, two
//   waves per SIMD.
// * Stages are 64 wide in k, one scale block, so each of the tile's 128 rows
//   of W has one 16-entry fp16 table per stage (built two stages ahead).  The
//   B operand of MFMA tile t at k-step s, lane (c, q), is W[n0 + 8c + t][k0 +
//   32s + 8q .. + 7]: one code dword of one row.  Lane L of wave t of the
//   workgroup decodes exactly that slot for both k-steps (one table read per
//   weight, pairs packed into dwords) and stores it as one 16-byte fragment,
//   one stage ahead of the MFMAs, double-buffered, one barrier per stage.
//   The 16 tables a wave's lookup instruction touches (rows 8c + t, c = 0..15)
//   sit contiguously in LDS.
//
// Bounds: rows of W past N read zero codes and zero scales through the buffer
// ranges (all-zero weights); fragment rows past the padded M read zero; C
// rows past M and columns past N are not stored.  N % 8 == 0 (whole 8-column
// groups per lane), K % 64 == 0 (the packed format).
#include <algorithm>

#include "nf4_kernel_util.h"
#include "nf4_launch.h"

#ifndef FWD_FRAG_DEPTH
#define FWD_FRAG_DEPTH 3
#endif

namespace nf4 {

constexpr int kFwBM = 512, kFwBN = 128;
constexpr uint32_t kFwTabStage = 128 * 32;          // 128 tables x 16 fp16
constexpr uint32_t kFwFragStage = 2 * 8 * 64 * 16;  // [k-step][tile][lane] x 16 B
constexpr uint32_t kFwTabBase = 0;
constexpr uint32_t kFwFragBase = 2 * kFwTabStage;
constexpr uint32_t kFwLds = kFwFragBase + 2 * kFwFragStage;

// LDS position (in tables) of stage row r = 8c + t: the rows of one tile t are contiguous
__device__ __forceinline__ uint32_t fw_tab_pos(uint32_t r) { return (r & 7u) * 16u + (r >> 3); }

// One workgroup's tile: NW waves (8, or 4 with each lane also taking the
// decode and table work of the lane 4 waves further), RB 16-row blocks per
// wave (tile rows 16 * RB * NW), AF k-steps of A fragments in flight.  The
// decode, table and fragment layouts are those of the eight-wave tile, so
// every variant gives bitwise the same result.
template <int NW, int RB, int AF>
__device__ __forceinline__ void forward_tile(uint32_t* smem, const void* __restrict__ Afrag,
                                             const float* __restrict__ S, const uint32_t* __restrict__ C32,
                                             float* __restrict__ out, int M, int N, int K, int k_chunk, int tiles_m,
                                             int tiles_n) {
  static_assert(AF == 1 || AF == 3, "fragment prefetch depth 1 or 3");
  static_assert(NW == 8 || NW == 4, "eight or four waves");
  constexpr int V = 8 / NW;  // decode slots (and tables) per lane
  constexpr int BM = 16 * RB * NW;
  constexpr int NAB = AF + 1;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ci = lane & 15, q = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = logical % tiles_n;
  const int rest = logical / tiles_n;
  const int mt = rest % tiles_m;
  const int split = rest / tiles_m;
  const int m0 = mt * BM, n0 = nt * kFwBN;
  const int kb = split * k_chunk;
  const int ke = min(K, kb + k_chunk);
  const int nst = (ke - kb) >> 6;

  const int mpad = (M + 15) & ~15;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(C32, (uint32_t)((size_t)N * (size_t)K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (uint32_t)((size_t)N * (size_t)(K / 64) * 4));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Afrag, (uint32_t)((size_t)mpad * (size_t)K * 2));
  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row
  auto stage_k = [&](int st) { return (uint32_t)(kb + 64 * min(st, nst - 1)); };

  // ---- MFMA role: rows m0 + 16 RB wave + 16 rb + ci, all 128 columns ----
  uint32_t voff_a[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    voff_a[rb] = ((uint32_t)((m0 + 16 * RB * wave) / 16 + rb) * (uint32_t)(K / 32) * 64u + (uint32_t)lane) * 16u;
  // B fragment slot of MFMA lane l inside its tile's 1 KiB: l ^ (4 (l / 16)), a permutation
  // inside each group of 16 lanes (the decode stores below stay conflict-free)
  const uint32_t rbase = kFwFragBase + 16u * (uint32_t)(lane ^ (4 * q));

  // ---- decode role: slot (k-step s, tile vw, MFMA lane dc + 16 dq): row 8 dc + vw, for the
  // eight-wave tile's wave vw = wave + NW v ----
  // Decode lane L takes dc = (L / 4) % 16, dq = L % 4, so the 32 lanes of a half-wave read the
  // tables of 8 rows (256 contiguous bytes: distinct banks) instead of 16
  const int dc = (lane >> 2) & 15, dq = lane & 3;
  uint32_t cvoff[V], tb[V], wb[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int vw = wave + NW * v;
    const uint32_t drow = (uint32_t)(8 * dc + vw);
    cvoff[v] = (uint32_t)(n0 + drow) * crow + 4u * (uint32_t)dq;
    tb[v] = kFwTabBase + fw_tab_pos(drow) * 32u;
    wb[v] = kFwFragBase + (uint32_t)vw * 1024u + 16u * (uint32_t)((dc + 16 * dq) ^ (4 * dq));  // + s * 8 KiB
  }

  // ---- table role: tables of stage rows tid / 4 + 16 NW u, levels 4 (tid % 4) .. + 3 ----
  uint32_t svoff[V], twaddr[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const uint32_t trow = (uint32_t)((tid >> 2) + 16 * NW * u);
    svoff[u] = (uint32_t)(n0 + trow) * srow;
    twaddr[u] = kFwTabBase + fw_tab_pos(trow) * 32u + 8u * (uint32_t)(tid & 3);
  }
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = kLevels[4 * (tid & 3) + i];

  floatx4 acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[rb][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto load_codes = [&](int st, uint32_t (&x)[V][2]) {
    const uint32_t k0b = stage_k(st) / 2;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s) x[v][s] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff[v], k0b + 16u * s, 0);
  };
  auto load_scales = [&](int st, float (&sc)[V]) {
#pragma unroll
    for (int u = 0; u < V; ++u)
      sc[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, svoff[u], 4u * (stage_k(st) / 64), 0));
  };
  auto build_tables = [&](const float (&sc)[V], uint32_t toff) {
#pragma unroll
    for (int u = 0; u < V; ++u) {
      u32x2 w;
      w[0] = pack_half2_rne(sc[u] * lv[0], sc[u] * lv[1]);
      w[1] = pack_half2_rne(sc[u] * lv[2], sc[u] * lv[3]);
      lds_store_u32x2(smem, twaddr[u] + toff, w);
    }
  };
  // A fragments of k-step j of the chunk (j = 2 * stage + s), RB row blocks
  auto load_af = [&](int j, u32x4 (&af)[RB]) {
    const uint32_t soff = (stage_k(j >> 1) / 32u + (uint32_t)(j & 1)) * 1024u;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      af[rb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a[rb], soff, 0));
  };
  // code of k = 8q + e, times two, in byte e / 2 of y (even e) or z (odd e)
  auto lookup = [&](auto ec, uint32_t x, uint32_t tbv, uint32_t toff) {
    constexpr int e = decltype(ec)::value;
    const uint32_t y = (e & 1) ? ((x >> 3) & 0x1E1E1E1Eu) : ((x << 1) & 0x1E1E1E1Eu);
    return lds_load_u16(smem, add_byte<(e >> 1)>(tbv, y) + toff);
  };

  u32x4 afr[NAB][RB];
  uint32_t xc[V][2];  // codes of the stage decoded during the current one
  float sc[V];        // scales of the tables built during the current stage

  // Prologue: tables of stages 0 and 1, stage 0 decoded into fragment buffer 0.
  {
    float s0[V], s1[V];
    load_scales(0, s0);
    load_scales(1, s1);
    uint32_t x0[V][2];
    load_codes(0, x0);
    load_codes(1, xc);
#pragma unroll
    for (int j = 0; j < AF; ++j) load_af(j, afr[j]);
    load_scales(2, sc);
    build_tables(s0, 0);
    build_tables(s1, kFwTabStage);
    __syncthreads();
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t lk[8];
        for_each_index(std::make_integer_sequence<int, 8>{},
                       [&](auto ec) { lk[decltype(ec)::value] = lookup(ec, x0[v][s], tb[v], 0u); });
        NF4_PHASE_BARRIER();
        u32x4 f;
#pragma unroll
        for (int p = 0; p < 4; ++p) f[p] = lk[2 * p] | (lk[2 * p + 1] << 16);
        lds_store_u32x4(smem, wb[v] + 8192u * s, f);
      }
    __syncthreads();
  }

  // One stage: MFMAs on fragment buffer P, decode of stage st+1 into buffer
  // P^1 with tables P^1, tables of stage st+2 into table buffer P.
  auto stage = [&](int st, auto par) {
    constexpr uint32_t P = decltype(par)::value;
    constexpr uint32_t toff_dec = (P ^ 1u) * kFwTabStage, toff_build = P * kFwTabStage;
    constexpr uint32_t frd = P * kFwFragStage, fwr = (P ^ 1u) * kFwFragStage;
    uint32_t xn[V][2];
    float scn[V];
    for_each_index(std::make_integer_sequence<int, 2>{}, [&](auto sc_) {
      constexpr int s = decltype(sc_)::value;
      constexpr int b = (2 * (int)P + s) % NAB;
      load_af(2 * st + s + AF, afr[(b + AF) % NAB]);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 af[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) af[rb] = afr[b][rb];
      auto read_b = [&](int t) { return lds_load_u32x4(smem, rbase + frd + (uint32_t)((s * 8 + t) * 1024)); };
      u32x4 bf[4];
      bf[0] = read_b(0);
      bf[1] = read_b(1);
      bf[2] = read_b(2);
      uint32_t lk[V][8];
      __builtin_amdgcn_sched_barrier(0);
      // 8 ticks, one per MFMA tile t (RB MFMAs, one per row block); B fragments
      // three ticks ahead through a ring of four; the decode of this
      // k-step's slots of the next stage (2 V table reads per tick for four
      // ticks, then the packs and stores) and the per-stage extras spread over
      // the ticks
      for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto tc) {
        constexpr int t = decltype(tc)::value;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(af[rb]), as_half8(bf[t % 4]), acc[rb][t], 0, 0, 0);
        if constexpr (t + 3 < 8) bf[(t + 3) % 4] = read_b(t + 3);
        if constexpr (t < 4) {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            lk[v][2 * t] = lookup(std::integral_constant<int, 2 * t>{}, xc[v][s], tb[v], toff_dec);
            lk[v][2 * t + 1] = lookup(std::integral_constant<int, 2 * t + 1>{}, xc[v][s], tb[v], toff_dec);
          }
        }
        if constexpr (t == 5) {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            u32x4 f;
#pragma unroll
            for (int p = 0; p < 4; ++p) f[p] = lk[v][2 * p] | (lk[v][2 * p + 1] << 16);
            lds_store_u32x4(smem, wb[v] + fwr + 8192u * s, f);
          }
        }
        if constexpr (t == 6 && s == 0) load_codes(st + 2, xn);
        if constexpr (t == 6 && s == 1) load_scales(st + 3, scn);
        if constexpr (t == 7 && s == 0) build_tables(sc, toff_build);
        // (the four-wave tiles, with two decode slots per lane, spill with the
        // full fixed order; the 256-row ones spread only their memory
        // instructions, measured up to 4% faster, and the 128-row ones keep
        // the compiler's order, where neither form gained)
        if constexpr (NW == 8) interleave_tick<RB>();
        if constexpr (NW == 4 && RB == 4) interleave_tick_memory<RB>();
        __builtin_amdgcn_sched_barrier(0);
        NF4_PHASE_BARRIER();  // race-check build: every tick's LDS accesses complete before the next
      });
    });
    __syncthreads();
#pragma unroll
    for (int v = 0; v < V; ++v) {
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

  // 16x16 accumulator layout: lane (ci, q), register r -> row 4q + r, column ci
  // of tile t, i.e. n = n0 + 8ci + t: eight consecutive outputs per row.
  float* __restrict__ dst = out + (size_t)split * (size_t)M * (size_t)N;
  const int col = n0 + 8 * ci;
  if (col < N) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * RB * wave + 16 * rb + 4 * q + r;
        if (row < M) {
          const floatx4 lo = {acc[rb][0][r], acc[rb][1][r], acc[rb][2][r], acc[rb][3][r]};
          const floatx4 hi = {acc[rb][4][r], acc[rb][5][r], acc[rb][6][r], acc[rb][7][r]};
          floatx4* o = reinterpret_cast<floatx4*>(dst + (size_t)row * (size_t)N + col);
          o[0] = lo;
          o[1] = hi;
        }
      }
    }
  }
}

// 512 x 128 tiles: eight waves of 64 rows, one workgroup per CU.
__global__ __launch_bounds__(512, 1) void nf4_forward_kernel(const void* __restrict__ Afrag,
                                                             const float* __restrict__ S,
                                                             const uint32_t* __restrict__ C32,
                                                             float* __restrict__ out, int M, int N, int K,
                                                             int k_chunk, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[kFwLds / 4];
  forward_tile<8, 4, FWD_FRAG_DEPTH>(smem, Afrag, S, C32, out, M, N, K, k_chunk, tiles_m, tiles_n);
}

// 256 x 128 tiles: four waves of 64 rows, two workgroups per CU.
__global__ __launch_bounds__(256, 2) void nf4_forward_mid_kernel(const void* __restrict__ Afrag,
                                                                 const float* __restrict__ S,
                                                                 const uint32_t* __restrict__ C32,
                                                                 float* __restrict__ out, int M, int N, int K,
                                                                 int k_chunk, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[kFwLds / 4];
  forward_tile<4, 4, 1>(smem, Afrag, S, C32, out, M, N, K, k_chunk, tiles_m, tiles_n);
}

// 128 x 128 tiles: four waves of 32 rows, three workgroups per CU.
__global__ __launch_bounds__(256, 3) void nf4_forward_small_kernel(const void* __restrict__ Afrag,
                                                                   const float* __restrict__ S,
                                                                   const uint32_t* __restrict__ C32,
                                                                   float* __restrict__ out, int M, int N, int K,
                                                                   int k_chunk, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[kFwLds / 4];
  forward_tile<4, 2, 1>(smem, Afrag, S, C32, out, M, N, K, k_chunk, tiles_m, tiles_n);
}

bool forward_supported(int64_t M, int64_t N, int64_t K) {
  return M > 0 && N > 0 && K > 0 && (N % 8) == 0 && (K % 64) == 0 &&
         (uint64_t)((M + 15) / 16) * 16 * (uint64_t)K * 2 < (1ull << 31) && (uint64_t)N * (uint64_t)K / 2 < (1ull << 31) &&
         (uint64_t)M * (uint64_t)N < (1ull << 40);
}

size_t forward_frag_bytes(int64_t M, int64_t K) { return (size_t)((M + 15) / 16) * 16 * (size_t)K * 2; }

int forward_tile_rows(int kernel) { return kernel == kForwardMid ? 256 : kernel == kForwardSmall ? 128 : kFwBM; }

hipError_t launch_forward(int kernel, int grid, const float* a, void* frags, const float* scales,
                          const uint32_t* codes, float* dst, int M, int N, int K, int k_chunk, int tiles_m,
                          int tiles_n, hipStream_t stream) {
  hipError_t e = launch_frag_pass(a, frags, M, K, /*natural=*/true, stream);
  if (e != hipSuccess) return e;
  return launch_forward_tiles(kernel, grid, frags, scales, codes, dst, M, N, K, k_chunk, tiles_m, tiles_n, stream);
}

hipError_t launch_forward_tiles(int kernel, int grid, const void* frags, const float* scales, const uint32_t* codes,
                                float* dst, int M, int N, int K, int k_chunk, int tiles_m, int tiles_n,
                                hipStream_t stream) {
  if (kernel == kForwardMid)
    hipLaunchKernelGGL(nf4_forward_mid_kernel, dim3(grid), dim3(256), 0, stream, frags, scales, codes, dst, M, N, K,
                       k_chunk, tiles_m, tiles_n);
  else if (kernel == kForwardSmall)
    hipLaunchKernelGGL(nf4_forward_small_kernel, dim3(grid), dim3(256), 0, stream, frags, scales, codes, dst, M, N,
                       K, k_chunk, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(nf4_forward_kernel, dim3(grid), dim3(512), 0, stream, frags, scales, codes, dst, M, N, K,
                       k_chunk, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace nf4
