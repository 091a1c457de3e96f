// nf4_grad_a: grad_A[M x K] = grad_out[M x N] . dequant(B_nf4[K x N])^T on gfx950.
//
// What is computed follows the subject page (aprender-gpu 0.32.0,
// src/kernels/backward/nf4_tensor_core.rs): grad_out is converted fp32 ->
// fp16 (Phase 1), each weight is decoded as fl32(scale * level) and converted
// to fp16 (Phase 2), the fp16 products are accumulated in fp32 over the
// shared dimension N (Phase 3) and grad_A is stored in fp32, overwriting
// (Phase 4).  How it is computed is this file's own design for CDNA4:
//
// * The reduction index n is the SLOW index of the stored weight W[N][K], but
//   an MFMA operand lane needs 8 consecutive reduction values at one output
//   column.  A decoding lane therefore loads one dword of codes (8 k) from
//   each of 8 consecutive rows and decodes that 8 x 8 block in registers; the
//   packed fp16 convert pairs rows (e, e+1), so every dword it produces is
//   already an MFMA B-operand pair -- no transpose pass.  The 8 columns of the
//   block go to 8 different MFMA tiles: column j of tile t is
//   k = k0 + 8*j + t, so one wave spans 256 consecutive k and each lane ends
//   up owning 8 consecutive outputs per row (two 128-bit stores).
// * Large M (tile kernel): a workgroup of 4 waves owns a BM x 256 output tile
//   (BM = 128 or 256).  Per 64-row stage of N each wave decodes one 16-row
//   MFMA k-step for the whole workgroup into LDS, already in B-fragment order
//   (lane-linear 16-byte slots: conflict-free ds_write_b128/ds_read_b128);
//   grad_out goes straight from global memory into A fragments because the
//   waves split M.  Stages are double-buffered: the global loads for stage
//   i+1 are issued before the MFMAs of stage i, and decoded after them.
// * Small M (skinny kernel, M <= 16): 16x16x32 MFMA with grad_out rows padded
//   to 16; each wave decodes straight into its own B operands (no LDS
//   round trip), 4 waves split N and are summed in a fixed order.
// * Enough workgroups for 256 CUs come from splitting N into chunks; each
//   chunk writes an fp32 partial and a separate kernel sums the partials in
//   chunk order.  No atomics anywhere: results are bitwise reproducible.
// * Workgroup ids are remapped so that one XCD (one L2) runs consecutive
//   tiles of the same grad_out row strip.
//
// The reduction order within a tile (which n pairs with which MFMA slot) is
// a fixed permutation shared by the A and B operands, so the products pair up
// exactly; fp32 accumulation is blocked (MFMA chunks of 16 or 32 products,
// then one fp32 add per chunk), which keeps the rounding error far below the
// 2e-3 * sum|g*w| acceptance bound at the largest N used.
#include <algorithm>

#include "nf4_kernel_util.h"
#include "nf4_launch.h"

namespace nf4 {

// ---------------------------------------------------------------------------
// Tile kernel (M > 16)
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256, (RB == 1 ? 2 : 1)) void grad_a_tile_kernel(
    const float* __restrict__ G, const float* __restrict__ S, const uint32_t* __restrict__ C32,
    float* __restrict__ out, int M, int N, int K, int n_chunk, int tiles_m, int tiles_k) {
  constexpr int BM = 128 * RB;
  __shared__ float lut[16];
  __shared__ u32x4 bfrag[2][4][8][64];  // [buffer][k-step][tile column t][lane], 64 KiB

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, h = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % tiles_k;
  const int rest = logical / tiles_k;
  const int mt = rest % tiles_m;
  const int split = rest / tiles_m;
  const int m0 = mt * BM, k0 = kt * 256;
  const int nb = split * n_chunk;
  const int ne = min(N, nb + n_chunk);
  const int nst = (ne - nb + 63) >> 6;

  if (tid < 16) lut[tid] = kLevels[tid];

  float* __restrict__ dst = out + (size_t)split * (size_t)M * (size_t)K;
  const int kk = k0 + 8 * j;  // decode / store column base of this lane
  const bool kval = kk < K;
  const size_t words_per_row = (size_t)(K >> 3);
  const size_t blocks_per_row = (size_t)(K >> 6);
  const bool vec_a = (N & 3) == 0;

  uint32_t x[8];
  float sc[8];
  float a[RB][32];
  u32x4 af[RB][4];
  floatx16 acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][t][r] = 0.f;

  // Rows of the k-step this wave decodes: n0 + 32*h + 8*wave + e.
  auto load_b = [&](int n0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = n0 + 32 * h + 8 * wave + e;
      const bool v = kval && n < ne;
      x[e] = v ? C32[(size_t)n * words_per_row + (kk >> 3)] : 0u;
      sc[e] = v ? S[(size_t)n * blocks_per_row + (kk >> 6)] : 0.f;
    }
  };
  // A lane (i = j, h) holds grad_out[row][n0 + 32*h + 8*s + e] for k-step s.
  auto load_a = [&](int n0) {
    const int nbase = n0 + 32 * h;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = m0 + wave * 32 * RB + 32 * rb + j;
      const float* src = G + (size_t)row * (size_t)N + nbase;
      if (row < M && vec_a && nbase + 32 <= ne) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const floatx4 q = reinterpret_cast<const floatx4*>(src)[v];
          a[rb][4 * v + 0] = q[0];
          a[rb][4 * v + 1] = q[1];
          a[rb][4 * v + 2] = q[2];
          a[rb][4 * v + 3] = q[3];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) a[rb][e] = (row < M && nbase + e < ne) ? src[e] : 0.f;
      }
    }
  };
  auto convert_a = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int p = 0; p < 4; ++p) af[rb][s][p] = pack_half2_rne(a[rb][8 * s + 2 * p], a[rb][8 * s + 2 * p + 1]);
  };
  auto decode_store = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = sc[e] * lut[(x[e] >> (4 * t)) & 15u];
      u32x4 v;
      v[0] = pack_half2_rne(f[0], f[1]);
      v[1] = pack_half2_rne(f[2], f[3]);
      v[2] = pack_half2_rne(f[4], f[5]);
      v[3] = pack_half2_rne(f[6], f[7]);
      bfrag[buf][wave][t][lane] = v;
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const half8 b = as_half8(bfrag[buf][s][t][lane]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(af[rb][s]), b, acc[rb][t], 0, 0, 0);
      }
    }
  };

  load_b(nb);
  load_a(nb);
  __syncthreads();  // lut visible
  decode_store(0);
  convert_a();
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) {
      load_b(nb + 64 * (st + 1));
      load_a(nb + 64 * (st + 1));
    }
    compute(buf);
    NF4_PHASE_BARRIER();  // race-check build: the stage's fragment reads complete before the next decode
    if (more) {
      decode_store(buf ^ 1);
      convert_a();
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane (j, h), register r -> row 8*(r/4) + 4*h + r%4, column j.
  if (kval) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wave * 32 * RB + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < M) {
          floatx4 lo = {acc[rb][0][r], acc[rb][1][r], acc[rb][2][r], acc[rb][3][r]};
          floatx4 hi = {acc[rb][4][r], acc[rb][5][r], acc[rb][6][r], acc[rb][7][r]};
          floatx4* o = reinterpret_cast<floatx4*>(dst + (size_t)row * (size_t)K + kk);
          o[0] = lo;
          o[1] = hi;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny kernel (1 <= M <= 16)
// ---------------------------------------------------------------------------
// 16x16x32 MFMA: A lane (i = lane%16, q = lane/16) holds A[i][8q..8q+7],
// B lane (c = lane%16, q) holds B[8q..8q+7][c], accumulator lane (c, q)
// register r holds C[4q + r][c].  A lane here loads two dwords of codes
// (16 k) from each of 8 rows, so column c of tile t (t = 0..15) is
// k = k0 + 16*c + t and a wave spans 256 k.
__global__ __launch_bounds__(256) void grad_a_skinny_kernel(const float* __restrict__ G, const float* __restrict__ S,
                                                            const uint32_t* __restrict__ C32, float* __restrict__ out,
                                                            int M, int N, int K, int n_chunk, int tiles_k) {
  __shared__ float lut[16];
  __shared__ floatx4 red[16][64];  // one wave's accumulators, 16 KiB

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, q = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % tiles_k;
  const int split = logical / tiles_k;
  const int k0 = kt * 256;
  const int nb = split * n_chunk;
  const int ne = min(N, nb + n_chunk);

  if (tid < 16) lut[tid] = kLevels[tid];
  __syncthreads();

  float* __restrict__ dst = out + (size_t)split * (size_t)M * (size_t)K;
  const int kk = k0 + 16 * c;
  const bool kval = kk < K;
  const size_t words_per_row = (size_t)(K >> 3);
  const size_t blocks_per_row = (size_t)(K >> 6);
  const bool arow = c < M;  // A lane row i = c
  const bool vec_a = (N & 3) == 0;

  floatx4 acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x2 x[8];
  float sc[8];
  float a[8];

  auto load = [&](int n0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = n0 + 8 * q + e;
      const bool v = kval && n < ne;
      const u32x2* p = reinterpret_cast<const u32x2*>(C32 + (size_t)n * words_per_row + (kk >> 3));
      x[e] = v ? *p : u32x2{0u, 0u};
      sc[e] = v ? S[(size_t)n * blocks_per_row + (kk >> 6)] : 0.f;
    }
    const int nbase = n0 + 8 * q;
    const float* src = G + (size_t)c * (size_t)N + nbase;
    if (arow && vec_a && nbase + 8 <= ne) {
      const floatx4 q0 = reinterpret_cast<const floatx4*>(src)[0];
      const floatx4 q1 = reinterpret_cast<const floatx4*>(src)[1];
      a[0] = q0[0]; a[1] = q0[1]; a[2] = q0[2]; a[3] = q0[3];
      a[4] = q1[0]; a[5] = q1[1]; a[6] = q1[2]; a[7] = q1[3];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (arow && nbase + e < ne) ? src[e] : 0.f;
    }
  };
  auto compute = [&]() {
    u32x4 av;
    av[0] = pack_half2_rne(a[0], a[1]);
    av[1] = pack_half2_rne(a[2], a[3]);
    av[2] = pack_half2_rne(a[4], a[5]);
    av[3] = pack_half2_rne(a[6], a[7]);
    const half8 ah = as_half8(av);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = (t < 8) ? x[e][0] : x[e][1];
        f[e] = sc[e] * lut[(word >> (4 * (t & 7))) & 15u];
      }
      u32x4 v;
      v[0] = pack_half2_rne(f[0], f[1]);
      v[1] = pack_half2_rne(f[2], f[3]);
      v[2] = pack_half2_rne(f[4], f[5]);
      v[3] = pack_half2_rne(f[6], f[7]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_half8(v), acc[t], 0, 0, 0);
    }
  };

  // Wave w takes the 32-row k-steps w, w+4, w+8, ... of this chunk.
  int n0 = nb + 32 * wave;
  if (n0 < ne) {
    load(n0);
    for (;;) {
      const int nn = n0 + 128;
      // keep this step's operands while the next step's loads are in flight
      u32x2 xc[8];
      float scc[8], ac[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { xc[e] = x[e]; scc[e] = sc[e]; ac[e] = a[e]; }
      if (nn < ne) load(nn);
      u32x2 xn[8];
      float scn[8], an[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { xn[e] = x[e]; scn[e] = sc[e]; an[e] = a[e]; x[e] = xc[e]; sc[e] = scc[e]; a[e] = ac[e]; }
      compute();
#pragma unroll
      for (int e = 0; e < 8; ++e) { x[e] = xn[e]; sc[e] = scn[e]; a[e] = an[e]; }
      if (nn >= ne) break;
      n0 = nn;
    }
  }

  // Fixed-order sum over the 4 waves: ((w0 + w1) + w2) + w3.
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    __syncthreads();
    if (wave == w) {
#pragma unroll
      for (int t = 0; t < 16; ++t) red[t][lane] = acc[t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[t] += red[t][lane];
    }
  }

  if (wave == 0 && kval) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      if (row < M) {
        floatx4* o = reinterpret_cast<floatx4*>(dst + (size_t)row * (size_t)K + kk);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          o[v] = floatx4{acc[4 * v + 0][r], acc[4 * v + 1][r], acc[4 * v + 2][r], acc[4 * v + 3][r]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split reduction and zero fill
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void grad_a_reduce_kernel(const floatx4* __restrict__ ws, floatx4* __restrict__ out,
                                                            int64_t n4, int splits) {
  // out = ((ws_0 + ws_1) + ws_2) + ...; the partials are loaded eight at a
  // time ahead of the adds, so a thread waits for one batch, not one load per
  // split (the sum order is the same)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    floatx4 s = ws[i];
    for (int p = 1; p < splits; p += 8) {
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p + u < splits) v[u] = ws[(int64_t)(p + u) * n4 + i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p + u < splits) s += v[u];
    }
    out[i] = s;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(floatx4* __restrict__ out, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    out[i] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// Launchers (called by the planner in nf4_plan.hip)
// ---------------------------------------------------------------------------
hipError_t launch_grad_a_tile(int rb, int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                              float* dst, int M, int N, int K, int n_chunk, int tiles_m, int tiles_k,
                              hipStream_t stream) {
  auto kern = rb == 2 ? grad_a_tile_kernel<2> : grad_a_tile_kernel<1>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, grad_out, scales, codes, dst, M, N, K, n_chunk, tiles_m,
                     tiles_k);
  return hipGetLastError();
}

hipError_t launch_grad_a_skinny(int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                                float* dst, int M, int N, int K, int n_chunk, int tiles_k, hipStream_t stream) {
  hipLaunchKernelGGL(grad_a_skinny_kernel, dim3(grid), dim3(256), 0, stream, grad_out, scales, codes, dst, M, N, K,
                     n_chunk, tiles_k);
  return hipGetLastError();
}

hipError_t launch_grad_a_reduce(int grid, const float* ws, float* out, int64_t n4, int splits, hipStream_t stream) {
  hipLaunchKernelGGL(grad_a_reduce_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const floatx4*>(ws),
                     reinterpret_cast<floatx4*>(out), n4, splits);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int grid, float* out, int64_t n4, hipStream_t stream) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<floatx4*>(out), n4);
  return hipGetLastError();
}

}  // namespace nf4
