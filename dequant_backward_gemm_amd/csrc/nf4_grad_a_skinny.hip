// Streaming kernel for grad_A = grad_out . dequant(W) with 1 <= M <= 16.
//
// Same arithmetic as the other grad_A kernels (grad_out rounded fp32 -> fp16,
// weights fp16(fl32(scale * level)), fp16 MFMA products accumulated in fp32
// over N).  At this size the work is streaming the packed weight once, so the
// kernel is organised for HBM bandwidth and decode throughput:
//
// * A workgroup (8 waves) owns a 128-column strip of grad_A over an N-chunk;
//   the waves take interleaved k-steps of 32 rows of N and are summed in a
//   fixed order at the end (LDS); the N-chunks' partials are summed, in chunk
//   order, by the last workgroup of the strip to finish.
// * Per k-step a wave builds the fp16 weight tables of its 32 rows x 2 scale
//   blocks in its own LDS area -- the 16 values fp16(fl32(scale * level)) a
//   code can stand for -- then decodes every weight with one 16-bit table
//   read straight into its MFMA B operands (no fragment round trip: every
//   decoded weight is used by this wave only).
// * MFMA 16x16x32 with grad_out rows padded to 16 (rows >= M read as zero).
//   B lane (c, q) holds rows n0 + 8q + e (e = 0..7) at column k0 + 8c + t of
//   tile t, so a lane's 8 columns are one code dword per row and the 8 tiles
//   give each lane 8 consecutive outputs per row.
// * grad_out is loaded with four lanes per 128-byte line (one row's 32
//   values of the k-step), rounded to fp16 and moved into the A layout (one
//   row per lane) through a 1 KiB per-wave LDS slot.
//
// N tails and chunk ends: rows n >= chunk end get scale 0 (so every table
// entry, hence every decoded weight, is +-0) and grad_out 0.  The scalar
// (row) part of a code load's offset is clamped to the last row, so it stays
// inside the array; the per-lane part beyond it reads zero through the
// buffer range check.  Columns past K only reach outputs that are not stored.
#include "nf4_kernel_util.h"
#include "nf4_launch.h"

namespace nf4 {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyBK = 128;
// Per-wave LDS in the loop: tables, then the grad_out staging slot.  The
// table of row 8q + e, block b sits at 256e + 64q + 32b: the 8 tables one
// lookup instruction reads (fixed e) are one contiguous 256-byte run, the
// layout measured closest to the LDS's per-instruction floor for random
// 16-bit reads.
constexpr int kSkTabBytes = 8 * 256;                  // 2048
constexpr int kSkWaveBytes = kSkTabBytes + 1024;      // + A staging
constexpr int kSkRedBytes = kSkinnyWaves * 16 * kSkinnyBK * 4;  // 64 KiB reduction buffer
static_assert(kSkinnyWaves * kSkWaveBytes <= kSkRedBytes, "loop LDS fits in the reduction buffer");

// One workgroup's strip and N-chunk: logical index `logical` of the
// problem's tiles_k x splits workgroups (strip fastest).
template <bool VEC_A>
__device__ __forceinline__ void stream_strip(const float* __restrict__ G, const float* __restrict__ S,
                                             const uint32_t* __restrict__ C32, float* out, float* __restrict__ grad_a,
                                             uint32_t* __restrict__ counters, int M, int N, int K, int n_chunk,
                                             int tiles_k, int splits, int logical) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[kSkRedBytes / 4];
  __shared__ uint32_t last_in_strip;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ci = lane & 15, q = lane >> 4;

  const int kt = logical % tiles_k;
  const int split = logical / tiles_k;
  const int k0 = kt * kSkinnyBK;
  const int nb = split * n_chunk;
  const int ne = min(N, nb + n_chunk);
  const int nsteps = (ne - nb + 31) >> 5;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(C32, (uint32_t)((size_t)N * (size_t)K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (uint32_t)((size_t)N * (size_t)(K / 64) * 4));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(G, (uint32_t)((size_t)M * (size_t)N * 4));
  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row

  const uint32_t wbase = (uint32_t)wave * kSkWaveBytes;
  // code dword of lane (ci, q): rows n0 + 8q + e, columns k0 + 8ci .. + 7
  const uint32_t cvoff = 8u * q * crow + (uint32_t)(k0 / 2 + 4 * ci);
  // table reads of lane (ci, q): row e at +256e, group q, block ci / 8, code c at +2c
  const uint32_t tlook = wbase + 64u * (uint32_t)q + 32u * (uint32_t)(ci >> 3);
  // table built by lane L: row 8q + e with e = L / 8, q = (L / 2) % 4, block L % 2, so that the 32-byte
  // tables eight consecutive lanes store sit at distinct offsets modulo 256 bytes (distinct banks)
  const int tkb = lane & 1, trow = 8 * ((lane >> 1) & 3) + (lane >> 3);
  const uint32_t tbuild = wbase + 256u * (trow & 7) + 64u * (trow >> 3) + 32u * tkb;
  const uint32_t svoff = (uint32_t)trow * srow + 4u * (uint32_t)(k0 / 64 + tkb);
  // grad_out as loaded by lane L: row L / 4, values 8 * (L % 4) .. + 7 of the k-step;
  // staged at the A-operand slot of lane 16 * (L % 4) + L / 4.  Slot s of the 1 KiB area sits at
  // 16 * (s ^ 4 * (s / 16 % 4)) bytes (a permutation inside each group of 16 slots), so that 16
  // consecutive lanes store to, and read from, 16 distinct 16-byte bank groups
  const int arow = lane >> 2, aq = lane & 3;
  // rows >= M read through an offset past the buffer's range: zero, no memory traffic
  const uint32_t avoff = (arow < M) ? (uint32_t)arow * (uint32_t)N * 4u + 32u * aq : 0x80000000u;
  auto aslot = [](uint32_t s) { return 16u * (s ^ (4u * ((s >> 4) & 3u))); };
  const uint32_t astore = wbase + kSkTabBytes + aslot((uint32_t)(16 * aq + arow));
  const uint32_t aread = wbase + kSkTabBytes + aslot((uint32_t)lane);

  floatx4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    uint32_t x[8];
    float sc;
    float a[8];
  };
  // (k-steps past the chunk are clamped to its last one: the loads stay
  // unconditional, so the wait counts never depend on a branch)
  auto load_step = [&](int j, Step& d) {
    const uint32_t n0 = (uint32_t)(nb + 32 * min(j, nsteps - 1));
#pragma unroll
    for (int e = 0; e < 8; ++e)
      d.x[e] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvoff, min(n0 + e, (uint32_t)N - 1u) * crow, 0);
    d.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, svoff, n0 * srow, 0));
    if constexpr (VEC_A) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const floatx4 g4 =
            __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rg, avoff + 16u * v, n0 * 4u, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) d.a[4 * v + i] = g4[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        d.a[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, avoff + 4u * i, n0 * 4u, 0));
    }
  };

  auto run_step = [&](int j, const Step& d) {
    const int n0 = nb + 32 * j;
    // Rows past the chunk can occur only in its last k-step: the row tests
    // below run there only (the branch is uniform over the wave; skipping
    // the selects in the other k-steps measured 0.2-0.9% faster).
    const bool full = n0 + 32 <= ne;
    // tables of this k-step (rows past the chunk get scale 0)
    {
      float sc = d.sc;
      if (!full) sc = (n0 + trow < ne) ? d.sc : 0.f;
      u32x4 w0, w1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        w0[c] = pack_half2_rne(sc * kLevels[2 * c], sc * kLevels[2 * c + 1]);
        w1[c] = pack_half2_rne(sc * kLevels[8 + 2 * c], sc * kLevels[8 + 2 * c + 1]);
      }
      lds_store_u32x4(smem, tbuild, w0);
      lds_store_u32x4(smem, tbuild + 16u, w1);
    }
    NF4_WAVE_DRAIN();  // race-check build: the wave's tables are complete before anything reads them
    // grad_out of the k-step into the A layout
    u32x4 af;
    {
      const int nl = n0 + 8 * aq;
      float g[8];
      if (full) {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = d.a[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = (nl + i < ne) ? d.a[i] : 0.f;
      }
      u32x4 h;
#pragma unroll
      for (int p = 0; p < 4; ++p) h[p] = pack_half2_rne(g[2 * p], g[2 * p + 1]);
      lds_store_u32x4(smem, astore, h);
      NF4_WAVE_DRAIN();
      af = lds_load_u32x4(smem, aread);
    }
    // decode (one table read per weight) and MFMA, tile by tile
    uint32_t y[8], z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = (d.x[e] << 1) & 0x1E1E1E1Eu;
      z[e] = (d.x[e] >> 3) & 0x1E1E1E1Eu;
    }
    // table reads of tile t + 1 are issued before tile t's are packed
    uint32_t lk[2][8];
    auto lookup = [&](auto tc, uint32_t (&l)[8]) {
      constexpr int t = decltype(tc)::value;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        l[e] = lds_load_u16(smem, add_byte<(t >> 1)>(tlook, (t & 1) ? z[e] : y[e]) + 256u * e);
    };
    lookup(std::integral_constant<int, 0>{}, lk[0]);
    for_each_index(std::make_integer_sequence<int, 8>{}, [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (t + 1 < 8) lookup(std::integral_constant<int, t + 1>{}, lk[(t + 1) & 1]);
      u32x4 b;
#pragma unroll
      for (int p = 0; p < 4; ++p) b[p] = lk[t & 1][2 * p] | (lk[t & 1][2 * p + 1] << 16);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(af), as_half8(b), acc[t], 0, 0, 0);
    });
    NF4_WAVE_DRAIN();  // race-check build: the step's table reads complete before the next step's builds
  };

  // Wave w takes k-steps w, w + 8, ... (cnt of them); the next one's loads are
  // in flight while one is decoded.  Two named buffers, a counted loop unrolled
  // twice whose body is one basic block: no loop-carried copy of a register a
  // load may still be writing (such a copy waits for the load), and no load
  // batch interleaved with another.
  const int cnt = (nsteps > wave) ? (nsteps - wave + kSkinnyWaves - 1) / kSkinnyWaves : 0;
  if (cnt > 0) {
    Step s0, s1;
    auto jj = [&](int i) { return wave + kSkinnyWaves * i; };
    load_step(jj(0), s0);
    int i = 0;
    for (; i + 2 <= cnt; i += 2) {
      load_step(jj(i + 1), s1);
      __builtin_amdgcn_sched_barrier(0);
      run_step(jj(i), s0);
      __builtin_amdgcn_sched_barrier(0);
      load_step(jj(i + 2), s0);
      __builtin_amdgcn_sched_barrier(0);
      run_step(jj(i + 1), s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < cnt) run_step(jj(i), s0);
  }

  // fixed-order sum of the 8 waves: ((w0 + w1) + w2) + ... + w7, rows < M only
  // (the padding rows' accumulators are zero and never stored)
  __syncthreads();
  {
    // accumulator lane (ci, q), register r: row 4q + r, columns 8ci + t
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * q + r < M) {
        const floatx4 lo = {acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        const floatx4 hi = {acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
        lds_store_u32x4(smem, (uint32_t)((wave * 16 + 4 * q + r) * kSkinnyBK + 8 * ci) * 4u,
                        __builtin_bit_cast(u32x4, lo));
        lds_store_u32x4(smem, (uint32_t)((wave * 16 + 4 * q + r) * kSkinnyBK + 8 * ci + 4) * 4u,
                        __builtin_bit_cast(u32x4, hi));
      }
    }
  }
  __syncthreads();
  {
    const int row = tid >> 5, c4 = tid & 31;  // 16 rows x 32 float4
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    if (row < M) {
      s = __builtin_bit_cast(floatx4, lds_load_u32x4(smem, (uint32_t)(row * kSkinnyBK + 4 * c4) * 4u));
#pragma unroll
      for (int w = 1; w < kSkinnyWaves; ++w)
        s += __builtin_bit_cast(floatx4,
                                lds_load_u32x4(smem, (uint32_t)((w * 16 + row) * kSkinnyBK + 4 * c4) * 4u));
    }
    const int col = k0 + 4 * c4;
    const bool mine = row < M && col < K;
    const uint32_t at = 4u * ((uint32_t)row * (uint32_t)K + (uint32_t)col);  // byte offset in one partial
    const uint32_t part = 4u * (uint32_t)M * (uint32_t)K;                    // bytes per partial
    if (splits == 1 || counters == nullptr) {
      if (mine) *reinterpret_cast<floatx4*>(reinterpret_cast<char*>(out) + (size_t)split * part + at) = s;
    } else {
      // Split reduction by the strip's last workgroup to finish.  The partials
      // are stored and loaded with device-scope coherence (sc1: they bypass
      // the XCDs' separate L2s), each wave waits for its stores to complete
      // before the workgroup's arrival is counted, and the workgroup that
      // sees the count reach `splits` sums the partials in split order,
      // ((p0 + p1) + p2) + ..., so the result does not depend on which
      // workgroup that is; it then resets the counter for the next call.
      // (A device-scope fence instead writes back and invalidates the whole
      // L2 per wave: measured 6x slower for the whole kernel.)
      constexpr int kDevice = 16;  // buffer cache policy: sc1
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(out, (uint32_t)splits * part);
      if (mine) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s), rp, at, (uint32_t)split * part,
                                                       kDevice);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));  // vmcnt(0): the stores are complete
      __syncthreads();
      if (tid == 0) last_in_strip = atomicAdd(&counters[kt], 1u) == (uint32_t)(splits - 1);
      __syncthreads();
      if (!last_in_strip) return;
      if (mine) {
        floatx4 t = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rp, at, 0, kDevice));
        for (int sp = 1; sp < splits; sp += 8) {
          floatx4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (sp + u < splits)
              v[u] = __builtin_bit_cast(floatx4,
                                        __builtin_amdgcn_raw_buffer_load_b128(rp, at, (uint32_t)(sp + u) * part, kDevice));
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (sp + u < splits) t += v[u];
        }
        *reinterpret_cast<floatx4*>(reinterpret_cast<char*>(grad_a) + at) = t;
      }
      if (tid == 0) __hip_atomic_store(&counters[kt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <bool VEC_A>
__global__ __launch_bounds__(512, 2) void grad_a_stream_kernel(const float* __restrict__ G,
                                                               const float* __restrict__ S,
                                                               const uint32_t* __restrict__ C32,
                                                               float* out, float* __restrict__ grad_a,
                                                               uint32_t* __restrict__ counters, int M, int N, int K,
                                                               int n_chunk, int tiles_k, int splits) {
  stream_strip<VEC_A>(G, S, C32, out, grad_a, counters, M, N, K, n_chunk, tiles_k, splits,
                      xcd_remap(blockIdx.x, gridDim.x));
}

// Several problems sharing M in one grid, each with the workgroups (and the
// N-chunks) its own launch would have, so each result is bitwise the one its
// own launch gives.  Problem p owns blocks [begin, begin + padded): its
// workgroup count rounded up to a multiple of 8, so that its blocks start on
// XCD 0 and the same XCD remap as a launch of its own applies inside it; the
// padding blocks exit at once.
__global__ __launch_bounds__(512, 2) void grad_a_stream_grouped_kernel(StreamGroup g) {
  int p = 0;
  while (p + 1 < g.count && (int)blockIdx.x >= g.p[p + 1].begin) ++p;
  const StreamProblem& w = g.p[p];
  const int local = (int)blockIdx.x - w.begin;
  const int logical = xcd_remap(local, w.padded);
  if (logical >= w.tiles_k * w.splits) return;
  stream_strip<true>(w.G, w.S, w.C32, w.part, w.grad_a, w.counters, g.M, w.N, w.K, w.n_chunk, w.tiles_k, w.splits,
                     logical);
}

bool stream_kernel_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N > 0 && (uint64_t)M * (uint64_t)N * 4 < (1ull << 31) &&
         (uint64_t)N * (uint64_t)K / 2 < (1ull << 31);
}

hipError_t launch_grad_a_stream_grouped(const StreamGroup& g, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(grad_a_stream_grouped_kernel, dim3(grid), dim3(512), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_grad_a_stream(int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                                float* dst, float* grad_a, uint32_t* counters, int M, int N, int K, int n_chunk,
                                int tiles_k, int splits, hipStream_t stream) {
  if (counters != nullptr && tiles_k > kWsCounters) return hipErrorInvalidValue;
  if ((N & 3) == 0)
    hipLaunchKernelGGL(grad_a_stream_kernel<true>, dim3(grid), dim3(512), 0, stream, grad_out, scales, codes, dst,
                       grad_a, counters, M, N, K, n_chunk, tiles_k, splits);
  else
    hipLaunchKernelGGL(grad_a_stream_kernel<false>, dim3(grid), dim3(512), 0, stream, grad_out, scales, codes, dst,
                       grad_a, counters, M, N, K, n_chunk, tiles_k, splits);
  return hipGetLastError();
}

}  // namespace nf4
