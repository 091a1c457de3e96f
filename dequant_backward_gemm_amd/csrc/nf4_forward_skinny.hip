// Streaming kernel for the forward product C = A . W^T with 1 <= M <= 16.
//
// Same arithmetic as nf4_forward's tile kernel (activations rounded fp32 ->
// fp16, weights fp16(fl32(scale * level)), fp16 MFMA products accumulated in
// fp32 over K).  At this size every weight is used by at most 16 rows, so the
// work is streaming the packed weight once, and the kernel is organised for
// the way HBM wants it read: long runs of each code row, in order.
//
// * Each wave owns 16T rows n of W (T MFMA tiles of 16 output columns; T = 2
//   measured best against 1 and 4: the activations loaded per step serve T
//   tiles) over a chunk of K and walks it in steps of 128 k (two scale
//   blocks).  Per step a lane loads 16 contiguous code bytes of its row per
//   tile, so one load instruction covers 64 bytes of each of 16 rows and
//   consecutive steps read consecutive bytes.  A workgroup is 8 such waves
//   over the same K chunk; each output is one wave's, so there is no
//   cross-wave sum.  K chunks (splits) go through fp32 partials, summed in
//   chunk order by the last workgroup of the strip to finish (or, without
//   arrival counters, by the reduce kernel).
// * The activations of a step (16 rows x 128 k) are the same for all 8
//   waves, so they are loaded once per workgroup -- one 16-byte load per
//   thread -- rounded to fp16 and written to LDS in the MFMA A layout (a
//   double buffer, one barrier per step); each wave then reads its four A
//   operands from there.  Loaded by every wave instead, at M = 16 they were
//   8 KiB per wave and step, four times the code bytes, and the kernel took
//   37 us against 25 at M = 1 on 18944 x 3584.
// * Decode: a lane's eight weights of one MFMA share a row and a scale block,
//   so the lane holds that one scale in a register and decodes each weight as
//   fp16(fl32(scale * level[code])), the level read from a 16-entry fp32
//   codebook in LDS (one 64-byte copy per wave).  Per-row tables of the 16
//   products would save the multiply, but the 16 columns one instruction
//   serves are 16 different rows, and 16 or 32 tables of 32 bytes collide in
//   the LDS banks (measured: ~7 conflict cycles per read on top of ~5); all
//   lanes reading the same 16 dwords never collide.
// * The reduction index inside a step is permuted so that the loads stay
//   whole: lane (c, q) holds k = 128s + 32q + 8u + j (j = 0..7) in MFMA u =
//   0..3 of step s, on both sides -- B lane (c, q): row c of the tile, code
//   dword u of its 16 bytes (block 2s + q/2, so one scale); A lane (i, q):
//   activation row i at the same k, 32 contiguous floats.  A rows past M read
//   zero.
// * K % 128 == 64 leaves a half step at the end: there lanes q = 2, 3 take
//   zero activations and a zero scale (every decoded weight +-0).
//
// Rows n >= N read zero codes and a zero scale through the buffers' range
// checks; columns n >= N are not stored.
#include "nf4_kernel_util.h"
#include "nf4_launch.h"

namespace nf4 {

constexpr int kFsWaves = 8;
constexpr int kFsTiles = 2;                       // MFMA tiles (16 columns each) per wave
constexpr int kFsCols = 16 * kFsTiles * kFsWaves;  // columns n of C per workgroup
constexpr int kFsTabBytes = 64;                   // per wave: the 16 fp32 levels
constexpr int kFsABytes = 4 * 64 * 16;             // one step's A operands: [u][lane] x 16 B

// One workgroup's strip and K-chunk: block `blk` of the problem's strips x
// splits workgroups (strip fastest).
template <int T>
__device__ __forceinline__ void forward_strip(const float* __restrict__ A, const float* __restrict__ S,
                                              const uint32_t* __restrict__ C32, float* out, float* __restrict__ c,
                                              uint32_t* __restrict__ counters, int M, int N, int K, int k_chunk,
                                              int strips, int splits, int blk) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[(kFsWaves * kFsTabBytes + 2 * kFsABytes) / 4];
  __shared__ uint32_t last_in_strip;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ci = lane & 15, q = lane >> 4;

  const int strip = blk % strips;
  const int split = blk / strips;
  const int n0 = strip * (16 * T * kFsWaves) + 16 * T * wave;  // this wave's rows n0 .. n0 + 16T - 1
  const int kbeg = split * k_chunk;
  const int kend = min(K, kbeg + k_chunk);
  const int nsteps = (kend - kbeg + 127) >> 7;

  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row
  // this wave's rows only: rows past N fall outside the ranges and read zero
  const int rows_here = max(0, min(16 * T, N - n0));
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(reinterpret_cast<const char*>(C32) + (size_t)min(n0, N) * crow, (uint32_t)rows_here * crow);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const char*>(S) + (size_t)min(n0, N) * srow, (uint32_t)rows_here * srow);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K * 4u);

  const uint32_t wbase = (uint32_t)wave * kFsTabBytes;
  if (lane < 16) lds_store_u32(smem, wbase + 4u * (uint32_t)lane, __builtin_bit_cast(uint32_t, kLevels[lane]));
  // code bytes of lane (ci, q): row ci, bytes k/2 for k = 128s + 32q .. + 31
  const uint32_t cvoff = (uint32_t)ci * crow + 16u * (uint32_t)q;
  // scale of lane (ci, q): row ci, block 2s + q / 2
  const uint32_t svoff = (uint32_t)ci * srow + 4u * (uint32_t)(q >> 1);
  // activations loaded by thread t: row t / 32, k = 128s + 4 (t % 32) .. + 3;
  // stored as A operand u of lane L = 16 (k / 32) + row at half 4 ((t % 32) & 1).
  // Operand u of lane L sits at slot L ^ (4u + L / 16) of the operand's 1 KiB
  // (a permutation inside each group of 16 lanes), so that the 32 threads of a
  // row store to 32 distinct 8-byte bank positions and 16 lanes read 16
  // distinct 16-byte slots
  const int arow = tid >> 5, af4 = tid & 31;
  const bool arow_ok = arow < M;
  const uint32_t avoff = ((uint32_t)arow * (uint32_t)K + 4u * (uint32_t)af4) * 4u;
  const uint32_t abase = kFsWaves * kFsTabBytes;
  const int au = (af4 >> 1) & 3, aq = af4 >> 3;
  const uint32_t astore =
      abase + (uint32_t)(au * 1024 + 16 * ((16 * aq + arow) ^ (4 * au + aq)) + 8 * (af4 & 1));
  uint32_t aread[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) aread[u] = abase + (uint32_t)(u * 1024 + 16 * (lane ^ (4 * u + q)));

  floatx4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    u32x4 x[T];
    float sc[T];
    floatx4 a;
  };
  // (steps past the chunk are clamped to its last one: the loads stay
  // unconditional, so the wait counts never depend on a branch)
  auto load_step = [&](int j, Step& d) {
    const int k0 = kbeg + 128 * min(j, nsteps - 1);
    const bool hi_ok = k0 + 64 < kend;  // the step's second block is inside the chunk
    const bool s_ok = q < 2 || hi_ok;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      d.x[t] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, cvoff + (uint32_t)(16 * t) * crow, (uint32_t)k0 / 2u, 0));
      const uint32_t soff = s_ok ? svoff + (uint32_t)(16 * t) * srow : 0x80000000u;
      d.sc[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff, (uint32_t)k0 / 16u, 0));
    }
    const uint32_t ao = (arow_ok && (af4 < 16 || hi_ok)) ? avoff : 0x80000000u;
    d.a = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(ra, ao, 4u * k0, 0));
  };

  // buffer b of the A double buffer: steps of parity b (a buffer is rewritten
  // two steps after it was read, with the previous step's barrier between)
  auto run_step = [&](const Step& d, uint32_t b) {
    {
      u32x2 h;
      h[0] = pack_half2_rne(d.a[0], d.a[1]);
      h[1] = pack_half2_rne(d.a[2], d.a[3]);
      lds_store_u32x2(smem, astore + b * kFsABytes, h);
    }
    __syncthreads();
    // decode and MFMA; the level reads of MFMA u + 1 are issued before MFMA u's
    // weights are formed
    // (u, t) pairs in the order u * T + t
    auto lookup = [&](auto ic, float (&l)[8]) {
      constexpr int u = decltype(ic)::value / T, t = decltype(ic)::value % T;
      const uint32_t x = d.x[t][u];
      const uint32_t y = (x << 2) & 0x3C3C3C3Cu;  // even k: low nibbles, times 4
      const uint32_t z = (x >> 2) & 0x3C3C3C3Cu;  // odd k: high nibbles, times 4
      l[0] = lds_load_f32(smem, add_byte<0>(wbase, y));
      l[1] = lds_load_f32(smem, add_byte<0>(wbase, z));
      l[2] = lds_load_f32(smem, add_byte<1>(wbase, y));
      l[3] = lds_load_f32(smem, add_byte<1>(wbase, z));
      l[4] = lds_load_f32(smem, add_byte<2>(wbase, y));
      l[5] = lds_load_f32(smem, add_byte<2>(wbase, z));
      l[6] = lds_load_f32(smem, add_byte<3>(wbase, y));
      l[7] = lds_load_f32(smem, add_byte<3>(wbase, z));
    };
    float lk[2][8];
    u32x4 af;
    lookup(std::integral_constant<int, 0>{}, lk[0]);
    for_each_index(std::make_integer_sequence<int, 4 * T>{}, [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int u = i / T, t = i % T;
      if constexpr (i + 1 < 4 * T) lookup(std::integral_constant<int, i + 1>{}, lk[(i + 1) & 1]);
      if constexpr (t == 0) af = lds_load_u32x4(smem, aread[u] + b * kFsABytes);
      u32x4 bf;
#pragma unroll
      for (int p = 0; p < 4; ++p) bf[p] = pack_half2_rne(d.sc[t] * lk[i & 1][2 * p], d.sc[t] * lk[i & 1][2 * p + 1]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(af), as_half8(bf), acc[t], 0, 0, 0);
    });
    NF4_PHASE_BARRIER();  // race-check build: the step's A reads complete before the next step's stores
  };

  // The next step's loads are in flight while one is decoded (two named
  // buffers, a counted loop unrolled twice, as in the backward streaming
  // kernel).
  if (nsteps > 0) {
    Step s0, s1;
    load_step(0, s0);
    int i = 0;
    for (; i + 2 <= nsteps; i += 2) {
      load_step(i + 1, s1);
      __builtin_amdgcn_sched_barrier(0);
      run_step(s0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_step(i + 2, s0);
      __builtin_amdgcn_sched_barrier(0);
      run_step(s1, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nsteps) run_step(s0, 0);
  }

  // accumulator lane (ci, q), register r of tile t: row 4q + r, column n0 + 16t + ci
  if (splits == 1 || counters == nullptr) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int col = n0 + 16 * t + ci;
      if (col < N) {
        float* dst = out + (size_t)split * (size_t)M * (size_t)N + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * q + r;
          const float v = acc[t][r];
          if (row < M) dst[(size_t)row * (size_t)N] = v;
        }
      }
    }
    return;
  }
  // Split sum by the strip's last workgroup to finish, as in the backward
  // streaming kernel: partials stored and loaded with device-scope coherence
  // (sc1, past the XCDs' separate L2s), each wave's stores complete before the
  // workgroup's arrival is counted, the chunks summed in order
  // ((p0 + p1) + p2) + ..., the counter reset for the next call.
  constexpr int kDevice = 16;  // buffer cache policy: sc1
  const uint32_t part = 4u * (uint32_t)M * (uint32_t)N;  // bytes per partial
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(out, (uint32_t)splits * part);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int col = n0 + 16 * t + ci;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      // (the element goes through a scalar first: __builtin_bit_cast of a
      // vector element reads element 0 whatever the index)
      const float v = acc[t][r];
      if (col < N && row < M)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rp,
                                              4u * ((uint32_t)row * (uint32_t)N + (uint32_t)col),
                                              (uint32_t)split * part, kDevice);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));  // vmcnt(0): the stores are complete
  __syncthreads();
  if (tid == 0) last_in_strip = atomicAdd(&counters[strip], 1u) == (uint32_t)(splits - 1);
  __syncthreads();
  if (!last_in_strip) return;
  // the strip's M x 256 outputs as float4 (N % 8 == 0: a strip's columns are whole float4s)
  const int c0 = strip * kFsCols;
  for (int e = tid; e < M * (kFsCols / 4); e += 64 * kFsWaves) {
    const int row = e / (kFsCols / 4), col = c0 + 4 * (e % (kFsCols / 4));
    if (col >= N) continue;
    const uint32_t at = 4u * ((uint32_t)row * (uint32_t)N + (uint32_t)col);
    floatx4 sum = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rp, at, 0, kDevice));
    for (int sp = 1; sp < splits; sp += 8) {
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < splits)
          v[u] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rp, at, (uint32_t)(sp + u) * part,
                                                                                   kDevice));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < splits) sum += v[u];
    }
    *reinterpret_cast<floatx4*>(reinterpret_cast<char*>(c) + at) = sum;
  }
  if (tid == 0) __hip_atomic_store(&counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int T>
__global__ __launch_bounds__(512, 2) void nf4_forward_stream_kernel(const float* __restrict__ A,
                                                                    const float* __restrict__ S,
                                                                    const uint32_t* __restrict__ C32,
                                                                    float* out, float* __restrict__ c,
                                                                    uint32_t* __restrict__ counters, int M, int N,
                                                                    int K, int k_chunk, int strips, int splits) {
  forward_strip<T>(A, S, C32, out, c, counters, M, N, K, k_chunk, strips, splits, (int)blockIdx.x);
}

// Several problems sharing M in one grid, each with the workgroups (and the
// K-chunks) its own launch would have, so each result is bitwise the one its
// own launch gives.  Problem p owns blocks [begin, begin + padded), padded =
// its workgroup count rounded up to a multiple of 8 (its blocks start on XCD
// 0, as in a launch of its own); the padding blocks exit at once.
__global__ __launch_bounds__(512, 2) void nf4_forward_stream_grouped_kernel(ForwardStreamGroup g) {
  int p = 0;
  while (p + 1 < g.count && (int)blockIdx.x >= g.p[p + 1].begin) ++p;
  const ForwardStreamProblem& w = g.p[p];
  const int blk = (int)blockIdx.x - w.begin;
  if (blk >= w.strips * w.splits) return;
  forward_strip<kFsTiles>(w.A, w.S, w.C32, w.part, w.c, w.counters, g.M, w.N, w.K, w.k_chunk, w.strips, w.splits,
                          blk);
}

hipError_t launch_forward_stream_grouped(const ForwardStreamGroup& g, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(nf4_forward_stream_grouped_kernel, dim3(grid), dim3(512), 0, stream, g);
  return hipGetLastError();
}


bool forward_stream_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N > 0 && (N % 8) == 0 && K > 0 && (K % 64) == 0 &&
         (uint64_t)M * (uint64_t)K * 4 < (1ull << 31) && (uint64_t)N * (uint64_t)K / 2 < (1ull << 31);
}

int forward_stream_strips(int64_t N) { return (int)((N + kFsCols - 1) / kFsCols); }

hipError_t launch_forward_stream(int grid, const float* a, const float* scales, const uint32_t* codes, float* dst,
                                 float* c, uint32_t* counters, int M, int N, int K, int k_chunk, int strips,
                                 int splits, hipStream_t stream) {
  if (counters != nullptr && strips > kWsCounters) return hipErrorInvalidValue;
  hipLaunchKernelGGL(nf4_forward_stream_kernel<kFsTiles>, dim3(grid), dim3(512), 0, stream, a, scales, codes, dst, c,
                     counters, M, N, K, k_chunk, strips, splits);
  return hipGetLastError();
}

}  // namespace nf4
