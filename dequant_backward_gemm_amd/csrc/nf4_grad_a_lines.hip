// Line-streaming kernel for grad_A = grad_out . dequant(W) with 1 <= M <= 16.
//
// Same arithmetic as the other grad_A kernels (grad_out rounded fp32 -> fp16,
// weights fp16(fl32(scale * level)), fp16 MFMA products accumulated in fp32
// over N).  At this size every weight is used once, so the kernel is built
// around two budgets: reading the packed codes in whole 128-byte lines, and
// decoding them fast enough to keep up.
//
// * A workgroup (8 waves) owns a 256-column strip of grad_A -- 128 code bytes,
//   one whole line, of every row -- over an N-chunk.  The waves take
//   interleaved k-steps of 16 rows and are summed in a fixed order at the end
//   (LDS); the N-chunks' partials are summed by the last workgroup of the
//   strip to finish.
// * Operand layout: a B register of the 16x16x32 MFMA holds the two weights of
//   ONE code byte (columns 2c and 2c+1 of one row), so each register decodes
//   from one row's scale.  Reduction index 8g + 2p + h (lane group g, register
//   p, half h) is row n0 + 4g + p, column parity h.  Two MFMAs per B operand
//   separate the parities: the "even" A operand holds fp16(grad_out) in the
//   low halves and zeros in the high halves, the "odd" one the reverse, so
//   their products land in the even and the odd output column of each byte.
//   (At M <= 16 the MFMA pipe has the slack: decode bounds the loop.)
// * Lane (j, g) of a wave loads 8 code bytes of each of its 4 rows
//   n0 + 4g + p: bytes 8j .. 8j+7 of the strip, i.e. columns 16j .. 16j+15;
//   byte t goes to MFMA tile t.  One load instruction covers 4 rows x 128
//   bytes: four whole lines.  Each lane ends up owning 16 consecutive
//   outputs per grad_A row.
// * Decode, two ways (rows p < 4 - CB the first, the others the second):
//     - table: per k-step the wave builds the tables of its 16 rows x 4 scale
//       blocks (one per lane: the 16 values fp16(fl32(scale * level)) a code
//       can stand for) in its own LDS area; each weight is one 16-bit table
//       read.  The 64 reads of an instruction hit 16 tables at random codes,
//       so they conflict in the LDS banks (measured ~4.4 cycles per
//       instruction, half of them conflict cycles);
//     - codebook: each weight's level is read from the one 16-entry fp32
//       codebook all lanes share (16 dwords in 16 banks: no conflicts), then
//       multiplied by the row's scale and converted, fp16(fl32(scale *
//       level)) -- two VALU instructions more per weight, no table to build.
//   The two give the same fp16 values, so any mix gives the same result.
// * Loads run kLnDepth k-steps ahead and tables one k-step ahead, in rings of
//   kLnDepth + 1 buffers; the loop is unrolled one ring turn so every buffer
//   index is a compile-time constant.
//
// Bounds: rows n >= chunk end get scale 0 (every decoded weight +-0) and
// grad_out 0.  The scalar (row) part of a load's offset is clamped to the last
// row, so it stays inside the array; the per-lane part beyond it reads zero
// through the buffer range check.  Code bytes and scale blocks past K (last
// strip) read neighbouring data or zero and only reach outputs that are never
// stored.
#include "nf4_kernel_util.h"
#include "nf4_launch.h"

namespace nf4 {

constexpr int kLnWaves = 8;
constexpr int kLnRows = 16;                               // rows of N per k-step of a wave
constexpr int kLnTabStep = 2048;                          // table bytes per k-step per wave
constexpr int kLnDepth = 3;                               // k-steps of loads in flight ahead of the decode
constexpr int kLnRing = kLnDepth + 1;                     // load buffers = table buffers
constexpr int kLnWaveTab = kLnRing * kLnTabStep;
constexpr int kLnCodebook = kLnWaves * kLnWaveTab;        // the shared fp32 codebook (64 bytes)
constexpr int kLnRedBytes = kLnWaves * 16 * kLinesBK * 4; // 128 KiB cross-wave reduction buffer
static_assert(kLnCodebook + 64 <= kLnRedBytes, "tables and codebook fit in the reduction buffer");

// The 4 B registers of one row (fp16 pairs: the weights of code bytes 0..3 of
// x, low nibble in the low half) from the row's table held as byte planes:
// pl = low bytes of entries 0..15 (4 dwords), ph = high bytes.  v_perm_b32
// looks up 4 nibbles at once in each 8-entry half of a plane; a byte mask
// from bit 3 of each nibble merges the halves; two rounds of v_perm_b32
// interleave low and high bytes into fp16 pairs: 27 VALU per 8 weights.
__device__ __forceinline__ void decode_planes(uint32_t x, const u32x4& pl, const u32x4& ph, uint32_t m55,
                                              uint32_t (&b)[4]) {
  const uint32_t xo = x >> 4;
  const uint32_t se = x & 0x07070707u;   // low 3 bits of the low nibbles
  const uint32_t so = xo & 0x07070707u;  // low 3 bits of the high nibbles
  // 0xFF in the bytes whose nibble is 8..15 (v_perm: selector 0x0D -> 0xFF, 0x05 -> byte 5 of {0, 0} = 0)
  const uint32_t me = __builtin_amdgcn_perm(0u, 0u, (x & 0x08080808u) | m55);
  const uint32_t mo = __builtin_amdgcn_perm(0u, 0u, (xo & 0x08080808u) | m55);
  auto look = [](uint32_t sel, uint32_t m, const u32x4& p) {
    const uint32_t lo = __builtin_amdgcn_perm(p[1], p[0], sel);  // entries 0..7
    const uint32_t hi = __builtin_amdgcn_perm(p[3], p[2], sel);  // entries 8..15
    return (m & hi) | (~m & lo);
  };
  const uint32_t le = look(se, me, pl), he = look(se, me, ph);
  const uint32_t lo = look(so, mo, pl), ho = look(so, mo, ph);
  const uint32_t p01 = __builtin_amdgcn_perm(he, le, 0x05010400u);
  const uint32_t p23 = __builtin_amdgcn_perm(he, le, 0x07030602u);
  const uint32_t q01 = __builtin_amdgcn_perm(ho, lo, 0x05010400u);
  const uint32_t q23 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);
  b[0] = __builtin_amdgcn_perm(q01, p01, 0x05040100u);
  b[1] = __builtin_amdgcn_perm(q01, p01, 0x07060302u);
  b[2] = __builtin_amdgcn_perm(q23, p23, 0x05040100u);
  b[3] = __builtin_amdgcn_perm(q23, p23, 0x07060302u);
}

// One workgroup's strip and N-chunk: logical index `logical` of the
// problem's tiles_k x splits workgroups (strip fastest).  VR: rows (of each
// lane's 4) decoded in registers from byte planes (the others: 16-bit table
// reads), CB: rows decoded through the shared codebook; VR + CB <= 4.
template <int VR, int CB>
__device__ __forceinline__ void lines_strip(const float* __restrict__ G, const float* __restrict__ S,
                                            const uint32_t* __restrict__ C32, float* out, float* __restrict__ grad_a,
                                            uint32_t* __restrict__ counters, int M, int N, int K, int n_chunk,
                                            int tiles_k, int splits, int logical) {
  static_assert(VR >= 0 && CB >= 0 && VR + CB <= 4, "at most 4 rows per lane");
  constexpr int TR = 4 - CB;  // rows decoded from per-k-step tables (16-bit reads or byte planes)
  constexpr int LR = TR - VR; // of which by 16-bit table reads
  __shared__ __attribute__((aligned(16))) uint32_t smem[kLnRedBytes / 4];
  __shared__ uint32_t last_in_strip;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;

  const int kt = logical % tiles_k;
  const int split = logical / tiles_k;
  const int k0 = kt * kLinesBK;
  const int nb = split * n_chunk;
  const int ne = min(N, nb + n_chunk);
  const int nsteps = (ne - nb + kLnRows - 1) / kLnRows;

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(C32, (uint32_t)((size_t)N * (size_t)K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (uint32_t)((size_t)N * (size_t)(K / 64) * 4));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(G, (uint32_t)((size_t)M * (size_t)N * 4));
  const uint32_t crow = (uint32_t)K / 2;   // bytes per code row
  const uint32_t srow = (uint32_t)K / 16;  // bytes per scale row

  if constexpr (CB > 0) {
    if (tid < 16) lds_store_u32(smem, kLnCodebook + 4u * (uint32_t)tid, __builtin_bit_cast(uint32_t, kLevels[tid]));
    __syncthreads();
  }

  const uint32_t wtab = (uint32_t)wave * kLnWaveTab;
  // codes of lane (j, g): rows n0 + 4g + p, bytes 8j .. 8j+7 of the strip
  const uint32_t cvoff = 4u * (uint32_t)g * crow + (uint32_t)(k0 / 2 + 8 * j);
  // table (row 4g + p, block b) of a k-step: 32 bytes at 512 p + 32 (4g + b)
  const uint32_t tidx = 4u * (uint32_t)g + (uint32_t)(j >> 2);
  // table built by lane L: row rr = L / 4 (= 4 gq + pq), block L % 4
  const int rr = lane >> 2, tblk = lane & 3;
  const int pq = rr & 3;
  const uint32_t bidx = 4u * (uint32_t)(rr >> 2) + (uint32_t)tblk;
  // fp16 layout: 32 bytes per table; plane layout: low planes at 16 idx, high planes at 256 + 16 idx
  const uint32_t tb_own = 512u * (uint32_t)pq + 32u * bidx;
  const uint32_t tb_lo = 512u * (uint32_t)pq + 16u * bidx;
  const uint32_t m55 = __builtin_amdgcn_readfirstlane(0x05050505u);
  const uint32_t svoff = (uint32_t)rr * srow + 4u * (uint32_t)(k0 / 64 + tblk);
  // the scale of a codebook-decoded row 4g + p, block j / 4
  const uint32_t cvs = 4u * (uint32_t)g * srow + 4u * (uint32_t)(k0 / 64 + (j >> 2));
  // grad_out of lane (i, g): row i, reduction rows n0 + 4g .. + 3; rows >= M
  // read through an offset past the buffer's range (zero, no traffic)
  const int arow = lane & 15;
  const uint32_t avoff = (arow < M) ? (uint32_t)arow * (uint32_t)N * 4u + 16u * (uint32_t)g : 0x80000000u;

  floatx4 acc[8][2];  // [tile][parity]
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t][0] = acc[t][1] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    float sc;           // the scale of the table this lane builds
    float cs[CB > 0 ? CB : 1];  // the scales of its codebook-decoded rows
    u32x2 x[4];         // codes of rows p = 0..3
    float a[4];         // grad_out, reduction rows n0 + 4g + p
  };
  const int cnt = (nsteps > wave) ? (nsteps - wave + kLnWaves - 1) / kLnWaves : 0;
  auto n0_of = [&](int i) { return nb + kLnRows * (wave + kLnWaves * i); };
  // (steps past the wave's last are clamped to it: the loads stay
  // unconditional; the scales first: loads complete in issue order, and the
  // table build that needs them comes a step before the decode)
  auto load_step = [&](int i, Step& d) {
    const uint32_t n0 = (uint32_t)n0_of(min(i, cnt - 1));
    if constexpr (TR > 0) d.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, svoff, n0 * srow, 0));
#pragma unroll
    for (int c = 0; c < CB; ++c)
      d.cs[c] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, cvs, min(n0 + (uint32_t)(TR + c), (uint32_t)N - 1u) * srow, 0));
#pragma unroll
    for (int p = 0; p < 4; ++p)
      d.x[p] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, cvoff, min(n0 + (uint32_t)p, (uint32_t)N - 1u) * crow, 0));
    const floatx4 v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rg, avoff, n0 * 4u, 0));
#pragma unroll
    for (int p = 0; p < 4; ++p) d.a[p] = v[p];
  };
  // tables of step i's table-decoded rows (its scale in d) into table buffer tb
  auto build_tables = [&](int i, const Step& d, uint32_t tb) {
    if constexpr (TR > 0) {
      const float sc = (n0_of(i) + rr < ne) ? d.sc : 0.f;
      uint32_t w[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) w[c] = pack_half2_rne(sc * kLevels[2 * c], sc * kLevels[2 * c + 1]);
      if (pq < LR) {
        lds_store_u32x4(smem, wtab + tb + tb_own, u32x4{w[0], w[1], w[2], w[3]});
        lds_store_u32x4(smem, wtab + tb + tb_own + 16u, u32x4{w[4], w[5], w[6], w[7]});
      } else if (pq < TR) {
        u32x4 lo, hi;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          lo[c] = __builtin_amdgcn_perm(w[2 * c + 1], w[2 * c], 0x06040200u);
          hi[c] = __builtin_amdgcn_perm(w[2 * c + 1], w[2 * c], 0x07050301u);
        }
        lds_store_u32x4(smem, wtab + tb + tb_lo, lo);
        lds_store_u32x4(smem, wtab + tb + tb_lo + 256u, hi);
      }
    }
  };
  // decode and MFMAs of step i from its loads and table buffer tb
  auto run_step = [&](int i, const Step& d, uint32_t tb) {
    const int nl = n0_of(i) + 4 * g;
    uint32_t bq[8][4];  // [tile][register p]
    // byte planes of the register-decoded rows (LDS reads issued first: they
    // do not wait for the codes)
    u32x4 pl[4], ph[4];
#pragma unroll
    for (int p = LR; p < TR; ++p) {
      const uint32_t base = wtab + tb + 512u * (uint32_t)p + 16u * tidx;
      pl[p] = lds_load_u32x4(smem, base);
      ph[p] = lds_load_u32x4(smem, base + 256u);
    }
    // 16-bit table rows: one table read per weight
    uint32_t lk[LR > 0 ? LR : 1][2][8];
#pragma unroll
    for (int p = 0; p < LR; ++p) {
      const uint32_t base = wtab + tb + 512u * (uint32_t)p + 32u * tidx;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = d.x[p][h];
        const uint32_t y = (x << 1) & 0x1E1E1E1Eu;  // low nibbles, times 2
        const uint32_t z = (x >> 3) & 0x1E1E1E1Eu;  // high nibbles, times 2
        lk[p][h][0] = lds_load_u16(smem, add_byte<0>(base, y));
        lk[p][h][1] = lds_load_u16(smem, add_byte<0>(base, z));
        lk[p][h][2] = lds_load_u16(smem, add_byte<1>(base, y));
        lk[p][h][3] = lds_load_u16(smem, add_byte<1>(base, z));
        lk[p][h][4] = lds_load_u16(smem, add_byte<2>(base, y));
        lk[p][h][5] = lds_load_u16(smem, add_byte<2>(base, z));
        lk[p][h][6] = lds_load_u16(smem, add_byte<3>(base, y));
        lk[p][h][7] = lds_load_u16(smem, add_byte<3>(base, z));
      }
    }
    // codebook rows: level read, fp32 multiply by the row's scale, fp16 convert
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      constexpr int p0 = TR;
      const int p = p0 + c;
      const float sc = (nl + p < ne) ? d.cs[c] : 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = d.x[p][h];
        const uint32_t y = (x << 2) & 0x3C3C3C3Cu;  // low nibbles, times 4
        const uint32_t z = (x >> 2) & 0x3C3C3C3Cu;  // high nibbles, times 4
        float q[8];
        q[0] = lds_load_f32(smem, add_byte<0>(kLnCodebook, y));
        q[1] = lds_load_f32(smem, add_byte<0>(kLnCodebook, z));
        q[2] = lds_load_f32(smem, add_byte<1>(kLnCodebook, y));
        q[3] = lds_load_f32(smem, add_byte<1>(kLnCodebook, z));
        q[4] = lds_load_f32(smem, add_byte<2>(kLnCodebook, y));
        q[5] = lds_load_f32(smem, add_byte<2>(kLnCodebook, z));
        q[6] = lds_load_f32(smem, add_byte<3>(kLnCodebook, y));
        q[7] = lds_load_f32(smem, add_byte<3>(kLnCodebook, z));
#pragma unroll
        for (int t = 0; t < 4; ++t) bq[4 * h + t][p] = pack_half2_rne(sc * q[2 * t], sc * q[2 * t + 1]);
      }
    }
    // register-decoded rows: 27 VALU per code dword
#pragma unroll
    for (int p = LR; p < TR; ++p) {
      uint32_t b0[4], b1[4];
      decode_planes(d.x[p][0], pl[p], ph[p], m55, b0);
      decode_planes(d.x[p][1], pl[p], ph[p], m55, b1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bq[t][p] = b0[t];
        bq[4 + t][p] = b1[t];
      }
    }
#pragma unroll
    for (int p = 0; p < LR; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) bq[4 * h + t][p] = lk[p][h][2 * t] | (lk[p][h][2 * t + 1] << 16);
    // grad_out -> the even and odd A operands (rows past the chunk give 0)
    u32x4 ae, ao;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float v = (nl + p < ne) ? d.a[p] : 0.f;
      ae[p] = pack_half2_rne(v, 0.f);
      ao[p] = pack_half2_rne(0.f, v);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 b = {bq[t][0], bq[t][1], bq[t][2], bq[t][3]};
      acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(ae), as_half8(b), acc[t][0], 0, 0, 0);
      acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(ao), as_half8(b), acc[t][1], 0, 0, 0);
    }
  };

  // Wave w takes k-steps w, w + 8, ... (cnt of them).  Step i's loads are
  // issued kLnDepth steps earlier and its tables built at the end of step
  // i - 1, both in rings of kLnRing buffers; the counted loop's body is one
  // ring turn with no branch inside, so every buffer index is a constant and
  // the wait counts at the loop head are the steady state's.  The tail (fewer
  // than kLnRing steps) runs the same step bodies under a wave-uniform test.
  if (cnt > 0) {
    Step sb[kLnRing];
    // (issued in step order, as the loop issues them, so the wait counts at the
    // loop head are the same on entry as on the back edge)
    for_each_index(std::make_integer_sequence<int, kLnDepth>{}, [&](auto uc) {
      load_step(decltype(uc)::value, sb[decltype(uc)::value]);
      __builtin_amdgcn_sched_barrier(0);
    });
    build_tables(0, sb[0], 0u);
    __builtin_amdgcn_sched_barrier(0);
    auto body = [&](int i, auto uc) {
      constexpr int u = decltype(uc)::value;
      load_step(i + kLnDepth, sb[(u + kLnDepth) % kLnRing]);
      __builtin_amdgcn_sched_barrier(0);
      run_step(i, sb[u], (uint32_t)u * kLnTabStep);
      NF4_WAVE_DRAIN();  // race-check build: the step's table reads complete before the next build
      build_tables(i + 1, sb[(u + 1) % kLnRing], (uint32_t)((u + 1) % kLnRing) * kLnTabStep);
      NF4_WAVE_DRAIN();
      __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + kLnRing <= cnt; i += kLnRing)
      for_each_index(std::make_integer_sequence<int, kLnRing>{}, [&](auto uc) { body(i + decltype(uc)::value, uc); });
    for_each_index(std::make_integer_sequence<int, kLnRing - 1>{}, [&](auto uc) {
      if (i + decltype(uc)::value < cnt) body(i + decltype(uc)::value, uc);
    });
  }

  // fixed-order sum of the 8 waves: ((w0 + w1) + w2) + ... + w7
  __syncthreads();
  {
    // accumulator lane (j, q), register r of tile t, parity h: row 4q + r,
    // column 16j + 2t + h of the strip
    const int q = g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * q + r < M) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const floatx4 f = {acc[2 * v][0][r], acc[2 * v][1][r], acc[2 * v + 1][0][r], acc[2 * v + 1][1][r]};
          lds_store_u32x4(smem, (uint32_t)((wave * 16 + 4 * q + r) * kLinesBK + 16 * j + 4 * v) * 4u,
                          __builtin_bit_cast(u32x4, f));
        }
      }
    }
  }
  __syncthreads();
  const uint32_t part = 4u * (uint32_t)M * (uint32_t)K;  // bytes per partial
  constexpr int kDevice = 16;                            // buffer cache policy: sc1
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(out, (uint32_t)splits * part);
  const bool split_sum = splits > 1 && counters != nullptr;
  // 16 rows x 64 float4 of the strip: two per thread
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int f = tid + 512 * e;
    const int row = f >> 6, c4 = f & 63;
    const int col = k0 + 4 * c4;
    if (row < M && col < K) {
      floatx4 s = __builtin_bit_cast(floatx4, lds_load_u32x4(smem, (uint32_t)(row * kLinesBK + 4 * c4) * 4u));
#pragma unroll
      for (int w = 1; w < kLnWaves; ++w)
        s += __builtin_bit_cast(floatx4, lds_load_u32x4(smem, (uint32_t)((w * 16 + row) * kLinesBK + 4 * c4) * 4u));
      const uint32_t at = 4u * ((uint32_t)row * (uint32_t)K + (uint32_t)col);
      if (!split_sum)
        *reinterpret_cast<floatx4*>(reinterpret_cast<char*>(out) + (size_t)split * part + at) = s;
      else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s), rp, at, (uint32_t)split * part, kDevice);
    }
  }
  if (!split_sum) return;
  // Split reduction by the strip's last workgroup to finish (partials stored
  // and loaded with device-scope coherence; each wave's stores complete
  // before the arrival is counted).  Its outputs (M rows x 64 float4) are
  // dealt to the 512 threads; when there are fewer outputs than threads, tpo
  // threads share an output, each summing a contiguous range of splits in
  // order, and the ranges' sums are added in range order.  The order is fixed
  // by (M, splits) alone, so the result does not depend on which workgroup
  // comes last.  All of a thread's partial loads are issued before the first
  // is used (one memory round trip).  The last workgroup then resets the
  // counter.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));  // vmcnt(0): the stores are complete
  __syncthreads();
  if (tid == 0) last_in_strip = atomicAdd(&counters[kt], 1u) == (uint32_t)(splits - 1);
  __syncthreads();
  if (!last_in_strip) return;
  const int F = M * 64;  // float4 outputs of the strip
  int tpo = 1;
  while (tpo < 8 && 2 * tpo * F <= 512 && 2 * tpo <= splits) tpo *= 2;
  const int r = tid % tpo;
  const int s_begin = r * splits / tpo, s_end = (r + 1) * splits / tpo;
  for (int o0 = 0; o0 < F; o0 += 512 / tpo) {
    const int o = o0 + tid / tpo;
    const int row = o >> 6, c4 = o & 63;
    const int col = k0 + 4 * c4;
    const bool mine = o < F && col < K;
    const uint32_t at = 4u * ((uint32_t)row * (uint32_t)K + (uint32_t)col);
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
    if (mine) {
      for (int sp = s_begin; sp < s_end; sp += 16) {
        floatx4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (sp + u < s_end)
            v[u] = __builtin_bit_cast(floatx4,
                                      __builtin_amdgcn_raw_buffer_load_b128(rp, at, (uint32_t)(sp + u) * part, kDevice));
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (sp + u < s_end) t = (sp + u == s_begin) ? v[u] : t + v[u];
      }
    }
    if (tpo > 1) {
      // the ranges' sums of an output through LDS, added in range order
      lds_store_u32x4(smem, 16u * (uint32_t)tid, __builtin_bit_cast(u32x4, t));
      __syncthreads();
      if (mine && r == 0) {
#pragma unroll 1
        for (int q = 1; q < tpo; ++q) t += __builtin_bit_cast(floatx4, lds_load_u32x4(smem, 16u * (uint32_t)(tid + q)));
      }
      __syncthreads();
    }
    if (mine && r == 0) *reinterpret_cast<floatx4*>(reinterpret_cast<char*>(grad_a) + at) = t;
  }
  if (tid == 0) __hip_atomic_store(&counters[kt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int VR, int CB>
__global__ __launch_bounds__(512, 1) void grad_a_lines_kernel(const float* __restrict__ G, const float* __restrict__ S,
                                                              const uint32_t* __restrict__ C32, float* out,
                                                              float* __restrict__ grad_a,
                                                              uint32_t* __restrict__ counters, int M, int N, int K,
                                                              int n_chunk, int tiles_k, int splits) {
  lines_strip<VR, CB>(G, S, C32, out, grad_a, counters, M, N, K, n_chunk, tiles_k, splits,
                  xcd_remap(blockIdx.x, gridDim.x));
}

bool lines_kernel_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N > 0 && (N % 4) == 0 && (uint64_t)M * (uint64_t)N * 4 < (1ull << 31) &&
         (uint64_t)N * (uint64_t)K / 2 < (1ull << 31);
}

hipError_t launch_grad_a_lines(int cb, int grid, const float* grad_out, const float* scales, const uint32_t* codes,
                               float* dst, float* grad_a, uint32_t* counters, int M, int N, int K, int n_chunk,
                               int tiles_k, int splits, hipStream_t stream) {
  if (counters != nullptr && tiles_k > kWsCounters) return hipErrorInvalidValue;
#define NF4_LINES_LAUNCH(V, C)                                                                                \
  hipLaunchKernelGGL((grad_a_lines_kernel<V, C>), dim3(grid), dim3(512), 0, stream, grad_out, scales, codes, dst, \
                     grad_a, counters, M, N, K, n_chunk, tiles_k, splits)
  // variant: 0..4 = that many rows in registers (byte planes), 5 = one row
  // through the codebook (the rest 16-bit table reads)
  switch (cb) {
    case 0: NF4_LINES_LAUNCH(0, 0); break;
    case 1: NF4_LINES_LAUNCH(1, 0); break;
    case 2: NF4_LINES_LAUNCH(2, 0); break;
    case 3: NF4_LINES_LAUNCH(3, 0); break;
    case 4: NF4_LINES_LAUNCH(4, 0); break;
    case 5: NF4_LINES_LAUNCH(0, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef NF4_LINES_LAUNCH
  return hipGetLastError();
}

}  // namespace nf4
